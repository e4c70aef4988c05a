"""Host sanitizer build of the C ABI layer (CPU only).

api.cpp (argument checks, dispatch into the launchers) and dispatch.cpp (the
per-shape table) are compiled with AddressSanitizer and UndefinedBehavior-
Sanitizer on their host code, linked with the ordinary kernel objects into
a separate library, and the CPU tests of the interface (test_abi,
test_binding, test_bench_coverage) run against it in a child process with
the sanitizer runtime preloaded.  Any sanitizer report fails the test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from fp8_block_scaled_rms_amd import build as b  # noqa: E402

OUT = os.path.join(b.BUILD, "asan")
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host",
                 "-fno-omit-frame-pointer"]
# the ordinary build's objects of every HIP source (kernels and their launchers)
KERNEL_OBJECTS = [src.replace(".hip", ".o") for src in b.SOURCES if src.endswith(".hip")]


def _asan_runtime(hipcc):
    r = subprocess.run([hipcc, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       stdout=subprocess.PIPE, text=True, check=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_abi_layer_under_asan_and_ubsan():
    hipcc = b._hipcc()
    runtime = _asan_runtime(hipcc)
    if runtime is None:
        pytest.skip("no AddressSanitizer runtime next to hipcc")
    for o in KERNEL_OBJECTS:
        if not os.path.exists(os.path.join(b.BUILD, o)):
            pytest.skip("the library has not been built (python -m fp8_block_scaled_rms_amd.build)")
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for src in ("api.cpp", "dispatch.cpp"):
        obj = os.path.join(OUT, src.replace(".cpp", ".o"))
        flags = [f for f in b.HIPCC_FLAGS]
        subprocess.run([hipcc, "-x", "hip", *flags, *HOST_SANITIZE, "-c",
                        os.path.join(b.CSRC, src), "-o", obj], check=True,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        objs.append(obj)
    lib = os.path.join(OUT, "libfp8q_asan.so")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, *objs,
                    *[os.path.join(b.BUILD, o) for o in KERNEL_OBJECTS]], check=True,
                   stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    env = dict(os.environ)
    env.update({"FP8Q_LIB": lib, "LD_PRELOAD": runtime,
                "ASAN_OPTIONS": "detect_leaks=0:detect_odr_violation=0:halt_on_error=1",
                "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})
    tests = [os.path.join(ROOT, "tests", t) for t in
             ("test_abi.py", "test_binding.py", "test_bench_coverage.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider", *tests], cwd=ROOT, env=env,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    out = r.stdout
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    # the child really loaded the sanitized library
    assert "passed" in out
