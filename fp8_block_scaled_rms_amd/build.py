"""Build libfp8q.so (HIP for gfx950) in-tree.

    python -m fp8_block_scaled_rms_amd.build          # or build() from Python

Steps: compile and run the SiLU table generator (host C++), compile the HIP
and C++ sources with hipcc for gfx950 in parallel, link the shared library
next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfp8q.so")

SOURCES = ["quant_kernels.hip", "gemm_kernels.hip", "probe_kernels.hip", "dispatch.cpp",
           "api.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # bit-exact quantization: no FMA contraction, IEEE fp32 division and sqrt
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
    # no packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: the blockwise scale FMA reads them
    # directly instead of copying each one out of the accumulation registers
    "-mllvm", "-amdgpu-mfma-vgpr-form=true",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", INCLUDE, "-I", CSRC, "-I", BUILD,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, cwd=None):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       cwd=cwd)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    return r.stdout


_M0_WORD = re.compile(r"\bm0\b")


def check_m0(asm_path: str) -> None:
    """The GEMM kernels write M0 from inline assembly (the LDS address of a
    direct global->LDS load) without the compiler knowing.  That is safe only
    while the compiler itself never keeps a value in M0: every instruction of
    the generated assembly that names M0 must be one of those writes, each
    followed by the wait state and the LDS-DMA load that reads it."""
    with open(asm_path) as f:
        lines = [ln.split(";")[0].strip() for ln in f]
    for i, ln in enumerate(lines):
        if not _M0_WORD.search(ln):
            continue
        ok = (re.fullmatch(r"s_mov_b32 m0, s\d+", ln) is not None and i + 2 < len(lines)
              and lines[i + 1] == "s_nop 0" and lines[i + 2].startswith("global_load_lds_dword"))
        if not ok:
            raise RuntimeError(f"{asm_path}:{i + 1}: unexpected use of M0: {ln!r}")


def build(verbose: bool = False, jobs: int = 4) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    # 1. SiLU table, generated on the host
    gen = os.path.join(BUILD, "gen_silu_table")
    _run(["g++", "-O2", "-std=c++17", "-o", gen, os.path.join(CSRC, "gen_silu_table.cpp")])
    _run([gen, os.path.join(BUILD, "silu_table.inc")])
    # 2. objects
    objs = []

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        # -save-temps keeps the gfx950 assembly next to the object (checked below)
        cmd = [hipcc, *HIPCC_FLAGS, "-save-temps", "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        out = _run(cmd, cwd=BUILD)
        if verbose and out.strip():
            print(out)
        return obj

    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    for src in SOURCES:
        check_m0(os.path.join(BUILD, os.path.splitext(src)[0] + "-hip-amdgcn-amd-amdhsa-gfx950.s"))
    # 3. link (write to a temp name, then rename: a loaded library is not
    #    clobbered in place)
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
