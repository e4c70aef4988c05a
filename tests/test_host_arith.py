"""The library's corrected-quotient routine (compiled for the host from the
same header the kernels use) against IEEE fp32 division."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_corrected_quotient_matches_ieee_division(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "div_check")
    subprocess.run([hipcc, "-x", "hip", "--offload-host-only", "-O2", "-std=c++17",
                    "-ffp-contract=off", "-I", os.path.join(ROOT, "fp8_block_scaled_rms_amd", "csrc"),
                    "-o", exe, os.path.join(ROOT, "tests", "host", "div_check.cpp")],
                   check=True, capture_output=True)
    r = subprocess.run([exe, "4"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout
    assert "mismatches 0" in r.stdout
