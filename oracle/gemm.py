"""fp64 dequantized FP8 matmuls and the GEMM acceptance rule.
TEST INFRASTRUCTURE ONLY.

The two GEMMs of the page "Helion in vLLM: FP8 inference of Qwen3"
(24-ai.news, 2026-06-10), section "Kernels integrated into vLLM":
scaled_mm and scaled_mm_blockwise.  Orientation "NT" (reading adopted): the
activation A is [M,K] and the weight B is [N,K] like a linear-layer weight,
Y = A B^T.

  scaled_mm:            Y[m,n] = sA[m] * sB[n] * sum_k D(A[m,k]) D(B[n,k])
  scaled_mm_blockwise:  Y[m,n] = sum_kb sA[m,kb] * sB[n//128, kb]
                                   * sum_{k in block kb} D(A[m,k]) D(B[n,k])

D is the e4m3 decode.  Every product D(a)D(b) is an integer multiple of
2^-18 and |sum| <= K * 448^2, so each inner sum is exact in float64 for
K < 171 196 whatever the summation order; numpy's float64 matmul therefore
returns the exact integer-grid sum.  The reference is kept in float64 (not
rounded to bf16); the method reaches it up to fp32 accumulation and the bf16
output rounding, which the acceptance rule below bounds.

Acceptance (no tolerance is printed on the pages; the reading adopted):
  out finite;  ||out - ref||_F / ||ref||_F <= 4e-3;
  |out - ref| / |ref| <= 1.6e-2 wherever |ref| > 1e-2 * rms(ref).

Pins (tests/test_oracle_gemm.py): brute force with exact rational
arithmetic (fractions.Fraction) on small shapes, closed forms for one-hot and
permutation weights, and blockwise == scaled_mm when every block scale of a
row (column) is equal.
"""
from __future__ import annotations

import numpy as np

from .e4m3 import decode

GROUP = 128
REL_FRO_TOL = 4e-3
REL_ELEM_TOL = 1.6e-2
ELEM_FLOOR = 1e-2


def scaled_mm(a, b, sa, sb) -> np.ndarray:
    """Per-token x per-channel scaled FP8 GEMM in float64.

    a: e4m3 [M,K]; b: e4m3 [N,K]; sa: fp32 [M]; sb: fp32 [N] -> float64 [M,N]."""
    A = decode(a)
    B = decode(b)
    P = A @ B.T
    sa64 = np.asarray(sa, dtype=np.float32).astype(np.float64)
    sb64 = np.asarray(sb, dtype=np.float32).astype(np.float64)
    return (sa64[:, None] * sb64[None, :]) * P


def scaled_mm_blockwise(a, sa, b, sb) -> np.ndarray:
    """1x128 activation x 128x128 weight block-scaled FP8 GEMM in float64.

    a: e4m3 [M,K]; sa: fp32 [M, K/128]; b: e4m3 [N,K]; sb: fp32 [N/128, K/128]
    -> float64 [M,N].  The sum over K-blocks runs in block order."""
    a = np.asarray(a, dtype=np.uint8)
    b = np.asarray(b, dtype=np.uint8)
    M, K = a.shape
    N = b.shape[0]
    KB = K // GROUP
    sa64 = np.asarray(sa, dtype=np.float32).astype(np.float64).reshape(M, KB)
    sb64 = np.asarray(sb, dtype=np.float32).astype(np.float64).reshape(N // GROUP, KB)
    sb_rows = np.repeat(sb64, GROUP, axis=0)  # [N, KB]: scale of row n's block
    out = np.zeros((M, N), dtype=np.float64)
    for kb in range(KB):
        ks = slice(kb * GROUP, (kb + 1) * GROUP)
        P = decode(a[:, ks]) @ decode(b[:, ks]).T
        out += (sa64[:, kb][:, None] * sb_rows[:, kb][None, :]) * P
    return out


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def acceptance(out, ref) -> dict:
    """Apply the GEMM acceptance rule to out (float64 values of the bf16
    output) against the float64 reference.  Returns a dict with 'ok' and the
    measured quantities."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    res = {"ok": True, "finite": bool(np.all(np.isfinite(out)))}
    if not res["finite"]:
        res["ok"] = False
        return res
    nref = np.linalg.norm(ref)
    diff = out - ref
    res["rel_fro"] = float(np.linalg.norm(diff) / nref) if nref > 0 else float(np.linalg.norm(diff))
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    big = np.abs(ref) > ELEM_FLOOR * rms
    if np.any(big):
        res["max_rel_elem"] = float(np.max(np.abs(diff[big]) / np.abs(ref[big])))
    else:
        res["max_rel_elem"] = 0.0
    res["ok"] = res["rel_fro"] <= REL_FRO_TOL and res["max_rel_elem"] <= REL_ELEM_TOL
    return res
