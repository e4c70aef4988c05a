"""W8A8 INT8: symmetric int8 activation quantizers and the per-token x
per-channel int8 GEMM.  TEST INFRASTRUCTURE ONLY.

The page "Helion can accelerate vLLM LLM inference on NVIDIA GPUs"
(aihirek.info), section "Autotuning picks the right variant", names W8A8_INT8
beside FP8_Dynamic and Block_FP8 among the quantized linear formats one GEMM
implementation serves.  The page fixes none of the arithmetic; the readings
adopted mirror the FP8 path (all in fp32 unless stated):

Quantizer, applied to a whole row (per token) or with one caller-given scale
for the whole tensor (static):
  amax  = max_i |y_i|
  scale = RN32(amax / 127)                 (IEEE fp32 division; symmetric)
  q_i   = clamp(rne(RN32(y_i / scale)), -127, 127)  as int8
  scale == 0 (all-zero row) -> q = 0.
The front ends (RMSNorm, SiLU-and-mul) are the FP8 path's (oracle.quant).

GEMM ("NT", A int8 [M,K], B int8 [N,K]):
  Y[m,n] = sA[m] * sB[n] * sum_k A[m,k] B[n,k]
The integer sum is exact (Python / numpy int64); the reference is kept in
float64.

Pins (tests/test_oracle_int8.py): the amax element maps to +-127, the
round-to-nearest error bound, power-of-two scaling invariance, sign
symmetry, zero rows, a static scale of 1 reducing to plain rounding, and the
GEMM against pure-Python integer loops on small shapes.
"""
from __future__ import annotations

import numpy as np

from . import quant

PER_TOKEN = 0
PER_TENSOR_STATIC = 2
_F127 = np.float32(127.0)


def encode(qf) -> np.ndarray:
    """fp32 quotients -> int8: round to nearest even, saturate to +-127."""
    q = np.rint(np.asarray(qf, dtype=np.float32).astype(np.float64))
    return np.clip(q, -127, 127).astype(np.int8)


def quantize_rows(y) -> tuple[np.ndarray, np.ndarray]:
    """Dynamic per-row quantization of fp32 y [M,K] -> (int8 [M,K], fp32 [M])."""
    y = np.asarray(y, dtype=np.float32)
    amax = np.max(np.abs(y), axis=-1) if y.shape[-1] else np.zeros(y.shape[:-1], np.float32)
    scale = (amax.astype(np.float32) / _F127).astype(np.float32)
    safe = np.where(scale == 0, np.float32(1.0), scale).astype(np.float32)
    qf = (y / safe[..., None]).astype(np.float32)
    q = encode(qf)
    q = np.where((scale == 0)[..., None], np.int8(0), q).astype(np.int8)
    return q, scale


def quantize_static(y, s) -> np.ndarray:
    s = np.float32(np.asarray(s, dtype=np.float32).reshape(-1)[0])
    if not (s > 0 and np.isfinite(s)):
        raise ValueError("a static scale must be positive and finite")
    with np.errstate(over="ignore"):
        qf = (np.asarray(y, dtype=np.float32) / s).astype(np.float32)
    return encode(qf)


def _rows(y, mode, scale):
    if mode == PER_TOKEN:
        return quantize_rows(y)
    if mode == PER_TENSOR_STATIC:
        s = np.float32(np.asarray(scale, dtype=np.float32).reshape(-1)[0])
        return quantize_static(y, s), np.array([s], np.float32)
    raise ValueError(f"int8 quantization supports modes 0 and 2, not {mode}")


def quantize(x_bits, mode: int, scale=None):
    """Standalone int8 quantization of a bf16 [M,K] matrix."""
    return _rows(quant._bf16_to_f32(x_bits), mode, scale)


def rmsnorm_quant(x_bits, w_bits, eps: float, mode: int, scale=None, inv_override=None):
    """Fused RMSNorm (the FP8 path's front end) + int8 quantization."""
    inv, _ = quant.rms_inv(x_bits, eps)
    if inv_override is not None:
        inv = np.asarray(inv_override, dtype=np.float32)
    return _rows(quant.rmsnorm_y(x_bits, w_bits, inv), mode, scale)


def silu_mul_quant(gate_up_bits, mode: int, scale=None):
    """Fused SiLU-and-mul (the FP8 path's front end) + int8 quantization."""
    return _rows(quant.silu_mul_y(gate_up_bits), mode, scale)


def quant_weight_per_channel(W) -> tuple[np.ndarray, np.ndarray]:
    """fp32 W [N,K] -> (int8 [N,K], fp32 scale [N]); test-setup only."""
    return quantize_rows(np.asarray(W, dtype=np.float32))


def scaled_mm(a, b, sa, sb) -> np.ndarray:
    """Y = sA sB^T * (A B^T) with the integer product exact; float64 [M,N]."""
    A = np.asarray(a, dtype=np.int8).astype(np.int64)
    B = np.asarray(b, dtype=np.int8).astype(np.int64)
    P = A @ B.T  # exact: |P| <= K * 127^2
    sa64 = np.asarray(sa, dtype=np.float32).astype(np.float64)
    sb64 = np.asarray(sb, dtype=np.float32).astype(np.float64)
    return (sa64[:, None] * sb64[None, :]) * P.astype(np.float64)
