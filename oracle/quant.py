"""Dynamic FP8 quantizers and their fused front ends.  TEST INFRASTRUCTURE ONLY.

Follows the kernels listed on the page "Helion in vLLM: FP8 inference of
Qwen3" (24-ai.news, 2026-06-10), section "Kernels integrated into vLLM":

  dynamic_per_token_scaled_fp8_quant, per_token_group_fp8_quant  -> quantize()
  rms_norm_dynamic_per_token_quant,  rms_norm_per_block_quant    -> rmsnorm_quant()
  silu_and_mul_dynamic_per_token_quant, silu_and_mul_per_block_quant
                                                                  -> silu_mul_quant()

"Dynamic" means the scale is computed from the data at run time.  The page
fixes neither the scale rule, the group size nor the arithmetic; the
readings adopted (all in fp32 unless stated):

Quantizer, applied to a vector y (a whole row per token, or one group of
128 consecutive elements of a row):
  amax  = max_i |y_i|                                   (exact)
  scale = RN32(amax / 448)                              (IEEE fp32 division)
  q_i   = E(RN32(y_i / scale))                          (IEEE fp32 division,
                                                         then e4m3 RNE encode)
  scale == 0 (all-zero group) -> codes are signed zeros.

RMSNorm front end, per row of length K (x and w are bf16, widened exactly):
  ss    = RN64(sum_i x_i^2)              (exactly rounded: math.fsum)
  inv   = RN32(1 / sqrt(ss/K + eps))     (every step in IEEE fp64; eps is the
                                          fp32 argument widened exactly)
  y_i   = RN32(RN32(x_i * w_i) * inv)    (x_i*w_i is exact in fp32)
No bf16 rounding of y before quantization (the fusion removes it).

SiLU-and-mul front end, per row of 2D (gate = columns [0,D), up = [D,2D)):
  y_i   = RN32(silu(g_i) * u_i),  silu correctly rounded to fp32 (oracle.silu)

Two further scale rules (same quantizer otherwise):
  power-of-two (UE8M0) scales, the format the page "Helion in vLLM: FP8
  inference of Qwen3", section "Practical limits", names as required by
  DeepGEMM on B200: scale = the smallest 2^e (e >= -127, the least UE8M0
  value) with 448 * 2^e >= amax; an all-zero group therefore gets 2^-127.
  static per-tensor scale: one caller-given scale s > 0 for the whole
  tensor, q_i = E(RN32(y_i / s)) (no amax; the encoder saturates).

Weight pre-quantization (inputs for the GEMMs, not on the hot path): the same
quantizer per output channel (a row of W) or per 128x128 block of W[N,K].

Pins (tests/test_oracle_quant.py): the amax element encodes to +-448 in
every non-zero group; the quantization error bound of a round-to-nearest
e4m3 code; power-of-two scaling invariance; sign symmetry; constant, one-hot
and all-zero rows; the division-vs-reciprocal tie vector in
tests/golden/e4m3_anchors.txt; RMSNorm closed forms (constant and one-hot
rows) and independence from the summation order.
"""
from __future__ import annotations

import math

import numpy as np

from . import e4m3
from .silu import silu_bf16

PER_TOKEN = 0
GROUP128 = 1
PER_TENSOR_STATIC = 2
PER_TOKEN_UE8M0 = 3
GROUP128_UE8M0 = 4
GROUP = 128
UE8M0_MIN_EXP = -127
_F448 = np.float32(448.0)


def _bf16_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def quantize_vectors(y) -> tuple[np.ndarray, np.ndarray]:
    """Quantize each vector along the last axis of the fp32 array y.

    Returns (codes uint8 with y's shape, scale fp32 with y.shape[:-1])."""
    y = np.asarray(y, dtype=np.float32)
    amax = np.max(np.abs(y), axis=-1) if y.shape[-1] else np.zeros(y.shape[:-1], np.float32)
    scale = (amax.astype(np.float32) / _F448).astype(np.float32)
    safe = np.where(scale == 0, np.float32(1.0), scale).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        qf = (y / safe[..., None]).astype(np.float32)
    codes = e4m3.encode(qf)
    zero_group = (scale == 0)[..., None]
    signed_zero = np.where(np.signbit(y), np.uint8(0x80), np.uint8(0x00))
    codes = np.where(zero_group, signed_zero, codes).astype(np.uint8)
    return codes, scale


def ue8m0_scale(amax) -> np.ndarray:
    """Power-of-two scales: for each fp32 amax the smallest s = 2^e with
    e >= -127 and 448 * s >= amax (exact comparisons in float64)."""
    a = np.asarray(amax, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.float32)
    for idx, v in np.ndenumerate(a):
        v = float(v)
        e = UE8M0_MIN_EXP
        if v > 0.0:
            # v < 2^p; 448 * 2^(p - 12) < 2^(p - 1) <= v, so start below the answer
            e = max(UE8M0_MIN_EXP, math.frexp(v)[1] - 12)
            while math.ldexp(448.0, e) < v:
                e += 1
        out[idx] = np.float32(math.ldexp(1.0, e))
    return out


def quantize_with_scale(y, scale) -> np.ndarray:
    """q = E(RN32(y / s)) with a given positive scale s broadcast over the
    last axis of y (s has y.shape[:-1], or is a scalar)."""
    y = np.asarray(y, dtype=np.float32)
    s = np.asarray(scale, dtype=np.float32)
    with np.errstate(over="ignore"):
        qf = (y / (s[..., None] if s.ndim else s)).astype(np.float32)
    return e4m3.encode(qf)


def quantize_vectors_ue8m0(y) -> tuple[np.ndarray, np.ndarray]:
    """Like quantize_vectors, with the power-of-two scale rule."""
    y = np.asarray(y, dtype=np.float32)
    amax = np.max(np.abs(y), axis=-1) if y.shape[-1] else np.zeros(y.shape[:-1], np.float32)
    scale = ue8m0_scale(amax)
    return quantize_with_scale(y, scale), scale


def _quantize_rows(y: np.ndarray, mode: int, static_scale=None) -> tuple[np.ndarray, np.ndarray]:
    M, K = y.shape
    if mode in (PER_TOKEN, PER_TOKEN_UE8M0):
        return (quantize_vectors if mode == PER_TOKEN else quantize_vectors_ue8m0)(y)
    if mode in (GROUP128, GROUP128_UE8M0):
        if K % GROUP:
            raise ValueError("group128 quantization needs K % 128 == 0")
        fn = quantize_vectors if mode == GROUP128 else quantize_vectors_ue8m0
        codes, scale = fn(y.reshape(M, K // GROUP, GROUP))
        return codes.reshape(M, K), scale.reshape(M, K // GROUP)
    if mode == PER_TENSOR_STATIC:
        s = np.float32(np.asarray(static_scale, dtype=np.float32).reshape(-1)[0])
        if not (s > 0 and np.isfinite(s)):
            raise ValueError("a static scale must be positive and finite")
        return quantize_with_scale(y, s), np.array([s], dtype=np.float32)
    raise ValueError(f"unknown quantization mode {mode}")


def quantize(x_bits, mode: int, scale=None) -> tuple[np.ndarray, np.ndarray]:
    """Standalone quantization of a bf16 [M,K] matrix (identity front end):
    dynamic per token (scale [M]) or per 1x128 group (scale [M,K/128]), with
    IEEE or power-of-two scales, or static per tensor with the given scale."""
    return _quantize_rows(_bf16_to_f32(x_bits), mode, scale)


def rms_inv(x_bits, eps: float) -> tuple[np.ndarray, np.ndarray]:
    """Per-row inverse RMS.  Returns (inv fp32 [M], the fp64 value it was
    rounded from [M])."""
    x = _bf16_to_f32(x_bits).astype(np.float64)
    M, K = x.shape
    eps64 = float(np.float32(eps))
    inv64 = np.empty(M, dtype=np.float64)
    for m in range(M):
        ss = math.fsum((x[m] * x[m]).tolist())  # every square is exact in fp64
        t = ss / K
        t = t + eps64
        inv64[m] = 1.0 / math.sqrt(t)
    return inv64.astype(np.float32), inv64


def rmsnorm_y(x_bits, w_bits, inv) -> np.ndarray:
    """y = RN32(RN32(x*w) * inv) for bf16 x [M,K], bf16 w [K], fp32 inv [M]."""
    x = _bf16_to_f32(x_bits)
    w = _bf16_to_f32(w_bits)
    xw = (x * w[None, :]).astype(np.float32)
    return (xw * np.asarray(inv, dtype=np.float32)[:, None]).astype(np.float32)


def rmsnorm_quant(x_bits, w_bits, eps: float, mode: int,
                  inv_override=None, scale=None) -> tuple[np.ndarray, np.ndarray]:
    """Fused RMSNorm + dynamic FP8 quantization of bf16 x [M,K].

    inv_override (fp32 [M]) replaces the computed inverse RMS; it exists only
    for the rounding-tie policy of the parity tests."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    inv, _ = rms_inv(x_bits, eps)
    if inv_override is not None:
        inv = np.asarray(inv_override, dtype=np.float32)
    y = rmsnorm_y(x_bits, w_bits, inv)
    return _quantize_rows(y, mode, scale)


def silu_mul_y(gate_up_bits) -> np.ndarray:
    """y = RN32(silu(gate) * up) for bf16 gate_up [M, 2D]."""
    gu = np.asarray(gate_up_bits, dtype=np.uint16)
    M, twoD = gu.shape
    D = twoD // 2
    s = silu_bf16(gu[:, :D])
    u = _bf16_to_f32(gu[:, D:])
    return (s * u).astype(np.float32)


def silu_mul_quant(gate_up_bits, mode: int, scale=None) -> tuple[np.ndarray, np.ndarray]:
    """Fused SiLU-and-mul + FP8 quantization of bf16 gate_up [M,2D]."""
    gu = np.asarray(gate_up_bits, dtype=np.uint16)
    if gu.shape[1] % 2:
        raise ValueError("gate_up must have an even number of columns")
    return _quantize_rows(silu_mul_y(gu), mode, scale)


def quant_weight_per_channel(W) -> tuple[np.ndarray, np.ndarray]:
    """fp32 W [N,K] -> (e4m3 codes [N,K], fp32 scale [N]), one scale per row."""
    return quantize_vectors(np.asarray(W, dtype=np.float32))


def quant_weight_block128(W) -> tuple[np.ndarray, np.ndarray]:
    """fp32 W [N,K] -> (e4m3 codes [N,K], fp32 scale [N/128, K/128]), one
    scale per 128x128 block."""
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    if N % GROUP or K % GROUP:
        raise ValueError("block quantization needs N and K multiples of 128")
    blocks = W.reshape(N // GROUP, GROUP, K // GROUP, GROUP).transpose(0, 2, 1, 3)
    codes, scale = quantize_vectors(blocks.reshape(N // GROUP, K // GROUP, GROUP * GROUP))
    codes = codes.reshape(N // GROUP, K // GROUP, GROUP, GROUP).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(codes.reshape(N, K)), scale
