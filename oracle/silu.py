"""Correctly rounded fp32 SiLU over every bf16 input.  TEST INFRASTRUCTURE ONLY.

SiLU feeds the fused SiLU-and-mul quantizers (page "Helion in vLLM: FP8
inference of Qwen3", 24-ai.news, section "Kernels integrated into vLLM":
silu_and_mul_dynamic_per_token_quant and silu_and_mul_per_block_quant).
The page does not fix how SiLU is rounded.  Reading adopted: the fp32 value
of silu(g) = g / (1 + exp(-g)) is the correctly rounded one (round to
nearest even) of the exact real value, for every bf16 gate g.  Since a bf16
gate has only 65 536 bit patterns, the oracle tabulates all of them.

Method: each finite gate is evaluated in decimal arithmetic with 60
significant digits, then rounded to fp32 by comparing the decimal value with
the exact midpoint of its two fp32 neighbours (no intermediate binary
rounding, hence no double rounding).  Two ranges are closed analytically:

* g > 200:  exp(-g) < 2^-288, so silu(g) = g (1 - d) with d far below half
  an fp32 ulp and the correctly rounded value is g itself;
* g < -200: |silu(g)| < 200 e^-200 < 2^-280, far below half the smallest
  fp32 subnormal, so the correctly rounded value is -0.0.

silu(+-0) = +-0.  Non-finite gates are outside the contract of the path:
+inf -> +inf, -inf -> -0.0, NaN -> NaN.

Pins (tests/test_oracle_silu.py): agreement with numpy's float64
exp-based evaluation rounded to fp32 on every finite gate with |g| < 200,
the fixed point silu(g) = g for large positive g, silu(g) = g/2 for tiny g,
the reflection identity silu(g) - silu(-g) = g within rounding, and a
handful of values checked against Python's float64 math.
"""
from __future__ import annotations

import decimal
import functools

import numpy as np

_CTX = decimal.Context(prec=60, Emin=-999999, Emax=999999)


def _round_decimal_to_f32(v: decimal.Decimal) -> np.float32:
    """Correctly round a (non-zero, finite) decimal value to fp32."""
    f = np.float32(float(v))  # within a couple of ulp of the answer
    # walk to the pair of adjacent fp32 values bracketing v
    lo = f
    while decimal.Decimal(float(lo)) > v:
        lo = np.nextafter(lo, np.float32(-np.inf))
    hi = np.nextafter(lo, np.float32(np.inf))
    while decimal.Decimal(float(hi)) < v:
        lo = hi
        hi = np.nextafter(lo, np.float32(np.inf))
    dlo = decimal.Decimal(float(lo))
    dhi = decimal.Decimal(float(hi))
    if dlo == v:
        return lo
    if dhi == v:
        return hi
    mid = _CTX.divide(_CTX.add(dlo, dhi), decimal.Decimal(2))
    # the exact value of silu at a non-zero rational point is irrational, so a
    # true tie cannot occur; refuse if 60 digits cannot tell the two apart
    gap = abs(_CTX.subtract(v, mid))
    if gap <= abs(v) * decimal.Decimal("1e-50"):
        raise ArithmeticError("SiLU value too close to an fp32 midpoint")
    if v < mid:
        return lo
    return hi


def silu_exact_f32(g: float) -> np.float32:
    """Correctly rounded fp32 silu(g) for one float value g (exact in fp32)."""
    if np.isnan(g):
        return np.float32(np.nan)
    if g == 0.0:
        return np.float32(g)  # keeps the sign of zero
    if np.isinf(g):
        return np.float32(np.inf) if g > 0 else np.float32(-0.0)
    if g > 200.0:
        return np.float32(g)
    if g < -200.0:
        return np.float32(-0.0)
    d = decimal.Decimal(float(g))  # exact
    e = _CTX.exp(_CTX.minus(d))
    v = _CTX.divide(d, _CTX.add(decimal.Decimal(1), e))
    return _round_decimal_to_f32(v)


@functools.lru_cache(maxsize=1)
def silu_table() -> np.ndarray:
    """fp32 [65536]: entry b is the correctly rounded silu of the bf16 gate
    whose bit pattern is b."""
    out = np.empty(65536, dtype=np.float32)
    gates = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    for b in range(65536):
        out[b] = silu_exact_f32(float(gates[b]))
    out.setflags(write=False)
    return out


def silu_bf16(gate_bits) -> np.ndarray:
    """Correctly rounded fp32 SiLU of bf16 gates given as uint16 bit patterns."""
    return silu_table()[np.asarray(gate_bits, dtype=np.uint16)]
