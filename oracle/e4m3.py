"""OCP e4m3 ("e4m3fn") codec.  TEST INFRASTRUCTURE ONLY.

The FP8 format of the path.  The page "Helion in vLLM: FP8 inference of
Qwen3" (24-ai.news), section "Kernels integrated into vLLM", names FP8
quantization kernels without fixing the format; the reading adopted is the
OCP 8-bit floating point e4m3 format (the one gfx950 implements natively):

  bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa;
  exponent 0  -> subnormal  (-1)^s * 2^-6 * m/8;
  exponent>=1 -> normal     (-1)^s * 2^(e-7) * (1 + m/8);
  0x7F and 0xFF are NaN; there is no infinity; the largest finite
  magnitude is 448 (0x7E).

Encoding (fp32 -> e4m3) rounds to nearest with ties to the even code and
saturates magnitudes >= 448 to +-448; the sign of zero and of values that
underflow is kept.

Pins (tests/test_oracle_e4m3.py): decode against torch's float8_e4m3fn
widening for all 256 codes and against hand-checked anchor values;
encode against a brute-force nearest-magnitude search, against torch's
float8_e4m3fn cast wherever that cast does not saturate to NaN, and
E(D(c)) == c for all 254 finite codes.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
NAN_CODES = (0x7F, 0xFF)


def _decode_magnitude(code7: int) -> float:
    e = (code7 >> 3) & 0xF
    m = code7 & 0x7
    if e == 0:
        return 2.0 ** -6 * (m / 8.0)
    return 2.0 ** (e - 7) * (1.0 + m / 8.0)


# The 127 finite non-negative magnitudes, index == code (0x00 .. 0x7E).
# They increase strictly with the code.
MAGNITUDES = np.array([_decode_magnitude(c) for c in range(0x7F)], dtype=np.float64)


def decode(codes) -> np.ndarray:
    """e4m3 bytes -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8)
    mag7 = (c & 0x7F).astype(np.int64)
    table = np.append(MAGNITUDES, np.nan)  # index 0x7F -> NaN
    v = table[mag7]
    return np.where((c & 0x80) != 0, -v, v)


def encode(values) -> np.ndarray:
    """fp32 values -> e4m3 bytes (RNE, ties to the even code, saturating).

    NaN inputs are outside the contract of the path; they map to 0x7F."""
    v = np.asarray(values, dtype=np.float32)
    sign = np.signbit(v)
    a = np.abs(v.astype(np.float64))  # exact
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    # first code whose magnitude is >= a
    hi = np.searchsorted(MAGNITUDES, a, side="left")
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    mlo = MAGNITUDES[lo]
    mhi = MAGNITUDES[hi]
    # compare 2a with mlo + mhi: both sides are exact in float64
    twice = 2.0 * a
    mid = mlo + mhi
    pick_hi = twice > mid
    tie = twice == mid
    pick_hi = np.where(tie, (hi & 1) == 0, pick_hi)
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == mhi, hi, code)  # exactly representable
    code = np.where(a >= E4M3_MAX, 0x7E, code)  # saturate
    code = code.astype(np.uint8) | np.where(sign, 0x80, 0).astype(np.uint8)
    return np.where(nan, np.uint8(0x7F), code).astype(np.uint8)
