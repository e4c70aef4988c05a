"""Pins of the oracle's e4m3 codec against things other than itself."""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _anchors():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_anchors.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()
            rows.append((int(code, 16), float(val)))
    return rows


def test_decode_anchor_values():
    for code, val in _anchors():
        got = e4m3.decode(np.array([code], np.uint8))[0]
        if np.isnan(val):
            assert np.isnan(got), hex(code)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), hex(code)


def test_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3.decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))
    assert set(np.flatnonzero(np.isnan(got)).tolist()) == {0x7F, 0xFF}


def test_encode_decode_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = e4m3.decode(codes).astype(np.float32)
    assert np.array_equal(e4m3.encode(vals), codes)


def _brute_force_encode(v: float) -> int:
    """Nearest finite magnitude by exhaustive exact search; ties to the even
    code; saturation at 448; sign kept."""
    a = Fraction(abs(v))
    sign = 0x80 if np.signbit(v) else 0
    if a >= 448:
        return 0x7E | sign
    best, bestd = None, None
    for c in range(0x7F):
        d = abs(Fraction(float(e4m3.MAGNITUDES[c])) - a)
        if bestd is None or d < bestd or (d == bestd and c % 2 == 0):
            best, bestd = c, d
    return best | sign


def test_encode_vs_brute_force_structured():
    rng = np.random.default_rng(1)
    vals = []
    # every midpoint between adjacent magnitudes, and its fp32 neighbours
    mags = e4m3.MAGNITUDES
    for c in range(0x7E):
        mid = np.float32((mags[c] + mags[c + 1]) / 2)
        vals += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))]
        vals += [np.float32(mags[c])]
    vals += [np.float32(x) for x in (448.0, 449.0, 463.99, 464.0, 465.0, 480.0, 1e4, 3e38,
                                     1e-30, 2.0 ** -10, 2.0 ** -11, 0.0)]
    vals += list(rng.uniform(-500, 500, 300).astype(np.float32))
    vals += list((rng.standard_normal(300) * 2.0 ** rng.integers(-14, 4, 300)).astype(np.float32))
    vals = np.array(vals, np.float32)
    vals = np.concatenate([vals, -vals])
    got = e4m3.encode(vals)
    want = np.array([_brute_force_encode(float(v)) for v in vals], np.uint8)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(float(vals[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


def _torch_encode(vals: np.ndarray) -> np.ndarray:
    return torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_vs_torch_exhaustive_fp32_range():
    """Every positive fp32 bit pattern from 2^-11 up to 464 (where torch's cast
    stops saturating), and their negatives, against torch's cast."""
    lo = np.float32(2.0 ** -11).view(np.uint32)
    hi = np.float32(464.0).view(np.uint32)
    step = 1 << 24
    for start in range(int(lo), int(hi) + 1, step):
        bits = np.arange(start, min(start + step, int(hi) + 1), dtype=np.uint32)
        vals = bits.view(np.float32)
        got = e4m3.encode(vals)
        want = _torch_encode(vals)
        assert np.array_equal(got, want), f"block at 0x{start:08x}"
        assert np.array_equal(e4m3.encode(-vals), want | 0x80)


def test_encode_underflow_and_zero_sign():
    tiny = np.array([0.0, -0.0, 1e-30, -1e-30, 2.0 ** -11, -(2.0 ** -11),
                     np.nextafter(np.float32(2.0 ** -10), np.float32(1))], np.float32)
    got = e4m3.encode(tiny)
    assert got.tolist() == [0x00, 0x80, 0x00, 0x80, 0x00, 0x80, 0x01]


def test_encode_saturates():
    big = np.array([448.0, 448.5, 464.0, 500.0, 1e10, 3.4e38], np.float32)
    assert e4m3.encode(big).tolist() == [0x7E] * 6
    assert e4m3.encode(-big).tolist() == [0xFE] * 6
