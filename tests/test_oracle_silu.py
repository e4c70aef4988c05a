"""Pins of the oracle's correctly rounded SiLU table."""
import math

import numpy as np

from oracle import silu


def _gates():
    return (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)


def test_table_matches_float64_evaluation():
    """numpy's float64 evaluation, rounded once to fp32, agrees on every finite
    gate with |g| < 200 (its error is ~1e-16, far from every fp32 midpoint)."""
    g = _gates()
    t = silu.silu_table()
    fin = np.isfinite(g) & (np.abs(g) < 200)
    g64 = g[fin].astype(np.float64)
    ref = (g64 / (1.0 + np.exp(-g64))).astype(np.float32)
    assert np.array_equal(t[fin].view(np.uint32), ref.view(np.uint32))


def test_fixed_points_and_limits():
    g = _gates()
    t = silu.silu_table()
    fin = np.isfinite(g)
    big = fin & (g >= 16.75)
    assert np.array_equal(t[big], g[big])
    # just below the threshold the deficit exceeds half an ulp
    b = np.float32(16.5)
    assert t[b.view(np.uint32) >> 16] < b
    tiny = fin & (np.abs(g) < 2.0 ** -24)
    assert np.array_equal(t[tiny], (g[tiny] * np.float32(0.5)).astype(np.float32))
    assert np.array_equal(np.signbit(t[tiny]), np.signbit(g[tiny]))
    neg = fin & (g <= -128)
    assert np.all(t[neg] == 0) and np.all(np.signbit(t[neg]))
    assert t[0x0000] == 0 and not np.signbit(t[0x0000])
    assert t[0x8000] == 0 and np.signbit(t[0x8000])


def test_reflection_identity():
    """silu(g) - silu(-g) = g exactly; the rounded table satisfies it to within
    one fp32 ulp of the larger term."""
    g = _gates()[:0x7F80]  # positive finite gates
    t = silu.silu_table()
    pos = t[np.arange(0x7F80)].astype(np.float64)
    neg = t[np.arange(0x7F80) | 0x8000].astype(np.float64)
    lhs = pos - neg
    ulp = np.spacing(np.maximum(np.abs(pos), np.abs(neg)).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(lhs - g.astype(np.float64)) <= ulp)


def test_spot_values_against_math():
    for v in (1.0, -1.0, 0.5, 3.0, -2.75, 10.0, -20.0):
        b = np.float32(v).view(np.uint32) >> 16
        want = np.float32(v / (1.0 + math.exp(-v)))
        assert silu.silu_bf16(np.array([b], np.uint16))[0] == want
