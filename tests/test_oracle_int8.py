"""Pins of the W8A8 INT8 oracle against closed forms, invariants and
pure-Python integer arithmetic."""
import numpy as np
import pytest

import synth
from oracle import int8, quant


def _rows(seed=0, n=300, L=512):
    rng = np.random.default_rng(seed)
    p = rng.integers(-20, 20, size=(n, 1)).astype(np.float32)
    y = rng.standard_normal((n, L)).astype(np.float32) * np.exp2(p)
    y[::5, rng.integers(0, L)] *= 20
    return y.astype(np.float32)


def test_amax_element_maps_to_127():
    y = _rows()
    q, s = int8.quantize_rows(y)
    r = np.arange(len(y))
    idx = np.argmax(np.abs(y), axis=1)
    assert np.array_equal(q[r, idx], np.where(y[r, idx] < 0, -127, 127).astype(np.int8))
    assert q.min() >= -127


def test_round_to_nearest_error_bound():
    y = _rows(1)
    q, s = int8.quantize_rows(y)
    err = np.abs(q.astype(np.float64) * s.astype(np.float64)[:, None] - y.astype(np.float64))
    assert np.all(err <= 0.5 * s.astype(np.float64)[:, None] * (1 + 2.0 ** -20))


def test_ties_round_to_even_and_saturate():
    # static scale 1: the quotient is the value itself
    y = np.array([[0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, 127.49, 300.0, -1e30]], np.float32)
    q = int8.quantize_static(y, np.float32(1.0))
    assert list(q[0]) == [0, 2, 2, 0, -2, -2, 126, 127, 127, -127]


def test_scaling_invariance_sign_and_zero_rows():
    y = _rows(2)
    q0, s0 = int8.quantize_rows(y)
    q1, s1 = int8.quantize_rows((y * np.float32(2.0 ** 7)).astype(np.float32))
    assert np.array_equal(q0, q1) and np.array_equal(s1, s0 * np.float32(128))
    q2, s2 = int8.quantize_rows(-y)
    assert np.array_equal(q2, -q0) and np.array_equal(s2, s0)
    z = np.zeros((2, 64), np.float32)
    z[1, ::2] = -0.0
    qz, sz = int8.quantize_rows(z)
    assert np.all(qz == 0) and np.all(sz == 0)


def test_scale_is_amax_over_127_ieee():
    y = _rows(3)
    _, s = int8.quantize_rows(y)
    amax = np.max(np.abs(y.astype(np.float64)), axis=1)
    assert np.all(np.abs(s.astype(np.float64) - amax / 127.0)
                  <= 0.5 * np.spacing(s).astype(np.float64))


def test_fused_front_ends_reuse_the_fp8_path_values():
    rng = synth.rng_for("int8-fused", 6, 256)
    x = synth.gen_activations(rng, 6, 256)
    w = synth.gen_rms_weight(rng, 256)
    inv, _ = quant.rms_inv(x, 1e-6)
    y = quant.rmsnorm_y(x, w, inv)
    q, s = int8.rmsnorm_quant(x, w, 1e-6, int8.PER_TOKEN)
    q2, s2 = int8.quantize_rows(y)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    gu = synth.gen_gate_up(rng, 6, 128)
    q3, _ = int8.silu_mul_quant(gu, int8.PER_TENSOR_STATIC, scale=np.float32(0.25))
    assert np.array_equal(q3, int8.encode((quant.silu_mul_y(gu) / np.float32(0.25))
                                          .astype(np.float32)))
    with pytest.raises(ValueError):
        int8.quantize(x, 1)


def test_gemm_against_python_integer_loops():
    rng = np.random.default_rng(7)
    M, N, K = 5, 7, 96
    a = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    b = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    sa = rng.random(M).astype(np.float32) + 0.5
    sb = rng.random(N).astype(np.float32) * 1e-3
    ref = int8.scaled_mm(a, b, sa, sb)
    for m in range(M):
        for n in range(N):
            p = sum(int(a[m, k]) * int(b[n, k]) for k in range(K))
            assert ref[m, n] == float(sa[m]) * float(sb[n]) * p


def test_gemm_extreme_accumulation_is_exact():
    # all +-127: |P| = K * 127^2 must not lose a unit
    K = 8192
    a = np.full((2, K), 127, np.int8)
    a[1] = -127
    b = np.full((3, K), -127, np.int8)
    b[2, ::2] = 127
    ref = int8.scaled_mm(a, b, np.ones(2, np.float32), np.ones(3, np.float32))
    assert ref[0, 0] == -K * 127 * 127 and ref[1, 0] == K * 127 * 127 and ref[0, 2] == 0
