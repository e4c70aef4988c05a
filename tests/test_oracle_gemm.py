"""Pins of the oracle's fp64 GEMMs against exact rational arithmetic and
closed forms, and checks of the acceptance rule."""
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import e4m3, gemm


def _fraction_decode(c: int) -> Fraction:
    """e4m3 decode in exact rational arithmetic, written from the format
    definition independently of oracle.e4m3."""
    s = -1 if c & 0x80 else 1
    e = (c >> 3) & 0xF
    m = c & 7
    if e == 0:
        return s * Fraction(m, 8) * Fraction(1, 64)
    return s * (1 + Fraction(m, 8)) * (Fraction(2) ** (e - 7))


def _rand_case(M, N, K, tag):
    rng = synth.rng_for("t", "gemm", tag, M, N, K)
    a = synth.gen_e4m3_codes(rng, (M, K))
    b = synth.gen_e4m3_codes(rng, (N, K))
    return rng, a, b


@pytest.mark.parametrize("M,N,K", [(3, 5, 128), (2, 3, 256)])
def test_scaled_mm_vs_fractions(M, N, K):
    rng, a, b = _rand_case(M, N, K, "mm")
    sa = synth.gen_scales(rng, M)
    sb = synth.gen_scales(rng, N)
    ref = gemm.scaled_mm(a, b, sa, sb)
    for m in range(M):
        for n in range(N):
            p = sum(_fraction_decode(int(a[m, k])) * _fraction_decode(int(b[n, k])) for k in range(K))
            exact = Fraction(float(sa[m])) * Fraction(float(sb[n])) * p
            assert abs(Fraction(ref[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 50)


@pytest.mark.parametrize("M,N,K", [(2, 128, 256), (3, 256, 384)])
def test_blockwise_vs_fractions(M, N, K):
    rng, a, b = _rand_case(M, N, K, "bw")
    sa = synth.gen_scales(rng, (M, K // 128))
    sb = synth.gen_scales(rng, (N // 128, K // 128))
    ref = gemm.scaled_mm_blockwise(a, sa, b, sb)
    for m in range(M):
        for n in list(range(0, N, 37)) + [N - 1]:
            exact = Fraction(0)
            for kb in range(K // 128):
                p = sum(_fraction_decode(int(a[m, k])) * _fraction_decode(int(b[n, k]))
                        for k in range(kb * 128, (kb + 1) * 128))
                exact += Fraction(float(sa[m, kb])) * Fraction(float(sb[n // 128, kb])) * p
            tol = Fraction(1, 2 ** 48) * max(abs(exact), Fraction(1, 2 ** 60))
            assert abs(Fraction(ref[m, n]) - exact) <= tol


def test_one_hot_weights_closed_form():
    """B row n holds a single 1.0 (code 0x38) at column perm[n]:
    Y[m,n] = sA[m] sB[n] D(A[m, perm[n]]) (scaled_mm) and
    Y[m,n] = sA[m, kb] sB[n//128, kb] D(A[m, j]), j = perm[n], kb = j//128."""
    M, N, K = 7, 256, 384
    rng, a, _ = _rand_case(M, N, K, "onehot")
    perm = rng.permutation(K)[:N]
    b = np.zeros((N, K), np.uint8)
    b[np.arange(N), perm] = 0x38
    sa = synth.gen_scales(rng, M)
    sb = synth.gen_scales(rng, N)
    y = gemm.scaled_mm(a, b, sa, sb)
    A = e4m3.decode(a)
    want = sa.astype(np.float64)[:, None] * sb.astype(np.float64)[None, :] * A[:, perm]
    assert np.array_equal(y, want)
    sab = synth.gen_scales(rng, (M, K // 128))
    sbb = synth.gen_scales(rng, (N // 128, K // 128))
    yb = gemm.scaled_mm_blockwise(a, sab, b, sbb)
    kb = perm // 128
    want_b = (sab.astype(np.float64)[:, kb] * sbb.astype(np.float64)[np.arange(N) // 128, kb][None, :]
              * A[:, perm])
    assert np.array_equal(yb, want_b)


def test_blockwise_with_uniform_block_scales_equals_scaled_mm():
    M, N, K = 5, 256, 512
    rng, a, b = _rand_case(M, N, K, "uni")
    sa = synth.gen_scales(rng, M)
    sb = synth.gen_scales(rng, N // 128)
    y = gemm.scaled_mm(a, b, sa, np.repeat(sb, 128))
    yb = gemm.scaled_mm_blockwise(a, np.repeat(sa[:, None], K // 128, axis=1), b,
                                  np.repeat(sb[:, None], K // 128, axis=1))
    # per-block rounding of the fp64 sums: bound by the magnitude of the terms
    mag = (sa.astype(np.float64)[:, None] * np.repeat(sb, 128).astype(np.float64)[None, :]
           * (np.abs(e4m3.decode(a)) @ np.abs(e4m3.decode(b)).T))
    assert np.all(np.abs(y - yb) <= 1e-14 * mag)


def _bf16_round(x64):
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x64.astype(np.float32))).astype(np.float64)


def test_acceptance_rule():
    rng, a, b = _rand_case(16, 256, 512, "acc")
    sa = synth.gen_scales(rng, 16)
    sb = synth.gen_scales(rng, 256)
    ref = gemm.scaled_mm(a, b, sa, sb)
    assert gemm.acceptance(_bf16_round(ref), ref)["ok"]
    bad = _bf16_round(ref)
    i = np.unravel_index(np.argmax(np.abs(ref)), ref.shape)
    bad[i] *= 1.05
    assert not gemm.acceptance(bad, ref)["ok"]
    perm = _bf16_round(ref)[:, ::-1]
    assert not gemm.acceptance(perm, ref)["ok"]
    nan = _bf16_round(ref)
    nan[0, 0] = np.nan
    assert not gemm.acceptance(nan, ref)["ok"]
