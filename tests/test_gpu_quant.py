"""GPU parity of the quantizers against the CPU oracle: bytes and scales must
be bit-identical.  Inputs are the seeded synthetic Qwen3-shaped workloads
(synth) plus edge cases.

Rounding-tie policy for RMSNorm (the only place two results can be right):
the GPU sums squares in fp64 in a different order than the oracle's exactly
rounded sum, so its fp32 inverse RMS may land on the other fp32 neighbour
when the fp64 value lies within 2^-40 (relative) of an fp32 midpoint.  Such a
row is accepted only if the oracle, re-run with that other neighbour, then
matches bit for bit.
"""
import numpy as np
import pytest
import torch

import fp8_block_scaled_rms_amd as fq
import synth
from oracle import e4m3, quant, silu
from gpu_util import DEV, bf16_dev, f32_dev, host, say

pytestmark = pytest.mark.gpu

EPS = 1e-6


def _rows_sample(M, n=192):
    if M <= n:
        return np.arange(M)
    rng = np.random.default_rng(M)
    rest = rng.choice(np.arange(1, M - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, M - 1], rest]))


def _static(scale):
    return None if scale is None else f32_dev(np.array([scale], np.float32))


def _check_rms(x, w, mode, rows=None, eps=EPS, scale=None):
    M, K = x.shape
    q, s = fq.rmsnorm_quant(bf16_dev(x), bf16_dev(w), eps, mode, scale=_static(scale))
    torch.cuda.synchronize()
    return compare_rms(host(q), host(s), x, w, mode, rows, eps, scale)


def compare_rms(q, s, x, w, mode, rows=None, eps=EPS, scale=None):
    """GPU outputs q, s (host arrays, all M rows) of rmsnorm_quant(x, w)
    against the oracle on `rows` (default all), with the tie policy above.
    Returns the number of rows accepted under the policy."""
    M, K = x.shape
    rows = np.arange(M) if rows is None else rows
    qr, sr = quant.rmsnorm_quant(x[rows], w, eps, mode, scale=scale)
    if mode == fq.PER_TENSOR_STATIC:  # the scale is an input: one value, all rows
        s = np.repeat(s, M)
        sr = np.repeat(sr, len(rows))
    qg, sg = q[rows], s[rows]
    bad = [i for i in range(len(rows))
           if not (np.array_equal(qg[i], qr[i]) and np.array_equal(sg[i].view(np.uint32),
                                                                    sr[i].view(np.uint32)))]
    if bad:
        inv32, inv64 = quant.rms_inv(x[rows][bad], eps)
        for j, i in enumerate(bad):
            lo = np.float32(inv64[j])
            other = np.nextafter(lo, np.float32(np.inf) if inv64[j] > lo else np.float32(0))
            mid = (float(lo) + float(other)) / 2
            assert abs(inv64[j] - mid) <= 2.0 ** -40 * inv64[j], f"row {rows[i]} differs"
            q2, s2 = quant.rmsnorm_quant(x[rows[i]:rows[i] + 1], w, eps, mode,
                                         inv_override=np.array([other], np.float32),
                                         scale=scale)
            assert np.array_equal(qg[i], q2[0]) and np.array_equal(sg[i], s2[0]), f"row {rows[i]}"
    return len(bad)


RMS_CASES = [
    # (name, M, K, mode)
    ("c1-tiny-group", 16, 256, fq.GROUP128),
    ("c2-per-token", 1, 2048, fq.PER_TOKEN),
    ("c2-per-token", 16, 2048, fq.PER_TOKEN),
    ("c2-per-token", 128, 2048, fq.PER_TOKEN),
    ("c2-per-token", 2048, 2048, fq.PER_TOKEN),
    ("c3-group", 1, 4096, fq.GROUP128),
    ("c3-group", 32, 4096, fq.GROUP128),
    ("c4-group", 2048, 5120, fq.GROUP128),
    ("ragged", 37, 5120, fq.PER_TOKEN),
    ("ragged", 3, 8, fq.PER_TOKEN),
    ("ragged", 5, 128, fq.GROUP128),
    ("ragged", 7, 2056, fq.PER_TOKEN),
    ("max-k", 4, 32768, fq.PER_TOKEN),
    ("max-k", 4, 32768, fq.GROUP128),
]


@pytest.mark.parametrize("name,M,K,mode", RMS_CASES)
def test_rmsnorm_quant_parity(name, M, K, mode):
    say("rmsnorm_quant", name, M, K, mode)
    rng = synth.rng_for(name, "rmsnorm_quant", M, K)
    x = synth.gen_activations(rng, M, K)
    w = synth.gen_rms_weight(rng, K)
    _check_rms(x, w, mode)


@pytest.mark.parametrize("mode", [fq.PER_TOKEN, fq.GROUP128])
def test_rmsnorm_quant_full_size_sampled(mode):
    """Qwen3-32B prefill size (M=8192, K=5120), in the bench's launch
    configuration; 192 sampled rows compared with the oracle."""
    M, K = 8192, 5120
    say("rmsnorm_quant sampled", M, K, mode)
    rng = synth.rng_for("c4-group", "rmsnorm_quant", M, K)
    x = synth.gen_activations(rng, M, K)
    w = synth.gen_rms_weight(rng, K)
    _check_rms(x, w, mode, rows=_rows_sample(M))


def test_rmsnorm_quant_edge_rows():
    K = 256
    rng = synth.rng_for("edge", "rmsnorm_quant", K)
    w = synth.gen_rms_weight(rng, K)
    rows = []
    rows.append(np.zeros(K, np.float32))                          # all zero
    z = np.zeros(K, np.float32); z[::3] = -0.0; rows.append(z)     # signed zeros
    rows.append(np.full(K, 0.75, np.float32))                     # constant
    rows.append(np.full(K, -3.0e-30, np.float32))                 # tiny scale path
    t = np.zeros(K, np.float32); t[5] = 1e-35; rows.append(t)     # one tiny element
    rows.append(np.full(K, 1.0e30, np.float32))                   # huge values
    h = rng.standard_normal(K).astype(np.float32); h[:128] = 0; rows.append(h)  # zero group
    o = np.zeros(K, np.float32); o[200] = -5.0; rows.append(o)    # one-hot
    x = synth.f32_to_bf16_bits(np.stack(rows))
    for mode in (fq.PER_TOKEN, fq.GROUP128):
        say("rmsnorm_quant edge", mode)
        _check_rms(x, w, mode)
        _check_rms(x, w, mode, eps=1e-30)


def _check_silu(gu, mode, rows=None, scale=None):
    M, twoD = gu.shape
    q, s = fq.silu_mul_quant(bf16_dev(gu), mode, scale=_static(scale))
    torch.cuda.synchronize()
    q, s = host(q), host(s)
    rows = np.arange(M) if rows is None else rows
    qr, sr = quant.silu_mul_quant(gu[rows], mode, scale=scale)
    assert np.array_equal(q[rows], qr)
    if mode == fq.PER_TENSOR_STATIC:
        assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))
    else:
        assert np.array_equal(s[rows].view(np.uint32), sr.view(np.uint32))


SILU_CASES = [
    ("c2-per-token", 1, 6144, fq.PER_TOKEN),
    ("c2-per-token", 16, 6144, fq.PER_TOKEN),
    ("c2-per-token", 128, 6144, fq.PER_TOKEN),
    ("c3-group", 1, 12288, fq.GROUP128),
    ("c3-group", 32, 12288, fq.GROUP128),
    ("c5-group", 64, 25600, fq.GROUP128),
    ("ragged", 9, 1000, fq.PER_TOKEN),
    ("ragged", 3, 384, fq.GROUP128),
    ("max-k", 2, 32768, fq.PER_TOKEN),
]


@pytest.mark.parametrize("name,M,D,mode", SILU_CASES)
def test_silu_mul_quant_parity(name, M, D, mode):
    say("silu_mul_quant", name, M, D, mode)
    rng = synth.rng_for(name, "silu_mul_quant", M, D)
    gu = synth.gen_gate_up(rng, M, D)
    _check_silu(gu, mode)


def test_silu_mul_quant_full_size_sampled():
    """Qwen3-32B MLP tail at M=4096, D=25600; sampled rows."""
    M, D = 4096, 25600
    say("silu_mul_quant sampled", M, D)
    rng = synth.rng_for("c5-group", "silu_mul_quant", M, D)
    gu = synth.gen_gate_up(rng, M, D)
    _check_silu(gu, fq.GROUP128, rows=_rows_sample(M, 96))


def test_silu_mul_quant_edge_rows():
    D = 256
    g = np.array([0.0, -0.0, 1e-30, -1e-30, 2.0 ** -26, 20.0, 200.0, -200.0, -100.0, -90.0,
                  1e10, -1e10, 16.5, -16.5, 0.5, -0.5], np.float32)
    gate = np.resize(g, (4, D)).astype(np.float32)
    up = np.ones((4, D), np.float32)
    up[1] = -1.0
    up[2] = 0.0
    up[3, ::2] = -0.0
    gu = synth.f32_to_bf16_bits(np.concatenate([gate, up], axis=1))
    for mode in (fq.PER_TOKEN, fq.GROUP128):
        say("silu_mul_quant edge", mode)
        _check_silu(gu, mode)


@pytest.mark.parametrize("mode", [fq.PER_TOKEN, fq.GROUP128])
def test_standalone_quant_parity(mode):
    M, K = 64, 4096
    say("quant", M, K, mode)
    rng = synth.rng_for("quant", M, K)
    x = synth.gen_activations(rng, M, K)
    q, s = fq.quant(bf16_dev(x), mode)
    torch.cuda.synchronize()
    qr, sr = quant.quantize(x, mode)
    assert np.array_equal(host(q), qr)
    assert np.array_equal(host(s).view(np.uint32), sr.view(np.uint32))


def _amax_over_448(lo=0x4000, hi=0x4380):
    """bf16 magnitudes a whose quotient RN32(a / RN32(a / 448)) is above 448
    (448 + 2^-15): the largest quotient a dynamic scale produces."""
    u = np.arange(lo, hi, dtype=np.uint32)
    a = (u << 16).view(np.float32)
    s = (a / np.float32(448)).astype(np.float32)
    return u[(a / s).astype(np.float32) > np.float32(448)].astype(np.uint16)


@pytest.mark.parametrize("mode", [fq.PER_TOKEN, fq.GROUP128])
def test_dynamic_quotient_above_448(mode):
    """The dynamic-scale encoders convert without a clamp: their quotients are
    at most 448 + 2^-15, which must encode to +-448.  Every group (or row)
    maximum here is such a value, of either sign."""
    M, K = 64, 4096
    say("quotient above 448", M, K, mode)
    cand = _amax_over_448()
    assert cand.size > 50
    rng = np.random.default_rng(448)
    x = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32) * 0.25)
    n_unit = K // 128 if mode == fq.GROUP128 else 1
    width = K // n_unit
    for m in range(M):
        for g in range(n_unit):
            col = g * width + int(rng.integers(width))
            sign = np.uint16(0x8000) if (m + g) % 2 else np.uint16(0)
            x[m, col] = cand[(m * n_unit + g) % cand.size] | sign
    q, s = fq.quant(bf16_dev(x), mode)
    torch.cuda.synchronize()
    qr, sr = quant.quantize(x, mode)
    assert np.array_equal(host(q), qr)
    assert np.array_equal(host(s).view(np.uint32), sr.view(np.uint32))
    # every unit's maximum had a quotient above 448 (checked in numpy fp32)
    y = (x.astype(np.uint32) << 16).view(np.float32).reshape(M, n_unit, width)
    qf = (y / sr.reshape(M, n_unit, 1)).astype(np.float32)
    assert int(np.count_nonzero(np.abs(qf) > np.float32(448))) == M * n_unit


def test_silu_exhaustive_all_bf16_gates():
    """Every one of the 65 536 bf16 gates (NaN patterns excluded) against the
    oracle's correctly rounded table."""
    say("silu exhaustive")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    g = bf16_dev(bits)
    y = torch.empty(65536, dtype=torch.float32, device=DEV)
    fq.fp8q_silu(y, g)
    torch.cuda.synchronize()
    got = host(y).view(np.uint32)
    want = silu.silu_table().view(np.uint32)
    exp = (bits.astype(np.uint32) >> 7) & 0xFF
    man = bits.astype(np.uint32) & 0x7F
    finite_or_inf = ~((exp == 0xFF) & (man != 0))
    bad = np.flatnonzero(finite_or_inf & (got != want))
    assert bad.size == 0, [(hex(int(b)), hex(int(got[b])), hex(int(want[b]))) for b in bad[:8]]


def test_e4m3_encoder_exhaustive_range():
    """The device encoder against the oracle on every fp32 bit pattern from
    2^-12 to 512 (both signs) and on special values."""
    lo = int(np.float32(2.0 ** -12).view(np.uint32))
    hi = int(np.float32(512.0).view(np.uint32))
    step = 1 << 24
    for start in range(lo, hi + 1, step):
        say("e4m3 encoder block", hex(start))
        bits = np.arange(start, min(start + step, hi + 1), dtype=np.uint32)
        vals = bits.view(np.float32)
        for v in (vals, -vals):
            x = f32_dev(v)
            q = torch.empty(v.size, dtype=torch.uint8, device=DEV)
            fq.fp8q_cvt_e4m3(q, x)
            torch.cuda.synchronize()
            assert np.array_equal(host(q), e4m3.encode(v)), hex(start)
    special = np.array([0.0, -0.0, 1e-45, -1e-45, 1e-40, -1e-40, 2.0 ** -10, -(2.0 ** -10),
                        448.0, 448.00003, -448.00003, 460.0, 464.0, 1e6, -1e6, 3.4e38, -3.4e38,
                        2.0 ** -9, 0.001953125 * 1.5, 0.001953125 * 2.5], np.float32)
    x = f32_dev(special)
    q = torch.empty(special.size, dtype=torch.uint8, device=DEV)
    fq.fp8q_cvt_e4m3(q, x)
    torch.cuda.synchronize()
    assert np.array_equal(host(q), e4m3.encode(special))


def test_quant_deterministic_and_no_op():
    M, K = 64, 5120
    rng = synth.rng_for("det", M, K)
    x = bf16_dev(synth.gen_activations(rng, M, K))
    w = bf16_dev(synth.gen_rms_weight(rng, K))
    a = fq.rmsnorm_quant(x, w, EPS, fq.PER_TOKEN)
    b = fq.rmsnorm_quant(x, w, EPS, fq.PER_TOKEN)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    # M == 0 is a no-op
    q, s = fq.rmsnorm_quant(x[:0], w, EPS, fq.GROUP128)
    assert q.shape == (0, K)


def test_quant_writes_stay_in_bounds():
    """Outputs carved out of larger buffers: the guard bytes around them must
    be untouched."""
    M, K = 37, 5120
    rng = synth.rng_for("canary", M, K)
    x = bf16_dev(synth.gen_activations(rng, M, K))
    w = bf16_dev(synth.gen_rms_weight(rng, K))
    for mode in (fq.PER_TOKEN, fq.GROUP128):
        ns = M if mode == fq.PER_TOKEN else M * K // 128
        qbuf = torch.full((M * K + 512,), 0xA5, dtype=torch.uint8, device=DEV)
        sbuf = torch.full((ns + 128,), -7.0, dtype=torch.float32, device=DEV)
        q = qbuf[256:256 + M * K].view(M, K)
        s = sbuf[64:64 + ns]
        fq.fp8q_rmsnorm_quant(q, s, x, w, EPS, mode)
        torch.cuda.synchronize()
        assert torch.all(qbuf[:256] == 0xA5) and torch.all(qbuf[256 + M * K:] == 0xA5)
        assert torch.all(sbuf[:64] == -7.0) and torch.all(sbuf[64 + ns:] == -7.0)


# ------------------------------------------- UE8M0 and static scale modes

UE8_CASES = [
    ("c2-per-token", 16, 2048, fq.PER_TOKEN_UE8M0),
    ("c2-per-token", 2048, 2048, fq.PER_TOKEN_UE8M0),
    ("c3-group", 32, 4096, fq.GROUP128_UE8M0),
    ("c4-group", 2048, 5120, fq.GROUP128_UE8M0),
    ("ragged", 37, 5120, fq.PER_TOKEN_UE8M0),
    ("ragged", 5, 128, fq.GROUP128_UE8M0),
    ("max-k", 4, 32768, fq.PER_TOKEN_UE8M0),
    ("max-k", 4, 32768, fq.GROUP128_UE8M0),
]


@pytest.mark.parametrize("name,M,K,mode", UE8_CASES)
def test_rmsnorm_quant_ue8m0_parity(name, M, K, mode):
    say("rmsnorm_quant ue8m0", name, M, K, mode)
    rng = synth.rng_for(name, "rmsnorm_quant", M, K)
    x = synth.gen_activations(rng, M, K)
    w = synth.gen_rms_weight(rng, K)
    _check_rms(x, w, mode)


@pytest.mark.parametrize("name,M,D,mode", [("c3-group", 32, 12288, fq.GROUP128_UE8M0),
                                           ("c5-group", 64, 25600, fq.GROUP128_UE8M0),
                                           ("c2-per-token", 128, 6144, fq.PER_TOKEN_UE8M0),
                                           ("ragged", 9, 1000, fq.PER_TOKEN_UE8M0)])
def test_silu_mul_quant_ue8m0_parity(name, M, D, mode):
    say("silu_mul_quant ue8m0", name, M, D, mode)
    rng = synth.rng_for(name, "silu_mul_quant", M, D)
    gu = synth.gen_gate_up(rng, M, D)
    _check_silu(gu, mode)


@pytest.mark.parametrize("scale", [0.05, 3.0e-3, 1.0e-30, 7.0e37, 1.0])
def test_static_scale_parity(scale):
    """Static per-tensor scale on all three front ends, scales on the fast
    quotient path (0.05, 3e-3, 1) and on the IEEE-division path (1e-30,
    7e37), with inputs that saturate."""
    M, K = 48, 2056
    say("static", scale)
    rng = synth.rng_for("static", M, K)
    x = synth.gen_activations(rng, M, K)
    w = synth.gen_rms_weight(rng, K)
    _check_rms(x, w, fq.PER_TENSOR_STATIC, scale=np.float32(scale))
    gu = synth.gen_gate_up(rng, M, K)
    _check_silu(gu, fq.PER_TENSOR_STATIC, scale=np.float32(scale))
    q, _ = fq.quant(bf16_dev(x), fq.PER_TENSOR_STATIC, scale=_static(np.float32(scale)))
    torch.cuda.synchronize()
    qr, _ = quant.quantize(x, fq.PER_TENSOR_STATIC, scale=np.float32(scale))
    assert np.array_equal(host(q), qr)


@pytest.mark.parametrize("mode", [fq.PER_TOKEN_UE8M0, fq.GROUP128_UE8M0])
def test_ue8m0_edge_rows(mode):
    """All-zero, tiny, huge and one-hot rows (scale 2^-127, the subnormal
    quotient path and the largest exponents)."""
    K = 256
    rng = synth.rng_for("edge-ue8", K)
    w = synth.gen_rms_weight(rng, K)
    rows = [np.zeros(K, np.float32), np.full(K, -3.0e-30, np.float32),
            np.full(K, 1.0e30, np.float32)]
    t = np.zeros(K, np.float32); t[5] = 1e-35; rows.append(t)
    o = np.zeros(K, np.float32); o[200] = -5.0; rows.append(o)
    x = synth.f32_to_bf16_bits(np.stack(rows))
    _check_rms(x, w, mode)
    q, s = fq.quant(bf16_dev(x), mode)
    torch.cuda.synchronize()
    qr, sr = quant.quantize(x, mode)
    assert np.array_equal(host(q), qr)
    assert np.array_equal(host(s).view(np.uint32), sr.view(np.uint32))
