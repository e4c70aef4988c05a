"""W8A8 INT8 on the GPU against the oracle: the int8 quantizers must match
bit for bit, and since the int8 GEMM sums exactly in int32, its output may
differ from the float64 reference only by the fp32 epilogue and the bf16
rounding: |out - ref| <= (2^-8 + 2^-21) |ref| for every element."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_rms_amd as fq
import synth
from oracle import gemm, int8, quant
from gpu_util import DEV, bf16_dev, bf16_host_f64, f32_dev, host, say

pytestmark = pytest.mark.gpu

EPS = 1e-6
I8 = fq.OP_SCALED_MM_INT8
BOUND = 2.0 ** -8 + 2.0 ** -21


def i8_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int8)).to(DEV)


def _i8_configs():
    names = [(i, fq.fp8q_gemm_config_name(i)) for i in range(fq.fp8q_gemm_num_configs())]
    return [(i, n) for i, n in names if n.startswith("i8_")]


def _m_for(name):
    if "_skinny_t" in name:
        return 16 * int(name.split("_skinny_t")[1].split("_")[0]) - 3
    return 200


def _close(y, ref):
    out = bf16_host_f64(y)
    err = np.abs(out - ref)
    bad = err > BOUND * np.abs(ref)
    assert not bad.any(), (int(bad.sum()), float(np.max(err / np.maximum(np.abs(ref), 1e-300))))


def _rand_gemm(rng, M, N, K):
    a = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    b = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    sa = synth.gen_scales(rng, (M,))
    sb = synth.gen_scales(rng, (N,))
    return a, b, sa, sb


# ------------------------------------------------------------ quantizers

@pytest.mark.parametrize("M,K,mode", [(1, 2048, fq.PER_TOKEN), (16, 2048, fq.PER_TOKEN),
                                      (2048, 2048, fq.PER_TOKEN), (37, 5120, fq.PER_TOKEN),
                                      (4, 32768, fq.PER_TOKEN), (48, 2056, fq.PER_TENSOR_STATIC)])
def test_rmsnorm_quant_int8_parity(M, K, mode):
    say("rmsnorm_quant_int8", M, K, mode)
    rng = synth.rng_for("int8-rms", M, K)
    x = synth.gen_activations(rng, M, K)
    w = synth.gen_rms_weight(rng, K)
    st = np.float32(0.05) if mode == fq.PER_TENSOR_STATIC else None
    q, s = fq.rmsnorm_quant_int8(bf16_dev(x), bf16_dev(w), EPS, mode,
                                 scale=None if st is None else f32_dev(np.array([st])))
    torch.cuda.synchronize()
    qr, sr = int8.rmsnorm_quant(x, w, EPS, mode, scale=st)
    q, s = host(q), host(s)
    bad = [m for m in range(M) if not np.array_equal(q[m], qr[m])]
    if mode == fq.PER_TOKEN:
        bad = sorted(set(bad) | {m for m in range(M) if s[m].view(np.uint32) != sr[m].view(np.uint32)})
    # the fp64 sum-of-squares tie policy of the FP8 tests: only rows whose
    # inverse RMS sits on an fp32 rounding tie may take the other neighbour
    if bad:
        inv32, inv64 = quant.rms_inv(x[bad], EPS)
        for j, m in enumerate(bad):
            lo = np.float32(inv64[j])
            other = np.nextafter(lo, np.float32(np.inf) if inv64[j] > lo else np.float32(0))
            mid = (float(lo) + float(other)) / 2
            assert abs(inv64[j] - mid) <= 2.0 ** -40 * inv64[j], f"row {m}"
            q2, s2 = int8.rmsnorm_quant(x[m:m + 1], w, EPS, mode, scale=st,
                                        inv_override=np.array([other], np.float32))
            assert np.array_equal(q[m], q2[0]), f"row {m}"
            if mode == fq.PER_TOKEN:
                assert s[m].view(np.uint32) == s2[0].view(np.uint32), f"row {m}"


@pytest.mark.parametrize("M,D,mode", [(16, 6144, fq.PER_TOKEN), (128, 6144, fq.PER_TOKEN),
                                      (9, 1000, fq.PER_TOKEN), (2, 32768, fq.PER_TOKEN),
                                      (33, 1024, fq.PER_TENSOR_STATIC)])
def test_silu_mul_quant_int8_parity(M, D, mode):
    say("silu_mul_quant_int8", M, D, mode)
    rng = synth.rng_for("int8-silu", M, D)
    gu = synth.gen_gate_up(rng, M, D)
    st = np.float32(0.3) if mode == fq.PER_TENSOR_STATIC else None
    q, s = fq.silu_mul_quant_int8(bf16_dev(gu), mode,
                                  scale=None if st is None else f32_dev(np.array([st])))
    torch.cuda.synchronize()
    qr, sr = int8.silu_mul_quant(gu, mode, scale=st)
    assert np.array_equal(host(q), qr)
    assert np.array_equal(host(s).view(np.uint32), sr.view(np.uint32))


def test_quant_int8_edge_rows():
    K = 256
    rows = [np.zeros(K, np.float32), np.full(K, -3.0e-30, np.float32),
            np.full(K, 1.0e30, np.float32)]
    t = np.linspace(-127.5, 127.5, K).astype(np.float32)  # ties at the half integers
    rows.append(t)
    o = np.zeros(K, np.float32); o[7] = -5.0; rows.append(o)
    x = synth.f32_to_bf16_bits(np.stack(rows))
    for mode, st in ((fq.PER_TOKEN, None), (fq.PER_TENSOR_STATIC, np.float32(1.0)),
                     (fq.PER_TENSOR_STATIC, np.float32(1e-30))):
        say("quant_int8 edge", mode, st)
        q, s = fq.quant_int8(bf16_dev(x), mode,
                             scale=None if st is None else f32_dev(np.array([st])))
        torch.cuda.synchronize()
        qr, sr = int8.quantize(x, mode, scale=st)
        assert np.array_equal(host(q), qr)
        assert np.array_equal(host(s).view(np.uint32), sr.view(np.uint32))


# ------------------------------------------------------------------ GEMM

@pytest.mark.parametrize("cfg,name", _i8_configs(), ids=[n for _, n in _i8_configs()])
def test_every_int8_variant(cfg, name):
    M, N, K = _m_for(name), 256, 3072
    say("int8 variant", name, M, N, K)
    rng = synth.rng_for("int8-variant", name, M, N, K)
    a, b, sa, sb = _rand_gemm(rng, M, N, K)
    y = fq.scaled_mm_int8(i8_dev(a), i8_dev(b), f32_dev(sa), f32_dev(sb), cfg=cfg)
    torch.cuda.synchronize()
    _close(y, int8.scaled_mm(a, b, sa, sb))


@pytest.mark.parametrize("M", [1, 17, 130])
@pytest.mark.parametrize("cfg,name", [c for c in _i8_configs() if "_tiled_" in c[1]],
                         ids=[n for _, n in _i8_configs() if "_tiled_" in n])
def test_int8_tiled_variant_few_tokens(cfg, name, M):
    """Fewer tokens than a tile (or a ragged last tile): loads past M clamp
    to the last row, and only rows below M are written."""
    N, K = 512, 640
    say("int8 tiled few tokens", name, M)
    rng = synth.rng_for("int8-few-tokens", name, M)
    a, b, sa, sb = _rand_gemm(rng, M, N, K)
    y = fq.scaled_mm_int8(i8_dev(a), i8_dev(b), f32_dev(sa), f32_dev(sb), cfg=cfg)
    torch.cuda.synchronize()
    assert y.shape == (M, N)
    _close(y, int8.scaled_mm(a, b, sa, sb))


@pytest.mark.parametrize("cfg,name", _i8_configs(), ids=[n for _, n in _i8_configs()])
def test_every_int8_variant_extreme_sums_exact(cfg, name):
    """All operands +-127 (the largest int32 sums) with unit scales and a
    one-hot pattern: the results are exactly representable in bf16 only
    where they are small, so compare with the bound; and a one-hot weight
    picks single products, which must come out exact."""
    M, N, K = _m_for(name), 256, 3072
    say("int8 variant extreme", name)
    rng = synth.rng_for("int8-extreme", name)
    a = np.where(rng.random((M, K)) < 0.5, 127, -127).astype(np.int8)
    b = np.where(rng.random((N, K)) < 0.5, 127, -127).astype(np.int8)
    ones_m, ones_n = np.ones(M, np.float32), np.ones(N, np.float32)
    y = fq.scaled_mm_int8(i8_dev(a), i8_dev(b), f32_dev(ones_m), f32_dev(ones_n), cfg=cfg)
    torch.cuda.synchronize()
    _close(y, int8.scaled_mm(a, b, ones_m, ones_n))
    oh = np.zeros((N, K), np.int8)
    oh[np.arange(N), rng.permutation(K)[:N]] = 1
    a2 = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    y = fq.scaled_mm_int8(i8_dev(a2), i8_dev(oh), f32_dev(ones_m), f32_dev(ones_n), cfg=cfg)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_host_f64(y), int8.scaled_mm(a2, oh, ones_m, ones_n))


C2 = [(M, N, K) for M in (1, 16, 128, 512, 2048) for N, K in ((4096, 2048), (2048, 2048),
                                                               (12288, 2048), (2048, 6144))]


@pytest.mark.parametrize("M,N,K", C2)
def test_int8_qwen3_1p7b_shapes(M, N, K):
    """The Qwen3-1.7B per-token linear shapes with realistic operands
    (int8-quantized activations and weights); large M compares sampled rows."""
    say("int8 c2", M, N, K, fq.fp8q_gemm_config_name(fq.fp8q_gemm_config_for(I8, M, N, K)))
    rng = synth.rng_for("int8-c2", M, N, K)
    x = synth.gen_activations(rng, M, K)
    a, sa = int8.quantize(x, int8.PER_TOKEN)
    b, sb = int8.quant_weight_per_channel(synth.gen_linear_weight(rng, N, K))
    y = fq.scaled_mm_int8(i8_dev(a), i8_dev(b), f32_dev(sa), f32_dev(sb))
    torch.cuda.synchronize()
    rows = np.arange(M) if M <= 128 else np.sort(np.random.default_rng(M).choice(M, 64, False))
    ref = int8.scaled_mm(a[rows], b, sa[rows], sb)
    _close(y[torch.from_numpy(rows).to(DEV)], ref)
    assert gemm.acceptance(bf16_host_f64(y[torch.from_numpy(rows).to(DEV)]), ref)["ok"]


def test_int8_gemm_deterministic_and_m_zero():
    rng = synth.rng_for("int8-det")
    a, b, sa, sb = _rand_gemm(rng, 37, 4096, 6144)
    args = (i8_dev(a), i8_dev(b), f32_dev(sa), f32_dev(sb))
    y1 = fq.scaled_mm_int8(*args)
    y2 = fq.scaled_mm_int8(*args)
    assert torch.equal(y1, y2)
    y0 = fq.scaled_mm_int8(args[0][:0], args[1], args[2][:0], args[3])
    assert y0.shape == (0, 4096)
