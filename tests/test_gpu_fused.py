"""The blockwise GEMM with SiLU-and-mul and group-128 quantization fused into
its epilogue (fp8q_scaled_mm_blockwise_silu_quant) against the two-kernel path
it replaces, bit for bit: the plain blockwise GEMM with the same 128x256-tile
variant (so the same fp32 sums and bf16 rounding), then silu_mul_quant in
group-128 mode -- and, on the host, the oracle's silu_mul_quant applied to
that bf16 product (the quantizer stage against the oracle)."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_rms_amd as fq
import synth
from oracle import gemm, quant
from gpu_util import DEV, bf16_host, bf16_host_f64, f32_dev, host, say, u8_dev

pytestmark = pytest.mark.gpu

BW = fq.OP_SCALED_MM_BLOCKWISE
TILE = "f16_tiled_m128_n256_w2x4_st3"


def _tile_cfg():
    return next(i for i in range(fq.fp8q_gemm_num_configs())
                if fq.fp8q_gemm_config_name(i) == TILE)


def _case(M, N, K, realistic, seed_tag):
    rng = synth.rng_for("fused", seed_tag, M, N, K)
    if realistic:
        x = synth.gen_activations(rng, M, K)
        a, sa = quant.quantize(x, quant.GROUP128)
        b, sb = quant.quant_weight_block128(synth.gen_linear_weight(rng, N, K))
    else:
        a = synth.gen_e4m3_codes(rng, (M, K))
        b = synth.gen_e4m3_codes(rng, (N, K))
        sa = synth.gen_scales(rng, (M, K // 128))
        sb = synth.gen_scales(rng, (N // 128, K // 128))
    return a, sa, b, sb


def _two_kernel(at, sat, bt, sbt):
    M, N = at.shape[0], bt.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    fq.fp8q_scaled_mm_blockwise(y, at, bt, sat, sbt, None, _tile_cfg())
    q, s = fq.silu_mul_quant(y, fq.GROUP128)
    return y, q, s


def _compare(M, N, K, realistic, tag, oracle_rows=None):
    a, sa, b, sb = _case(M, N, K, realistic, tag)
    at, bt, sat, sbt = u8_dev(a), u8_dev(b), f32_dev(sa), f32_dev(sb)
    qf, sf = fq.scaled_mm_blockwise_silu_quant(at, bt, sat, sbt)
    y, q2, s2 = _two_kernel(at, sat, bt, sbt)
    torch.cuda.synchronize()
    assert torch.equal(qf, q2), int((qf != q2).sum())
    assert torch.equal(sf.view(torch.int32), s2.view(torch.int32))
    rows = np.arange(M) if oracle_rows is None else oracle_rows
    ridx = torch.from_numpy(rows).to(DEV)
    yb = bf16_host(y[ridx])
    qo, so = quant.silu_mul_quant(yb, quant.GROUP128)
    assert np.array_equal(host(qf[ridx]), qo)
    assert np.array_equal(host(sf[ridx]).view(np.uint32), so.view(np.uint32))
    return a, sa, b, sb, y


@pytest.mark.parametrize("M,N,K", [(1, 256, 128), (200, 512, 384), (130, 768, 1024),
                                   (384, 2560, 640)])
def test_fused_matches_two_kernels_random(M, N, K):
    say("fused silu quant random", M, N, K)
    _compare(M, N, K, False, "random")


@pytest.mark.parametrize("M,N,K", [(256, 1024, 5120), (77, 51200, 512)])
def test_fused_matches_two_kernels_realistic(M, N, K):
    say("fused silu quant realistic", M, N, K)
    a, sa, b, sb, y = _compare(M, N, K, True, "realistic")
    # the GEMM stage itself against the fp64 oracle
    rows = np.arange(min(M, 32))
    ref = gemm.scaled_mm_blockwise(a[rows], sa[rows], b, sb)
    assert gemm.acceptance(bf16_host_f64(y[torch.from_numpy(rows).to(DEV)]), ref)["ok"]


def test_fused_qwen3_32b_gate_up_m2048():
    """The Qwen3-32B prefill gate_up at M=2048 (N = 2 x 25600, K = 5120): every
    output against the two-kernel path, sampled rows against the oracle."""
    M, N, K = 2048, 51200, 5120
    say("fused silu quant c4", M, N, K)
    rows = np.sort(np.random.default_rng(7).choice(M, 24, replace=False))
    _compare(M, N, K, True, "c4", oracle_rows=rows)


def test_fused_zero_groups_and_m_zero():
    """Weight rows that are zero give all-zero groups (scale 0, codes +-0) in
    some output tiles; M = 0 is a no-op."""
    M, N, K = 64, 512, 256
    say("fused silu quant zero groups", M, N, K)
    rng = synth.rng_for("fused-zero", M, N, K)
    a = synth.gen_e4m3_codes(rng, (M, K))
    b = synth.gen_e4m3_codes(rng, (N, K))
    b[0:128] = 0          # gate rows of output tile 0: silu(0) * up = 0
    b[256 + 128:] = 0     # up rows of output tile 1
    sa = synth.gen_scales(rng, (M, K // 128))
    sb = synth.gen_scales(rng, (N // 128, K // 128))
    at, bt, sat, sbt = u8_dev(a), u8_dev(b), f32_dev(sa), f32_dev(sb)
    qf, sf = fq.scaled_mm_blockwise_silu_quant(at, bt, sat, sbt)
    _, q2, s2 = _two_kernel(at, sat, bt, sbt)
    torch.cuda.synchronize()
    assert torch.equal(qf, q2) and torch.equal(sf.view(torch.int32), s2.view(torch.int32))
    assert torch.all(sf == 0.0)
    assert torch.all((qf & 0x7F) == 0)
    q0, s0 = fq.scaled_mm_blockwise_silu_quant(at[:0], bt, sat[:0], sbt)
    assert q0.shape == (0, N // 2) and s0.shape == (0, N // 256)


def test_fused_writes_stay_in_bounds():
    M, N, K = 200, 512, 256
    say("fused silu quant canary", M, N, K)
    a, sa, b, sb = _case(M, N, K, False, "canary")
    at, bt, sat, sbt = u8_dev(a), u8_dev(b), f32_dev(sa), f32_dev(sb)
    qbuf = torch.full((M * N // 2 + 1024,), 0x5A, dtype=torch.uint8, device=DEV)
    sbuf = torch.full((M * N // 256 + 128,), -7.0, dtype=torch.float32, device=DEV)
    q = qbuf[512:512 + M * N // 2].view(M, N // 2)
    s = sbuf[64:64 + M * N // 256].view(M, N // 256)
    fq.fp8q_scaled_mm_blockwise_silu_quant(q, s, at, bt, sat, sbt)
    torch.cuda.synchronize()
    assert torch.all(qbuf[:512] == 0x5A) and torch.all(qbuf[512 + M * N // 2:] == 0x5A)
    assert torch.all(sbuf[:64] == -7.0) and torch.all(sbuf[64 + M * N // 256:] == -7.0)
