"""GPU parity of the FP8 GEMMs against the CPU oracle.

* Every compiled variant (tiled, skinny, every split-K factor) on a ragged
  shape, for both scaled_mm and scaled_mm_blockwise: the oracle acceptance
  rule on random codes, and exact bf16 results on one-hot weights with
  power-of-two scales (each output is then a single exactly representable
  product, so any misplaced element, row, column or block scale shows).
* The table's choice at every Qwen3 workload shape: full comparison where
  the oracle is quick, sampled rows at the largest sizes.
* Determinism and guard bytes.
"""
import numpy as np
import pytest
import torch

import fp8_block_scaled_rms_amd as fq
import synth
from oracle import gemm, quant
from gpu_util import DEV, bf16_dev, bf16_host, bf16_host_f64, f32_dev, host, say, u8_dev

pytestmark = pytest.mark.gpu

MM, BW = fq.OP_SCALED_MM, fq.OP_SCALED_MM_BLOCKWISE


def _configs():
    """Every variant of the FP8 ops.  These are the exact (f16_) engine's: the
    i8_ ones serve the int8 op (tests/test_gpu_int8.py), and the FP8-MFMA
    engine's f8_ variants, registered only on an explicit non-conforming
    opt-in, are a measurement (tests/fp8_mfma_study.py), not a tested path."""
    names = [(i, fq.fp8q_gemm_config_name(i)) for i in range(fq.fp8q_gemm_num_configs())]
    return [(i, n) for i, n in names if n.startswith("f16_")]


def _check_engine(name, op, y, a, sa, b, sb):
    res = gemm.acceptance(bf16_host_f64(y), _ref(op, a, sa, b, sb))
    assert res["ok"], res


def _m_for(name):
    if "_skinny_t" in name:
        return 16 * int(name.split("_skinny_t")[1].split("_")[0]) - 3
    return 200


def _run(op, a, sa, b, sb, cfg=None):
    at, bt = u8_dev(a), u8_dev(b)
    sat, sbt = f32_dev(sa), f32_dev(sb)
    if op == MM:
        y = fq.scaled_mm(at, bt, sat, sbt, cfg=cfg)
    else:
        y = fq.scaled_mm_blockwise(at, bt, sat, sbt, cfg=cfg)
    torch.cuda.synchronize()
    return y


def _ref(op, a, sa, b, sb):
    return gemm.scaled_mm(a, b, sa, sb) if op == MM else gemm.scaled_mm_blockwise(a, sa, b, sb)


def _scales(rng, op, M, N, K, pow2=False):
    if op == MM:
        shp_a, shp_b = (M,), (N,)
    else:
        shp_a, shp_b = (M, K // 128), (N // 128, K // 128)
    if pow2:
        return (np.exp2(rng.integers(-6, 3, shp_a)).astype(np.float32),
                np.exp2(rng.integers(-6, 3, shp_b)).astype(np.float32))
    return synth.gen_scales(rng, shp_a), synth.gen_scales(rng, shp_b)


@pytest.mark.parametrize("op", [MM, BW], ids=["mm", "blockwise"])
@pytest.mark.parametrize("cfg,name", _configs(), ids=[n for _, n in _configs()])
def test_every_variant_random(cfg, name, op):
    M, N, K = _m_for(name), 256, 3072
    say("gemm variant random", name, op, M, N, K)
    rng = synth.rng_for("variant", name, op, M, N, K)
    a = synth.gen_e4m3_codes(rng, (M, K))
    b = synth.gen_e4m3_codes(rng, (N, K))
    sa, sb = _scales(rng, op, M, N, K)
    y = _run(op, a, sa, b, sb, cfg)
    _check_engine(name, op, y, a, sa, b, sb)


def _tiled_configs():
    return [c for c in _configs() if "_tiled_" in c[1]]


@pytest.mark.parametrize("K", [128, 256, 384, 512])
@pytest.mark.parametrize("cfg,name", _tiled_configs(), ids=[n for _, n in _tiled_configs()])
def test_every_tiled_variant_short_k(cfg, name, K):
    """K of 1 to 4 blocks: fewer K blocks than pipeline stages (and, with
    split-K, workgroup rows left without blocks)."""
    M, N = 200, 256
    for op in (MM, BW):
        say("gemm tiled short K", name, op, M, N, K)
        rng = synth.rng_for("short-k", name, op, M, N, K)
        a = synth.gen_e4m3_codes(rng, (M, K))
        b = synth.gen_e4m3_codes(rng, (N, K))
        sa, sb = _scales(rng, op, M, N, K)
        y = _run(op, a, sa, b, sb, cfg)
        _check_engine(name, op, y, a, sa, b, sb)


@pytest.mark.parametrize("M", [1, 17, 130])
@pytest.mark.parametrize("cfg,name", [c for c in _tiled_configs() if c[1].startswith("f16_")],
                         ids=[n for _, n in _tiled_configs() if n.startswith("f16_")])
def test_every_tiled_variant_few_tokens(cfg, name, M):
    """Fewer tokens than a tile (or a ragged last tile): every token-row load
    past M clamps to the last row, and only rows below M are written."""
    N, K = 512, 640
    for op in (MM, BW):
        say("gemm tiled few tokens", name, op, M, N, K)
        rng = synth.rng_for("few-tokens", name, op, M, N, K)
        a = synth.gen_e4m3_codes(rng, (M, K))
        b = synth.gen_e4m3_codes(rng, (N, K))
        sa, sb = _scales(rng, op, M, N, K)
        y = _run(op, a, sa, b, sb, cfg)
        _check_engine(name, op, y, a, sa, b, sb)


@pytest.mark.parametrize("op", [MM, BW], ids=["mm", "blockwise"])
@pytest.mark.parametrize("cfg,name", _configs(), ids=[n for _, n in _configs()])
def test_every_variant_one_hot_exact(cfg, name, op):
    M, N, K = _m_for(name), 256, 3072
    say("gemm variant one-hot", name, op, M, N, K)
    rng = synth.rng_for("onehot", name, op, M, N, K)
    a = synth.gen_e4m3_codes(rng, (M, K))
    perm = rng.permutation(K)[:N]
    b = np.zeros((N, K), np.uint8)
    b[np.arange(N), perm] = 0x38  # 1.0
    sa, sb = _scales(rng, op, M, N, K, pow2=True)
    y = bf16_host_f64(_run(op, a, sa, b, sb, cfg))
    ref = _ref(op, a, sa, b, sb)  # exactly representable in bf16 here
    assert np.array_equal(y, ref)


def _gemm_case(config, op, M, N, K, realistic):
    rng = synth.rng_for(config, "gemm", op, M, N, K)
    if realistic:
        x = synth.gen_activations(rng, M, K)
        a, sa = quant.quantize(x, quant.PER_TOKEN if op == MM else quant.GROUP128)
        W = synth.gen_linear_weight(rng, N, K)
        b, sb = quant.quant_weight_per_channel(W) if op == MM else quant.quant_weight_block128(W)
    else:
        a = synth.gen_e4m3_codes(rng, (M, K))
        b = synth.gen_e4m3_codes(rng, (N, K))
        sa, sb = _scales(rng, op, M, N, K)
    return a, sa, b, sb


C2 = [(M, N, K) for M in (1, 16, 128, 512) for N, K in ((4096, 2048), (2048, 2048),
                                                         (12288, 2048), (2048, 6144))]
C3 = [(M, N, K) for M in (1, 2, 4, 8, 16, 32) for N, K in ((6144, 4096), (4096, 4096),
                                                            (24576, 4096), (4096, 12288))]


@pytest.mark.parametrize("M,N,K", C2)
def test_scaled_mm_qwen3_1p7b_shapes(M, N, K):
    say("scaled_mm c2", M, N, K, fq.fp8q_gemm_config_name(fq.fp8q_gemm_config_for(MM, M, N, K)))
    a, sa, b, sb = _gemm_case("c2", MM, M, N, K, realistic=True)
    y = _run(MM, a, sa, b, sb)
    res = gemm.acceptance(bf16_host_f64(y), gemm.scaled_mm(a, b, sa, sb))
    assert res["ok"], res


@pytest.mark.parametrize("M,N,K", C3)
def test_blockwise_qwen3_8b_decode_shapes(M, N, K):
    say("blockwise c3", M, N, K, fq.fp8q_gemm_config_name(fq.fp8q_gemm_config_for(BW, M, N, K)))
    a, sa, b, sb = _gemm_case("c3", BW, M, N, K, realistic=(N * K <= 4096 * 4096))
    y = _run(BW, a, sa, b, sb)
    res = gemm.acceptance(bf16_host_f64(y), gemm.scaled_mm_blockwise(a, sa, b, sb))
    assert res["ok"], res


def _sampled_rows(M, n):
    rng = np.random.default_rng(M + 7)
    return np.sort(np.concatenate([[0, M - 1], rng.choice(np.arange(1, M - 1), n - 2, False)]))


LARGE = [
    (MM, 2048, 4096, 2048), (MM, 2048, 2048, 2048), (MM, 2048, 12288, 2048),
    (MM, 2048, 2048, 6144),
    (BW, 2048, 10240, 5120), (BW, 2048, 5120, 8192), (BW, 2048, 51200, 5120),
    (BW, 2048, 5120, 25600),
    (BW, 8192, 10240, 5120), (BW, 8192, 5120, 8192), (BW, 8192, 51200, 5120),
    (BW, 8192, 5120, 25600),
    (BW, 64, 5120, 25600), (BW, 4096, 5120, 25600),
]


@pytest.mark.parametrize("op,M,N,K", LARGE)
def test_large_shapes_sampled_rows(op, M, N, K):
    """Full-size Qwen3 prefill / MLP-tail shapes in the table's launch
    configuration; 48 sampled rows (all columns) against the oracle."""
    say("gemm large", op, M, N, K, fq.fp8q_gemm_config_name(fq.fp8q_gemm_config_for(op, M, N, K)))
    a, sa, b, sb = _gemm_case("large", op, M, N, K, realistic=False)
    y = _run(op, a, sa, b, sb)
    rows = _sampled_rows(M, 48) if M > 48 else np.arange(M)
    ya = bf16_host_f64(y[torch.from_numpy(rows).to(DEV)])
    ref = _ref(op, a[rows], sa[rows], b, sb)
    res = gemm.acceptance(ya, ref)
    assert res["ok"], res


def test_c1_tiny_pipeline_end_to_end():
    """rmsnorm_quant (group128) -> scaled_mm_blockwise on the tiny blockwise
    workload (M=16, K=256, N=512), against the oracle pipeline."""
    M, K, N = 16, 256, 512
    rng = synth.rng_for("c1", M, N, K)
    x = synth.gen_activations(rng, M, K, outlier_frac=0.0)
    w = synth.gen_rms_weight(rng, K)
    W = synth.gen_linear_weight(rng, N, K)
    b, sb = quant.quant_weight_block128(W)
    q, s = fq.rmsnorm_quant(bf16_dev(x), bf16_dev(w), 1e-6, fq.GROUP128)
    y = fq.scaled_mm_blockwise(q, u8_dev(b), s, f32_dev(sb))
    torch.cuda.synchronize()
    qr, sr = quant.rmsnorm_quant(x, w, 1e-6, quant.GROUP128)
    assert np.array_equal(host(q), qr) and np.array_equal(host(s), sr)
    res = gemm.acceptance(bf16_host_f64(y), gemm.scaled_mm_blockwise(qr, sr, b, sb))
    assert res["ok"], res


@pytest.mark.parametrize("op,M,N,K", [(BW, 8, 4096, 12288), (MM, 2048, 2048, 6144),
                                      (BW, 200, 1024, 1024)])
def test_gemm_deterministic(op, M, N, K):
    a, sa, b, sb = _gemm_case("det", op, M, N, K, realistic=False)
    y1 = bf16_host(_run(op, a, sa, b, sb))
    y2 = bf16_host(_run(op, a, sa, b, sb))
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("cfg,name", _configs(), ids=[n for _, n in _configs()])
def test_gemm_writes_stay_in_bounds(cfg, name):
    M, N, K = _m_for(name), 256, 3072
    rng = synth.rng_for("canary", name)
    a = u8_dev(synth.gen_e4m3_codes(rng, (M, K)))
    b = u8_dev(synth.gen_e4m3_codes(rng, (N, K)))
    sa, sb = [f32_dev(s) for s in _scales(rng, BW, M, N, K)]
    buf = torch.full((M * N + 1024,), 3.0, dtype=torch.bfloat16, device=DEV)
    y = buf[512:512 + M * N].view(M, N)
    nws = fq.fp8q_workspace_size(BW, M, N, K, cfg)
    wsbuf = torch.full(((nws // 4) + 128,), -1.0, dtype=torch.float32, device=DEV)
    ws = wsbuf[64:64 + nws // 4] if nws else None
    fq.fp8q_scaled_mm_blockwise(y, a, b, sa, sb, ws, cfg)
    torch.cuda.synchronize()
    assert torch.all(buf[:512] == 3.0) and torch.all(buf[512 + M * N:] == 3.0)
    assert torch.all(wsbuf[:64] == -1.0) and torch.all(wsbuf[64 + nws // 4:] == -1.0)


HYBRIDS = ["f16_tiled_m128_n256_w2x4_st3_h2", "f16_tiled_m128_n256_w2x4_st3_h4"]


def _hybrid_parts(name, M, N):
    """The hybrid's two variants and the columns its unsplit part takes: the
    bn-wide column tiles of every token-tile row that fill whole rounds of
    resident workgroups (one eight-wave 128x256 or two four-wave 128x128
    workgroups per CU)."""
    part_a, split = name.rsplit("_h", 1)
    bn = int(part_a.split("_n")[1].split("_")[0])
    per_cu = 1 if bn == 256 else 2
    slots = per_cu * torch.cuda.get_device_properties(0).multi_processor_count
    rows, cols = -(-M // 128), N // bn
    na = (rows * cols // slots) * slots // rows * bn
    return part_a, "f16_tiled_m128_n128_w2x2_st2_s" + split, min(na, cols * bn)


@pytest.mark.parametrize("M", [2048, 1999])
@pytest.mark.parametrize("name", HYBRIDS)
@pytest.mark.parametrize("op", [MM, BW], ids=["mm", "blockwise"])
def test_hybrid_columns_equal_their_two_variants(op, name, M):
    """A hybrid variant at a shape with more tiles than one round of
    workgroups (M=2048, and a ragged M=1999; N=5120): the columns that fill whole rounds equal,
    bit for bit, the unsplit variant's output, and the rest the split
    128x128 variant's, each run alone on the whole problem; nothing outside
    y or the workspace is written, and sampled rows meet the acceptance
    rule."""
    N, K = 5120, 1024
    part_a, part_b, na = _hybrid_parts(name, M, N)
    assert 0 < na < N
    names = {fq.fp8q_gemm_config_name(i): i for i in range(fq.fp8q_gemm_num_configs())}
    say("gemm hybrid", name, op, M, N, K, "columns", na)
    rng = synth.rng_for("hybrid", name, op, M, N, K)
    a_h = synth.gen_e4m3_codes(rng, (M, K))
    b_h = synth.gen_e4m3_codes(rng, (N, K))
    sa_h, sb_h = _scales(rng, op, M, N, K)
    a, b, sa, sb = u8_dev(a_h), u8_dev(b_h), f32_dev(sa_h), f32_dev(sb_h)

    def run(cfg, guard=False):
        buf = torch.full((M * N + 1024,), 3.0, dtype=torch.bfloat16, device=DEV)
        y = buf[512:512 + M * N].view(M, N)
        nws = fq.fp8q_workspace_size(op, M, N, K, cfg)
        wsbuf = torch.full(((nws // 4) + 128,), -1.0, dtype=torch.float32, device=DEV)
        ws = wsbuf[64:64 + nws // 4] if nws else None
        if op == MM:
            fq.fp8q_scaled_mm(y, a, b, sa, sb, ws, cfg)
        else:
            fq.fp8q_scaled_mm_blockwise(y, a, b, sa, sb, ws, cfg)
        torch.cuda.synchronize()
        if guard:
            assert torch.all(buf[:512] == 3.0) and torch.all(buf[512 + M * N:] == 3.0)
            assert torch.all(wsbuf[:64] == -1.0) and torch.all(wsbuf[64 + nws // 4:] == -1.0)
        return y

    y_h = run(names[name], guard=True)
    y_a = run(names[part_a])
    y_b = run(names[part_b])
    assert torch.equal(y_h[:, :na].view(torch.int16), y_a[:, :na].view(torch.int16))
    assert torch.equal(y_h[:, na:].view(torch.int16), y_b[:, na:].view(torch.int16))
    rows_s = synth.rng_for("hybrid-rows", name, op).choice(M, 48, replace=False)
    rows_s.sort()
    sa_rows = sa_h[rows_s]
    res = gemm.acceptance(bf16_host_f64(y_h)[rows_s], _ref(op, a_h[rows_s], sa_rows, b_h, sb_h))
    assert res["ok"], res


@pytest.mark.parametrize("name", HYBRIDS)
def test_hybrid_ue8m0_columns_equal_their_two_variants(name):
    """The UE8M0 entry point on a hybrid variant, with power-of-two scales at
    a shape where both parts run (eight-wave tiles fold the scales into the
    widening, four-wave tiles take the general path): each part's columns
    equal, bit for bit, that variant run alone through the same entry point,
    and sampled rows meet the acceptance rule."""
    M, N, K = 2048, 5120, 1024
    part_a, part_b, na = _hybrid_parts(name, M, N)
    assert 0 < na < N
    names = {fq.fp8q_gemm_config_name(i): i for i in range(fq.fp8q_gemm_num_configs())}
    say("gemm hybrid ue8m0", name, M, N, K, "columns", na)
    rng = synth.rng_for("hybrid-ue8m0", name, M, N, K)
    a_h = synth.gen_e4m3_codes(rng, (M, K))
    b_h = synth.gen_e4m3_codes(rng, (N, K))
    sa_h, sb_h = _scales(rng, BW, M, N, K, pow2=True)
    a, b, sa, sb = u8_dev(a_h), u8_dev(b_h), f32_dev(sa_h), f32_dev(sb_h)
    y_h = fq.scaled_mm_blockwise_ue8m0(a, b, sa, sb, cfg=names[name])
    y_a = fq.scaled_mm_blockwise_ue8m0(a, b, sa, sb, cfg=names[part_a])
    y_b = fq.scaled_mm_blockwise_ue8m0(a, b, sa, sb, cfg=names[part_b])
    torch.cuda.synchronize()
    assert torch.equal(y_h[:, :na].view(torch.int16), y_a[:, :na].view(torch.int16))
    assert torch.equal(y_h[:, na:].view(torch.int16), y_b[:, na:].view(torch.int16))
    rows_s = synth.rng_for("hybrid-ue8m0-rows", name).choice(M, 48, replace=False)
    rows_s.sort()
    res = gemm.acceptance(bf16_host_f64(y_h)[rows_s], _ref(BW, a_h[rows_s], sa_h[rows_s], b_h, sb_h))
    assert res["ok"], res


def test_gemm_m_zero_is_noop():
    a = torch.empty((0, 256), dtype=torch.uint8, device=DEV)
    b = torch.zeros((256, 256), dtype=torch.uint8, device=DEV)
    y = fq.scaled_mm(a, b, torch.empty(0, device=DEV), torch.ones(256, device=DEV))
    assert y.shape == (0, 256)


# ------------------------------------- power-of-two (UE8M0) blockwise scales

def _ue8m0_weight_blocks(W):
    """W fp32 [N,K] -> e4m3 codes and power-of-two scales per 128x128 block
    (the oracle's quantizer with the UE8M0 scale rule)."""
    N, K = W.shape
    blocks = W.reshape(N // 128, 128, K // 128, 128).transpose(0, 2, 1, 3)
    codes, scale = quant.quantize_vectors_ue8m0(blocks.reshape(N // 128, K // 128, 128 * 128))
    codes = codes.reshape(N // 128, K // 128, 128, 128).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(codes.reshape(N, K)), scale


def _run_ue8(a, sa, b, sb, cfg=None):
    y = fq.scaled_mm_blockwise_ue8m0(u8_dev(a), u8_dev(b), f32_dev(sa), f32_dev(sb), cfg=cfg)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("cfg,name", [c for c in _configs() if c[1].startswith("f16_")],
                         ids=[n for _, n in _configs() if n.startswith("f16_")])
def test_ue8m0_every_variant_one_hot_exact(cfg, name):
    """Power-of-two scales (the folded path of the tiled kernels) with one-hot
    weights: every output is one scaled e4m3 value, exact in bf16."""
    M, N, K = _m_for(name), 256, 3072
    say("ue8m0 variant one-hot", name)
    rng = synth.rng_for("ue8-onehot", name)
    a = synth.gen_e4m3_codes(rng, (M, K))
    b = np.zeros((N, K), np.uint8)
    b[np.arange(N), rng.permutation(K)[:N]] = 0x38
    sa, sb = _scales(rng, BW, M, N, K, pow2=True)
    y = bf16_host_f64(_run_ue8(a, sa, b, sb, cfg))
    assert np.array_equal(y, _ref(BW, a, sa, b, sb))


@pytest.mark.parametrize("M,N,K", [(256, 2048, 5120), (200, 1024, 8192), (2048, 10240, 5120)])
def test_ue8m0_realistic_against_oracle(M, N, K):
    """UE8M0 activations from the GPU quantizer and power-of-two weight block
    scales, in the table's launch configuration."""
    say("ue8m0 realistic", M, N, K)
    rng = synth.rng_for("ue8-real", M, N, K)
    x = synth.gen_activations(rng, M, K)
    qa, sa_t = fq.quant(bf16_dev(x), fq.GROUP128_UE8M0)
    a, sa = host(qa), host(sa_t)
    b, sb = _ue8m0_weight_blocks(synth.gen_linear_weight(rng, N, K))
    y = _run_ue8(a, sa, b, sb)
    rows = _sampled_rows(M, 64) if M > 64 else np.arange(M)
    ref = gemm.scaled_mm_blockwise(a[rows], sa[rows], b, sb)
    res = gemm.acceptance(bf16_host_f64(y[torch.from_numpy(rows).to(DEV)]), ref)
    assert res["ok"], res


@pytest.mark.parametrize("name", ["f16_tiled_m128_n256_w2x4_st3", "f16_tiled_m256_n128_w4x2_st3"])
def test_ue8m0_mixed_folding_waves(name):
    """Eight-wave tiles whose waves take different paths in one workgroup:
    token rows with power-of-two scales fold them into the widening, rows
    with general scales run the per-block FMA, with the same barriers.  Also
    a ragged M (the last tile's rows clamp) and a long K."""
    M, N, K = 328, 512, 5120
    cfg = next(i for i, n in _configs() if n == name)
    say("ue8m0 mixed folding", name, M, N, K)
    rng = synth.rng_for("ue8-mixed", name)
    a = synth.gen_e4m3_codes(rng, (M, K))
    b = synth.gen_e4m3_codes(rng, (N, K))
    sa, sb = _scales(rng, BW, M, N, K, pow2=True)
    sa_gen, _ = _scales(rng, BW, M, N, K)
    rows = (np.arange(M) // 64) % 2 == 1          # every other 64-row band: general scales
    sa[rows] = sa_gen[rows]
    y = bf16_host_f64(_run_ue8(a, sa, b, sb, cfg))
    res = gemm.acceptance(y, _ref(BW, a, sa, b, sb))
    assert res["ok"], res


def test_ue8m0_four_wave_tiles_run_the_general_path():
    """Folding measured slower in the four-wave tiles, so there the UE8M0
    entry runs the general blockwise kernel: bit for bit its result."""
    M, N, K = 200, 256, 3072
    cfg = next(i for i, n in _configs() if n == "f16_tiled_m128_n128_w2x2_st2")
    say("ue8m0 four-wave general path", M, N, K)
    rng = synth.rng_for("ue8-fourwave")
    a = synth.gen_e4m3_codes(rng, (M, K))
    b = synth.gen_e4m3_codes(rng, (N, K))
    sa, sb = _scales(rng, BW, M, N, K, pow2=True)
    assert torch.equal(_run_ue8(a, sa, b, sb, cfg), _run(BW, a, sa, b, sb, cfg))


def test_ue8m0_falls_back_on_general_or_spread_scales():
    """In a folding (eight-wave) tile, scales that are not powers of two take
    the general path (same bytes as scaled_mm_blockwise); so do power-of-two
    scales whose exponents span more than the f16 window, which must still
    match the oracle."""
    M, N, K = 200, 256, 3072
    cfg = next(i for i, n in _configs() if n == "f16_tiled_m128_n256_w2x4_st3")
    say("ue8m0 fallback", M, N, K)
    rng = synth.rng_for("ue8-fallback")
    a = synth.gen_e4m3_codes(rng, (M, K))
    b = synth.gen_e4m3_codes(rng, (N, K))
    sa, sb = _scales(rng, BW, M, N, K)  # general fp32 scales
    y_ue8 = _run_ue8(a, sa, b, sb, cfg)
    y_gen = _run(BW, a, sa, b, sb, cfg)
    assert torch.equal(y_ue8, y_gen)
    sa2 = np.exp2(rng.integers(-4, 4, (M, K // 128))).astype(np.float32)
    sa2[::3, 5] = np.float32(2.0 ** -40)  # 36+ binades below the rest of those rows
    sb2 = np.exp2(rng.integers(-4, 4, (N // 128, K // 128))).astype(np.float32)
    y = bf16_host_f64(_run_ue8(a, sa2, b, sb2, cfg))
    res = gemm.acceptance(y, _ref(BW, a, sa2, b, sb2))
    assert res["ok"], res


def test_calls_on_a_side_stream_are_ordered_by_that_stream():
    """The library enqueues on the stream it is given: a chain on a side
    stream (quantizer -> GEMM) reads the quantizer's output in order, and the
    result equals the same chain on the default stream."""
    M, N, K = 96, 2048, 4096
    rng = synth.rng_for("stream", M, N, K)
    x = bf16_dev(synth.gen_activations(rng, M, K))
    w = bf16_dev(synth.gen_rms_weight(rng, K))
    b = u8_dev(synth.gen_e4m3_codes(rng, (N, K)))
    sb = f32_dev(synth.gen_scales(rng, (N // 128, K // 128)))
    q0, s0 = fq.rmsnorm_quant(x, w, 1e-6, fq.GROUP128)
    y0 = fq.scaled_mm_blockwise(q0, b, s0, sb)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q1, s1 = fq.rmsnorm_quant(x, w, 1e-6, fq.GROUP128)
        y1 = fq.scaled_mm_blockwise(q1, b, s1, sb)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(q0, q1) and torch.equal(s0, s1) and torch.equal(y0, y1)


def test_rows_past_32bit_byte_offsets():
    """M*K beyond 2^32 bytes of A (M = 2^20 + 256, K = 4096): the tiled
    kernels address a tile's token rows with 32-bit offsets from the tile's
    first row and clamp the last tile's rows, which must not wrap.  Rows on
    both sides of the 2^32 boundary against the oracle; then the fused
    SiLU-and-mul epilogue on the same operands against the two-kernel path
    with the same tile, on every row."""
    M, N, K = (1 << 20) + 256, 256, 4096
    say("rows past 2^32 bytes", M, N, K)
    g = torch.Generator(device=DEV)
    g.manual_seed(4242)
    a = torch.randint(0, 255, (M, K), generator=g, device=DEV, dtype=torch.uint8) & 0xF7
    b = torch.randint(0, 255, (N, K), generator=g, device=DEV, dtype=torch.uint8) & 0xF7
    sa = torch.rand((M, K // 128), generator=g, device=DEV) + 0.5
    sb = torch.rand((N // 128, K // 128), generator=g, device=DEV) + 0.5
    name = "f16_tiled_m128_n256_w2x4_st3"
    cfg = next(i for i, n in _configs() if n == name)
    y = fq.scaled_mm_blockwise(a, b, sa, sb, cfg=cfg)
    torch.cuda.synchronize()
    edge = (1 << 32) // K  # first row whose byte offset from A passes 2^32
    rows = np.array([0, 1, 127, edge - 129, edge - 1, edge, edge + 1, edge + 200, M - 129,
                     M - 128, M - 2, M - 1])
    ri = torch.from_numpy(rows).to(DEV)
    ref = gemm.scaled_mm_blockwise(host(a[ri]), host(sa[ri]), host(b), host(sb))
    res = gemm.acceptance(bf16_host_f64(y[ri]), ref)
    assert res["ok"], res
    q2, s2 = fq.silu_mul_quant(y, fq.GROUP128)
    del y
    q1, s1 = fq.scaled_mm_blockwise_silu_quant(a, b, sa, sb)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2)
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))
