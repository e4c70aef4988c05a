"""GPU parity of every launch bench.py times, at its own size and in its own
launch configuration (the table's variant, the quantizer's own unit shape).

The case list is bench.launch_plan(): one case per distinct (kind, mode, M,
K, N).  Full-size inputs are periodic so that the oracle, which is slow,
computes only their distinct rows while every output element is checked:

* token rows: P distinct rows drawn by synth (the workload's distribution),
  row m of the input is row m % P (P prime, so a kernel that reads a
  neighbouring row or tile shows);
* weight rows (GEMMs): the first PN rows are drawn, row n is row n % PN, with
  PN = 7 weight blocks of 128 rows (not a multiple of any tile height).

Quantizers: bytes and scales bit-exact.  The P source rows go through the
oracle (with the RMSNorm rounding-tie policy of test_gpu_quant); every other
row must equal its source row's output bit for bit.
GEMMs: every output against the oracle's fp64 reference (periodic in both
dimensions) under the acceptance rule of oracle.gemm, evaluated on the GPU
for size.
Fused gate_up + SiLU-and-mul quantization: every output bit-identical to the
two-kernel path (the same tile variant's GEMM, then silu_mul_quant), the
GEMM stage against the oracle as above, and sampled rows of the quantizer
stage against the oracle applied to that GEMM's bf16 output.
"""
import functools

import numpy as np
import pytest
import torch

import bench
import fp8_block_scaled_rms_amd as fq
import synth
from oracle import gemm, quant
from gpu_util import DEV, bf16_dev, bf16_host, f32_dev, host, say, u8_dev
from test_gpu_quant import compare_rms

pytestmark = pytest.mark.gpu

P_QUANT = 193     # distinct token rows of a quantizer input
P_GEMM = 37       # distinct token rows of a GEMM input
PN_BLOCKS = 7     # distinct 128-row weight blocks of a GEMM input
EPS = 1e-6

QUANT_KINDS = ("rmsnorm_quant", "quant", "silu_mul_quant")


def cases():
    """Distinct (kind, mode, M, K, N) launches of one bench step, in plan order."""
    seen, out = set(), []
    for L in bench.launch_plan():
        key = (L.kind, L.mode, L.M, L.K, L.N)
        if key not in seen:
            seen.add(key)
            out.append(key)
    return out


def _ids(c):
    kind, mode, M, K, N = c
    return f"{kind}-m{mode}-M{M}-K{K}" + (f"-N{N}" if N else "")


def _periodic(M, P):
    return torch.arange(M, device=DEV) % P


# ------------------------------------------------------------- quantizers

def _quant_case(kind, mode, M, K):
    P = min(M, P_QUANT)
    rng = synth.rng_for("bench-launch", kind, mode, M, K)
    idx = _periodic(M, P)
    if kind == "silu_mul_quant":
        src = synth.gen_gate_up(rng, P, K)
        q, s = fq.silu_mul_quant(bf16_dev(src)[idx], mode)
        qr, sr = quant.silu_mul_quant(src, mode)
    elif kind == "quant":
        src = synth.gen_activations(rng, P, K)
        q, s = fq.quant(bf16_dev(src)[idx], mode)
        qr, sr = quant.quantize(src, mode)
    else:
        src = synth.gen_activations(rng, P, K)
        w = synth.gen_rms_weight(rng, K)
        q, s = fq.rmsnorm_quant(bf16_dev(src)[idx].contiguous(), bf16_dev(w), EPS, mode)
        qr = None
    torch.cuda.synchronize()
    if qr is not None:
        assert np.array_equal(host(q[:P]), qr)
        assert np.array_equal(host(s[:P]).view(np.uint32), sr.view(np.uint32))
    else:
        # rows [0, P) of the full-size launch are the P source rows: against
        # the oracle with the rounding-tie policy
        compare_rms(host(q[:P]), host(s[:P]), src, w, mode)
    # every row equals its source row
    assert torch.equal(q, q[idx]), "a row differs from its source row"
    assert torch.equal(s.view(torch.int32), s[idx].view(torch.int32))


# ------------------------------------------------------------------ GEMMs

@functools.lru_cache(maxsize=4)
def _weights(op, K, PN):
    """PN realistic weight rows (N(0, 0.02), quantized per output channel or
    per 128x128 block by the oracle) for a K."""
    rng = synth.rng_for("bench-launch-weights", op, K, PN)
    W = synth.gen_linear_weight(rng, PN, K)
    return quant.quant_weight_per_channel(W) if op == "scaled_mm" else \
        quant.quant_weight_block128(W)


def _gemm_inputs(kind, M, K, N):
    op = "scaled_mm" if kind == "scaled_mm" else "blockwise"
    P = min(M, P_GEMM)
    PN = min(N, 128 * PN_BLOCKS)
    rng = synth.rng_for("bench-launch", kind, M, K, N)
    x = synth.gen_activations(rng, P, K)
    a, sa = quant.quantize(x, quant.PER_TOKEN if op == "scaled_mm" else quant.GROUP128)
    b, sb = _weights(op, K, PN)
    ridx, cidx = _periodic(M, P), _periodic(N, PN)
    a_d = u8_dev(a)[ridx].contiguous()
    sa_d = f32_dev(sa)[ridx].contiguous()
    b_d = u8_dev(b)[cidx].contiguous()
    if op == "scaled_mm":
        sb_d = f32_dev(sb)[cidx].contiguous()
        ref = gemm.scaled_mm(a, b, sa, sb)
    else:
        sb_d = f32_dev(sb)[_periodic(N // 128, PN // 128)].contiguous()
        ref = gemm.scaled_mm_blockwise(a, sa, b, sb)
    return (a_d, b_d, sa_d, sb_d), torch.from_numpy(ref).to(DEV), ridx, cidx


def _acceptance_periodic(y, ref_p, ridx, cidx):
    """oracle.gemm's acceptance rule for y [M, N] (bf16, on the GPU) against
    the reference ref[m, n] = ref_p[ridx[m], cidx[n]] (float64), evaluated
    on the GPU."""
    ref = ref_p[ridx][:, cidx]
    out = y.double()
    if not bool(torch.isfinite(out).all()):
        return {"ok": False, "finite": False}
    diff = out - ref
    nref = float(torch.linalg.vector_norm(ref))
    rel_fro = float(torch.linalg.vector_norm(diff)) / nref
    rms = float(torch.sqrt(torch.mean(ref * ref)))
    big = ref.abs() > gemm.ELEM_FLOOR * rms
    max_rel = float((diff.abs()[big] / ref.abs()[big]).max()) if bool(big.any()) else 0.0
    ok = rel_fro <= gemm.REL_FRO_TOL and max_rel <= gemm.REL_ELEM_TOL
    return {"ok": ok, "finite": True, "rel_fro": rel_fro, "max_rel_elem": max_rel}


def _gemm_case(kind, M, K, N):
    (a, b, sa, sb), ref_p, ridx, cidx = _gemm_inputs(kind, M, K, N)
    if kind == "scaled_mm":
        y = fq.scaled_mm(a, b, sa, sb)
    else:
        y = fq.scaled_mm_blockwise(a, b, sa, sb)
    torch.cuda.synchronize()
    res = _acceptance_periodic(y, ref_p, ridx, cidx)
    assert res["ok"], res


def _fused_case(M, K, N):
    """gate_up GEMM with the SiLU-and-mul quantizer in its epilogue."""
    (a, b, sa, sb), ref_p, ridx, cidx = _gemm_inputs("scaled_mm_blockwise", M, K, N)
    qf, sf = fq.scaled_mm_blockwise_silu_quant(a, b, sa, sb)
    tile = next(i for i in range(fq.fp8q_gemm_num_configs())
                if fq.fp8q_gemm_config_name(i) == "f16_tiled_m128_n256_w2x4_st3")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    fq.fp8q_scaled_mm_blockwise(y, a, b, sa, sb, None, tile)
    q2, s2 = fq.silu_mul_quant(y, fq.GROUP128)
    torch.cuda.synchronize()
    assert torch.equal(qf, q2), int((qf != q2).sum())
    assert torch.equal(sf.view(torch.int32), s2.view(torch.int32))
    res = _acceptance_periodic(y, ref_p, ridx, cidx)
    assert res["ok"], res
    rows = np.sort(np.random.default_rng(M).choice(M, 16, replace=False))
    r = torch.from_numpy(rows).to(DEV)
    qo, so = quant.silu_mul_quant(bf16_host(y[r]), quant.GROUP128)
    assert np.array_equal(host(qf[r]), qo)
    assert np.array_equal(host(sf[r]).view(np.uint32), so.view(np.uint32))


@pytest.mark.parametrize("case", cases(), ids=[_ids(c) for c in cases()])
def test_bench_launch(case):
    kind, mode, M, K, N = case
    say("bench launch", _ids(case))
    if kind in QUANT_KINDS:
        _quant_case(kind, mode, M, K)
    elif kind == "scaled_mm_blockwise_silu_quant":
        _fused_case(M, K, N)
    else:
        _gemm_case(kind, M, K, N)
