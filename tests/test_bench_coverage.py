"""CPU checks that the GPU parity tests reach every kernel instantiation the
benchmark times.

bench.launch_plan() lists every launch of a bench step; the GPU test
test_gpu_bench_launches runs one case per distinct (kind, mode, M, K, N) of
that list at the same size, so it reaches the same quantizer unit shape
(threads per unit, chunks per thread: the kernel's template arguments) and
the same table variant.  The choice is replayed here through the library's
host-only queries, for the MI355X's 256 compute units.
"""
import bench
import fp8_block_scaled_rms_amd as fq

import test_gpu_bench_launches as gpu_cases

NUM_CUS = 256
FRONT = {"quant": fq.FRONT_IDENT, "rmsnorm_quant": fq.FRONT_RMSNORM,
         "silu_mul_quant": fq.FRONT_SILU}
OP = {"scaled_mm": fq.OP_SCALED_MM, "scaled_mm_blockwise": fq.OP_SCALED_MM_BLOCKWISE}


def _instantiation(kind, mode, M, K, N):
    if kind in FRONT:
        tpr, ch, _ = fq.fp8q_quant_launch_config(FRONT[kind], mode, M, K, NUM_CUS)
        return ("quant", FRONT[kind], mode, tpr, ch)
    if kind in OP:
        cfg = fq.fp8q_gemm_config_for(OP[kind], M, N, K)
        assert cfg >= 0, (kind, M, N, K)
        return ("gemm", OP[kind], fq.fp8q_gemm_config_name(cfg))
    return ("fused", kind)


def test_gpu_cases_cover_every_bench_launch():
    tested = set(gpu_cases.cases())
    for L in bench.launch_plan():
        assert (L.kind, L.mode, L.M, L.K, L.N) in tested, L.label


def test_every_bench_instantiation_is_tested():
    tested = {_instantiation(*c) for c in gpu_cases.cases()}
    timed = {_instantiation(L.kind, L.mode, L.M, L.K, L.N) for L in bench.launch_plan()}
    assert timed <= tested, sorted(map(str, timed - tested))


def test_named_instantiations_are_reached():
    """Quantizer instantiations the bench times at large row counts (among
    them 1.7B SiLU-and-mul and attention-output quantization at M=2048 and
    the 32B attention output at K=8192): each is reached by a bench launch,
    hence by a GPU case."""
    timed = {_instantiation(L.kind, L.mode, L.M, L.K, L.N) for L in bench.launch_plan()}
    # (front end, mode, threads per unit, chunks per thread)
    for want in [(fq.FRONT_SILU, fq.PER_TOKEN, 128, 6),
                 (fq.FRONT_IDENT, fq.PER_TOKEN, 128, 2),
                 (fq.FRONT_IDENT, fq.GROUP128, 64, 4)]:
        assert ("quant",) + want in timed, want


def test_quant_launch_config_matches_the_call_checks():
    """The host query rejects what the calls reject."""
    assert fq.lib().fp8q_quant_launch_config(1, 1, 4, 200, NUM_CUS, None, None, None) != 0
    import pytest
    with pytest.raises(fq.Fp8qError):
        fq.fp8q_quant_launch_config(fq.FRONT_RMSNORM, fq.GROUP128, 4, 200, NUM_CUS)
    with pytest.raises(fq.Fp8qError):
        fq.fp8q_quant_launch_config(fq.FRONT_RMSNORM, 9, 4, 256, NUM_CUS)
    with pytest.raises(fq.Fp8qError):
        fq.fp8q_quant_launch_config(7, fq.PER_TOKEN, 4, 256, NUM_CUS)
    tpr, ch, grid = fq.fp8q_quant_launch_config(fq.FRONT_RMSNORM, fq.GROUP128, 8192, 5120,
                                                NUM_CUS)
    assert tpr in (64, 128, 256) and ch * 8 * tpr >= 5120 and grid > 0


def test_rmsnorm_launches_loop_over_rows():
    """RMSNorm launches are sized so that workgroups loop over rows (each
    wave prefetches its next row): at the bench's large row counts a
    workgroup handles more than one unit, so the GPU cases at those sizes run
    the prefetching loop, including a prefetch past the last row."""
    for M, K in [(2048, 5120), (8192, 5120), (2048, 2048)]:
        tpr, ch, grid = fq.fp8q_quant_launch_config(fq.FRONT_RMSNORM, fq.GROUP128, M, K, NUM_CUS)
        units_per_block = 256 // tpr
        assert grid <= NUM_CUS * 3, (M, K, grid)  # at most 12 waves per compute unit
        assert grid * units_per_block < M, (M, K, tpr, grid)
    # the other front ends keep their larger grids
    _, _, grid = fq.fp8q_quant_launch_config(fq.FRONT_IDENT, fq.GROUP128, 8192, 8192, NUM_CUS)
    assert grid > NUM_CUS * 3
