"""The compiled-in GEMM dispatch table is a function of the committed
measurements (CPU only): regenerating it from csrc/tune_results.jsonl gives
csrc/tune_table.inc byte for byte, every shape the tuner measures has
results, and every variant the table names is one the library registers."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from fp8_block_scaled_rms_amd import tune  # noqa: E402
import fp8_block_scaled_rms_amd as fq  # noqa: E402


def test_table_regenerates_byte_for_byte():
    rows = tune.exact_choices(tune.load_results(tune.RESULTS_FILE))
    with open(tune.TABLE_FILE) as f:
        assert f.read() == tune.table_text(rows)


def test_every_tuned_shape_is_measured():
    done = tune.load_results(tune.RESULTS_FILE)
    shapes = {k[:4] for k in done}
    missing = [sh for sh in tune.SHAPES if tuple(sh) not in shapes]
    assert not missing, missing


def test_table_names_registered_exact_variants():
    names = {fq.fp8q_gemm_config_name(i) for i in range(fq.fp8q_gemm_num_configs())}
    names = {n.decode() if isinstance(n, bytes) else n for n in names}
    rows = tune.exact_choices(tune.load_results(tune.RESULTS_FILE))
    for op, M, N, K, name in rows:
        assert name in names, name
        assert name.startswith("i8_" if op == tune.I8 else "f16_"), (op, name)


def test_noalloc_test_shapes_split_k():
    """tests/test_zz_no_alloc.py exercises the scratch array on shapes whose
    table variant splits K; a regenerated table must keep them splitting."""
    pairs = [((4096, 5120, 25600), (64, 5120, 25600)), ((64, 5120, 25600), (32, 4096, 12288)),
             ((32, 4096, 12288), (16, 4096, 12288))]
    for pair in pairs:
        needs = [fq.fp8q_workspace_size(fq.OP_SCALED_MM_BLOCKWISE, *s) for s in pair]
        assert all(n > 0 for n in needs), (pair, needs)
        assert needs[1] < needs[0], (pair, needs)  # the second call is the smaller
        assert needs[0] <= 64 << 20
    big = fq.fp8q_workspace_size(fq.OP_SCALED_MM_BLOCKWISE, 1024, 5120, 25600)
    assert big > 64 << 20  # the oversized case the no-alloc entry rejects


def test_choice_is_the_fastest_and_ties_break_by_name():
    done = {(1, 8, 256, 512, "f16_b"): 2.0, (1, 8, 256, 512, "f16_a"): 2.0,
            (1, 8, 256, 512, "f8_c"): 1.0, (1, 16, 256, 512, "f16_b"): 3.0,
            (1, 16, 256, 512, "f16_a"): 4.0}
    assert tune.exact_choices(done) == [(1, 8, 256, 512, "f16_a"), (1, 16, 256, 512, "f16_b")]
    text = tune.table_text(tune.exact_choices(done))
    assert text.splitlines()[-2:] == ['{1, 256, 512, 8, "f16_a"},',
                                      '{1, 256, 512, 1073741824, "f16_b"},']
