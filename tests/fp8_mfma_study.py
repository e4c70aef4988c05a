"""Measurement (GPU): the FP8-MFMA engine against the GEMM contract.

Runs the non-conforming f8_ variants (registered only with
FP8Q_NONCONFORMING_FP8_MFMA=1, set here before the library loads) and the
exact engine's table choice on the realistic Qwen3 inputs of
tests/fp8_mfma_model.py, and writes a markdown table of the contract's
quantities against the oracle, plus how closely the hardware follows the
truncation model.  Not a pytest module: nothing here is a pass/fail check of
a selectable variant.

    FP8Q_NONCONFORMING_FP8_MFMA=1 python tests/fp8_mfma_study.py OUT.md
"""
import os
import sys

os.environ["FP8Q_NONCONFORMING_FP8_MFMA"] = "1"
HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import fp8_block_scaled_rms_amd as fq  # noqa: E402
import fp8_mfma_model as m  # noqa: E402
from gpu_util import bf16_host_f64, f32_dev, u8_dev  # noqa: E402
from oracle import gemm  # noqa: E402

M, N = 256, 1024
VARIANT = "f8_tiled_m128_n128_w2x2_st2"


def main(out_path):
    names = {fq.fp8q_gemm_config_name(i): i for i in range(fq.fp8q_gemm_num_configs())}
    f8 = names[VARIANT]
    lines = [f"# FP8-MFMA engine against the GEMM contract ({M} tokens x {N} weight rows "
             "per workload, realistic inputs)", "",
             "Command: `FP8Q_NONCONFORMING_FP8_MFMA=1 python tests/fp8_mfma_study.py OUT.md`",
             "", f"FP8 engine variant `{VARIANT}` "
             "(v_mfma_scale_f32_16x16x128_f8f6f4); exact engine: the table's f16_ variant.", "",
             "| workload GEMM | K | FP8 engine max rel. elem | FP8 rel. Frobenius | elements over "
             "1.6e-2 | exact engine max rel. elem | exact rel. Frobenius | FP8 engine outputs equal "
             "to the truncation model's |",
             "|---|---|---|---|---|---|---|---|"]
    for name, op, K, src in m.CONFIGS:
        print("[case]", name, K, flush=True)
        a, sa, b, sb = m.config_inputs(op, K, src, M=M, N=N, seed_tag="fp8-mfma-study")
        ref = m.reference(op, a, sa, b, sb)
        at, bt, sat, sbt = u8_dev(a), u8_dev(b), f32_dev(sa), f32_dev(sb)
        run = fq.scaled_mm if op == "mm" else fq.scaled_mm_blockwise
        y8 = bf16_host_f64(run(at, bt, sat, sbt, cfg=f8))
        yx = bf16_host_f64(run(at, bt, sat, sbt))
        torch.cuda.synchronize()
        r8, rx = gemm.acceptance(y8, ref), gemm.acceptance(yx, ref)
        rms = np.sqrt(np.mean(ref * ref))
        big = np.abs(ref) > gemm.ELEM_FLOOR * rms
        over = int(np.sum(np.abs(y8 - ref)[big] > gemm.REL_ELEM_TOL * np.abs(ref)[big]))
        model = m.fp8_mfma_gemm(a[:16], b, sa[:16], sb, op == "bw")
        same = float(np.mean(y8[:16] == model))
        lines.append(f"| {name} | {K} | {r8['max_rel_elem']:.2e} | {r8['rel_fro']:.2e} | "
                     f"{over} of {int(big.sum())} | {rx['max_rel_elem']:.2e} | "
                     f"{rx['rel_fro']:.2e} | {100 * same:.1f} % |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else "fp8_mfma_study.md")
