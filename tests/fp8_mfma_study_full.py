"""Measurement (GPU): the FP8-MFMA engine against the GEMM contract at the
full Qwen3 workload shapes.

The committed small study (tests/fp8_mfma_study.py) samples 256 x 1024
outputs per workload through the CPU oracle.  Here every output of the
real shapes is checked: operands are made on the GPU with the bench's
recipe (activations through the library's RMSNorm or SiLU-and-mul
quantizer, N(0, 0.02) weights quantized per channel or per 128x128 block
with torch ops), and the reference is the exact dequantized product in
fp64 (torch matmul on the GPU: every e4m3 x fp32-scale value is exact in
fp64, and K <= 25600 sums keep ~1e-13 relative accuracy, far inside the
contract).  Both engines are compared with it: the FP8-MFMA engine (a
non-conforming f8_ variant, registered only with
FP8Q_NONCONFORMING_FP8_MFMA=1, set here before the library loads) and the
exact engine (the table's f16_ choice).  Not a pytest module.

    python tests/fp8_mfma_study_full.py OUT.md
"""
import os
import sys

os.environ["FP8Q_NONCONFORMING_FP8_MFMA"] = "1"
HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

import torch  # noqa: E402

import fp8_block_scaled_rms_amd as fq  # noqa: E402

REL_FRO_TOL, REL_ELEM_TOL, ELEM_FLOOR = 4e-3, 1.6e-2, 1e-2
F8_VARIANT = "f8_tiled_m128_n128_w2x2_st2"

# (name, op, M, N, K, activation source)
SHAPES = [
    ("qwen3-1.7b qkv (per-token)", "mm", 2048, 4096, 2048, "x"),
    ("qwen3-1.7b gate_up (per-token)", "mm", 2048, 12288, 2048, "x"),
    ("qwen3-1.7b down (per-token)", "mm", 2048, 2048, 6144, "silu"),
    ("qwen3-8b gate_up (blockwise, decode M=32)", "bw", 32, 24576, 4096, "x"),
    ("qwen3-8b down (blockwise, decode M=32)", "bw", 32, 4096, 12288, "silu"),
    ("qwen3-32b qkv (blockwise)", "bw", 8192, 10240, 5120, "x"),
    ("qwen3-32b o_proj (blockwise)", "bw", 8192, 5120, 8192, "x"),
    ("qwen3-32b gate_up (blockwise)", "bw", 8192, 51200, 5120, "x"),
    ("qwen3-32b down (blockwise)", "bw", 8192, 5120, 25600, "silu"),
    ("qwen3-32b MLP tail down (blockwise)", "bw", 4096, 5120, 25600, "silu"),
]


def inputs(op, M, N, K, src, gen, dev):
    mode = fq.PER_TOKEN if op == "mm" else fq.GROUP128
    if src == "x":
        x = torch.randn((M, K), generator=gen, device=dev)
        cols = torch.randperm(K, generator=gen, device=dev)[: int(round(0.01 * K))]
        x[:, cols] *= 20.0
        w = (1.0 + 0.1 * torch.randn((K,), generator=gen, device=dev)).to(torch.bfloat16)
        a, sa = fq.rmsnorm_quant(x.to(torch.bfloat16).contiguous(), w, 1e-6, mode)
    else:
        gu = (2.0 * torch.randn((M, 2 * K), generator=gen, device=dev)).to(torch.bfloat16)
        a, sa = fq.silu_mul_quant(gu, mode)
    wt = 0.02 * torch.randn((N, K), generator=gen, device=dev)
    if op == "mm":
        sb = wt.abs().amax(dim=1) / 448.0
        b = (wt / sb[:, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    else:
        blk = wt.view(N // 128, 128, K // 128, 128)
        sb = blk.abs().amax(dim=(1, 3)) / 448.0
        b = (blk / sb[:, None, :, None]).clamp(-448, 448).to(torch.float8_e4m3fn)
        b = b.view(torch.uint8).view(N, K)
    return a, sa.float().contiguous(), b.contiguous(), sb.float().contiguous()


def dequant(q, s, op):
    v = q.view(torch.float8_e4m3fn).to(torch.float64)
    if op == "mm" or s.dim() == 1:
        return v * s.to(torch.float64)[:, None]
    R, K = v.shape
    if s.shape[0] == R:  # activation groups [M, K/128]
        return (v.view(R, K // 128, 128) * s.to(torch.float64)[:, :, None]).view(R, K)
    return (v.view(R // 128, 128, K // 128, 128)  # weight blocks [N/128, K/128]
            * s.to(torch.float64)[:, None, :, None]).view(R, K)


def check(y, ref):
    """Contract quantities of y (bf16) against the fp64 reference, by rows."""
    ref_sq = float((ref * ref).sum())
    rms = (ref_sq / ref.numel()) ** 0.5
    err_sq, max_rel, over, counted = 0.0, 0.0, 0, 0
    for r0 in range(0, ref.shape[0], 1024):
        rr = ref[r0:r0 + 1024]
        d = y[r0:r0 + 1024].to(torch.float64) - rr
        err_sq += float((d * d).sum())
        big = rr.abs() > ELEM_FLOOR * rms
        rel = (d.abs() / rr.abs().clamp_min(1e-300))[big]
        counted += int(big.sum())
        if rel.numel():
            max_rel = max(max_rel, float(rel.max()))
            over += int((rel > REL_ELEM_TOL).sum())
    return {"rel_fro": (err_sq / ref_sq) ** 0.5, "max_rel": max_rel, "over": over,
            "counted": counted}


def main(out_path):
    dev = "cuda:0"
    names = {fq.fp8q_gemm_config_name(i): i for i in range(fq.fp8q_gemm_num_configs())}
    f8 = names[F8_VARIANT]
    gen = torch.Generator(device=dev)
    lines = ["# FP8-MFMA engine against the GEMM contract at the full Qwen3 shapes", "",
             "Command: `python tests/fp8_mfma_study_full.py OUT.md` (sets "
             "FP8Q_NONCONFORMING_FP8_MFMA=1 itself)", "",
             f"FP8 engine: `{F8_VARIANT}` (v_mfma_scale_f32_16x16x128_f8f6f4). Exact engine: "
             "the table's f16_ variant. Reference: the dequantized product in fp64 on the GPU. "
             f"Contract: rel. Frobenius <= {REL_FRO_TOL}, rel. error <= {REL_ELEM_TOL} per "
             f"element wherever |ref| > {ELEM_FLOOR} rms(ref).", "",
             "| GEMM | M x N x K | outputs checked | FP8 engine: over 1.6e-2 | max rel. | "
             "rel. Frobenius | exact engine: over 1.6e-2 | max rel. | rel. Frobenius |",
             "|---|---|---|---|---|---|---|---|---|"]
    for i, (name, op, M, N, K, src) in enumerate(SHAPES):
        print("[case]", name, M, N, K, flush=True)
        gen.manual_seed(0x5EED + i)
        a, sa, b, sb = inputs(op, M, N, K, src, gen, dev)
        ref = dequant(a, sa, op) @ dequant(b, sb, op).t().contiguous()
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        run = fq.fp8q_scaled_mm if op == "mm" else fq.fp8q_scaled_mm_blockwise
        res = []
        for cfg in (f8, fq.fp8q_gemm_config_for(fq.OP_SCALED_MM if op == "mm"
                                                else fq.OP_SCALED_MM_BLOCKWISE, M, N, K)):
            nws = fq.fp8q_workspace_size(fq.OP_SCALED_MM if op == "mm"
                                         else fq.OP_SCALED_MM_BLOCKWISE, M, N, K, cfg)
            ws = torch.empty((nws + 3) // 4, dtype=torch.float32, device=dev) if nws else None
            run(y, a, b, sa, sb, ws, cfg)
            torch.cuda.synchronize()
            res.append(check(y, ref))
            del ws
        r8, rx = res
        lines.append(f"| {name} | {M} x {N} x {K} | {r8['counted']} | {r8['over']} | "
                     f"{r8['max_rel']:.2e} | {r8['rel_fro']:.2e} | {rx['over']} | "
                     f"{rx['max_rel']:.2e} | {rx['rel_fro']:.2e} |")
        print(lines[-1], flush=True)
        del a, sa, b, sb, ref, y
        torch.cuda.empty_cache()
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else "fp8_mfma_study_full.md")
