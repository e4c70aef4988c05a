"""Measure every applicable GEMM variant per shape on the GPU and write the
per-shape dispatch table (csrc/tune_table.inc).

The table is how the library picks, per (op, N, K, M), between the tiled
kernel, the weight-streaming small-M kernel and their split-K / tile-shape
parameters (page "Helion can accelerate vLLM LLM inference on NVIDIA GPUs",
aihirek.info, section "Autotuning picks the right variant": the algorithm is
a tuned parameter chosen per shape instead of a hand-written rule).

    python -m fp8_block_scaled_rms_amd.tune --out results.jsonl [--write-table PATH]
        [--engine exact|fp8|all] [--shapes default|quick|large|int8|small|tail]
        [--remeasure]
    python -m fp8_block_scaled_rms_amd.tune --from-results RESULTS --write-table PATH

Results are appended to a JSONL file, one line per (shape, variant), and a
rerun skips what the file already holds (resumable).  Timing: HIP events
around a batch of back-to-back launches on the current stream (mean per
launch, median of three batches); every repetition reads its own copy of
the weights, rotating through >= 1 GiB of copies, so no run is served by the
256 MB last-level cache.

The committed table is a pure function of the committed results file
(csrc/tune_results.jsonl): --from-results rewrites it without a GPU, byte
for byte (a CPU test checks that it does).
"""
from __future__ import annotations

import argparse
import json
import os
import sys

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import fp8_block_scaled_rms_amd as fq  # noqa: E402

MM, BW, I8 = fq.OP_SCALED_MM, fq.OP_SCALED_MM_BLOCKWISE, fq.OP_SCALED_MM_INT8

# every GEMM of the Qwen3 FP8 workloads
SHAPES = (
    [(MM, M, N, K) for M in (1, 16, 128, 512, 2048)
     for N, K in ((4096, 2048), (2048, 2048), (12288, 2048), (2048, 6144))]
    + [(BW, M, N, K) for M in (1, 2, 4, 8, 16, 32)
       for N, K in ((6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288))]
    + [(BW, M, N, K) for M in (2048, 8192)
       for N, K in ((10240, 5120), (5120, 8192), (51200, 5120), (5120, 25600))]
    + [(BW, 64, 5120, 25600), (BW, 4096, 5120, 25600), (BW, 16, 512, 256)]
    # W8A8 INT8 on the Qwen3-1.7B per-token shapes
    + [(I8, M, N, K) for M in (1, 16, 128, 512, 2048)
       for N, K in ((4096, 2048), (2048, 2048), (12288, 2048), (2048, 6144))]
)
# M buckets between measured M values are served by the next larger one
QUICK = [(BW, 8192, 51200, 5120), (BW, 2048, 10240, 5120), (BW, 32, 24576, 4096),
         (BW, 1, 4096, 4096), (MM, 2048, 12288, 2048), (MM, 128, 12288, 2048)]
LARGE = [(BW, M, N, K) for M in (2048, 8192)
         for N, K in ((10240, 5120), (5120, 8192), (51200, 5120), (5120, 25600))]
# shapes whose 128x256 tiles leave the last round of workgroups part-empty
# (where the hybrid variants can differ from their unsplit part)
TAIL = [(BW, 2048, 10240, 5120), (BW, 2048, 5120, 8192), (BW, 2048, 5120, 25600),
        (BW, 4096, 5120, 25600)]


def variants(op, M, N, K, engine):
    out = []
    for i in range(fq.fp8q_gemm_num_configs()):
        name = fq.fp8q_gemm_config_name(i)
        if (op == I8) != name.startswith("i8_"):  # engines serve their own op only
            continue
        if op != I8 and engine == "exact" and not name.startswith("f16_"):
            continue
        if op != I8 and engine == "fp8" and not name.startswith("f8_"):
            continue
        if "_skinny_" in name:
            tm = int(name.split("_skinny_t")[1].split("_")[0])
            if M > 16 * tm or (tm > 1 and M <= 8 * tm):  # too small a fit is pointless
                continue
            rw = int(name.split("_r")[1].split("_")[0])
            if N % (16 * rw):
                continue
        else:
            if M <= 16:
                continue
            bn = int(name.split("_n")[1].split("_")[0])
            if N % bn:
                continue
        out.append((i, name))
    return out


BATCHES = 3

# GPU clock cycles of the spin kernel that the timed launches queue behind
# (a few milliseconds, longer than the host needs to issue them)
QUEUE_AHEAD_CYCLES = 8_000_000


def time_shape(op, M, N, K, cands, reps=10):
    dev = "cuda:0"
    g = torch.Generator(device=dev)
    g.manual_seed(M * 7919 + N * 31 + K)
    wbytes = N * K
    copies = max(1, min(reps, (1 << 30) // max(wbytes, 1) + 1))
    if op == I8:
        a = torch.randint(-127, 128, (M, K), generator=g, device=dev, dtype=torch.int8)
        bs = [torch.randint(-127, 128, (N, K), generator=g, device=dev, dtype=torch.int8)
              for _ in range(copies)]
    else:
        a = torch.randint(0, 255, (M, K), generator=g, device=dev, dtype=torch.uint8) & 0xF7
        bs = [torch.randint(0, 255, (N, K), generator=g, device=dev, dtype=torch.uint8) & 0xF7
              for _ in range(copies)]
    if op in (MM, I8):
        sa = torch.rand(M, generator=g, device=dev) + 0.5
        sb = torch.rand(N, generator=g, device=dev) + 0.5
    else:
        sa = torch.rand(M, K // 128, generator=g, device=dev) + 0.5
        sb = torch.rand(N // 128, K // 128, generator=g, device=dev) + 0.5
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    res = {}
    for cfg, name in cands:
        nws = fq.fp8q_workspace_size(op, M, N, K, cfg)
        ws = torch.empty((nws + 3) // 4, dtype=torch.float32, device=dev) if nws else None

        def run(b):
            if op == MM:
                fq.fp8q_scaled_mm(y, a, b, sa, sb, ws, cfg)
            elif op == I8:
                fq.fp8q_scaled_mm_int8(y, a, b, sa, sb, ws, cfg)
            else:
                fq.fp8q_scaled_mm_blockwise(y, a, b, sa, sb, ws, cfg)

        for w in range(2):
            run(bs[w % copies])
        # Back-to-back launches between two events, all queued behind a spin
        # kernel: the GPU then runs them without waiting for the host, whose
        # per-call cost through this binding (about 10 us) exceeds a small
        # kernel's duration.  Per-launch events would add their own overhead.
        batches = []
        for _ in range(BATCHES):
            torch.cuda.synchronize()
            torch.cuda._sleep(QUEUE_AHEAD_CYCLES)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for r in range(reps):
                run(bs[r % copies])
            e1.record()
            torch.cuda.synchronize()
            batches.append(e0.elapsed_time(e1) * 1e3 / reps)
        res[name] = sorted(batches)[BATCHES // 2]
    return res


RESULTS_FILE = os.path.join(HERE, "csrc", "tune_results.jsonl")
TABLE_FILE = os.path.join(HERE, "csrc", "tune_table.inc")


def load_results(path):
    """{(op, M, N, K, variant): us}; a later line for the same key wins."""
    done = {}
    if os.path.exists(path):
        with open(path) as f:
            for line in f:
                if line.strip():
                    r = json.loads(line)
                    done[(r["op"], r["M"], r["N"], r["K"], r["variant"])] = r["us"]
    return done


def exact_choices(done):
    """Per measured shape, the fastest variant of the engine that meets the
    GEMM tolerance: f16_ (e4m3 widened exactly to f16) for the FP8 ops, i8_
    for int8.  The FP8-MFMA engine's (f8_) grouped truncation is outside the
    tolerance, so its times never pick a table row."""
    per_shape = {}
    for (op, M, N, K, name), us in done.items():
        if name.startswith(("f16_", "i8_")):
            per_shape.setdefault((op, M, N, K), {})[name] = us
    # ties go to the name that sorts first, so the choice is a function of the times
    return [(op, M, N, K, min(sorted(c), key=c.get))
            for (op, M, N, K), c in sorted(per_shape.items())]


def table_text(rows):
    """rows: list of (op, M, N, K, best_name).  One table row per measured M;
    the row's M_max is that M, the largest measured M of a family also
    serves everything above it."""
    fam = {}
    for op, M, N, K, name in rows:
        fam.setdefault((op, N, K), []).append((M, name))
    lines = ["// Per-shape GEMM variant table: {op, N, K, M_max, variant name}.",
             "// op 0 = scaled_mm, 1 = scaled_mm_blockwise, 2 = scaled_mm_int8.  For a call",
             "// (op, M, N, K) the first row with the same op, N and K and M <= M_max wins;",
             "// shapes absent from the table use the built-in rule in dispatch.cpp.",
             "// Generated from the MI355X times in tune_results.jsonl (no hand edits) by",
             "// python -m fp8_block_scaled_rms_amd.tune --from-results RESULTS --write-table",
             "// TABLE, with RESULTS and TABLE that file and this one (in csrc/)."]
    for (op, N, K), ms in sorted(fam.items()):
        ms.sort()
        for j, (M, name) in enumerate(ms):
            m_max = M if j + 1 < len(ms) else 1 << 30
            lines.append(f'{{{op}, {N}, {K}, {m_max}, "{name}"}},')
    return "\n".join(lines) + "\n"


def write_table(rows, path):
    with open(path, "w") as f:
        f.write(table_text(rows))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default="tune_results.jsonl")
    ap.add_argument("--engine", default="exact", choices=["exact", "fp8", "all"])
    ap.add_argument("--shapes", default="default",
                    choices=["default", "quick", "large", "int8", "small", "tail"])
    ap.add_argument("--remeasure", action="store_true",
                    help="first drop the results file's rows of the selected shapes, so that "
                         "every variant of each is timed again in this run")
    ap.add_argument("--write-table", default=None, help="path of the table to write")
    ap.add_argument("--from-results", default=None,
                    help="write the table from this results file without measuring")
    ap.add_argument("--reps", type=int, default=20)
    args = ap.parse_args()
    if args.from_results:
        if not args.write_table:
            ap.error("--from-results needs --write-table")
        write_table(exact_choices(load_results(args.from_results)), args.write_table)
        return
    shapes = {"default": SHAPES, "quick": QUICK, "large": LARGE, "tail": TAIL,
              "int8": [sh for sh in SHAPES if sh[0] == I8],
              "small": [sh for sh in SHAPES if sh[0] != I8 and sh[1] <= 128]}[args.shapes]
    if args.remeasure and os.path.exists(args.out):
        keep = []
        with open(args.out) as f:
            for line in f:
                r = json.loads(line) if line.strip() else None
                if r is not None and (r["op"], r["M"], r["N"], r["K"]) not in shapes:
                    keep.append(line if line.endswith("\n") else line + "\n")
        with open(args.out, "w") as f:
            f.writelines(keep)
    done = load_results(args.out)
    with open(args.out, "a") as f:
        for op, M, N, K in shapes:
            cands = variants(op, M, N, K, args.engine)
            todo = [(c, n) for c, n in cands if (op, M, N, K, n) not in done]
            if todo:
                res = time_shape(op, M, N, K, todo, args.reps)
                for n, us in res.items():
                    done[(op, M, N, K, n)] = us
                    f.write(json.dumps({"op": op, "M": M, "N": N, "K": K, "variant": n,
                                        "us": round(us, 3)}) + "\n")
                f.flush()
            mine = {n: done[(op, M, N, K, n)] for _, n in cands}
            best = min(mine, key=mine.get)
            flops = 2.0 * M * N * K
            byts = M * K + N * K + 2 * M * N
            print(f"op{op} M={M:5d} N={N:6d} K={K:6d} best {best:30s} {mine[best]:9.1f}us "
                  f"{flops / mine[best] / 1e6:8.1f}TF {byts / mine[best] / 1e3:7.0f}GB/s "
                  f"({len(mine)} variants)", flush=True)
    if args.write_table:
        # the same function of the results file as --from-results
        write_table(exact_choices(load_results(args.out)), args.write_table)


if __name__ == "__main__":
    main()
