"""Benchmark of the FP8 quantized-linear hot path on one MI355X.

One step = the FP8 linear layers of a Qwen3 decoder layer for every workload
of the Qwen3 FP8 inference runs (page "Helion in vLLM: FP8 inference of
Qwen3", 24-ai.news, sections "Kernels integrated into vLLM" and "Whole-model
speedup"), M from 1 to 8192:

  qwen3-1.7b per-token (hidden 2048)  M in 1,16,128,512,2048:
      rmsnorm_quant -> scaled_mm qkv; quant(attn out) -> scaled_mm o_proj;
      rmsnorm_quant -> scaled_mm gate_up; silu_mul_quant -> scaled_mm down
  qwen3-8b block decode (hidden 4096)  M in 1,2,4,8,16,32:   same chain with
      1x128 group quantization and scaled_mm_blockwise
  qwen3-32b block prefill (hidden 5120) M in 2048,8192:       same chain
  qwen3-32b MLP tail                    M in 64,4096:
      silu_mul_quant(gate_up [M,51200]) -> scaled_mm_blockwise down
  tiny blockwise linear                 M = 16: rmsnorm_quant -> 512x256 GEMM

Inputs are seeded synthetic data of the stated distributions (X ~ N(0,1)
with 1 % outlier columns x20, RMSNorm weight 1+N(0,0.1), gate_up ~ N(0,2),
weights N(0,0.02) quantized per output channel or per 128x128 block), all
resident in HBM before timing.  Every (workload, M) has its own weight copy,
so no GEMM finds its weights in the 256 MB last-level cache from a previous
launch of the same step.

value = GEMM FLOPs of one step / wall time of one step (quantizer kernels
included in the time).  The roofline entry is for the dominant kernel (the
largest share of step time), timed with HIP events on its launch stream
during the timed steps.  The CPU baseline runs the oracle on a bounded
sample of that kernel's workload.  After the timed region, decode_chain
reports the Qwen3-8B decode layer's 8-launch chain per M, launched eagerly
and replayed from a HIP graph, w8a8_int8 the int8 GEMMs on the Qwen3-1.7B
shapes, and ue8m0_blockwise the prefill GEMMs with power-of-two scales.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
F16_PEAK_TFLOPS = 2500.0      # MI355X dense f16/bf16 MFMA
INT8_PEAK_TOPS = 5000.0       # MI355X dense int8 MFMA
HBM_PEAK_GBS = 8000.0

PER_TOKEN, GROUP128 = 0, 1
MM, BW = 0, 1

WORKLOADS = {
    # name: (mode, hidden, (qkv_n, o_k, gate_up_n, inter), Ms)
    "qwen3-1.7b-per-token": (PER_TOKEN, 2048, (4096, 2048, 12288, 6144), (1, 16, 128, 512, 2048)),
    "qwen3-8b-block-decode": (GROUP128, 4096, (6144, 4096, 24576, 12288), (1, 2, 4, 8, 16, 32)),
    "qwen3-32b-block-prefill": (GROUP128, 5120, (10240, 8192, 51200, 25600), (2048, 8192)),
}
MLP_TAIL = ("qwen3-32b-mlp-tail", (64, 4096), 25600, 5120)
TINY = ("tiny-blockwise", 16, 256, 512)
# Workloads whose gate_up projection and SiLU-and-mul quantization run as one
# kernel (fp8q_scaled_mm_blockwise_silu_quant: group-128 mode, large M).
FUSED_MLP = ("qwen3-32b-block-prefill",)
# name and op id under which the fused kernel is reported and its traffic
# recorded (it is not one of the table's variants)
FUSED_VARIANT = "f16_tiled_m128_n256_w2x4_st3_silu_quant"
SQ = 4


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--detail", default=None, help="write a per-kernel breakdown JSON here")
    p.add_argument("--cpu-sample-rows", type=int, default=2048)
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy (3 times), the known-size "
                        "reference for scaling the FETCH_SIZE / WRITE_SIZE counters")
    return p.parse_args()


# HBM traffic of the dominant kernel, measured offline with rocprofv3 PMC
# counters (FETCH_SIZE and WRITE_SIZE, each scaled by the same counter's
# reading for a plain copy of known size).  The record names the kernel
# variant, the shape and a hash of the kernel sources; when any of them
# differs from the kernel measured now, the traffic is reported as null.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic_qwen3_32b_prefill_gate_up_m8192.md")
KERNEL_SOURCES = ("fp8_block_scaled_rms_amd/csrc/gemm_kernels.hip",
                  "fp8_block_scaled_rms_amd/csrc/gemm_kernels.h",
                  "fp8_block_scaled_rms_amd/csrc/fp8q_common.hpp",
                  "fp8_block_scaled_rms_amd/csrc/silu_table.hpp")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(variant, op, M, N, K):
    """Bytes per launch from the committed PMC record, or None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if line.startswith("traffic_record: "):
                r = json.loads(line[len("traffic_record: "):])
                if (r["variant"] == variant and (r["op"], r["M"], r["N"], r["K"]) == (op, M, N, K)
                        and r["kernel_src_sha256_16"] == kernel_source_hash()):
                    return int(r["bytes_per_launch"])
    return None


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                      "launches": 3}), flush=True)


class Step:
    """All launches of one step, with pre-allocated buffers and bound C calls."""

    def __init__(self, fq, torch, dev):
        self.fq, self.torch, self.dev = fq, torch, dev
        self.lib = fq.lib()
        self.calls = []     # (label, kind, flops, bytes, callable)
        self.operands = {}  # GEMM label -> (a, sa, b, sb)
        self.keep = []      # tensors that must stay alive
        self.gen = torch.Generator(device=dev)
        self.gen.manual_seed(20260610)
        self.ws = None
        self.ws_bytes = 0
        self._ws_need = 0
        self.stream = torch.cuda.current_stream().cuda_stream

    # ------------------------------------------------------------ data
    def randn(self, shape, std=1.0):
        t = self.torch.randn(shape, generator=self.gen, device=self.dev, dtype=self.torch.float32)
        return t * std

    def activations(self, M, K):
        x = self.randn((M, K))
        n_out = int(round(0.01 * K))
        cols = self.torch.randperm(K, generator=self.gen, device=self.dev)[:n_out]
        x[:, cols] *= 20.0
        return x.to(self.torch.bfloat16).contiguous()

    def weight(self, N, K, mode):
        """N(0,0.02) fp32 weights quantized with torch ops: per output channel
        (mode PER_TOKEN) or per 128x128 block (GROUP128).  Input preparation
        only; not part of the timed path."""
        torch = self.torch
        w = self.randn((N, K), 0.02)
        if mode == PER_TOKEN:
            s = w.abs().amax(dim=1) / 448.0
            q = (w / s[:, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
        else:
            blk = w.view(N // 128, 128, K // 128, 128)
            s = blk.abs().amax(dim=(1, 3)) / 448.0
            q = (blk / s[:, None, :, None]).clamp(-448, 448).to(torch.float8_e4m3fn)
            q = q.view(torch.uint8).view(N, K)
        del w
        return q.contiguous(), s.float().contiguous()

    def empty(self, shape, dtype):
        t = self.torch.empty(shape, dtype=dtype, device=self.dev)
        self.keep.append(t)
        return t

    # --------------------------------------------------------- launches
    def _check(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what}: status {rc} "
                               f"{self.lib.fp8q_status_string(rc).decode()}")

    def add_rmsnorm(self, label, x, w, mode):
        torch, L = self.torch, self.lib
        M, K = x.shape
        q = self.empty((M, K), torch.uint8)
        s = self.empty((M,) if mode == PER_TOKEN else (M, K // 128), torch.float32)
        args = (q.data_ptr(), s.data_ptr(), x.data_ptr(), w.data_ptr(), M, K, 1e-6, mode,
                self.stream)
        fn = L.fp8q_rmsnorm_quant
        self.calls.append((label, "rmsnorm_quant", 0, 3 * M * K + 2 * K + s.numel() * 4,
                           lambda: self._check(fn(*args), label)))
        self.keep += [x, w]
        return q, s

    def add_silu(self, label, gu, mode):
        torch, L = self.torch, self.lib
        M, twoD = gu.shape
        D = twoD // 2
        q = self.empty((M, D), torch.uint8)
        s = self.empty((M,) if mode == PER_TOKEN else (M, D // 128), torch.float32)
        args = (q.data_ptr(), s.data_ptr(), gu.data_ptr(), M, D, mode, self.stream)
        fn = L.fp8q_silu_mul_quant
        self.calls.append((label, "silu_mul_quant", 0, 5 * M * D + s.numel() * 4,
                           lambda: self._check(fn(*args), label)))
        self.keep.append(gu)
        return q, s

    def add_quant(self, label, x, mode):
        torch, L = self.torch, self.lib
        M, K = x.shape
        q = self.empty((M, K), torch.uint8)
        s = self.empty((M,) if mode == PER_TOKEN else (M, K // 128), torch.float32)
        args = (q.data_ptr(), s.data_ptr(), x.data_ptr(), M, K, mode, self.stream)
        fn = L.fp8q_quant
        self.calls.append((label, "quant", 0, 3 * M * K + s.numel() * 4,
                           lambda: self._check(fn(*args), label)))
        self.keep.append(x)
        return q, s

    def add_gemm(self, label, op, a, sa, b, sb):
        torch, L = self.torch, self.lib
        M, K = a.shape
        N = b.shape[0]
        y = self.empty((M, N), torch.bfloat16)
        need = L.fp8q_workspace_size(op, M, N, K)
        self._ws_need = max(self._ws_need, need)
        nbytes = M * K + N * K + 2 * M * N + sa.numel() * 4 + sb.numel() * 4
        flops = 2 * M * N * K
        step = self

        if op == MM:
            fn = L.fp8q_scaled_mm

            def call():
                step._check(fn(y.data_ptr(), a.data_ptr(), b.data_ptr(), sa.data_ptr(),
                               sb.data_ptr(), M, N, K, step.ws_ptr, step.ws_bytes, step.stream),
                            label)
        else:
            fn = L.fp8q_scaled_mm_blockwise

            def call():
                step._check(fn(y.data_ptr(), a.data_ptr(), sa.data_ptr(), b.data_ptr(),
                               sb.data_ptr(), M, N, K, step.ws_ptr, step.ws_bytes, step.stream),
                            label)
        cfg = L.fp8q_gemm_config_for(op, M, N, K)
        kind = ("scaled_mm" if op == MM else "scaled_mm_blockwise")
        self.operands[label] = (a, sa, b, sb)
        self.calls.append((label, kind, flops, nbytes, call))
        self.keep += [a, sa, b, sb]
        return y, cfg

    def add_gemm_silu(self, label, a, sa, b, sb):
        """gate_up GEMM (b: gate rows then up rows) with SiLU-and-mul and
        group-128 quantization in its epilogue."""
        torch, L = self.torch, self.lib
        M, K = a.shape
        N = b.shape[0]
        q = self.empty((M, N // 2), torch.uint8)
        s = self.empty((M, N // 256), torch.float32)
        nbytes = M * K + N * K + M * (N // 2) + sa.numel() * 4 + sb.numel() * 4 + s.numel() * 4
        fn = L.fp8q_scaled_mm_blockwise_silu_quant
        args = (q.data_ptr(), s.data_ptr(), a.data_ptr(), sa.data_ptr(), b.data_ptr(),
                sb.data_ptr(), M, N, K, self.stream)
        self.operands[label] = (a, sa, b, sb)
        self.calls.append((label, "scaled_mm_blockwise_silu_quant", 2 * M * N * K, nbytes,
                           lambda: self._check(fn(*args), label)))
        self.keep += [a, sa, b, sb]
        return q, s

    def finalize(self):
        if self._ws_need:
            self.ws = self.torch.empty(((self._ws_need + 3) // 4,), dtype=self.torch.float32,
                                       device=self.dev)
            self.ws_bytes = self._ws_need
        self.ws_ptr = self.ws.data_ptr() if self.ws is not None else None

    def run(self, timer=None):
        for label, kind, flops, nbytes, call in self.calls:
            if timer is not None and label in timer:
                ev0 = self.torch.cuda.Event(enable_timing=True)
                ev1 = self.torch.cuda.Event(enable_timing=True)
                ev0.record()
                call()
                ev1.record()
                timer[label][0].append(ev0)
                timer[label][1].append(ev1)
            else:
                call()


def build(step: Step):
    torch = step.torch
    cfg_of = {}
    for name, (mode, hidden, (qkv_n, o_k, gu_n, inter), Ms) in WORKLOADS.items():
        op = MM if mode == PER_TOKEN else BW
        for M in Ms:
            tag = f"{name}/M{M}"
            wqkv = step.weight(qkv_n, hidden, mode)
            wo = step.weight(hidden, o_k, mode)
            wgu = step.weight(gu_n, hidden, mode)
            wdn = step.weight(hidden, inter, mode)
            x = step.activations(M, hidden)
            rw = (1.0 + step.randn((hidden,), 0.1)).to(torch.bfloat16)
            q, s = step.add_rmsnorm(f"{tag}/rmsnorm_quant", x, rw, mode)
            _, c = step.add_gemm(f"{tag}/qkv", op, q, s, *wqkv)
            cfg_of[f"{tag}/qkv"] = c
            attn = step.activations(M, o_k)
            q, s = step.add_quant(f"{tag}/quant_attn", attn, mode)
            _, c = step.add_gemm(f"{tag}/o_proj", op, q, s, *wo)
            cfg_of[f"{tag}/o_proj"] = c
            x2 = step.activations(M, hidden)
            q, s = step.add_rmsnorm(f"{tag}/rmsnorm_quant2", x2, rw, mode)
            if name in FUSED_MLP:
                q, s = step.add_gemm_silu(f"{tag}/gate_up_silu_mul_quant", q, s, *wgu)
                cfg_of[f"{tag}/gate_up_silu_mul_quant"] = FUSED_VARIANT
            else:
                gu, c = step.add_gemm(f"{tag}/gate_up", op, q, s, *wgu)
                cfg_of[f"{tag}/gate_up"] = c
                q, s = step.add_silu(f"{tag}/silu_mul_quant", gu, mode)
            _, c = step.add_gemm(f"{tag}/down", op, q, s, *wdn)
            cfg_of[f"{tag}/down"] = c
    name, Ms, D, hidden = MLP_TAIL
    for M in Ms:
        tag = f"{name}/M{M}"
        wdn = step.weight(hidden, D, GROUP128)
        gu = (step.randn((M, 2 * D), 2.0)).to(torch.bfloat16)
        q, s = step.add_silu(f"{tag}/silu_mul_quant", gu, GROUP128)
        _, c = step.add_gemm(f"{tag}/down", BW, q, s, *wdn)
        cfg_of[f"{tag}/down"] = c
    name, M, K, N = TINY
    tag = f"{name}/M{M}"
    w = step.weight(N, K, GROUP128)
    x = step.activations(M, K)
    rw = (1.0 + step.randn((K,), 0.1)).to(torch.bfloat16)
    q, s = step.add_rmsnorm(f"{tag}/rmsnorm_quant", x, rw, GROUP128)
    _, c = step.add_gemm(f"{tag}/linear", BW, q, s, *w)
    cfg_of[f"{tag}/linear"] = c
    step.finalize()
    torch.cuda.synchronize()
    return cfg_of


def queue_ahead(torch, cycles: int):
    """Queue a spin kernel of `cycles` GPU clock cycles: launches issued next
    wait behind it, so the GPU then runs them without waiting for the host,
    whose cost per call through the binding (about 10 us) exceeds the
    duration of a small kernel.  Events around them then time the kernels,
    not the host."""
    torch.cuda.synchronize()
    torch.cuda._sleep(cycles)


def variant_name(fq, cfg):
    """A table variant's name from its id; the fused kernel's name as is."""
    if cfg is None or isinstance(cfg, str):
        return cfg
    name = fq.fp8q_gemm_config_name(cfg)
    return name.decode() if isinstance(name, bytes) else name


def per_kernel_times(step: Step, reps: int = 3):
    """Event-timed GPU duration of every launch (median over reps).  Each
    timed pass is issued right behind an untimed one, which keeps the GPU
    busy (its large GEMMs take milliseconds) while the host issues the timed
    pass, so no launch of the timed pass waits for the host."""
    torch = step.torch
    times = {label: [] for label, *_ in step.calls}
    for _ in range(reps):
        torch.cuda.synchronize()
        step.run()
        evs = []
        for label, kind, flops, nbytes, call in step.calls:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            call()
            e1.record()
            evs.append((label, e0, e1))
        torch.cuda.synchronize()
        for label, e0, e1 in evs:
            times[label].append(e0.elapsed_time(e1) * 1e3)  # us
    return {k: float(np.median(v)) for k, v in times.items()}


def cpu_baseline(step: Step, label: str, rows: int):
    """The oracle computing what the dominant kernel computes (the blockwise
    or per-token GEMM; for the fused kernel also the bf16 rounding and the
    group-128 SiLU-and-mul quantization) on its first `rows` tokens."""
    import threadpoolctl

    from oracle import gemm as ogemm
    from oracle import quant as oquant

    entry = next(c for c in step.calls if c[0] == label)
    a, sa, b, sb = step.operands[label]
    K = a.shape[1]
    N = b.shape[0]
    a_h = a[:rows].cpu().numpy()
    sa_h = sa[:rows].cpu().numpy()
    b_h = b.cpu().numpy()
    sb_h = sb.cpu().numpy()
    info = threadpoolctl.threadpool_info()
    blas_threads = max([i.get("num_threads", 1) for i in info] or [1])
    t0 = time.perf_counter()
    if entry[1] == "scaled_mm":
        ogemm.scaled_mm(a_h, b_h, sa_h, sb_h)
        what = "fp64 dequantized matmul"
    else:
        y = ogemm.scaled_mm_blockwise(a_h, sa_h, b_h, sb_h)
        what = "fp64 dequantized matmul"
        if entry[1] == "scaled_mm_blockwise_silu_quant":
            import synth
            oquant.silu_mul_quant(synth.f32_to_bf16_bits(y.astype(np.float32)), oquant.GROUP128)
            what += ", bf16 rounding, SiLU-and-mul group-128 quantization"
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * N * K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"{label} ({entry[1]}), first {rows} of {a.shape[0]} tokens, "
                      f"N={N}, K={K}: {what}, {dt:.1f} s"}


def decode_chain_latency(step: Step, Ms=(1, 8, 32), reps: int = 50):
    """The Qwen3-8B block-decode layer chain (8 launches) per M, launched
    eagerly through the C ABI and replayed from a HIP graph: the GPU time per
    chain back to back (between two events on the current stream, the chains
    queued behind a spin kernel so that the GPU never waits for the host), and
    the wall-clock latency of one chain from an idle GPU (issue, then
    synchronize; median of 20)."""
    from fp8_block_scaled_rms_amd.graph import LinearChain

    torch = step.torch
    mode, hidden, (qkv_n, o_k, gu_n, inter), _ = WORKLOADS["qwen3-8b-block-decode"]
    wts = {"qkv": step.weight(qkv_n, hidden, mode), "o_proj": step.weight(hidden, o_k, mode),
           "gate_up": step.weight(gu_n, hidden, mode), "down": step.weight(hidden, inter, mode)}
    rw = (1.0 + step.randn((hidden,), 0.1)).to(torch.bfloat16)
    out = {"workload": "qwen3-8b-block-decode", "launches_per_chain": 8}
    for M in Ms:
        chain = LinearChain(step.activations(M, hidden), step.activations(M, o_k),
                            step.activations(M, hidden), rw, wts, mode)
        chain.capture()
        res = {}
        for kind, fn in (("eager_us", chain.run), ("graph_us", chain.replay)):
            for _ in range(3):
                fn()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            queue_ahead(torch, 8_000_000)  # ~4 ms: longer than issuing the chains
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            res[kind] = round(e0.elapsed_time(e1) * 1e3 / reps, 2)
            lat = []
            for _ in range(20):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                fn()
                torch.cuda.synchronize()
                lat.append(time.perf_counter() - t0)
            res[kind.replace("_us", "_single_us")] = round(float(np.median(lat)) * 1e6, 1)
        out[f"M{M}"] = res
    return out


def ue8m0_gemm(step: Step, reps: int = 6):
    """Qwen3-32B prefill GEMMs with power-of-two (UE8M0) block scales: the
    blockwise GEMM on its general path vs the UE8M0 entry point, which folds
    the scales into the f16 widening (same operands, weights rotated over two
    copies)."""
    torch, L = step.torch, step.lib
    g = step.gen
    out = {}
    for M, N, K in ((8192, 51200, 5120), (2048, 10240, 5120)):
        a = torch.randint(0, 255, (M, K), generator=g, device=step.dev, dtype=torch.uint8) & 0xF7
        bs = [torch.randint(0, 255, (N, K), generator=g, device=step.dev, dtype=torch.uint8) & 0xF7
              for _ in range(2)]
        sa = torch.exp2(torch.randint(-8, 1, (M, K // 128), generator=g, device=step.dev)
                        .float())
        sb = torch.exp2(torch.randint(-14, -5, (N // 128, K // 128), generator=g,
                                      device=step.dev).float())
        y = torch.empty((M, N), dtype=torch.bfloat16, device=step.dev)
        res = {}
        for kind, fn, op in (("general_us", L.fp8q_scaled_mm_blockwise, BW),
                             ("ue8m0_folded_us", L.fp8q_scaled_mm_blockwise_ue8m0, 3)):
            need = L.fp8q_workspace_size(op, M, N, K)
            ws = torch.empty(((need + 3) // 4,), dtype=torch.float32, device=step.dev) if need \
                else None
            wsp = ws.data_ptr() if ws is not None else None

            def run(i):
                rc = fn(y.data_ptr(), a.data_ptr(), sa.data_ptr(), bs[i % 2].data_ptr(),
                        sb.data_ptr(), M, N, K, wsp, need, step.stream)
                if rc != 0:
                    raise RuntimeError(f"blockwise GEMM status {rc}")
            run(0)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(reps):
                run(i)
            e1.record()
            torch.cuda.synchronize()
            res[kind] = round(e0.elapsed_time(e1) * 1e3 / reps, 1)
        res["ue8m0_tflops"] = round(2.0 * M * N * K / res["ue8m0_folded_us"] / 1e6, 1)
        res["general_tflops"] = round(2.0 * M * N * K / res["general_us"] / 1e6, 1)
        out[f"M{M}_N{N}_K{K}"] = res
    return out


def int8_sweep(step: Step, reps: int = 20):
    """W8A8 INT8 on the Qwen3-1.7B per-token linear shapes: every GEMM shape
    per M, back-to-back launches between two events (queued behind a spin
    kernel; weights rotated over 8 copies).  Reported against the dense int8
    MFMA peak (5.0 POP/s) and HBM."""
    torch, L = step.torch, step.lib
    hidden, (qkv_n, o_k, gu_n, inter), Ms = 2048, (4096, 2048, 12288, 6144), (1, 16, 128, 512,
                                                                                2048)
    shapes = [(qkv_n, hidden), (hidden, o_k), (gu_n, hidden), (hidden, inter)]
    g = step.gen
    out = {"workload": "qwen3-1.7b-per-token (int8)", "peak_tops": INT8_PEAK_TOPS, "per_M": {}}
    tot_ops = tot_us = 0.0
    st = step.stream
    for M in Ms:
        per = {}
        for N, K in shapes:
            a = torch.randint(-127, 128, (M, K), generator=g, device=step.dev, dtype=torch.int8)
            bs = [torch.randint(-127, 128, (N, K), generator=g, device=step.dev,
                                dtype=torch.int8) for _ in range(8)]
            sa = torch.rand(M, generator=g, device=step.dev) * 1e-2
            sb = torch.rand(N, generator=g, device=step.dev) * 1e-3
            y = torch.empty((M, N), dtype=torch.bfloat16, device=step.dev)
            need = L.fp8q_workspace_size(2, M, N, K)
            ws = torch.empty(((need + 3) // 4,), dtype=torch.float32, device=step.dev) if need \
                else None
            wsp = ws.data_ptr() if ws is not None else None

            def run(i):
                rc = L.fp8q_scaled_mm_int8(y.data_ptr(), a.data_ptr(), bs[i % 8].data_ptr(),
                                           sa.data_ptr(), sb.data_ptr(), M, N, K, wsp, need, st)
                if rc != 0:
                    raise RuntimeError(f"int8 GEMM status {rc}")
            for i in range(3):
                run(i)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            queue_ahead(torch, 4_000_000)  # ~2 ms: longer than issuing the launches
            e0.record()
            for i in range(reps):
                run(i)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            ops = 2.0 * M * N * K
            tot_ops += ops
            tot_us += us
            cfg = L.fp8q_gemm_config_for(2, M, N, K)
            per[f"{N}x{K}"] = {"us": round(us, 2), "tops": round(ops / us / 1e6, 1),
                               "gbs": round((M * K + N * K + 2 * M * N) / us / 1e3, 0),
                               "variant": L.fp8q_gemm_config_name(cfg).decode()}
        out["per_M"][f"M{M}"] = per
    out["gemm_tops"] = round(tot_ops / tot_us / 1e6, 1)
    big = out["per_M"]["M2048"][f"{gu_n}x{hidden}"]
    out["largest_gemm_frac_of_int8_peak"] = round(big["tops"] / INT8_PEAK_TOPS, 4)
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import torch

    import fp8_block_scaled_rms_amd as fq

    dev = "cuda:0"
    torch.cuda.set_device(0)
    step = Step(fq, torch, dev)
    cfg_of = build(step)
    total_flops = sum(c[2] for c in step.calls)

    # warm up, then find the dominant kernel from one event-timed pass
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    kt = per_kernel_times(step)
    dominant = max(kt, key=kt.get)

    # timed region: K steps, events around the dominant kernel's launches
    timer = {dominant: ([], [])}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step.run(timer)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    durs = [a.elapsed_time(b) * 1e-3 for a, b in zip(*timer[dominant])]  # seconds
    dom_avg = float(np.mean(durs))
    dom = next(c for c in step.calls if c[0] == dominant)
    dom_cfg_name = variant_name(fq, cfg_of.get(dominant))
    exact = dom_cfg_name is None or dom_cfg_name.startswith("f16_")
    if dom[2] > 0:
        achieved = dom[2] / dom_avg / 1e12
        peak = F16_PEAK_TFLOPS if exact else FP8_PEAK_TFLOPS
        a_t, _, b_t, _ = step.operands[dominant]
        dom_op = {"scaled_mm": MM, "scaled_mm_blockwise": BW,
                  "scaled_mm_blockwise_silu_quant": SQ}[dom[1]]
        traffic = measured_traffic(dom_cfg_name, dom_op, a_t.shape[0], b_t.shape[0],
                                   a_t.shape[1])
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                "algorithmic_bytes": dom[3],
                "kernel": dominant, "variant": dom_cfg_name,
                "avg_launch_us": round(dom_avg * 1e6, 2),
                "frac_of_fp8_peak": round(achieved / FP8_PEAK_TFLOPS, 4)}
    else:
        achieved = dom[3] / dom_avg / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": dominant, "avg_launch_us": round(dom_avg * 1e6, 2)}

    # per-workload summary from the event-timed pass
    summary = {}
    for label, kind, flops, nbytes, _ in step.calls:
        wl = label.split("/")[0]
        s = summary.setdefault(wl, {"gemm_us": 0.0, "quant_us": 0.0, "gemm_flops": 0.0})
        if flops:
            s["gemm_us"] += kt[label]
            s["gemm_flops"] += flops
        else:
            s["quant_us"] += kt[label]
    per_wl = {wl: {"gemm_tflops": round(s["gemm_flops"] / (s["gemm_us"] * 1e-6) / 1e12, 1),
                   "gemm_us": round(s["gemm_us"], 1), "quant_us": round(s["quant_us"], 1)}
              for wl, s in summary.items()}

    chain = decode_chain_latency(step)
    w8a8 = int8_sweep(step)
    ue8 = ue8m0_gemm(step)

    cpu = None
    if not args.no_cpu_baseline and dom[2] > 0:
        cpu = cpu_baseline(step, dominant, args.cpu_sample_rows)

    value = total_flops / (ms_per_step * 1e-3) / 1e12
    line = {
        "metric": "FP8 block-scaled GEMM TFLOP/s & % FP8 MFMA peak, Qwen3 shapes M=1..8192",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": "synthetic",
        "config": {"workload": "qwen3-fp8-linear-sweep",
                   "parts": list(WORKLOADS) + [MLP_TAIL[0], TINY[0]],
                   "gemm_flops_per_step": total_flops,
                   "launches_per_step": len(step.calls),
                   "parallelism": "single-gpu"},
        "frac_of_fp8_peak": round(value / FP8_PEAK_TFLOPS, 4),
        "roofline": roof,
        "cpu_baseline": cpu,
        "per_workload": per_wl,
        "decode_chain": chain,
        "w8a8_int8": w8a8,
        "ue8m0_blockwise": ue8,
    }
    if args.detail:
        detail = {label: {"kind": kind, "us": round(kt[label], 2), "flops": flops,
                          "bytes": nbytes,
                          "variant": variant_name(fq, cfg_of.get(label))}
                  for label, kind, flops, nbytes, _ in step.calls}
        with open(args.detail, "w") as f:
            json.dump(detail, f, indent=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
