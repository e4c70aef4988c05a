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
       python bench.py --decode-study   small-M GEMMs beside a read-only kernel
                                        streaming the same weight bytes
       python bench.py --chain-study    the decode chain eagerly and as a graph
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


class Launch(tuple):
    """One launch of a bench step: label, kind, quantization mode, M, K and N.
    kind is rmsnorm_quant, quant, silu_mul_quant (K = D, the output columns),
    scaled_mm, scaled_mm_blockwise or scaled_mm_blockwise_silu_quant (N = 2D
    weight rows); N is None for the quantizers."""
    __slots__ = ()

    def __new__(cls, label, kind, mode, M, K, N=None):
        return super().__new__(cls, (label, kind, mode, M, K, N))

    label = property(lambda s: s[0])
    kind = property(lambda s: s[1])
    mode = property(lambda s: s[2])
    M = property(lambda s: s[3])
    K = property(lambda s: s[4])
    N = property(lambda s: s[5])


def launch_plan():
    """Every launch of one step, in issue order (build() enqueues exactly
    these; the GPU parity tests run each one at its own size)."""
    plan = []
    for name, (mode, hidden, (qkv_n, o_k, gu_n, inter), Ms) in WORKLOADS.items():
        gemm = "scaled_mm" if mode == PER_TOKEN else "scaled_mm_blockwise"
        for M in Ms:
            tag = f"{name}/M{M}"
            plan.append(Launch(f"{tag}/rmsnorm_quant", "rmsnorm_quant", mode, M, hidden))
            plan.append(Launch(f"{tag}/qkv", gemm, mode, M, hidden, qkv_n))
            plan.append(Launch(f"{tag}/quant_attn", "quant", mode, M, o_k))
            plan.append(Launch(f"{tag}/o_proj", gemm, mode, M, o_k, hidden))
            plan.append(Launch(f"{tag}/rmsnorm_quant2", "rmsnorm_quant", mode, M, hidden))
            if name in FUSED_MLP:
                plan.append(Launch(f"{tag}/gate_up_silu_mul_quant",
                                   "scaled_mm_blockwise_silu_quant", mode, M, hidden, gu_n))
            else:
                plan.append(Launch(f"{tag}/gate_up", gemm, mode, M, hidden, gu_n))
                plan.append(Launch(f"{tag}/silu_mul_quant", "silu_mul_quant", mode, M,
                                   gu_n // 2))
            plan.append(Launch(f"{tag}/down", gemm, mode, M, inter, hidden))
    name, Ms, D, hidden = MLP_TAIL
    for M in Ms:
        tag = f"{name}/M{M}"
        plan.append(Launch(f"{tag}/silu_mul_quant", "silu_mul_quant", GROUP128, M, D))
        plan.append(Launch(f"{tag}/down", "scaled_mm_blockwise", GROUP128, M, D, hidden))
    name, M, K, N = TINY
    tag = f"{name}/M{M}"
    plan.append(Launch(f"{tag}/rmsnorm_quant", "rmsnorm_quant", GROUP128, M, K))
    plan.append(Launch(f"{tag}/linear", "scaled_mm_blockwise", GROUP128, M, K, N))
    return plan


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--detail", default=None, help="write a per-kernel breakdown JSON here")
    p.add_argument("--cpu-sample-rows", type=int, default=2048)
    p.add_argument("--decode-study", action="store_true",
                   help="only time the small-M (HBM-bound) GEMM launches of a step, each beside "
                        "a read-only kernel streaming the same weight bytes, and print that "
                        "comparison as one JSON line")
    p.add_argument("--chain-study", action="store_true",
                   help="only run the decode-chain comparison (eager vs HIP graph) and print "
                        "it as one JSON line, for a kernel trace of the two")
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
                  "fp8_block_scaled_rms_amd/csrc/gemm_common.hpp",
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


class LaunchCall:
    """One C-ABI launch with its arguments bound (the stream is appended).
    Calling it with `override` {argument position: pointer} issues the same
    launch with those arguments replaced."""

    def __init__(self, step, label, fn, args, rot):
        self.step, self.label, self.fn, self.args, self.rot = step, label, fn, args, rot

    def __call__(self, override=None):
        args = self.args if not override else [override.get(i, v)
                                                for i, v in enumerate(self.args)]
        rc = self.fn(*args, self.step.stream)
        if rc != 0:
            raise RuntimeError(f"{self.label}: status {rc} "
                               f"{self.step.lib.fp8q_status_string(rc).decode()}")


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
        self._ws_calls = []
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
    def _add(self, label, kind, flops, nbytes, fn, args, rot):
        """Record one launch: fn(*args, stream).  rot maps argument positions
        to the tensors they point at that the per-kernel timing rotates over
        distinct copies (the inputs a launch streams from HBM)."""
        call = LaunchCall(self, label, fn, list(args), rot)
        self.calls.append((label, kind, flops, nbytes, call))
        return call

    def add_rmsnorm(self, label, x, w, mode):
        torch, L = self.torch, self.lib
        M, K = x.shape
        q = self.empty((M, K), torch.uint8)
        s = self.empty((M,) if mode == PER_TOKEN else (M, K // 128), torch.float32)
        args = (q.data_ptr(), s.data_ptr(), x.data_ptr(), w.data_ptr(), M, K, 1e-6, mode)
        self._add(label, "rmsnorm_quant", 0, 3 * M * K + 2 * K + s.numel() * 4,
                  L.fp8q_rmsnorm_quant, args, {2: x})
        self.keep += [x, w]
        return q, s

    def add_silu(self, label, gu, mode):
        torch, L = self.torch, self.lib
        M, twoD = gu.shape
        D = twoD // 2
        q = self.empty((M, D), torch.uint8)
        s = self.empty((M,) if mode == PER_TOKEN else (M, D // 128), torch.float32)
        args = (q.data_ptr(), s.data_ptr(), gu.data_ptr(), M, D, mode)
        self._add(label, "silu_mul_quant", 0, 5 * M * D + s.numel() * 4,
                  L.fp8q_silu_mul_quant, args, {2: gu})
        self.keep.append(gu)
        return q, s

    def add_quant(self, label, x, mode):
        torch, L = self.torch, self.lib
        M, K = x.shape
        q = self.empty((M, K), torch.uint8)
        s = self.empty((M,) if mode == PER_TOKEN else (M, K // 128), torch.float32)
        args = (q.data_ptr(), s.data_ptr(), x.data_ptr(), M, K, mode)
        self._add(label, "quant", 0, 3 * M * K + s.numel() * 4, L.fp8q_quant, args, {2: x})
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
        fn = L.fp8q_scaled_mm if op == MM else L.fp8q_scaled_mm_blockwise
        # the workspace (arguments 8 and 9) is set by finalize()
        args = (y.data_ptr(), a.data_ptr(), b.data_ptr(), sa.data_ptr(), sb.data_ptr(), M, N, K,
                None, 0)
        call = self._add(label, "scaled_mm" if op == MM else "scaled_mm_blockwise",
                         2 * M * N * K, nbytes, fn, args, {2: b})
        self._ws_calls.append(call)
        cfg = L.fp8q_gemm_config_for(op, M, N, K)
        self.operands[label] = (a, sa, b, sb)
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
        args = (q.data_ptr(), s.data_ptr(), a.data_ptr(), b.data_ptr(), sa.data_ptr(),
                sb.data_ptr(), M, N, K)
        self._add(label, "scaled_mm_blockwise_silu_quant", 2 * M * N * K, nbytes,
                  L.fp8q_scaled_mm_blockwise_silu_quant, args, {3: b})
        self.operands[label] = (a, sa, b, sb)
        self.keep += [a, sa, b, sb]
        return q, s

    def finalize(self):
        if self._ws_need:
            self.ws = self.torch.empty(((self._ws_need + 3) // 4,), dtype=self.torch.float32,
                                       device=self.dev)
            self.ws_bytes = self._ws_need
        self.ws_ptr = self.ws.data_ptr() if self.ws is not None else None
        for call in self._ws_calls:
            call.args[8] = self.ws_ptr
            call.args[9] = self.ws_bytes

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
    plan = launch_plan()
    got = [(c[0], c[1]) for c in step.calls]
    if got != [(p.label, p.kind) for p in plan]:
        raise RuntimeError("bench launches differ from launch_plan()")
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


ROTATE_BYTES = 1 << 30   # streamed inputs rotate over at least this many bytes of copies
REALTIME_MHZ = 100.0     # rate of s_memrealtime on gfx9-family GPUs


def per_kernel_times(step: Step, batches: int = 3):
    """GPU time of every launch of the step.  Each launch is timed as R
    back-to-back launches between two events (R = 100, or fewer for launches
    above 50 us, so that a batch lasts a few milliseconds), queued behind a
    spin kernel so that the GPU never waits for the host; the inputs the
    launch streams (a GEMM's weights, a quantizer's input rows) rotate over
    distinct copies of >= 1 GiB in total, so that the 256 MB last-level cache
    cannot serve them from an earlier launch.  Median over `batches`."""
    torch = step.torch
    # a first pass with events around single launches sizes the batches
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
    single = {label: e0.elapsed_time(e1) * 1e3 for label, e0, e1 in evs}
    out = {}
    for label, kind, flops, nbytes, call in step.calls:
        t1 = single[label]
        reps = 100 if t1 < 50.0 else max(3, int(np.ceil(5000.0 / t1)))
        rot_bytes = sum(t.numel() * t.element_size() for t in call.rot.values())
        copies = int(min(reps, max(1, -(-ROTATE_BYTES // max(rot_bytes, 1)))))
        pools = {}
        for pos, t in call.rot.items():
            pool = torch.empty((copies,) + tuple(t.shape), dtype=t.dtype, device=step.dev)
            pool.copy_(t.unsqueeze(0).expand_as(pool))
            pools[pos] = [pool[i].data_ptr() for i in range(copies)]
            pools.setdefault("_keep", []).append(pool)
        overrides = [{pos: ptrs[r % copies] for pos, ptrs in pools.items() if pos != "_keep"}
                     for r in range(reps)]
        call(overrides[0])  # warm the code path
        times = []
        for _ in range(batches):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            queue_ahead(torch, 2_000_000 + 60_000 * reps)  # longer than issuing the batch
            e0.record()
            for r in range(reps):
                call(overrides[r])
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3 / reps)
        out[label] = float(np.median(times))
        del pools
    return out


def size_matched_probes(step: Step, launches, batches: int = 3):
    """For each (label, is_gemm, nbytes): the streaming probe
    (include/fp8q_probe.h) moving the same bytes, timed like
    per_kernel_times (100 back-to-back launches behind a spin kernel, source
    and destination rotating over 1 GiB and 512 MiB, median of `batches`).
    A GEMM launch gets the read-only loop over its byte count; a quantizer
    the copy loop moving the same total (half read, half written, where the
    quantizer reads two to four bytes per byte it writes).  Small launches
    carry the fixed costs of starting and draining a kernel, which these
    probes pay too: the ratio is the launch's distance from a plain stream
    of its own size."""
    torch, L = step.torch, step.lib
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs = 8 * cus
    src_pool = 1 << 30
    dst_pool = 1 << 29
    src = torch.ones(src_pool, dtype=torch.uint8, device=step.dev)
    dst = torch.empty(dst_pool, dtype=torch.uint8, device=step.dev)
    scratch = torch.empty(wgs * 256 * 4, dtype=torch.uint8, device=step.dev)
    reps = 100
    out = {}
    for label, is_gemm, nbytes in launches:
        kind = 2 if is_gemm else 3
        n = (int(nbytes if is_gemm else nbytes // 2) // 4096) * 4096
        nsrc = max(1, src_pool // n)
        ndst = max(1, dst_pool // n)

        def run(r):
            d = scratch.data_ptr() if is_gemm else dst.data_ptr() + (r % ndst) * n
            rc = L.fp8q_probe_stream(kind, src.data_ptr() + (r % nsrc) * n, d, n, wgs,
                                     step.stream)
            if rc != 0:
                raise RuntimeError(f"probe_stream status {rc}")

        run(0)
        times = []
        for _ in range(batches):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            queue_ahead(torch, 2_000_000 + 60_000 * reps)
            e0.record()
            for r in range(reps):
                run(r)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3 / reps)
        out[label] = (float(np.median(times)), 2 * n if not is_gemm else n)
    del src, dst, scratch
    return out


def decode_study(step: Step, reps: int = 50):
    """Every small-M GEMM launch of a step (the 8B block decode, the 32B MLP
    tail at M=64, the 1.7B gate_up at M<=128) timed as in per_kernel_times,
    beside the read-only probe kernel (include/fp8q_probe.h) streaming the
    same weight bytes from the same rotated copies: the gap is what the GEMM
    costs beyond reading its weights."""
    torch, L = step.torch, step.lib
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(8 * cus * 256, dtype=torch.int32, device=step.dev)
    out = {}
    for label, kind, flops, nbytes, call in step.calls:
        wl, M = label.split("/")[0], int(label.split("/")[1][1:])
        small = flops and (wl == "qwen3-8b-block-decode" or
                           (wl == "qwen3-32b-mlp-tail" and M == 64) or
                           (wl == "qwen3-1.7b-per-token" and label.endswith("/gate_up")
                            and M <= 128))
        if not small:
            continue
        (pos, wt), = call.rot.items()
        wbytes = wt.numel() * wt.element_size()
        copies = int(min(reps, max(1, -(-ROTATE_BYTES // wbytes))))
        pool = torch.empty((copies,) + tuple(wt.shape), dtype=wt.dtype, device=step.dev)
        pool.copy_(wt.unsqueeze(0).expand_as(pool))
        ptrs = [pool[i].data_ptr() for i in range(copies)]
        res = {"bytes": int(nbytes), "weight_bytes": int(wbytes)}
        for what in ("gemm", "read_only"):
            def run(r):
                if what == "gemm":
                    call({pos: ptrs[r % copies]})
                else:
                    rc = L.fp8q_probe_stream(2, ptrs[r % copies], sink.data_ptr(), wbytes,
                                             8 * cus, step.stream)
                    if rc != 0:
                        raise RuntimeError(f"probe_stream status {rc}")
            run(0)
            ts = []
            for _ in range(3):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                queue_ahead(torch, 2_000_000 + 60_000 * reps)
                e0.record()
                for r in range(reps):
                    run(r)
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3 / reps)
            res[f"{what}_us"] = round(float(np.median(ts)), 2)
        res["gemm_gbs"] = round(nbytes / res["gemm_us"] / 1e3, 0)
        res["read_only_gbs"] = round(wbytes / res["read_only_us"] / 1e3, 0)
        res["gemm_over_read_only"] = round(res["gemm_us"] / res["read_only_us"], 3)
        out[label] = res
        del pool
    return out


def measure_ceilings(step: Step):
    """What this GPU reaches on plain loops (include/fp8q_probe.h): dense
    f16 and FP8 matrix instructions on every CU (and the shader clock
    meanwhile, from the s_memtime / s_memrealtime stamps of every
    workgroup), and HBM streaming (read, and device-to-device copy)."""
    torch, L = step.torch, step.lib
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    res = {"compute_units": cus}
    wgs = 4 * cus  # 16 waves per CU
    stamps = torch.zeros((wgs, 4), dtype=torch.int64, device=step.dev)
    sink = torch.zeros(wgs, dtype=torch.float32, device=step.dev)
    for kind, name in ((0, "mfma_f16"), (1, "mfma_fp8")):
        iters = 4000 if kind == 0 else 2000
        runs = []
        for _ in range(4):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            rc = L.fp8q_probe_mfma(kind, iters, wgs, stamps.data_ptr(), sink.data_ptr(),
                                   step.stream)
            e1.record()
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"probe_mfma status {rc}")
            t = e0.elapsed_time(e1) * 1e-3
            st = stamps.cpu().numpy().astype(np.float64)
            ratio = np.median((st[:, 1] - st[:, 0]) / (st[:, 3] - st[:, 2]))
            flops = L.fp8q_probe_mfma_flops_per_iter(kind) * iters * wgs * 4  # 4 waves
            runs.append((flops / t / 1e12, ratio))
        best = max(runs)
        res[f"{name}_tflops"] = round(best[0], 1)
        # shader clock: s_memtime ticks per tick of s_memrealtime, the
        # GPU's constant 100 MHz counter, over each workgroup's loop
        res[f"{name}_sclk_mhz"] = round(best[1] * REALTIME_MHZ, 0)
    n = 4 << 30
    src = torch.ones(n, dtype=torch.uint8, device=step.dev)
    dst = torch.empty(n // 2, dtype=torch.uint8, device=step.dev)
    scratch = torch.empty(wgs * 2 * 256 * 4, dtype=torch.uint8, device=step.dev)
    for kind, name, nbytes, nread, moved in ((2, "hbm_read", n, n, n),
                                             (3, "hbm_copy", n // 2, n // 2, n)):
        best = 0.0
        for _ in range(4):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            out = scratch if kind == 2 else dst
            rc = L.fp8q_probe_stream(kind, src.data_ptr(), out.data_ptr(), nread, 2 * wgs,
                                     step.stream)
            e1.record()
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"probe_stream status {rc}")
            best = max(best, moved / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        res[f"{name}_gbs"] = round(best, 0)
    del src, dst, scratch
    return res


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


STACK = 8  # layers in the decode-stack graphs


def _chain_times(torch, fn, per, reps):
    """(GPU time per layer back to back, wall-clock latency per layer of one
    call from an idle GPU) of fn, which issues `per` layers' chains."""
    for _ in range(3):
        fn()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    # longer than the host takes to issue the chains (~4 ms for one layer's,
    # ~75 ms for a stack's when issued eagerly)
    queue_ahead(torch, 8_000_000 if per == 1 else 20_000_000 * per)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    back_to_back = e0.elapsed_time(e1) * 1e3 / (reps * per)
    lat = []
    for _ in range(20):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        lat.append(time.perf_counter() - t0)
    return round(back_to_back, 2), round(float(np.median(lat)) * 1e6 / per, 1)


def _stack(step: Step, workload, M, stack_wts, rw):
    from fp8_block_scaled_rms_amd.graph import LinearChain

    mode, hidden, (qkv_n, o_k, gu_n, inter), _ = WORKLOADS[workload]
    return [LinearChain(step.activations(M, hidden), step.activations(M, o_k),
                        step.activations(M, hidden), rw, w, mode) for w in stack_wts]


def _layer_weights(step: Step, workload):
    mode, hidden, (qkv_n, o_k, gu_n, inter), _ = WORKLOADS[workload]
    return {"qkv": step.weight(qkv_n, hidden, mode), "o_proj": step.weight(hidden, o_k, mode),
            "gate_up": step.weight(gu_n, hidden, mode), "down": step.weight(hidden, inter, mode)}


def decode_chain_latency(step: Step, Ms=(1, 8, 32), reps: int = 50):
    """The Qwen3-8B block-decode layer chain (8 launches) per M, launched
    eagerly through the C ABI and replayed from a HIP graph: the GPU time per
    chain back to back (between two events on the current stream, the chains
    queued behind a spin kernel so that the GPU never waits for the host), and
    the wall-clock latency of one chain from an idle GPU (issue, then
    synchronize; median of 20).  The same for a stack of STACK layers with
    distinct weights (a decode step's linear work, its weights larger than
    the last-level cache): eagerly, layer after layer, and as one graph
    holding every layer's launches (capture_stack); those figures are per
    layer.  The stack is also timed for the Qwen3-1.7B per-token layer, whose
    kernels take less GPU time than the host needs to issue them."""
    from fp8_block_scaled_rms_amd.graph import LinearChain, capture_stack

    torch = step.torch
    workload = "qwen3-8b-block-decode"
    mode, hidden, (qkv_n, o_k, gu_n, inter), _ = WORKLOADS[workload]
    stack_wts = [_layer_weights(step, workload) for _ in range(STACK)]
    rw = (1.0 + step.randn((hidden,), 0.1)).to(torch.bfloat16)
    out = {"workload": workload, "launches_per_chain": 8, "stack_layers": STACK}
    for M in Ms:
        chain = LinearChain(step.activations(M, hidden), step.activations(M, o_k),
                            step.activations(M, hidden), rw, stack_wts[0], mode)
        chain.capture()
        stack = _stack(step, workload, M, stack_wts, rw)
        stack_graph = capture_stack(stack)

        def stack_eager():
            for c in stack:
                c.run()

        res = {}
        for kind, fn, per in (("eager", chain.run, 1), ("graph", chain.replay, 1),
                              ("stack_eager", stack_eager, STACK),
                              ("stack_graph", stack_graph.replay, STACK)):
            sfx = "_per_layer" if per > 1 else ""
            res[f"{kind}_us{sfx}"], res[f"{kind}_single_us{sfx}"] = _chain_times(
                torch, fn, per, reps)
        out[f"M{M}"] = res
        del stack, stack_graph, chain
    del stack_wts

    workload = "qwen3-1.7b-per-token"
    mode, hidden, _, _ = WORKLOADS[workload]
    small_wts = [_layer_weights(step, workload) for _ in range(STACK)]
    rw = (1.0 + step.randn((hidden,), 0.1)).to(torch.bfloat16)
    small = {"workload": workload, "stack_layers": STACK}
    for M in (1, 16):
        stack = _stack(step, workload, M, small_wts, rw)
        stack_graph = capture_stack(stack)

        def stack_eager():
            for c in stack:
                c.run()

        res = {}
        for kind, fn in (("stack_eager", stack_eager), ("stack_graph", stack_graph.replay)):
            res[f"{kind}_us_per_layer"], res[f"{kind}_single_us_per_layer"] = _chain_times(
                torch, fn, STACK, reps)
        small[f"M{M}"] = res
        del stack, stack_graph
    out["stack_" + workload] = small
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
                rc = fn(y.data_ptr(), a.data_ptr(), bs[i % 2].data_ptr(), sa.data_ptr(),
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


def library_context(step: Step, kt, reps: int = 5):
    """Context from the installed libraries on the same GPU (not part of the
    path, and not a target): torch's f16 matmul (hipBLASLt) and FP8
    _scaled_mm with per-tensor scales on the dominant GEMM's shape, which
    compute neither the blockwise scales nor the exact FP8 sums, and torch
    eager compositions of two fused quantizers (the pages compare their
    kernels with the framework's own ops), each against this library's
    launch of the same work."""
    torch = step.torch
    out = {}
    M, N, K = 8192, 51200, 5120

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    a = step.randn((M, K)).to(torch.float16)
    bt = step.randn((K, N), 0.02).to(torch.float16)  # [K, N] contiguous: no transposed operand
    us = timed(lambda: torch.matmul(a, bt))
    out["torch_matmul_f16_us"] = round(us, 1)
    out["torch_matmul_f16_tflops"] = round(2.0 * M * N * K / us / 1e6, 1)
    del a, bt
    try:
        a8 = step.randn((M, K)).to(torch.float8_e4m3fn)
        b8 = (step.randn((N, K), 0.02) * 64).to(torch.float8_e4m3fn)
        one = torch.ones((), device=step.dev)
        us = timed(lambda: torch._scaled_mm(a8, b8.t(), scale_a=one, scale_b=one,
                                            out_dtype=torch.bfloat16))
        out["torch_scaled_mm_fp8_per_tensor_us"] = round(us, 1)
        out["torch_scaled_mm_fp8_per_tensor_tflops"] = round(2.0 * M * N * K / us / 1e6, 1)
        del a8, b8
    except Exception as e:  # not every build of torch has it for this GPU
        out["torch_scaled_mm_fp8_per_tensor"] = f"unavailable: {type(e).__name__}"
    out["this_library_fused_gate_up_us"] = round(
        kt["qwen3-32b-block-prefill/M8192/gate_up_silu_mul_quant"], 1)

    def rms_group(x, w):
        xf = x.float()
        y = xf * torch.rsqrt(xf.pow(2).mean(dim=1, keepdim=True) + 1e-6) * w.float()
        g = y.view(x.shape[0], -1, 128)
        s = g.abs().amax(dim=2, keepdim=True) / 448.0
        return (g / s).to(torch.float8_e4m3fn), s

    def silu_group(gu):
        D = gu.shape[1] // 2
        y = torch.nn.functional.silu(gu[:, :D].float()) * gu[:, D:].float()
        g = y.view(gu.shape[0], -1, 128)
        s = g.abs().amax(dim=2, keepdim=True) / 448.0
        return (g / s).to(torch.float8_e4m3fn), s

    x = step.activations(8192, 5120)
    w = (1.0 + step.randn((5120,), 0.1)).to(torch.bfloat16)
    us = timed(lambda: rms_group(x, w))
    out["torch_eager_rmsnorm_group128_quant_M8192_K5120_us"] = round(us, 1)
    out["this_library_rmsnorm_group128_quant_us"] = round(
        kt["qwen3-32b-block-prefill/M8192/rmsnorm_quant"], 1)
    del x
    gu = (step.randn((4096, 51200), 2.0)).to(torch.bfloat16)
    us = timed(lambda: silu_group(gu))
    out["torch_eager_silu_mul_group128_quant_M4096_D25600_us"] = round(us, 1)
    out["this_library_silu_mul_group128_quant_us"] = round(
        kt["qwen3-32b-mlp-tail/M4096/silu_mul_quant"], 1)
    del gu
    torch.cuda.empty_cache()
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
    if args.chain_study:
        print(json.dumps({"decode_chain": decode_chain_latency(step)}), flush=True)
        return
    cfg_of = build(step)
    total_flops = sum(c[2] for c in step.calls)
    if args.decode_study:
        for _ in range(2):
            step.run()
        torch.cuda.synchronize()
        study = decode_study(step)
        for label in study:
            study[label]["variant"] = variant_name(fq, cfg_of.get(label))
        print(json.dumps({"decode_study": study}), flush=True)
        return

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
    ceil = measure_ceilings(step)
    if dom[2] > 0:
        # The metric's peak is the FP8 one; the exact engine (f16_ variants)
        # runs f16 matrix instructions, whose dense peak is half of it: that
        # fraction, and those of the ceilings measured on this GPU, are
        # reported beside it.
        achieved = dom[2] / dom_avg / 1e12
        a_t, _, b_t, _ = step.operands[dominant]
        dom_op = {"scaled_mm": MM, "scaled_mm_blockwise": BW,
                  "scaled_mm_blockwise_silu_quant": SQ}[dom[1]]
        traffic = measured_traffic(dom_cfg_name, dom_op, a_t.shape[0], b_t.shape[0],
                                   a_t.shape[1])
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / FP8_PEAK_TFLOPS, 4),
                "traffic": traffic, "algorithmic_bytes": dom[3],
                "kernel": dominant, "variant": dom_cfg_name,
                "avg_launch_us": round(dom_avg * 1e6, 2),
                "engine": "f16" if (dom_cfg_name or "").startswith("f16_") else "other",
                "frac_of_f16_peak": round(achieved / F16_PEAK_TFLOPS, 4),
                "frac_of_measured_f16_ceiling": round(achieved / ceil["mfma_f16_tflops"], 4),
                "sclk_mhz_of_mfma_probe": ceil["mfma_f16_sclk_mhz"]}
    else:
        achieved = dom[3] / dom_avg / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": dominant, "avg_launch_us": round(dom_avg * 1e6, 2),
                "frac_of_measured_copy_ceiling": round(achieved / ceil["hbm_copy_gbs"], 4)}

    # the HBM-bound launches with a target: quantizers of >= 16 MB, and the
    # small-M GEMMs (8B decode, 32B MLP tail at M=64, 1.7B gate_up at M<=128)
    hbm = {}
    for label, kind, flops, nbytes, _ in step.calls:
        wl, mtag = label.split("/")[0], label.split("/")[1]
        M = int(mtag[1:])
        small_gemm = flops and (wl == "qwen3-8b-block-decode" or
                                (wl == "qwen3-32b-mlp-tail" and M == 64) or
                                (wl == "qwen3-1.7b-per-token" and label.endswith("/gate_up")
                                 and M <= 128))
        if (not flops and nbytes >= 16e6) or small_gemm:
            gbs = nbytes / (kt[label] * 1e-6) / 1e9
            # GEMMs mostly read (weights); quantizers read 2-4 B and write
            # 1 B per element: compared with the read-only and the copy
            # ceiling respectively
            ref = ceil["hbm_read_gbs"] if flops else ceil["hbm_copy_gbs"]
            hbm[label] = {"us": round(kt[label], 2), "gbs": round(gbs, 0),
                          "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                          "frac_of_measured_ceiling": round(gbs / ref, 4)}
    sizes = {label: (bool(flops), nbytes) for label, kind, flops, nbytes, _ in step.calls}
    probes = size_matched_probes(step, [(label,) + sizes[label] for label in hbm])
    for label, (pus, pbytes) in probes.items():
        hbm[label]["size_matched_probe_us"] = round(pus, 2)
        hbm[label]["size_matched_probe_gbs"] = round(pbytes / (pus * 1e-6) / 1e9, 0)
        hbm[label]["probe_over_kernel_time"] = round(pus / kt[label], 4)

    # per-workload summary from the batched per-kernel times
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
    libctx = library_context(step, kt)

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
        "ceilings": ceil,
        "hbm_bound_launches": hbm,
        "per_workload": per_wl,
        "decode_chain": chain,
        "w8a8_int8": w8a8,
        "ue8m0_blockwise": ue8,
        "library_context": libctx,
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
