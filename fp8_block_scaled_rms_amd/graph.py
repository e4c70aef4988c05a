"""The FP8 linear chain of one decoder layer, launched eagerly or replayed
from a HIP graph.

Decode steps are launch-bound: the page "Helion in vLLM: FP8 inference of
Qwen3" (24-ai.news), section "Practical limits", and the page "Helion can
accelerate vLLM LLM inference on NVIDIA GPUs" (aihirek.info), section
"Performance costs tuning and operations", both put the per-call dispatch
cost at tens of microseconds and run decode under graphs.  The chain is

    x    --rmsnorm_quant-->  QKV GEMM        -> y_qkv
    attn --quant-->          o_proj GEMM     -> y_o
    h    --rmsnorm_quant-->  gate_up GEMM    -> y_gu --silu_mul_quant--> down GEMM -> y_down

with per-token scales and scaled_mm, or 1x128 groups and
scaled_mm_blockwise.  Attention is not part of the path: `attn` is an input
buffer standing in for its output.

Every buffer is allocated once, when the chain is built.  run() enqueues the
seven launches on the current stream through the C ABI (ctypes calls bound
in advance); capture() records the same launches into a torch.cuda.CUDAGraph,
whose replay then costs one launch.  None of the chain's launches records a
memset or allocates, so a replay reads the inputs in place and rewrites
every output.  capture_stack() records the chains of several layers, each
with its own weights, into one graph.
"""
from __future__ import annotations

import torch

from . import (GROUP128, OP_SCALED_MM, OP_SCALED_MM_BLOCKWISE, PER_TOKEN, _check, lib)


class LinearChain:
    """weights: dict with keys 'qkv', 'o_proj', 'gate_up', 'down', each a
    (codes uint8 [N,K], scale fp32 [N] or [N/128,K/128]) pair, quantized
    per output channel (mode PER_TOKEN) or per 128x128 block (GROUP128)."""

    def __init__(self, x, attn, h, rms_w, weights, mode: int, eps: float = 1e-6):
        if mode not in (PER_TOKEN, GROUP128):
            raise ValueError("the chain runs the per-token or the group128 path")
        dev = x.device
        self.mode = mode
        self.x, self.attn, self.h, self.rms_w = x, attn, h, rms_w
        self.weights = weights
        M = x.shape[0]
        op = OP_SCALED_MM if mode == PER_TOKEN else OP_SCALED_MM_BLOCKWISE
        L = lib()

        def qbuf(K):
            q = torch.empty((M, K), dtype=torch.uint8, device=dev)
            s = torch.empty((M,) if mode == PER_TOKEN else (M, K // 128), dtype=torch.float32,
                            device=dev)
            return q, s

        def ybuf(name):
            return torch.empty((M, weights[name][0].shape[0]), dtype=torch.bfloat16, device=dev)

        self.q_x, self.s_x = qbuf(x.shape[1])
        self.q_a, self.s_a = qbuf(attn.shape[1])
        self.q_h, self.s_h = qbuf(h.shape[1])
        self.y_qkv, self.y_o, self.y_gu, self.y_down = (ybuf("qkv"), ybuf("o_proj"),
                                                        ybuf("gate_up"), ybuf("down"))
        D = self.y_gu.shape[1] // 2
        self.q_g, self.s_g = qbuf(D)

        gemms = [("qkv", self.q_x, self.s_x, self.y_qkv), ("o_proj", self.q_a, self.s_a, self.y_o),
                 ("gate_up", self.q_h, self.s_h, self.y_gu), ("down", self.q_g, self.s_g,
                                                              self.y_down)]
        need = max(L.fp8q_workspace_size(op, M, w[0].shape[0], w[0].shape[1])
                   for w in (weights[n] for n, *_ in gemms))
        self.ws = (torch.empty(((need + 3) // 4,), dtype=torch.float32, device=dev)
                   if need else None)
        ws_p = self.ws.data_ptr() if self.ws is not None else None

        # (function, args without the stream, label)
        calls = [(L.fp8q_rmsnorm_quant, (self.q_x.data_ptr(), self.s_x.data_ptr(), x.data_ptr(),
                                         rms_w.data_ptr(), M, x.shape[1], eps, mode),
                  "rmsnorm_quant"),
                 (L.fp8q_quant, (self.q_a.data_ptr(), self.s_a.data_ptr(), attn.data_ptr(), M,
                                 attn.shape[1], mode), "quant")]
        for name, qa, sa, y in gemms[:3]:
            b, sb = weights[name]
            N, K = b.shape
            if mode == PER_TOKEN:
                args = (y.data_ptr(), qa.data_ptr(), b.data_ptr(), sa.data_ptr(), sb.data_ptr(),
                        M, N, K, ws_p, need)
                calls.append((L.fp8q_scaled_mm, args, name))
            else:
                args = (y.data_ptr(), qa.data_ptr(), b.data_ptr(), sa.data_ptr(), sb.data_ptr(),
                        M, N, K, ws_p, need)
                calls.append((L.fp8q_scaled_mm_blockwise, args, name))
            if name == "o_proj":
                calls.append((L.fp8q_rmsnorm_quant,
                              (self.q_h.data_ptr(), self.s_h.data_ptr(), h.data_ptr(),
                               rms_w.data_ptr(), M, h.shape[1], eps, mode), "rmsnorm_quant2"))
        calls.append((L.fp8q_silu_mul_quant, (self.q_g.data_ptr(), self.s_g.data_ptr(),
                                              self.y_gu.data_ptr(), M, D, mode),
                      "silu_mul_quant"))
        b, sb = weights["down"]
        N, K = b.shape
        if mode == PER_TOKEN:
            args = (self.y_down.data_ptr(), self.q_g.data_ptr(), b.data_ptr(),
                    self.s_g.data_ptr(), sb.data_ptr(), M, N, K, ws_p, need)
            calls.append((L.fp8q_scaled_mm, args, "down"))
        else:
            args = (self.y_down.data_ptr(), self.q_g.data_ptr(), b.data_ptr(),
                    self.s_g.data_ptr(), sb.data_ptr(), M, N, K, ws_p, need)
            calls.append((L.fp8q_scaled_mm_blockwise, args, "down"))
        # execution order: rmsnorm_quant, qkv, quant, o_proj, rmsnorm_quant2, gate_up,
        # silu_mul_quant, down
        order = ["rmsnorm_quant", "qkv", "quant", "o_proj", "rmsnorm_quant2", "gate_up",
                 "silu_mul_quant", "down"]
        by_label = {c[2]: c for c in calls}
        self.calls = [by_label[n] for n in order]
        self.graph = None

    def outputs(self):
        return {"y_qkv": self.y_qkv, "y_o": self.y_o, "y_gate_up": self.y_gu,
                "y_down": self.y_down}

    def run(self) -> None:
        """Enqueue the chain on the current stream."""
        st = torch.cuda.current_stream().cuda_stream
        for fn, args, label in self.calls:
            _check(fn(*args, st), label)

    def capture(self) -> torch.cuda.CUDAGraph:
        """Record the chain into a graph (after one eager warm-up on a side
        stream, which also performs every one-time set-up of the library)."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run()
        torch.cuda.synchronize()
        self.graph = g
        return g

    def replay(self) -> None:
        self.graph.replay()


def capture_stack(chains) -> torch.cuda.CUDAGraph:
    """Record the chains of several decoder layers back to back into one
    graph, as a decode step of a whole stack runs them (each chain with its
    own weights and buffers).  One replay then issues every layer's launches
    with a single host call, and the GPU runs them without the gap that
    separates two replays."""
    chains = list(chains)
    if not chains:
        raise ValueError("capture_stack needs at least one chain")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in chains:
            c.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in chains:
            c.run()
    torch.cuda.synchronize()
    return g
