"""The decoder-layer FP8 linear chain under a HIP graph: every stage of the
eager chain against the oracle, and every graph replay against the eager
result, with eager work, input changes and synchronizations between the
replays."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_rms_amd as fq
from fp8_block_scaled_rms_amd.graph import LinearChain
import synth
from oracle import gemm, quant
from gpu_util import DEV, bf16_dev, bf16_host, bf16_host_f64, f32_dev, host, say, u8_dev

pytestmark = pytest.mark.gpu

EPS = 1e-6


def _weights(rng, shapes, mode):
    out = {}
    for name, (N, K) in shapes.items():
        W = synth.gen_linear_weight(rng, N, K)
        if mode == fq.PER_TOKEN:
            c, s = quant.quant_weight_per_channel(W)
        else:
            c, s = quant.quant_weight_block128(W)
        out[name] = (c, s)
    return out


def _build(tag, M, hidden, qkv_n, o_k, gu_n, inter, mode):
    rng = synth.rng_for("graph", tag, M)
    x = synth.gen_activations(rng, M, hidden)
    attn = synth.gen_activations(rng, M, o_k)
    h = synth.gen_activations(rng, M, hidden)
    w = synth.gen_rms_weight(rng, hidden)
    shapes = {"qkv": (qkv_n, hidden), "o_proj": (hidden, o_k), "gate_up": (gu_n, hidden),
              "down": (hidden, inter)}
    wts = _weights(rng, shapes, mode)
    dev_w = {n: (u8_dev(c), f32_dev(s)) for n, (c, s) in wts.items()}
    chain = LinearChain(bf16_dev(x), bf16_dev(attn), bf16_dev(h), bf16_dev(w), dev_w, mode, EPS)
    return chain, (x, attn, h, w, wts)


def _ref_gemm(mode, a, sa, b, sb):
    if mode == fq.PER_TOKEN:
        return gemm.scaled_mm(a, b, sa, sb)
    return gemm.scaled_mm_blockwise(a, sa, b, sb)


def _check_eager_against_oracle(chain, host_in, mode):
    x, attn, h, w, wts = host_in
    q, s = quant.rmsnorm_quant(x, w, EPS, mode)
    assert np.array_equal(host(chain.q_x), q) and np.array_equal(host(chain.s_x), s)
    q, s = quant.quantize(attn, mode)
    assert np.array_equal(host(chain.q_a), q) and np.array_equal(host(chain.s_a), s)
    q, s = quant.rmsnorm_quant(h, w, EPS, mode)
    assert np.array_equal(host(chain.q_h), q) and np.array_equal(host(chain.s_h), s)
    for name, qa, sa, y in (("qkv", chain.q_x, chain.s_x, chain.y_qkv),
                            ("o_proj", chain.q_a, chain.s_a, chain.y_o),
                            ("gate_up", chain.q_h, chain.s_h, chain.y_gu)):
        ref = _ref_gemm(mode, host(qa), host(sa), *wts[name])
        res = gemm.acceptance(bf16_host_f64(y), ref)
        assert res["ok"], (name, res)
    # the SiLU stage consumes the GPU's own gate_up output (bf16)
    q, s = quant.silu_mul_quant(bf16_host(chain.y_gu), mode)
    assert np.array_equal(host(chain.q_g), q) and np.array_equal(host(chain.s_g), s)
    ref = _ref_gemm(mode, host(chain.q_g), host(chain.s_g), *wts["down"])
    res = gemm.acceptance(bf16_host_f64(chain.y_down), ref)
    assert res["ok"], ("down", res)


def _snapshot(chain):
    return {k: v.clone() for k, v in chain.outputs().items()} | {
        "q_g": chain.q_g.clone(), "s_g": chain.s_g.clone()}


def _same(a, b):
    return all(torch.equal(a[k], b[k]) for k in a)


CASES = [
    # tag, M, hidden, qkv_n, o_k, gate_up_n, intermediate, mode
    ("small-group", 4, 512, 768, 512, 2048, 1024, fq.GROUP128),
    ("small-per-token", 16, 512, 1024, 512, 2048, 1024, fq.PER_TOKEN),
]


@pytest.mark.parametrize("tag,M,hidden,qkv_n,o_k,gu_n,inter,mode", CASES)
def test_chain_eager_matches_oracle_and_graph_replays_match_eager(tag, M, hidden, qkv_n, o_k,
                                                                   gu_n, inter, mode):
    say("graph chain", tag, M)
    chain, host_in = _build(tag, M, hidden, qkv_n, o_k, gu_n, inter, mode)
    chain.run()
    torch.cuda.synchronize()
    _check_eager_against_oracle(chain, host_in, mode)
    eager = _snapshot(chain)

    chain.capture()
    for rep in range(3):
        # clobber the outputs, replay, compare
        for t in chain.outputs().values():
            t.fill_(7.0)
        chain.replay()
        torch.cuda.synchronize()
        assert _same(_snapshot(chain), eager), f"replay {rep}"
        # eager work of the program between replays
        chain.run()
        junk = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        assert _same(_snapshot(chain), eager) and torch.isfinite(junk)

    # new inputs in place: the replay must read them, and match eager again
    chain.x.copy_(torch.roll(chain.x, 1, dims=0))
    chain.h.mul_(0.5)
    chain.run()
    torch.cuda.synchronize()
    eager2 = _snapshot(chain)
    assert not _same(eager2, eager)
    for t in chain.outputs().values():
        t.fill_(7.0)
    chain.replay()
    torch.cuda.synchronize()
    assert _same(_snapshot(chain), eager2)


def test_chain_graph_at_qwen3_8b_decode_shape():
    """Full Qwen3-8B decode shapes (hidden 4096, QKV 6144, gate_up 24576,
    down K 12288) at M = 8: three replays equal the eager chain."""
    M = 8
    say("graph chain qwen3-8b", M)
    g = torch.Generator(device=DEV)
    g.manual_seed(8)
    dev = DEV

    def w(N, K):
        b = torch.randint(0, 0x7F, (N, K), generator=g, device=dev, dtype=torch.uint8)
        b |= (torch.randint(0, 2, (N, K), generator=g, device=dev, dtype=torch.uint8) << 7)
        s = torch.rand(N // 128, K // 128, generator=g, device=dev) * 1e-3 + 1e-4
        return b, s

    wts = {"qkv": w(6144, 4096), "o_proj": w(4096, 4096), "gate_up": w(24576, 4096),
           "down": w(4096, 12288)}
    x = torch.randn(M, 4096, generator=g, device=dev).to(torch.bfloat16)
    attn = torch.randn(M, 4096, generator=g, device=dev).to(torch.bfloat16)
    h = torch.randn(M, 4096, generator=g, device=dev).to(torch.bfloat16)
    rw = (1 + 0.1 * torch.randn(4096, generator=g, device=dev)).to(torch.bfloat16)
    chain = LinearChain(x, attn, h, rw, wts, fq.GROUP128, EPS)
    chain.run()
    torch.cuda.synchronize()
    eager = _snapshot(chain)
    chain.capture()
    for rep in range(3):
        for t in chain.outputs().values():
            t.fill_(-1.0)
        chain.replay()
        torch.cuda.synchronize()
        assert _same(_snapshot(chain), eager), f"replay {rep}"
        chain.run()
        torch.cuda.synchronize()


@pytest.mark.parametrize("mode", [fq.GROUP128, fq.PER_TOKEN], ids=["group128", "per-token"])
def test_stack_of_layers_in_one_graph_matches_eager(mode):
    """Three layers with distinct weights and inputs recorded into one graph
    (capture_stack): every replay reproduces every layer's eager outputs,
    with eager work between the replays."""
    from fp8_block_scaled_rms_amd.graph import capture_stack

    say("graph stack of 3 layers", mode)
    chains = []
    for layer in range(3):
        chain, host_in = _build(f"stack{layer}-{mode}", 8, 512, 768, 512, 2048, 1024, mode)
        chain.run()
        torch.cuda.synchronize()
        _check_eager_against_oracle(chain, host_in, mode)
        chains.append(chain)
    eager = [_snapshot(c) for c in chains]
    assert not _same(eager[0], eager[1])
    g = capture_stack(chains)
    for rep in range(3):
        for c in chains:
            for t in c.outputs().values():
                t.fill_(7.0)
        g.replay()
        torch.cuda.synchronize()
        for layer, c in enumerate(chains):
            assert _same(_snapshot(c), eager[layer]), f"replay {rep}, layer {layer}"
        for c in chains:
            c.run()
        junk = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for layer, c in enumerate(chains):
            assert _same(_snapshot(c), eager[layer])
