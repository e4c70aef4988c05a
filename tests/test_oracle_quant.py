"""Pins of the oracle's quantizers against closed forms, invariants and
independent library evaluations."""
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import e4m3, quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _groups(seed=0, n=400, L=128):
    rng = np.random.default_rng(seed)
    scale_pow = rng.integers(-20, 20, size=(n, 1)).astype(np.float32)
    y = rng.standard_normal((n, L)).astype(np.float32) * np.exp2(scale_pow)
    y[::7, rng.integers(0, L)] *= 20
    return y.astype(np.float32)


def test_amax_element_encodes_to_448():
    y = _groups()
    codes, scale = quant.quantize_vectors(y)
    idx = np.argmax(np.abs(y), axis=1)
    amax_codes = codes[np.arange(len(y)), idx]
    want = np.where(y[np.arange(len(y)), idx] < 0, 0xFE, 0x7E)
    assert np.array_equal(amax_codes, want)
    # and no code exceeds the max magnitude
    assert np.all((codes & 0x7F) <= 0x7E)


def test_quantization_error_bound():
    y = _groups(1)
    codes, scale = quant.quantize_vectors(y)
    deq = e4m3.decode(codes) * scale.astype(np.float64)[:, None]
    err = np.abs(deq - y.astype(np.float64))
    bound = np.maximum(2.0 ** -4 * np.abs(y.astype(np.float64)),
                       2.0 ** -10 * scale.astype(np.float64)[:, None]) * (1 + 2.0 ** -20)
    assert np.all(err <= bound)


def test_scale_is_amax_over_448_ieee():
    y = _groups(2)
    _, scale = quant.quantize_vectors(y)
    amax = np.max(np.abs(y.astype(np.float64)), axis=1)
    # correctly rounded quotient: compare with torch's fp32 division
    ref = (torch.from_numpy(amax.astype(np.float32)) / torch.tensor(448.0)).numpy()
    assert np.array_equal(scale, ref)
    # and it is within half an ulp of the exact quotient
    exact = amax / 448.0
    assert np.all(np.abs(scale.astype(np.float64) - exact) <= 0.5 * np.spacing(scale).astype(np.float64))


def test_power_of_two_invariance():
    y = _groups(3)
    c0, s0 = quant.quantize_vectors(y)
    for j in (-5, 3, 11):
        c1, s1 = quant.quantize_vectors((y * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(c0, c1)
        assert np.array_equal(s1, (s0 * np.float32(2.0 ** j)).astype(np.float32))


def test_sign_flip():
    y = _groups(4)
    c0, s0 = quant.quantize_vectors(y)
    c1, s1 = quant.quantize_vectors(-y)
    assert np.array_equal(s0, s1)
    assert np.array_equal(c1, c0 ^ 0x80)


def test_constant_zero_and_tiny_groups():
    L = 128
    c, s = quant.quantize_vectors(np.full((1, L), 3.25, np.float32))
    assert np.all(c == 0x7E) and s[0] == np.float32(np.float32(3.25) / np.float32(448))
    z = np.zeros((1, L), np.float32)
    z[0, 1::2] = -0.0
    c, s = quant.quantize_vectors(z)
    assert s[0] == 0
    assert np.array_equal(c[0], np.where(np.signbit(z[0]), 0x80, 0x00).astype(np.uint8))


def test_tie_vector_from_golden():
    with open(os.path.join(GOLDEN, "quant_tie_vector.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for y0, y1, sbits, c0, c1, c1_recip in rows:
        y = np.array([float(y0), float(y1)], np.float32)
        codes, scale = quant.quantize_vectors(y)
        assert scale.view(np.uint32) == int(sbits, 16)
        assert codes.tolist() == [int(c0, 16), int(c1, 16)]
        assert int(c1, 16) != int(c1_recip, 16)


def test_per_token_and_group_layouts():
    rng = synth.rng_for("t", "layout")
    x = synth.gen_activations(rng, 5, 384)
    qt, st = quant.quantize(x, quant.PER_TOKEN)
    qg, sg = quant.quantize(x, quant.GROUP128)
    assert qt.shape == (5, 384) and st.shape == (5,)
    assert qg.shape == (5, 384) and sg.shape == (5, 3)
    xf = synth.bf16_bits_to_f32(x)
    for m in range(5):
        c, s = quant.quantize_vectors(xf[m])
        assert np.array_equal(qt[m], c) and st[m] == s
        for g in range(3):
            c, s = quant.quantize_vectors(xf[m, g * 128:(g + 1) * 128])
            assert np.array_equal(qg[m, g * 128:(g + 1) * 128], c) and sg[m, g] == s


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_constant_row_reduces_to_quantized_weight():
    """x = c (a power of two) everywhere and eps far below half an ulp of c^2:
    inv = 1/|c| exactly, so y = w * sign(c) and the codes are those of w."""
    K = 256
    rng = synth.rng_for("t", "rms-const")
    w = synth.gen_rms_weight(rng, K)
    wf = synth.bf16_bits_to_f32(w)
    for c in (0.25, -4.0, 2.0 ** 10):
        x = synth.f32_to_bf16_bits(np.full((1, K), c, np.float32))
        for mode in (quant.PER_TOKEN, quant.GROUP128):
            q, s = quant.rmsnorm_quant(x, w, 2.0 ** -80, mode)
            q2, s2 = quant._quantize_rows((wf * np.float32(np.sign(c)))[None, :], mode)
            assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_rmsnorm_one_hot_row():
    """x = c e_j, K = 256, c a power of two, tiny eps: inv = 16/c exactly,
    y_j = 16 w_j, so code_j = +-448 and every other code is a signed zero."""
    K = 256
    rng = synth.rng_for("t", "rms-onehot")
    w = synth.gen_rms_weight(rng, K)
    wf = synth.bf16_bits_to_f32(w)
    for j, c in ((0, 1.0), (77, -8.0), (255, 0.5)):
        xf = np.zeros((1, K), np.float32)
        xf[0, j] = c
        q, s = quant.rmsnorm_quant(synth.f32_to_bf16_bits(xf), w, 2.0 ** -90, quant.PER_TOKEN)
        # x_i = +0 off the hot index: y_i = (+0 * w_i) * inv has the sign of w_i
        want = np.where(np.signbit(wf), 0x80, 0x00).astype(np.uint8)
        want[j] = 0xFE if (c * wf[j]) < 0 else 0x7E
        assert np.array_equal(q[0], want)
        assert s[0] == np.float32(np.float32(16 * abs(wf[j])) / np.float32(448))


def test_rmsnorm_y_vs_float64_formula():
    """y agrees with an fp64 torch evaluation of x * w / sqrt(mean(x^2) + eps)
    to within 1.5 fp32 ulp (the exact product rounded twice)."""
    rng = synth.rng_for("t", "rms-f64")
    M, K = 64, 2048
    x = synth.gen_activations(rng, M, K)
    w = synth.gen_rms_weight(rng, K)
    inv, _ = quant.rms_inv(x, 1e-6)
    y = quant.rmsnorm_y(x, w, inv).astype(np.float64)
    xt = torch.from_numpy(synth.bf16_bits_to_f32(x).astype(np.float64))
    wt = torch.from_numpy(synth.bf16_bits_to_f32(w).astype(np.float64))
    ref = (xt * torch.rsqrt(xt.pow(2).mean(-1, keepdim=True) + float(np.float32(1e-6))) * wt).numpy()
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(y - ref) <= 1.5 * ulp)


def test_rmsnorm_inv_order_independent():
    """fp64 sums in three orders round to the same fp32 inverse RMS."""
    rng = synth.rng_for("t", "rms-order")
    M, K = 200, 5120
    x = synth.gen_activations(rng, M, K)
    inv, _ = quant.rms_inv(x, 1e-6)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    sq = xf * xf
    eps = float(np.float32(1e-6))
    for ss in (np.sum(sq, axis=1), np.cumsum(sq, axis=1)[:, -1],
               sq.reshape(M, 40, 128).sum(axis=2).sum(axis=1)):
        alt = (1.0 / np.sqrt(ss / K + eps)).astype(np.float32)
        assert np.array_equal(alt, inv)


def test_rmsnorm_shapes_and_modes():
    rng = synth.rng_for("t", "rms-shapes")
    x = synth.gen_activations(rng, 3, 256)
    w = synth.gen_rms_weight(rng, 256)
    q, s = quant.rmsnorm_quant(x, w, 1e-6, quant.GROUP128)
    assert q.shape == (3, 256) and s.shape == (3, 2)
    q, s = quant.rmsnorm_quant(x[:0], w, 1e-6, quant.PER_TOKEN)
    assert q.shape == (0, 256) and s.shape == (0,)


# -------------------------------------------------------------- SiLU-mul

def test_silu_mul_y_vs_torch_float64():
    rng = synth.rng_for("t", "silu-mul")
    M, D = 16, 1024
    gu = synth.gen_gate_up(rng, M, D)
    y = quant.silu_mul_y(gu).astype(np.float64)
    g = torch.from_numpy(synth.bf16_bits_to_f32(gu[:, :D]).astype(np.float64))
    u = torch.from_numpy(synth.bf16_bits_to_f32(gu[:, D:]).astype(np.float64))
    ref = (torch.nn.functional.silu(g) * u).numpy()
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(y - ref) <= 1.5 * ulp + 1e-45)


def test_silu_mul_gate_first_half():
    """With up = 1, y is silu(gate); with gate large (silu(g) = g), y = g*up."""
    D = 128
    g = np.linspace(-6, 6, D).astype(np.float32)
    gu = synth.f32_to_bf16_bits(np.concatenate([g, np.ones(D, np.float32)])[None, :])
    y = quant.silu_mul_y(gu)[0]
    gb = synth.bf16_bits_to_f32(gu[0, :D]).astype(np.float64)
    ref = gb / (1 + np.exp(-gb))
    assert np.allclose(y, ref, rtol=1e-6, atol=0)
    gu2 = synth.f32_to_bf16_bits(np.concatenate([np.full(D, 32.0, np.float32), g])[None, :])
    y2 = quant.silu_mul_y(gu2)[0]
    assert np.array_equal(y2, (np.float32(32) * synth.bf16_bits_to_f32(gu2[0, D:])).astype(np.float32))


# ------------------------------------------------------- weight quantizers

def test_weight_block128_matches_blockwise_loop():
    rng = synth.rng_for("t", "wq")
    W = synth.gen_linear_weight(rng, 256, 384)
    codes, scale = quant.quant_weight_block128(W)
    assert codes.shape == (256, 384) and scale.shape == (2, 3)
    for i in range(2):
        for j in range(3):
            blk = W[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            amax = np.float32(np.max(np.abs(blk)))
            assert scale[i, j] == np.float32(amax / np.float32(448))
            c = e4m3.encode((blk / scale[i, j]).astype(np.float32))
            assert np.array_equal(codes[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128], c)


def test_weight_per_channel():
    rng = synth.rng_for("t", "wq-ch")
    W = synth.gen_linear_weight(rng, 8, 256)
    codes, scale = quant.quant_weight_per_channel(W)
    for n in range(8):
        amax = np.float32(np.max(np.abs(W[n])))
        assert scale[n] == np.float32(amax / np.float32(448))
        assert np.array_equal(codes[n], e4m3.encode((W[n] / scale[n]).astype(np.float32)))


# ------------------------------------------------ power-of-two (UE8M0) scales

def test_ue8m0_scale_closed_forms():
    """Values fixed by the definition: the smallest 2^e (e >= -127) with
    448 * 2^e >= amax."""
    f = np.float32
    above_448 = np.nextafter(f(448), f(1e9))
    above_175 = np.nextafter(f(1.75), f(1e9))
    cases = [(448.0, 1.0), (above_448, 2.0), (1.0, 2.0 ** -8), (1.75, 2.0 ** -8),
             (above_175, 2.0 ** -7), (0.0, 2.0 ** -127), (1e-45, 2.0 ** -127),
             (3.4e38, 2.0 ** 120), (224.0, 0.5), (56.0, 0.125)]
    amax = np.array([c[0] for c in cases], np.float32)
    want = np.array([c[1] for c in cases], np.float32)
    assert np.array_equal(quant.ue8m0_scale(amax).view(np.uint32), want.view(np.uint32))


def test_ue8m0_scale_properties():
    rng = np.random.default_rng(11)
    amax = (rng.random(5000) * np.exp2(rng.integers(-140, 120, 5000))).astype(np.float32)
    s = quant.ue8m0_scale(amax).astype(np.float64)
    m, e = np.frexp(s)
    assert np.all(m == 0.5)                                   # a power of two
    a = amax.astype(np.float64)
    assert np.all(448.0 * s >= a)                             # covers amax
    assert np.all((s == 2.0 ** -127) | (448.0 * s / 2 < a))   # and is the smallest


def test_ue8m0_quantizer_invariants():
    y = _groups(21)
    codes, scale = quant.quantize_vectors_ue8m0(y)
    rows = np.arange(len(y))
    idx = np.argmax(np.abs(y), axis=1)
    # amax / scale lies in (224, 448], so the amax element encodes to 0x76..0x7E
    mag = codes[rows, idx] & 0x7F
    assert np.all((mag >= 0x76) & (mag <= 0x7E))
    # error of round-to-nearest at the code's own spacing
    deq = e4m3.decode(codes) * scale.astype(np.float64)[:, None]
    err = np.abs(deq - y.astype(np.float64))
    bound = np.maximum(2.0 ** -4 * np.abs(y.astype(np.float64)),
                       2.0 ** -10 * scale.astype(np.float64)[:, None]) * (1 + 2.0 ** -20)
    assert np.all(err <= bound)
    # power-of-two invariance: y * 2^j -> same codes, scale * 2^j
    c2, s2 = quant.quantize_vectors_ue8m0((y * np.float32(2.0 ** 5)).astype(np.float32))
    assert np.array_equal(c2, codes) and np.array_equal(s2, scale * np.float32(32))


def test_ue8m0_equals_ieee_rule_when_amax_is_448_times_a_power_of_two():
    """Where amax / 448 is itself a power of two both scale rules agree, so
    the two quantizers must give the same bytes."""
    y = _groups(22)
    rows = np.arange(len(y))
    idx = np.argmax(np.abs(y), axis=1)
    target = np.exp2(np.floor(np.log2(np.abs(y[rows, idx]))) - 3).astype(np.float32) * np.float32(448)
    z = np.clip(y, -target[:, None] * np.float32(0.99), target[:, None] * np.float32(0.99))
    z[rows, idx] = np.where(y[rows, idx] < 0, -target, target)
    c_ieee, s_ieee = quant.quantize_vectors(z)
    c_ue8, s_ue8 = quant.quantize_vectors_ue8m0(z)
    assert np.array_equal(s_ieee, s_ue8)
    assert np.array_equal(c_ieee, c_ue8)


def test_ue8m0_all_zero_group_and_layouts():
    x = np.zeros((3, 256), np.float32)
    x[1, 130] = -2.5
    bits = synth.f32_to_bf16_bits(x)
    q, s = quant.quantize(bits, quant.GROUP128_UE8M0)
    assert s.shape == (3, 2)
    assert s[0, 0] == np.float32(2.0 ** -127) and s[1, 1] == np.float32(2.0 ** -7)
    assert q[1, 130] == 0xFA  # -2.5 / 2^-7 = -320 = -1.25 * 2^8: exponent 15, mantissa 2
    assert np.all(q[0] == 0)
    qt, st = quant.quantize(bits, quant.PER_TOKEN_UE8M0)
    assert st.shape == (3,) and st[1] == np.float32(2.0 ** -7) and qt[1, 130] == 0xFA


# ---------------------------------------------------- static per-tensor scale

def test_static_scale_reduces_to_dynamic_and_to_plain_encode():
    rng = synth.rng_for("static", 8, 512)
    x = synth.gen_activations(rng, 8, 512)
    # with the dynamic per-token scale of a one-row tensor the codes agree
    q_dyn, s_dyn = quant.quantize(x[:1], quant.PER_TOKEN)
    q_st, s_st = quant.quantize(x[:1], quant.PER_TENSOR_STATIC, scale=s_dyn)
    assert np.array_equal(q_dyn, q_st) and s_st[0] == s_dyn[0]
    # scale 1 is the plain encoder of the bf16 values
    q1, _ = quant.quantize(x, quant.PER_TENSOR_STATIC, scale=np.float32(1.0))
    assert np.array_equal(q1, e4m3.encode(synth.bf16_bits_to_f32(x)))


def test_static_scale_saturates_and_keeps_zero_signs():
    y = np.array([[1e30, -1e30, 448.0 * 3, -0.0, 0.0, 2.0 ** -20]], np.float32)
    q, s = quant.quantize(synth.f32_to_bf16_bits(y), quant.PER_TENSOR_STATIC, scale=np.float32(2.0))
    assert list(q[0][:5]) == [0x7E, 0xFE, 0x7E, 0x80, 0x00]
    with pytest.raises(ValueError):
        quant.quantize(synth.f32_to_bf16_bits(y), quant.PER_TENSOR_STATIC, scale=np.float32(0.0))


def test_static_mode_on_fused_front_ends():
    rng = synth.rng_for("static-fused", 4, 256)
    x = synth.gen_activations(rng, 4, 256)
    w = synth.gen_rms_weight(rng, 256)
    inv, _ = quant.rms_inv(x, 1e-6)
    y = quant.rmsnorm_y(x, w, inv)
    q, s = quant.rmsnorm_quant(x, w, 1e-6, quant.PER_TENSOR_STATIC, scale=np.float32(0.01))
    assert np.array_equal(q, e4m3.encode((y / np.float32(0.01)).astype(np.float32)))
    gu = synth.gen_gate_up(rng, 4, 128)
    q2, _ = quant.silu_mul_quant(gu, quant.PER_TENSOR_STATIC, scale=np.float32(0.5))
    y2 = quant.silu_mul_y(gu)
    assert np.array_equal(q2, e4m3.encode((y2 / np.float32(0.5)).astype(np.float32)))
