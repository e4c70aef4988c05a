"""Seeded synthetic inputs for the FP8 quantized-linear path.

This module only draws random data in the storage formats the path consumes
(bf16 bit patterns, fp32 arrays, raw e4m3 bytes).  It performs none of the
method's arithmetic: no normalisation, no activation, no amax, no scale, no
e4m3 encoding.  Both the CPU oracle (in tests) and the GPU path consume the
arrays it returns, so it is the only code the two sides share.

Workload shapes follow the Qwen3 FP8 inference runs described on the page
"Helion in vLLM: FP8 inference of Qwen3" (24-ai.news, 2026-06-10), section
"Whole-model speedup" (Qwen3 1.7B / 8B / 32B); the value distributions are
the ones stated for the benchmark workloads:

* activations X ~ N(0, 1) with 1 % of the columns (chosen by the seed)
  multiplied by 20 before the bf16 cast;
* RMSNorm weight 1 + N(0, 0.1);
* gate_up ~ N(0, 2) (2 is the standard deviation);
* linear weights W ~ N(0, 0.02).

Every generator takes a ``numpy.random.Generator``; ``rng_for`` derives one
from a string key with CRC32 so that a (config, op, M, N, K) tuple always
yields the same bytes on every machine.
"""
from __future__ import annotations

import zlib

import numpy as np

__all__ = [
    "rng_for",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "gen_activations",
    "gen_rms_weight",
    "gen_gate_up",
    "gen_linear_weight",
    "gen_e4m3_codes",
    "gen_scales",
]


def rng_for(*key) -> np.random.Generator:
    """PCG64 generator seeded with crc32 of the '|'-joined key."""
    seed = zlib.crc32("|".join(str(k) for k in key).encode())
    return np.random.default_rng(seed)


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even) and return
    the 16-bit patterns as uint16.  Inputs must be finite."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to fp32 exactly."""
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def gen_activations(rng, M: int, K: int, outlier_frac: float = 0.01,
                    outlier_mult: float = 20.0) -> np.ndarray:
    """X ~ N(0,1) [M,K] with round(outlier_frac*K) distinct seeded columns
    scaled by outlier_mult, returned as bf16 bits [M,K]."""
    x = rng.standard_normal((M, K), dtype=np.float32)
    n_out = int(round(outlier_frac * K))
    if n_out > 0:
        cols = rng.choice(K, size=n_out, replace=False)
        x[:, cols] *= np.float32(outlier_mult)
    return f32_to_bf16_bits(x)


def gen_rms_weight(rng, K: int, std: float = 0.1) -> np.ndarray:
    """RMSNorm weight 1 + N(0, std) as bf16 bits [K]."""
    w = np.float32(1.0) + np.float32(std) * rng.standard_normal(K, dtype=np.float32)
    return f32_to_bf16_bits(w)


def gen_gate_up(rng, M: int, D: int, std: float = 2.0) -> np.ndarray:
    """gate_up ~ N(0, std) as bf16 bits [M, 2D]; columns [0,D) are the gate,
    [D,2D) the up projection."""
    g = np.float32(std) * rng.standard_normal((M, 2 * D), dtype=np.float32)
    return f32_to_bf16_bits(g)


def gen_linear_weight(rng, N: int, K: int, std: float = 0.02) -> np.ndarray:
    """Full-precision linear weight W ~ N(0, std) as fp32 [N, K]."""
    return np.float32(std) * rng.standard_normal((N, K), dtype=np.float32)


def gen_e4m3_codes(rng, shape, allow_negative: bool = True) -> np.ndarray:
    """Uniformly random finite OCP e4m3 byte codes (the two NaN codes 0x7F
    and 0xFF are never drawn)."""
    c = rng.integers(0, 0x7F, size=shape, dtype=np.uint8)  # 0x00..0x7E
    if allow_negative:
        sign = rng.integers(0, 2, size=shape, dtype=np.uint8) << 7
        c = c | sign
    return c


def gen_scales(rng, shape, lo: float = 2.0 ** -12, hi: float = 2.0 ** -4) -> np.ndarray:
    """Positive fp32 scales, log-uniform in [lo, hi)."""
    e = rng.uniform(np.log2(lo), np.log2(hi), size=shape)
    return np.exp2(e).astype(np.float32)
