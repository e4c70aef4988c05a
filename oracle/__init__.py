"""CPU oracle for the FP8 quantized-linear path.  TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct numpy / standard-library implementations of
what the path computes.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package; the product
library never calls it and shares no code, table or constant with it.

Sources.  The operations are the ones listed on the page "Helion in vLLM:
FP8 inference of Qwen3" (24-ai.news, 2026-06-10), section "Kernels
integrated into vLLM": per-token and per-token-group FP8 quantization, the
same fused behind an RMSNorm or a SiLU-and-mul, scaled_mm and
scaled_mm_blockwise.  The page says only "FP8"; the format (OCP e4m3), the
scale rule amax/448, the 1x128 activation groups, the 128x128 weight blocks,
fp32 accumulation and bf16 output are the readings adopted for the whole
project (each one is listed with its reason in the design notes).

Modules
  e4m3   -- OCP e4m3 decode (closed form) and round-to-nearest-even encode
  quant  -- the dynamic quantizer and the fused RMSNorm / SiLU-mul front ends,
            plus weight pre-quantization (per channel, per 128x128 block)
  silu   -- correctly rounded fp32 SiLU over every bf16 input
  gemm   -- fp64 dequantized matmuls (scaled_mm, scaled_mm_blockwise) and the
            GEMM acceptance rule
  int8   -- W8A8 INT8: symmetric int8 quantizers and the exact-integer GEMM

Every function here is pinned by a test under tests/ against something other
than itself (library routines, exhaustive enumeration, closed forms, exact
rational arithmetic); see each module's docstring.
"""
from . import e4m3, quant, silu, gemm, int8  # noqa: F401

PER_TOKEN = 0
GROUP128 = 1
GROUP = 128
