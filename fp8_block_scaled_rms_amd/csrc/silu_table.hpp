// Correctly rounded SiLU of bf16 gates for the fp8q kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

// Correctly rounded SiLU over bf16 gates: table for |g| in [2^-25, 2^7),
// closed rules outside it (silu(g) = g/2 exactly in fp32 below 2^-25;
// silu(g) = g above 2^7; silu(g) rounds to -0 below -2^7).  The table (8192
// fp32 bit patterns, written at build time by gen_silu_table.cpp) is copied
// into LDS by the kernels that use it; each translation unit holds its own
// copy in device memory.
static __device__ const uint32_t kSiluTable[8192] = {
#include "silu_table.inc"
};
constexpr uint32_t kSiluLo = 102u << 7;  // |g| >= 2^-25
constexpr uint32_t kSiluHi = 134u << 7;  // |g| <  2^7

// Branch-free: the table is read for every gate, at the clamped magnitude (an
// in-range index), and selects pick the closed rules.  With branches, each
// lookup's LDS read had to complete before the next gate's code could run
// (the paths join on the result register), so reads never overlapped.
// Where every product of a row is kept in registers (the per-token SiLU
// quantizer), the overlapping reads cost more registers than they save time,
// and silu_bf16_branchy (same values) serves.
__device__ __forceinline__ float silu_bf16(uint32_t bits, const float* tab) {
  const uint32_t a = bits & 0x7FFFu;
  const float g = __uint_as_float(bits << 16);
  const uint32_t ac = a < kSiluLo ? kSiluLo : (a >= kSiluHi ? kSiluHi - 1u : a);
  const float t = tab[(ac - kSiluLo) | ((bits & 0x8000u) >> 3)];
  const float big = (bits & 0x8000u) ? -0.0f : g;
  const float r = a >= kSiluHi ? big : t;
  return a < kSiluLo ? g * 0.5f : r;
}
__device__ __forceinline__ float silu_bf16_branchy(uint32_t bits, const float* tab) {
  const uint32_t a = bits & 0x7FFFu;
  const float g = __uint_as_float(bits << 16);
  if (a < kSiluLo) return g * 0.5f;
  if (a >= kSiluHi) return (bits & 0x8000u) ? -0.0f : g;
  return tab[(a - kSiluLo) | ((bits & 0x8000u) >> 3)];
}

}  // namespace fp8q
