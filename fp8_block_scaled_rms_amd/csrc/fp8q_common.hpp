// Shared device helpers of the fp8q kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

constexpr float kE4M3Max = 448.0f;
constexpr int kGroup = 128;  // 1x128 activation groups, 128x128 weight blocks

// ------------------------------------------------------ buffer loads --
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Buffer resource for raw loads from [base, base + bytes) (bytes < 2^32).
// A load whose offset lies outside that range returns zeros and reads no
// memory, so a resource doubles as a branch-free mask.  Word 3 is the gfx9
// family's raw buffer format (32-bit data format, no swizzle, no thread-id
// offset).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 bit_cast_u4(v4u v) { return make_uint4(v[0], v[1], v[2], v[3]); }

// ---------------------------------------------------------------- bf16 --
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// ---------------------------------------------------- quotient y / s --
// The quantizers need RN32(y / s) exactly (IEEE fp32 division) for fp32 y
// and s > 0.  It is formed from an fp64 product: q = RN32(RN64(y * r)) with
// r an fp64 reciprocal of s of relative error at most 2^-53 (1 + 2^-30):
// RN64(1/s), or the refined reciprocal of recip_refine below.
// Why that is exact:
//  * q64 = RN64(y * r) differs from y/s by a relative error below 2^-51.9.
//  * RN32(q64) != RN32(y/s) needs an fp32 rounding boundary (a midpoint m of
//    two adjacent fp32 values, a number with a 25-bit odd significand when
//    y/s >= 2^-126) between q64 and y/s, or at q64.
//  * y/s is never a midpoint: y = m * s would give y an odd significand of at
//    least 25 bits.  And it is never close to one: y - m*s is a non-zero
//    multiple of 2^min(ey, em + es) (ulp exponents of y, m and s), so at
//    least 2^-24 |y| or 2^-49 |m s|, since y, m and s have at most 24, 25 and
//    24 significant bits.  So |y/s - m| >= 2^-49 |m|, while |q64 - y/s| <
//    2^-51.9 |y/s|: no boundary lies between them.
//  * Quotients below 2^-126 (where fp32 midpoints have fewer bits) keep
//    their sign and a magnitude below 2^-125; every such quotient encodes to
//    a signed zero in e4m3 and int8, the only use made of them.
//  * q64 cannot overflow; a huge quotient converts to +-inf, which the
//    encoders saturate (only a static scale allows it).
// Three fp64-unit instructions (widen, multiply, narrow) per element, where
// a two-step fp32 correction of y * RN32(1/s) takes six.
// tests/host/div_check.cpp checks it against IEEE division on the host.
__host__ __device__ __forceinline__ float div_rn_f64(float y, double r) {
  return static_cast<float>(static_cast<double>(y) * r);
}

// Scale of a group and the fp64 reciprocal used by its quotients; a zero
// scale (all-zero group, or amax below 448 * 2^-150) takes r = 1, so the
// quotients are the signed zeros (or values below 2^-140) that encode to
// +-0, as the definition asks of a zero scale.
struct GroupScale {
  float s;
  double r;
};
__host__ __device__ __forceinline__ double recip_or_one(float s) {
  return s > 0.0f ? 1.0 / static_cast<double>(s) : 1.0;
}

// fp64 reciprocal of s from an fp32 seed within 4 ulp of 1/s (the hardware
// reciprocal is within 1 ulp), by two Newton steps r += r (1 - s r), each
// with one rounding of the residual and one of the update.  A seed of
// relative error d0 <= 2^-21 leaves at most d0^2 + 2^-53 (1 + d0) <= 2^-41.9
// after the first step and 2^-53 (1 + 2^-30) after the second, which keeps
// the quotient's fp64 product within the 2^-51.9 the exactness argument
// above needs.  For s in [2^-110, 2^120], where 1/s and the seed are normal
// fp32 numbers (scales of groups with amax >= 2^-100 lie in [2^-109, 2^120)).
__host__ __device__ __forceinline__ double recip_refine(float s, float seed) {
  const double d = s;
  double r = seed;
  r = fma(r, fma(-d, r, 1.0), r);
  r = fma(r, fma(-d, r, 1.0), r);
  return r;
}
__device__ __forceinline__ float rcp_seed(float s) { return __builtin_amdgcn_rcpf(s); }

// Scale s = RN32(amax / d) for d = 448 (e4m3) or 127 (int8) and its
// reciprocal.  Above amax = 2^-100 (scales of 2^-109 and more, normal
// quotients): s by the same fp64-product argument with r = RN64(1/d) (d has
// 3 and 7 significant bits), the reciprocal by recip_refine.  Below: IEEE
// division and the correctly rounded fp64 reciprocal.
__host__ __device__ __forceinline__ float scale_div(float amax, double recip_d, float d) {
  if (__builtin_expect(amax >= 0x1p-100f, 1)) return div_rn_f64(amax, recip_d);
  return amax / d;
}
constexpr double kRecip448 = 1.0 / 448.0;  // RN64 (constant-folded IEEE division)
constexpr double kRecip127 = 1.0 / 127.0;
__device__ __forceinline__ GroupScale scale_and_recip(float amax, double recip_d, float d) {
  GroupScale g;
  if (__builtin_expect(amax >= 0x1p-100f, 1)) {
    g.s = div_rn_f64(amax, recip_d);
    g.r = recip_refine(g.s, rcp_seed(g.s));
  } else {
    g.s = amax / d;
    g.r = recip_or_one(g.s);
  }
  return g;
}
__device__ __forceinline__ GroupScale make_scale(float amax) {
  return scale_and_recip(amax, kRecip448, kE4M3Max);
}
// Symmetric int8 scale amax / 127 (W8A8 INT8).
__device__ __forceinline__ GroupScale make_scale_i8(float amax) {
  return scale_and_recip(amax, kRecip127, 127.0f);
}

// Power-of-two (UE8M0) scale: the smallest s = 2^e, e >= -127, with
// 448 * s >= amax.  For amax in [2^k, 2^(k+1)) that is 2^(k-8) when
// amax <= 448 * 2^(k-8) = 1.75 * 2^k, else 2^(k-7); amax below 2^-126 (or
// zero) gets the least UE8M0 value 2^-127.  The reciprocal is exact.
__device__ __forceinline__ GroupScale make_scale_ue8m0(float amax) {
  int e = -127;
  if (amax >= 0x1p-126f) {
    const uint32_t biased = (__float_as_uint(amax) >> 23) & 0xFFu;  // k + 127
    const float bound = __uint_as_float((biased << 23) | 0x600000u);  // 1.75 * 2^k
    const int k = static_cast<int>(biased) - 127;
    e = (amax <= bound) ? k - 8 : k - 7;
    if (e < -127) e = -127;
  }
  GroupScale g;
  g.s = (e >= -126) ? __uint_as_float(static_cast<uint32_t>(e + 127) << 23) : 0x1p-127f;
  g.r = recip_or_one(g.s);
  return g;
}

// A caller-given (static) scale s > 0.
__device__ __forceinline__ GroupScale static_scale(float s) {
  GroupScale g;
  g.s = s;
  g.r = recip_or_one(s);
  return g;
}

// y / s rounded to fp32 (any scale: dynamic, power of two or static).
__device__ __forceinline__ float quotient(float y, const GroupScale& g) {
  return div_rn_f64(y, g.r);
}

// ------------------------------------------------------------- e4m3 --
// Four fp32 values -> four OCP e4m3 bytes (little-endian order a,b,c,d),
// round to nearest even, saturating to +-448.  The clamp makes the
// saturation explicit; the hardware conversion rounds to nearest even.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, -kE4M3Max, kE4M3Max);
  b = __builtin_amdgcn_fmed3f(b, -kE4M3Max, kE4M3Max);
  c = __builtin_amdgcn_fmed3f(c, -kE4M3Max, kE4M3Max);
  d = __builtin_amdgcn_fmed3f(d, -kE4M3Max, kE4M3Max);
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return static_cast<uint32_t>(v);
}
// The same for quotients by a dynamic scale (amax / 448 rounded, or the
// power of two at or above it): |v| <= 448 (1 + 2^-23), so no clamp.  The
// hardware conversion rounds to nearest even over the whole of (448, 464]
// to +-448 (a NaN code appears only above 464, where no such quotient
// lies); tests/test_gpu_quant.py checks the amax elements whose quotient is
// 448 + 2^-15.
__device__ __forceinline__ uint32_t pack4_e4m3_dynamic(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return static_cast<uint32_t>(v);
}

// ------------------------------------------------------------- int8 --
// Four fp32 quotients -> four int8 bytes: round to nearest even (the
// default rounding mode), saturating to +-127.  Clamping first is the same
// as clamping after: +-127 are integers.
__device__ __forceinline__ uint32_t i8_byte(float v) {
  const float r = __builtin_rintf(__builtin_amdgcn_fmed3f(v, -127.0f, 127.0f));
  return static_cast<uint32_t>(static_cast<int>(r)) & 0xFFu;
}
__device__ __forceinline__ uint32_t pack4_i8(float a, float b, float c, float d) {
  return i8_byte(a) | (i8_byte(b) << 8) | (i8_byte(c) << 16) | (i8_byte(d) << 24);
}

// ------------------------------------------------------ reductions --
// DPP controls for lane moves inside rows of 16 lanes.
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror

// Maxima of amax candidates: non-negative floats (|y| or +0, never NaN or
// -0), which order as their bit patterns do as unsigned integers.  The
// integer max needs none of the NaN-quieting moves the compiler adds around
// a float max of values that come from lane moves.
__device__ __forceinline__ uint32_t u32_max(uint32_t v, uint32_t w) { return v > w ? v : w; }
// max over each aligned group of 16 lanes; every lane gets its group's max.
__device__ __forceinline__ float max16(float v) {
  uint32_t u = __float_as_uint(v);
  u = u32_max(u, __builtin_amdgcn_mov_dpp(u, kDppQuadXor1, 0xF, 0xF, false));
  u = u32_max(u, __builtin_amdgcn_mov_dpp(u, kDppQuadXor2, 0xF, 0xF, false));
  u = u32_max(u, __builtin_amdgcn_mov_dpp(u, kDppHalfMirror, 0xF, 0xF, false));
  u = u32_max(u, __builtin_amdgcn_mov_dpp(u, kDppMirror, 0xF, 0xF, false));
  return __uint_as_float(u);
}
// max over the whole wave (all lanes get it).
__device__ __forceinline__ float max64(float v) {
  uint32_t u = __float_as_uint(max16(v));
  u = u32_max(u, static_cast<uint32_t>(__shfl_xor(static_cast<int>(u), 16)));
  u = u32_max(u, static_cast<uint32_t>(__shfl_xor(static_cast<int>(u), 32)));
  return __uint_as_float(u);
}
// fp64 sum over the wave; butterfly order, every lane gets the same value.
__device__ __forceinline__ double sum64(double v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace fp8q
