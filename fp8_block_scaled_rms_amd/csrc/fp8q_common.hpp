// Shared device helpers of the fp8q kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

constexpr float kE4M3Max = 448.0f;
constexpr int kGroup = 128;  // 1x128 activation groups, 128x128 weight blocks

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
// Correctly rounded fp32 quotient y / s given r = RN(1/s), for
// 2^-76 <= s < 2^126 and |y| <= 449 s.  Markstein's correction (P. Markstein,
// "Computation of elementary functions on the IBM RISC System/6000
// processor", IBM J. Res. Dev. 34(1), 1990): one correction step turns the
// product y*r (within ~2 ulp) into a faithful quotient, and a second step
// with an exact remainder then yields the correctly rounded quotient.  That
// holds whenever |y| >= 2^-100 and |y/s| >= 2^-125 (the remainders are then
// exact); otherwise the result still has the sign of y and magnitude below
// 2^-22, which is all the e4m3 encoder needs (such quotients encode to +-0).
// copysign restores the sign of a zero quotient (the correction turns -0
// into +0).  tests/host/div_check.cpp checks this against IEEE division.
__host__ __device__ __forceinline__ float div_rn_corrected(float y, float s, float r) {
  float q0 = y * r;
  float e0 = fmaf(-q0, s, y);
  float q1 = fmaf(e0, r, q0);
  float e1 = fmaf(-q1, s, y);
  float q2 = fmaf(e1, r, q1);
  return copysignf(q2, y);
}

// Scale of a group from its amax, the reciprocal used by the corrected
// quotient, and whether the fast quotient is valid for that scale.
struct GroupScale {
  float s;
  float r;
  bool fast;
};
__device__ __forceinline__ GroupScale make_scale(float amax) {
  GroupScale g;
  g.s = amax / kE4M3Max;  // IEEE division (correctly rounded build flags)
  g.fast = g.s >= 0x1p-76f;
  g.r = g.fast ? 1.0f / g.s : 1.0f;
  return g;
}
// Symmetric int8 scale amax / 127 (W8A8 INT8).
__device__ __forceinline__ GroupScale make_scale_i8(float amax) {
  GroupScale g;
  g.s = amax / 127.0f;  // IEEE division
  g.fast = g.s >= 0x1p-76f;
  g.r = g.fast ? 1.0f / g.s : 1.0f;
  return g;
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
  g.fast = g.s >= 0x1p-76f;
  g.r = g.fast ? 1.0f / g.s : 1.0f;
  return g;
}

// A caller-given (static) scale s > 0: the fast quotient where its proof
// holds, IEEE division elsewhere.
__device__ __forceinline__ GroupScale static_scale(float s) {
  GroupScale g;
  g.s = s;
  g.fast = s >= 0x1p-76f && s < 0x1p126f;
  g.r = g.fast ? 1.0f / s : 1.0f;
  return g;
}

// y / s rounded to fp32; a zero scale (all-zero group) passes y (a signed
// zero) through.
__device__ __forceinline__ float quotient(float y, const GroupScale& g) {
  if (g.fast) return div_rn_corrected(y, g.s, g.r);
  return g.s == 0.0f ? y : y / g.s;
}
// The same for a static scale, where |y| may exceed 448 s by any factor: y
// is first clamped to +-449 s (any quotient of magnitude >= 448 encodes to
// +-448 anyway), which keeps the fast quotient inside its proven range.
__device__ __forceinline__ float quotient_static(float y, const GroupScale& g) {
  if (g.fast) {
    const float lim = 449.0f * g.s;
    return div_rn_corrected(__builtin_amdgcn_fmed3f(y, -lim, lim), g.s, g.r);
  }
  return y / g.s;
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
// DPP lane moves inside rows of 16 lanes.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror

// max over each aligned group of 16 lanes; every lane gets its group's max.
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v));
  return v;
}
// max over the whole wave (all lanes get it).
__device__ __forceinline__ float max64(float v) {
  v = max16(v);
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
// fp64 sum over the wave; butterfly order, every lane gets the same value.
__device__ __forceinline__ double sum64(double v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace fp8q
