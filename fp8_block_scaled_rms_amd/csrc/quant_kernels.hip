// Fused front end + dynamic FP8 (OCP e4m3) quantization kernels for gfx950.
//
// One kernel template covers the quantizers named on the page "Helion in
// vLLM: FP8 inference of Qwen3" (24-ai.news), section "Kernels integrated
// into vLLM":
//   kIdent  dynamic_per_token_scaled_fp8_quant / per_token_group_fp8_quant
//   kRms    rms_norm_dynamic_per_token_quant   / rms_norm_per_block_quant
//   kSilu   silu_and_mul_dynamic_per_token_quant / silu_and_mul_per_block_quant
// each with a per-token (one scale per row) or per-1x128-group scale.
//
// The work is HBM-bound (3 B per element for RMSNorm, 5 B per output element
// for SiLU-and-mul), so the design is about streaming: a work unit is a whole
// row (per-token mode, and RMSNorm, whose inverse RMS spans the row) or a
// 2048*CH-column segment of a row (group mode).  A 256-thread workgroup owns a
// unit; thread t owns the 8-element (16-byte) chunks t, t+256, ... so every
// load and store is a coalesced 128-bit access, and the 16 consecutive lanes
// that hold one 128-element group reduce its amax with four DPP moves.
// Workgroups loop over units (grid-stride) so that per-workgroup set-up (the
// SiLU table in LDS) is amortised.
#include "fp8q_common.hpp"
#include "quant_kernels.h"

namespace fp8q {

namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 8;  // bf16 elements per 16-byte chunk
constexpr int kSeg = kThreads * kChunk;  // columns covered per CH step

// Correctly rounded SiLU over bf16 gates: table for |g| in [2^-25, 2^7),
// closed rules outside it (silu(g) = g/2 exactly in fp32 below 2^-25;
// silu(g) = g above 2^7; silu(g) rounds to -0 below -2^7).
__device__ const uint32_t kSiluTable[8192] = {
#include "silu_table.inc"
};
constexpr uint32_t kSiluLo = 102u << 7;  // |g| >= 2^-25
constexpr uint32_t kSiluHi = 134u << 7;  // |g| <  2^7

__device__ __forceinline__ float silu_bf16(uint32_t bits, const float* tab) {
  const uint32_t a = bits & 0x7FFFu;
  const float g = __uint_as_float(bits << 16);
  if (a < kSiluLo) return g * 0.5f;
  if (a >= kSiluHi) return (bits & 0x8000u) ? -0.0f : g;
  return tab[(a - kSiluLo) | ((bits & 0x8000u) >> 3)];
}

__device__ __forceinline__ void load_silu_table(float* lds) {
  const uint4* src = reinterpret_cast<const uint4*>(kSiluTable);
  uint4* dst = reinterpret_cast<uint4*>(lds);
  for (int i = threadIdx.x; i < 8192 / 4; i += kThreads) dst[i] = src[i];
  __syncthreads();
}

// Reduce across the 4 waves of the workgroup through LDS (fixed order).
__device__ __forceinline__ double block_sum(double v, double* red) {
  v = sum64(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  double t = ((red[0] + red[1]) + red[2]) + red[3];
  __syncthreads();
  return t;
}
__device__ __forceinline__ float block_max(float v, float* red) {
  v = max64(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float t = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return t;
}

template <int OP, int MODE, int CH>
__global__ __launch_bounds__(kThreads) void quant_kernel(uint8_t* __restrict__ q,
                                                         float* __restrict__ scale,
                                                         const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ w, int M,
                                                         int K, float eps) {
  __shared__ double red64[4];
  __shared__ float red32[4];
  extern __shared__ float silu_tab[];
  if constexpr (OP == kSilu) load_silu_table(silu_tab);

  const int tid = threadIdx.x;
  const int nchunk = K / kChunk;              // chunks per row
  const int seg_cols = (MODE == kPerToken || OP == kRms) ? K : kSeg * CH;
  const int nseg = (K + seg_cols - 1) / seg_cols;
  const long units = static_cast<long>(M) * nseg;
  const long in_stride = (OP == kSilu) ? 2L * K : K;  // elements per input row

  for (long unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const int row = static_cast<int>(unit / nseg);
    const int seg = static_cast<int>(unit % nseg);
    const int c0 = seg * (seg_cols / kChunk);  // first chunk of this unit
    const uint16_t* xr = x + row * in_stride;

    // ---- load and front end: y (fp32) per element, kept in registers
    float y[CH][kChunk];
    bool valid[CH];
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = c0 + tid + i * kThreads;
      valid[i] = (c < nchunk) && (c < c0 + seg_cols / kChunk);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (valid[i]) v = *reinterpret_cast<const uint4*>(xr + c * kChunk);
      const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
      if constexpr (OP == kIdent) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          y[i][2 * j] = bf16_lo(vv[j]);
          y[i][2 * j + 1] = bf16_hi(vv[j]);
        }
      } else if constexpr (OP == kRms) {
        uint4 wv = make_uint4(0, 0, 0, 0);
        if (valid[i]) wv = *reinterpret_cast<const uint4*>(w + c * kChunk);
        const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x0 = bf16_lo(vv[j]), x1 = bf16_hi(vv[j]);
          const double d0 = x0, d1 = x1;
          ss = fma(d0, d0, ss);
          ss = fma(d1, d1, ss);
          y[i][2 * j] = x0 * bf16_lo(ww[j]);      // exact in fp32
          y[i][2 * j + 1] = x1 * bf16_hi(ww[j]);
        }
      } else {  // kSilu
        uint4 u = make_uint4(0, 0, 0, 0);
        if (valid[i]) u = *reinterpret_cast<const uint4*>(xr + K + c * kChunk);
        const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          y[i][2 * j] = silu_bf16(vv[j] & 0xFFFFu, silu_tab) * bf16_lo(uu[j]);
          y[i][2 * j + 1] = silu_bf16(vv[j] >> 16, silu_tab) * bf16_hi(uu[j]);
        }
      }
    }

    if constexpr (OP == kRms) {
      const double tot = block_sum(ss, red64);
      const double t = tot / static_cast<double>(K) + static_cast<double>(eps);
      const float inv = static_cast<float>(1.0 / sqrt(t));
#pragma unroll
      for (int i = 0; i < CH; ++i)
#pragma unroll
        for (int j = 0; j < kChunk; ++j) y[i][j] = y[i][j] * inv;
    }

    // ---- amax per chunk, then per group (16 lanes) or per row (block)
    float cmax[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      float m = 0.0f;
#pragma unroll
      for (int j = 0; j < kChunk; ++j) m = fmaxf(m, fabsf(y[i][j]));
      cmax[i] = valid[i] ? m : 0.0f;
    }

    if constexpr (MODE == kPerToken) {
      float m = cmax[0];
#pragma unroll
      for (int i = 1; i < CH; ++i) m = fmaxf(m, cmax[i]);
      const float amax = block_max(m, red32);
      const GroupScale g = make_scale(amax);
      if (tid == 0) scale[row] = g.s;
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        if (!valid[i]) continue;
        const int c = c0 + tid + i * kThreads;
        uint2 out;
        out.x = pack4_e4m3(quotient(y[i][0], g), quotient(y[i][1], g), quotient(y[i][2], g),
                           quotient(y[i][3], g));
        out.y = pack4_e4m3(quotient(y[i][4], g), quotient(y[i][5], g), quotient(y[i][6], g),
                           quotient(y[i][7], g));
        *reinterpret_cast<uint2*>(q + static_cast<long>(row) * K + c * kChunk) = out;
      }
    } else {
      const int ngroups = K / kGroup;
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const float amax = max16(cmax[i]);  // all 16 lanes of a group agree
        if (!valid[i]) continue;
        const int c = c0 + tid + i * kThreads;
        const GroupScale g = make_scale(amax);
        if ((tid & 15) == 0) scale[static_cast<long>(row) * ngroups + c / 16] = g.s;
        uint2 out;
        out.x = pack4_e4m3(quotient(y[i][0], g), quotient(y[i][1], g), quotient(y[i][2], g),
                           quotient(y[i][3], g));
        out.y = pack4_e4m3(quotient(y[i][4], g), quotient(y[i][5], g), quotient(y[i][6], g),
                           quotient(y[i][7], g));
        *reinterpret_cast<uint2*>(q + static_cast<long>(row) * K + c * kChunk) = out;
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void cvt_e4m3_kernel(uint8_t* __restrict__ q,
                                                            const float* __restrict__ x,
                                                            long n) {
  const long n4 = n / 4;
  for (long i = blockIdx.x * static_cast<long>(kThreads) + threadIdx.x; i < n4;
       i += static_cast<long>(gridDim.x) * kThreads) {
    const float4 v = reinterpret_cast<const float4*>(x)[i];
    reinterpret_cast<uint32_t*>(q)[i] = pack4_e4m3(v.x, v.y, v.z, v.w);
  }
  // tail (n % 4 elements) by the first thread
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    for (long i = n4 * 4; i < n; ++i) q[i] = static_cast<uint8_t>(pack4_e4m3(x[i], 0.f, 0.f, 0.f));
  }
}

__global__ __launch_bounds__(kThreads) void silu_kernel(float* __restrict__ y,
                                                        const uint16_t* __restrict__ g,
                                                        long n) {
  extern __shared__ float silu_tab[];
  load_silu_table(silu_tab);
  for (long i = blockIdx.x * static_cast<long>(kThreads) + threadIdx.x; i < n;
       i += static_cast<long>(gridDim.x) * kThreads)
    y[i] = silu_bf16(g[i], silu_tab);
}

constexpr size_t kSiluLds = 8192 * sizeof(float);

template <int OP, int MODE, int CH>
hipError_t launch_quant_t(uint8_t* q, float* scale, const uint16_t* x, const uint16_t* w,
                          int M, int K, float eps, int grid, hipStream_t st) {
  const size_t lds = (OP == kSilu) ? kSiluLds : 0;
  hipLaunchKernelGGL((quant_kernel<OP, MODE, CH>), dim3(grid), dim3(kThreads), lds, st, q,
                     scale, x, w, M, K, eps);
  return hipGetLastError();
}

template <int OP, int MODE>
hipError_t launch_quant_ch(int ch, uint8_t* q, float* scale, const uint16_t* x,
                           const uint16_t* w, int M, int K, float eps, int grid,
                           hipStream_t st) {
  switch (ch) {
    case 1: return launch_quant_t<OP, MODE, 1>(q, scale, x, w, M, K, eps, grid, st);
    case 2: return launch_quant_t<OP, MODE, 2>(q, scale, x, w, M, K, eps, grid, st);
    case 3: return launch_quant_t<OP, MODE, 3>(q, scale, x, w, M, K, eps, grid, st);
    case 4: return launch_quant_t<OP, MODE, 4>(q, scale, x, w, M, K, eps, grid, st);
    case 6: return launch_quant_t<OP, MODE, 6>(q, scale, x, w, M, K, eps, grid, st);
    case 8: return launch_quant_t<OP, MODE, 8>(q, scale, x, w, M, K, eps, grid, st);
    case 12: return launch_quant_t<OP, MODE, 12>(q, scale, x, w, M, K, eps, grid, st);
    case 16: return launch_quant_t<OP, MODE, 16>(q, scale, x, w, M, K, eps, grid, st);
    default: return hipErrorInvalidValue;
  }
}

int pick_ch(int chunks_per_thread) {
  static const int kAllowed[] = {1, 2, 3, 4, 6, 8, 12, 16};
  for (int c : kAllowed)
    if (c >= chunks_per_thread) return c;
  return -1;
}

}  // namespace

int quant_max_k() { return kSeg * 16; }

hipError_t launch_quant(int op, int mode, uint8_t* q, float* scale, const uint16_t* x,
                        const uint16_t* w, int M, int K, float eps, int num_cus,
                        hipStream_t st) {
  // A row (or segment) is spread over 256 threads, CH 16-byte chunks each.
  const bool whole_row = (mode == kPerToken) || (op == kRms);
  const int chunks = (K / kChunk + kThreads - 1) / kThreads;
  const int ch = whole_row ? pick_ch(chunks) : 1;
  if (ch < 0) return hipErrorInvalidValue;
  const int seg_cols = whole_row ? K : kSeg * ch;
  const long units = static_cast<long>(M) * ((K + seg_cols - 1) / seg_cols);
  const long cap = static_cast<long>(num_cus) * 8;
  const int grid = static_cast<int>(units < cap ? units : cap);
  if (op == kIdent) {
    return mode == kPerToken
               ? launch_quant_ch<kIdent, kPerToken>(ch, q, scale, x, w, M, K, eps, grid, st)
               : launch_quant_ch<kIdent, kGroup128>(ch, q, scale, x, w, M, K, eps, grid, st);
  }
  if (op == kRms) {
    return mode == kPerToken
               ? launch_quant_ch<kRms, kPerToken>(ch, q, scale, x, w, M, K, eps, grid, st)
               : launch_quant_ch<kRms, kGroup128>(ch, q, scale, x, w, M, K, eps, grid, st);
  }
  return mode == kPerToken
             ? launch_quant_ch<kSilu, kPerToken>(ch, q, scale, x, w, M, K, eps, grid, st)
             : launch_quant_ch<kSilu, kGroup128>(ch, q, scale, x, w, M, K, eps, grid, st);
}

hipError_t launch_cvt_e4m3(uint8_t* q, const float* x, long n, int num_cus, hipStream_t st) {
  const long blocks = (n / 4 + kThreads - 1) / kThreads;
  const long cap = static_cast<long>(num_cus) * 8;
  const int grid = static_cast<int>(blocks < 1 ? 1 : (blocks < cap ? blocks : cap));
  hipLaunchKernelGGL(cvt_e4m3_kernel, dim3(grid), dim3(kThreads), 0, st, q, x, n);
  return hipGetLastError();
}

hipError_t launch_silu(float* y, const uint16_t* g, long n, int num_cus, hipStream_t st) {
  const long blocks = (n + kThreads - 1) / kThreads;
  const long cap = static_cast<long>(num_cus) * 4;
  const int grid = static_cast<int>(blocks < 1 ? 1 : (blocks < cap ? blocks : cap));
  hipLaunchKernelGGL(silu_kernel, dim3(grid), dim3(kThreads), kSiluLds, st, y, g, n);
  return hipGetLastError();
}

}  // namespace fp8q
