// Fused front end + dynamic FP8 (OCP e4m3) or INT8 quantization kernels for
// gfx950.
//
// One kernel template covers the quantizers named on the page "Helion in
// vLLM: FP8 inference of Qwen3" (24-ai.news), section "Kernels integrated
// into vLLM":
//   kIdent  dynamic_per_token_scaled_fp8_quant / per_token_group_fp8_quant
//   kRms    rms_norm_dynamic_per_token_quant   / rms_norm_per_block_quant
//   kSilu   silu_and_mul_dynamic_per_token_quant / silu_and_mul_per_block_quant
// each with a per-token (one scale per row) or per-1x128-group scale, the
// scale being amax/448 or the power of two UE8M0 needs (page above, section
// "Practical limits"), or with one caller-given static scale per tensor.
//
// The work is HBM-bound (3 B per element for RMSNorm, 5 B per output element
// for SiLU-and-mul), so the design is about streaming.  A work unit is a whole
// row (per-token mode, and RMSNorm, whose inverse RMS spans the row) or a
// 512*CH-column segment of a row (group and static modes).  A unit belongs to one 64-lane
// wave -- rows up to 8192 columns and every group-mode segment -- so its
// reductions are DPP/shuffle moves inside the wave with no barrier; longer
// rows take the whole 256-thread workgroup and reduce across its waves in LDS.
// Lane t of a unit owns the 8-element (16-byte) chunks t, t+TPR, ... and
// issues all of their loads before any arithmetic, so every access is a
// coalesced 128-bit one and each lane keeps up to 16 (x2 for the weight or
// the up half) loads in flight.  The 16 consecutive lanes that hold one
// 128-element group reduce its amax with four DPP moves.  Workgroups loop
// over units (grid-stride) so per-workgroup set-up (the SiLU table in LDS) is
// amortised.
#include "fp8q_common.hpp"
#include "silu_table.hpp"
#include "quant_kernels.h"

namespace fp8q {

namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 8;  // bf16 elements per 16-byte chunk

__device__ __forceinline__ void load_silu_table(float* lds) {
  const uint4* src = reinterpret_cast<const uint4*>(kSiluTable);
  uint4* dst = reinterpret_cast<uint4*>(lds);
  for (int i = threadIdx.x; i < 8192 / 4; i += kThreads) dst[i] = src[i];
  __syncthreads();
}

// Reductions over the TPR threads of a unit: inside the wave first, then for
// TPR = 128 / 256 across its 2 / 4 waves through LDS, in a fixed order.
// Every wave of the workgroup must call these (they hold barriers when
// TPR > 64).
template <int TPR>
__device__ __forceinline__ double unit_sum(double v, double* red) {
  v = sum64(v);
  if constexpr (TPR == 64) return v;
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  double t;
  if constexpr (TPR == 128)
    t = red[wave & ~1] + red[wave | 1];
  else
    t = ((red[0] + red[1]) + red[2]) + red[3];
  __syncthreads();
  return t;
}
template <int TPR>
__device__ __forceinline__ float unit_max(float v, float* red) {
  v = max64(v);
  if constexpr (TPR == 64) return v;
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float t;
  if constexpr (TPR == 128)
    t = fmaxf(red[wave & ~1], red[wave | 1]);
  else
    t = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return t;
}

// A work unit is processed by TPR threads: one wave (TPR = 64; reductions
// stay inside the wave, no barrier), two waves or the whole 256-thread
// workgroup (TPR = 128 / 256: long rows, or few rows; cross-wave reductions
// go through LDS).  Thread t of a unit owns the 8-element chunks t, t + TPR,
// ..., CH of them.
template <int FMT>
__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d) {
  if constexpr (FMT == kFmtI8) return pack4_i8(a, b, c, d);
  return pack4_e4m3(a, b, c, d);
}

template <int OP, int MODE, int TPR, int CH, int FMT>
__global__ __launch_bounds__(kThreads) void quant_kernel(uint8_t* __restrict__ q,
                                                         float* __restrict__ scale,
                                                         const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ w, int M,
                                                         int K, float eps) {
  static_assert(TPR == 64 || TPR == 128 || TPR == kThreads, "unit = 1, 2 or 4 waves");
  constexpr int kUnitsPerBlock = kThreads / TPR;
  __shared__ double red64[4];
  __shared__ float red32[4];
  extern __shared__ float silu_tab[];
  if constexpr (OP == kSilu) load_silu_table(silu_tab);

  const int sub = static_cast<int>(threadIdx.x) / TPR;
  const int tid = static_cast<int>(threadIdx.x) % TPR;
  const int nchunk = K / kChunk;  // chunks per row
  constexpr bool kWholeRow = mode_is_row(MODE) || (OP == kRms);
  const int unit_chunks = kWholeRow ? nchunk : TPR * CH;
  const int nseg = (nchunk + unit_chunks - 1) / unit_chunks;
  const long units = static_cast<long>(M) * nseg;
  const long in_stride = (OP == kSilu) ? 2L * K : K;  // elements per input row

  for (long ub = blockIdx.x; ub * kUnitsPerBlock < units; ub += gridDim.x) {
    // a unit past the end still takes part in the barriers, with no loads or
    // stores
    const long unit_raw = ub * kUnitsPerBlock + sub;
    const bool active = unit_raw < units;
    const long unit = active ? unit_raw : 0;
    const int row = static_cast<int>(unit / nseg);
    const int seg = static_cast<int>(unit % nseg);
    const int c0 = seg * unit_chunks;  // first chunk of this unit
    const int c_end = (c0 + unit_chunks < nchunk) ? c0 + unit_chunks : nchunk;
    const uint16_t* xr = x + row * in_stride;

    // ---- load (all chunks first) and front end: y (fp32) per element
    uint4 xv[CH], wv[CH];
    bool valid[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = c0 + tid + i * TPR;
      valid[i] = active && c < c_end;
      xv[i] = valid[i] ? *reinterpret_cast<const uint4*>(xr + c * kChunk) : make_uint4(0, 0, 0, 0);
      if constexpr (OP == kRms)
        wv[i] = valid[i] ? *reinterpret_cast<const uint4*>(w + c * kChunk) : make_uint4(0, 0, 0, 0);
      if constexpr (OP == kSilu)
        wv[i] = valid[i] ? *reinterpret_cast<const uint4*>(xr + K + c * kChunk)
                         : make_uint4(0, 0, 0, 0);  // up
    }
    float y[CH][kChunk];
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const uint32_t vv[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
      const uint32_t ww[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (OP == kIdent) {
          y[i][2 * j] = bf16_lo(vv[j]);
          y[i][2 * j + 1] = bf16_hi(vv[j]);
        } else if constexpr (OP == kRms) {
          const float x0 = bf16_lo(vv[j]), x1 = bf16_hi(vv[j]);
          const double d0 = x0, d1 = x1;
          ss = fma(d0, d0, ss);
          ss = fma(d1, d1, ss);
          y[i][2 * j] = x0 * bf16_lo(ww[j]);  // exact in fp32
          y[i][2 * j + 1] = x1 * bf16_hi(ww[j]);
        } else {  // kSilu: gate in xv, up in wv
          y[i][2 * j] = silu_bf16(vv[j] & 0xFFFFu, silu_tab) * bf16_lo(ww[j]);
          y[i][2 * j + 1] = silu_bf16(vv[j] >> 16, silu_tab) * bf16_hi(ww[j]);
        }
      }
    }

    if constexpr (OP == kRms) {
      const double tot = unit_sum<TPR>(ss, red64);
      const double t = tot / static_cast<double>(K) + static_cast<double>(eps);
      const float inv = static_cast<float>(1.0 / sqrt(t));
#pragma unroll
      for (int i = 0; i < CH; ++i)
#pragma unroll
        for (int j = 0; j < kChunk; ++j) y[i][j] = y[i][j] * inv;
    }

    // ---- amax per chunk, then per group (16 lanes) or per row
    float cmax[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      float m = 0.0f;
#pragma unroll
      for (int j = 0; j < kChunk; ++j) m = fmaxf(m, fabsf(y[i][j]));
      cmax[i] = valid[i] ? m : 0.0f;
    }

    if constexpr (mode_is_row(MODE)) {
      float m = cmax[0];
#pragma unroll
      for (int i = 1; i < CH; ++i) m = fmaxf(m, cmax[i]);
      const float amax = unit_max<TPR>(m, red32);
      const GroupScale g = FMT == kFmtI8      ? make_scale_i8(amax)
                           : mode_is_ue8(MODE) ? make_scale_ue8m0(amax)
                                               : make_scale(amax);
      if (active && tid == 0) scale[row] = g.s;
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        if (!valid[i]) continue;
        const int c = c0 + tid + i * TPR;
        uint2 out;
        out.x = pack4<FMT>(quotient(y[i][0], g), quotient(y[i][1], g), quotient(y[i][2], g),
                           quotient(y[i][3], g));
        out.y = pack4<FMT>(quotient(y[i][4], g), quotient(y[i][5], g), quotient(y[i][6], g),
                           quotient(y[i][7], g));
        *reinterpret_cast<uint2*>(q + static_cast<long>(row) * K + c * kChunk) = out;
      }
    } else if constexpr (mode_is_group(MODE)) {
      const int ngroups = K / kGroup;
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const float amax = max16(cmax[i]);  // all 16 lanes of a group agree
        if (!valid[i]) continue;
        const int c = c0 + tid + i * TPR;
        const GroupScale g = mode_is_ue8(MODE) ? make_scale_ue8m0(amax) : make_scale(amax);
        if ((tid & 15) == 0) scale[static_cast<long>(row) * ngroups + c / 16] = g.s;
        uint2 out;
        out.x = pack4<FMT>(quotient(y[i][0], g), quotient(y[i][1], g), quotient(y[i][2], g),
                           quotient(y[i][3], g));
        out.y = pack4<FMT>(quotient(y[i][4], g), quotient(y[i][5], g), quotient(y[i][6], g),
                           quotient(y[i][7], g));
        *reinterpret_cast<uint2*>(q + static_cast<long>(row) * K + c * kChunk) = out;
      }
    } else {  // kStaticTensor: the caller's scale, read once per unit
      const GroupScale g = static_scale(scale[0]);
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        if (!valid[i]) continue;
        const int c = c0 + tid + i * TPR;
        uint2 out;
        out.x = pack4<FMT>(quotient_static(y[i][0], g), quotient_static(y[i][1], g),
                           quotient_static(y[i][2], g), quotient_static(y[i][3], g));
        out.y = pack4<FMT>(quotient_static(y[i][4], g), quotient_static(y[i][5], g),
                           quotient_static(y[i][6], g), quotient_static(y[i][7], g));
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

template <int OP, int MODE, int TPR, int CH, int FMT>
hipError_t launch_quant_t(uint8_t* q, float* scale, const uint16_t* x, const uint16_t* w,
                          int M, int K, float eps, int grid, hipStream_t st) {
  const size_t lds = (OP == kSilu) ? kSiluLds : 0;
  hipLaunchKernelGGL((quant_kernel<OP, MODE, TPR, CH, FMT>), dim3(grid), dim3(kThreads), lds, st, q,
                     scale, x, w, M, K, eps);
  return hipGetLastError();
}

template <int OP, int MODE, int TPR, int FMT>
hipError_t launch_quant_ch(int ch, uint8_t* q, float* scale, const uint16_t* x,
                           const uint16_t* w, int M, int K, float eps, int grid,
                           hipStream_t st) {
  switch (ch) {
    case 1: return launch_quant_t<OP, MODE, TPR, 1, FMT>(q, scale, x, w, M, K, eps, grid, st);
    case 2: return launch_quant_t<OP, MODE, TPR, 2, FMT>(q, scale, x, w, M, K, eps, grid, st);
    case 4: return launch_quant_t<OP, MODE, TPR, 4, FMT>(q, scale, x, w, M, K, eps, grid, st);
    case 6: return launch_quant_t<OP, MODE, TPR, 6, FMT>(q, scale, x, w, M, K, eps, grid, st);
    case 8: return launch_quant_t<OP, MODE, TPR, 8, FMT>(q, scale, x, w, M, K, eps, grid, st);
    case 10: return launch_quant_t<OP, MODE, TPR, 10, FMT>(q, scale, x, w, M, K, eps, grid, st);
    case 12: return launch_quant_t<OP, MODE, TPR, 12, FMT>(q, scale, x, w, M, K, eps, grid, st);
    case 16: return launch_quant_t<OP, MODE, TPR, 16, FMT>(q, scale, x, w, M, K, eps, grid, st);
    default: return hipErrorInvalidValue;
  }
}

// Units of more than one wave only exist for whole-row units (per-token
// modes and RMSNorm); other combinations instantiate the one-wave kernel only.
template <int OP, int MODE, int FMT>
hipError_t launch_quant_tpr(int tpr, int ch, uint8_t* q, float* scale, const uint16_t* x,
                            const uint16_t* w, int M, int K, float eps, int grid,
                            hipStream_t st) {
  if (tpr == 64)
    return launch_quant_ch<OP, MODE, 64, FMT>(ch, q, scale, x, w, M, K, eps, grid, st);
  if constexpr (mode_is_row(MODE) || OP == kRms) {
    if (tpr == 128)
      return launch_quant_ch<OP, MODE, 128, FMT>(ch, q, scale, x, w, M, K, eps, grid, st);
    return launch_quant_ch<OP, MODE, kThreads, FMT>(ch, q, scale, x, w, M, K, eps, grid, st);
  }
  return hipErrorInvalidValue;
}

template <int OP, int FMT>
hipError_t launch_quant_mode(int mode, int tpr, int ch, uint8_t* q, float* scale,
                             const uint16_t* x, const uint16_t* w, int M, int K, float eps,
                             int grid, hipStream_t st) {
  if constexpr (FMT == kFmtI8) {
    if (mode == kPerToken)
      return launch_quant_tpr<OP, kPerToken, FMT>(tpr, ch, q, scale, x, w, M, K, eps, grid, st);
    if (mode == kStaticTensor)
      return launch_quant_tpr<OP, kStaticTensor, FMT>(tpr, ch, q, scale, x, w, M, K, eps, grid,
                                                      st);
    return hipErrorInvalidValue;
  }
  switch (mode) {
    case kPerToken:
      return launch_quant_tpr<OP, kPerToken, FMT>(tpr, ch, q, scale, x, w, M, K, eps, grid, st);
    case kGroup128:
      return launch_quant_tpr<OP, kGroup128, FMT>(tpr, ch, q, scale, x, w, M, K, eps, grid, st);
    case kStaticTensor:
      return launch_quant_tpr<OP, kStaticTensor, FMT>(tpr, ch, q, scale, x, w, M, K, eps, grid, st);
    case kPerTokenUe8:
      return launch_quant_tpr<OP, kPerTokenUe8, FMT>(tpr, ch, q, scale, x, w, M, K, eps, grid, st);
    case kGroup128Ue8:
      return launch_quant_tpr<OP, kGroup128Ue8, FMT>(tpr, ch, q, scale, x, w, M, K, eps, grid, st);
    default:
      return hipErrorInvalidValue;
  }
}

int pick_ch(int chunks_per_thread) {
  static const int kAllowed[] = {1, 2, 4, 6, 8, 10, 12, 16};
  for (int c : kAllowed)
    if (c >= chunks_per_thread) return c;
  return -1;
}

}  // namespace

int quant_max_k() { return kThreads * kChunk * 16; }

hipError_t launch_quant(int op, int mode, int fmt, uint8_t* q, float* scale,
                        const uint16_t* x, const uint16_t* w, int M, int K, float eps,
                        int num_cus, hipStream_t st) {
  const bool whole_row = mode_is_row(mode) || (op == kRms);
  const int nchunk = K / kChunk;
  // Chunks a lane may hold before its registers cut occupancy too far (the
  // SiLU front end keeps gate, up and the product live at once); measured
  // per front end at the workload shapes.
  const int ch_max = (op == kRms) ? 8 : (op == kSilu) ? 6 : 4;
  // Waves wanted in flight before a unit is made smaller for parallelism.
  const long want_waves = 16L * num_cus;
  int tpr, ch, unit_chunks;
  if (whole_row) {
    // one wave per row while a lane holds at most ch_max chunks (and there
    // are enough rows to fill the chip), else 2 or 4 waves per row
    tpr = 64;
    while (tpr < kThreads && ((nchunk + tpr - 1) / tpr > ch_max ||
                              static_cast<long>(M) * (tpr / 64) < want_waves))
      tpr *= 2;
    ch = pick_ch((nchunk + tpr - 1) / tpr);
    unit_chunks = nchunk;
  } else {
    // row segments of whole 128-column groups, one wave each: as few
    // segments per row as ch_max allows, more when rows are few
    tpr = 64;
    int nseg = (nchunk + 64 * ch_max - 1) / (64 * ch_max);
    while (static_cast<long>(M) * nseg < want_waves && nseg * 16 < nchunk) nseg *= 2;
    ch = pick_ch((nchunk + nseg * 64 - 1) / (nseg * 64));
    unit_chunks = 64 * ch;
  }
  if (ch < 0) return hipErrorInvalidValue;
  const long units = static_cast<long>(M) * ((nchunk + unit_chunks - 1) / unit_chunks);
  const long blocks = (units + (kThreads / tpr) - 1) / (kThreads / tpr);
  // the SiLU table costs 32 KiB of LDS fill per workgroup: fewer, looping ones
  const long cap = static_cast<long>(num_cus) * (op == kSilu ? 4 : 16);
  const int grid = static_cast<int>(blocks < cap ? blocks : cap);
  if (fmt == kFmtI8) {
    if (op == kIdent)
      return launch_quant_mode<kIdent, kFmtI8>(mode, tpr, ch, q, scale, x, w, M, K, eps, grid,
                                               st);
    if (op == kRms)
      return launch_quant_mode<kRms, kFmtI8>(mode, tpr, ch, q, scale, x, w, M, K, eps, grid, st);
    return launch_quant_mode<kSilu, kFmtI8>(mode, tpr, ch, q, scale, x, w, M, K, eps, grid, st);
  }
  if (op == kIdent)
    return launch_quant_mode<kIdent, kFmtE4m3>(mode, tpr, ch, q, scale, x, w, M, K, eps, grid,
                                               st);
  if (op == kRms)
    return launch_quant_mode<kRms, kFmtE4m3>(mode, tpr, ch, q, scale, x, w, M, K, eps, grid, st);
  return launch_quant_mode<kSilu, kFmtE4m3>(mode, tpr, ch, q, scale, x, w, M, K, eps, grid, st);
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
