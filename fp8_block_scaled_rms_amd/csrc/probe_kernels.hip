// Ceiling probes for the measurement: what this GPU reaches on plain
// matrix-core and memory-streaming loops, and its shader clock meanwhile.
// They compute nothing of the FP8 path; the benchmark reports the path's
// kernels against these measured ceilings beside the published peaks.
//
//  * mfma: every wave issues a long run of independent matrix instructions
//    (8 accumulators, so no instruction waits for the previous one), either
//    v_mfma_f32_16x16x32_f16 (the exact engine's instruction) or
//    v_mfma_scale_f32_16x16x128_f8f6f4 on e4m3 operands (the FP8 rate).
//    Thread 0 of each workgroup stamps s_memtime (shader clock cycles) and
//    s_memrealtime (a constant 100 MHz counter) before and after its loop.
//  * read: each workgroup streams a contiguous slice of a buffer with 16-byte
//    loads, 8 in flight per thread, folded into one word per thread that it
//    stores (so the loads cannot be dropped).
//  * copy: the same slices, loaded and stored.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8q_probe.h"

namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kProbeThreads = 256;

__device__ __forceinline__ uint64_t memtime() {
  uint64_t t;
  asm volatile("s_memtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t) :: "memory");
  return t;
}
__device__ __forceinline__ uint64_t memrealtime() {
  uint64_t t;
  asm volatile("s_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t) :: "memory");
  return t;
}

template <int KIND>
__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(long iters,
                                                                   uint64_t* __restrict__ stamps,
                                                                   float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  uint64_t t0 = 0, r0 = 0;
  if (threadIdx.x == 0) {
    t0 = memtime();
    r0 = memrealtime();
  }
  v4f acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = v4f{0, 0, 0, 0};
  if constexpr (KIND == FP8Q_PROBE_MFMA_F16) {
    v8h a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = static_cast<_Float16>((lane + i) & 7);
      b[i] = static_cast<_Float16>((lane * 3 + i) & 7);
    }
    for (long it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[i], 0, 0, 0);
    }
  } else {
    v8i a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = 0x38383838 + ((lane + i) & 3);  // e4m3 values near 1
      b[i] = 0x30303030 + ((lane * 5 + i) & 3);
    }
    for (long it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[i], 0, 0, 0, 127, 0,
                                                                  127);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  if (s == -1.0f) sink[blockIdx.x] = s;  // never true: keeps the loop
  if (threadIdx.x == 0) {
    const uint64_t t1 = memtime(), r1 = memrealtime();
    stamps[4 * blockIdx.x + 0] = t0;
    stamps[4 * blockIdx.x + 1] = t1;
    stamps[4 * blockIdx.x + 2] = r0;
    stamps[4 * blockIdx.x + 3] = r1;
  }
}

// Each workgroup streams one contiguous slice, 8 loads per thread in
// flight (128 bytes per thread per iteration).
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint4* __restrict__ src,
                                                                   long n16,
                                                                   uint32_t* __restrict__ out) {
  uint32_t acc = 0;
  const long per = (n16 + gridDim.x - 1) / gridDim.x;
  const long lo = blockIdx.x * per;
  const long hi = (lo + per < n16) ? lo + per : n16;
  long i = lo + threadIdx.x;
  for (; i + (kUnroll - 1) * kProbeThreads < hi; i += kUnroll * kProbeThreads) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * kProbeThreads];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < hi; i += kProbeThreads) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[blockIdx.x * static_cast<long>(kProbeThreads) + threadIdx.x] = acc;
}

__global__ __launch_bounds__(kProbeThreads) void copy_probe_kernel(const uint4* __restrict__ src,
                                                                   uint4* __restrict__ dst,
                                                                   long n16) {
  const long per = (n16 + gridDim.x - 1) / gridDim.x;
  const long lo = blockIdx.x * per;
  const long hi = (lo + per < n16) ? lo + per : n16;
  long i = lo + threadIdx.x;
  for (; i + (kUnroll - 1) * kProbeThreads < hi; i += kUnroll * kProbeThreads) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * kProbeThreads];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) dst[i + u * kProbeThreads] = v[u];
  }
  for (; i < hi; i += kProbeThreads) dst[i] = src[i];
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

int fp8q_probe_mfma(int kind, int64_t iters, int workgroups, uint64_t* stamps, float* sink,
                    void* stream) {
  if (iters <= 0 || workgroups <= 0 || !stamps || !sink) return 1;
  if (kind != FP8Q_PROBE_MFMA_F16 && kind != FP8Q_PROBE_MFMA_FP8) return 1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (kind == FP8Q_PROBE_MFMA_F16)
    hipLaunchKernelGGL(mfma_probe_kernel<FP8Q_PROBE_MFMA_F16>, dim3(workgroups),
                       dim3(kProbeThreads), 0, st, static_cast<long>(iters), stamps, sink);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<FP8Q_PROBE_MFMA_FP8>, dim3(workgroups),
                       dim3(kProbeThreads), 0, st, static_cast<long>(iters), stamps, sink);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

int64_t fp8q_probe_mfma_flops_per_iter(int kind) {
  // 8 instructions per loop iteration and wave
  if (kind == FP8Q_PROBE_MFMA_F16) return 8LL * 2 * 16 * 16 * 32;
  if (kind == FP8Q_PROBE_MFMA_FP8) return 8LL * 2 * 16 * 16 * 128;
  return 0;
}

int fp8q_probe_stream(int kind, const void* src, void* dst, int64_t bytes, int workgroups,
                      void* stream) {
  if (!src || !dst || bytes <= 0 || bytes % 16 || workgroups <= 0) return 1;
  if (!aligned16(src) || !aligned16(dst)) return 3;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const long n16 = static_cast<long>(bytes / 16);
  if (kind == FP8Q_PROBE_READ)
    hipLaunchKernelGGL(read_probe_kernel, dim3(workgroups), dim3(kProbeThreads), 0, st,
                       static_cast<const uint4*>(src), n16, static_cast<uint32_t*>(dst));
  else if (kind == FP8Q_PROBE_COPY)
    hipLaunchKernelGGL(copy_probe_kernel, dim3(workgroups), dim3(kProbeThreads), 0, st,
                       static_cast<const uint4*>(src), static_cast<uint4*>(dst), n16);
  else
    return 1;
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

}  // extern "C"
