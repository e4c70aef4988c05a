// C ABI of the fp8q library: argument checks on the host (before any HIP
// call), device check (gfx950 only), dispatch, launch.  Nothing here
// allocates device memory or synchronizes.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "dispatch.h"
#include "fp8q.h"
#include "gemm_kernels.h"
#include "quant_kernels.h"

namespace {

thread_local int g_last_hip = 0;

constexpr int kMaxDevices = 64;
// largest GEMM K: 256 rows of K bytes stay below 2^32
constexpr int64_t kMaxGemmK = int64_t{1} << 22;
// per device: 0 unknown, 1 gfx950, 2 other arch; CU count
std::atomic<int> g_dev_state[kMaxDevices];
std::atomic<int> g_dev_cus[kMaxDevices];

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks the current device; returns FP8Q_OK and its CU count.
int device_check(int* num_cus) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    (void)hipGetLastError();  // clear the sticky error of the failed query
    return FP8Q_ERR_NO_DEVICE;
  }
  if (dev >= kMaxDevices) return FP8Q_ERR_NO_DEVICE;
  int st = g_dev_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return FP8Q_ERR_NO_DEVICE;
    }
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    g_dev_state[dev].store(st, std::memory_order_release);
  }
  if (st != 1) return FP8Q_ERR_ARCH;
  *num_cus = g_dev_cus[dev].load(std::memory_order_relaxed);
  return FP8Q_OK;
}

int launched(hipError_t e) {
  if (e == hipSuccess) return FP8Q_OK;
  g_last_hip = static_cast<int>(e);
  return FP8Q_ERR_HIP;
}

int check_quant_args(const void* q, const float* scale, const void* x, int64_t M, int64_t K,
                     int mode, int fmt) {
  if (M < 0 || K <= 0) return FP8Q_ERR_INVALID_ARG;
  if (mode < FP8Q_PER_TOKEN || mode > FP8Q_GROUP128_UE8M0) return FP8Q_ERR_BAD_MODE;
  if (fmt == fp8q::kFmtI8 && mode != FP8Q_PER_TOKEN && mode != FP8Q_PER_TENSOR_STATIC)
    return FP8Q_ERR_BAD_MODE;
  if (M == 0) return FP8Q_OK;
  if (!q || !scale || !x) return FP8Q_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(scale) || !aligned16(x)) return FP8Q_ERR_ALIGNMENT;
  const bool group = mode == FP8Q_GROUP128 || mode == FP8Q_GROUP128_UE8M0;
  if (K % (group ? 128 : 8) != 0) return FP8Q_ERR_UNSUPPORTED_SHAPE;
  if (K > fp8q::quant_max_k()) return FP8Q_ERR_UNSUPPORTED_SHAPE;
  if (M > INT_MAX || M * K > (int64_t)1 << 40) return FP8Q_ERR_UNSUPPORTED_SHAPE;
  return FP8Q_OK;
}

int run_quant(int op, int fmt, void* q, float* scale, const void* x, const void* w, int64_t M,
              int64_t K, float eps, int mode, void* stream) {
  int num_cus = 0;
  int rc = device_check(&num_cus);
  if (rc != FP8Q_OK) return rc;
  return launched(fp8q::launch_quant(op, mode, fmt, static_cast<uint8_t*>(q), scale,
                                     static_cast<const uint16_t*>(x),
                                     static_cast<const uint16_t*>(w), static_cast<int>(M),
                                     static_cast<int>(K), eps, num_cus,
                                     static_cast<hipStream_t>(stream)));
}

int check_gemm_args(int op, const void* y, const void* a, const void* b, const float* sa,
                    const float* sb, int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N <= 0 || K <= 0) return FP8Q_ERR_INVALID_ARG;
  if (M == 0) return FP8Q_OK;
  if (!y || !a || !b || !sa || !sb) return FP8Q_ERR_INVALID_ARG;
  if (!aligned16(y) || !aligned16(a) || !aligned16(b) || !aligned16(sa) || !aligned16(sb))
    return FP8Q_ERR_ALIGNMENT;
  if (K % 128 != 0 || N % 128 != 0) return FP8Q_ERR_UNSUPPORTED_SHAPE;
  if (M > INT_MAX || N > INT_MAX || K > INT_MAX) return FP8Q_ERR_UNSUPPORTED_SHAPE;
  // the tiled kernels address a tile's rows with 32-bit byte offsets
  if (K > kMaxGemmK) return FP8Q_ERR_UNSUPPORTED_SHAPE;
  // int32 sums of int8 products stay exact for K * 127^2 < 2^31
  if (op == FP8Q_OP_SCALED_MM_INT8 && K > 131072) return FP8Q_ERR_UNSUPPORTED_SHAPE;
  return FP8Q_OK;
}

int run_gemm(int op, void* y, const void* a, const float* sa, const void* b, const float* sb,
             int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes, int cfg,
             void* stream) {
  int rc = check_gemm_args(op, y, a, b, sa, sb, M, N, K);
  if (rc != FP8Q_OK || M == 0) return rc;
  if (cfg < 0) cfg = fp8q::dispatch_gemm(op, M, N, K);
  if (cfg < 0 || cfg >= fp8q::gemm_num_configs() || !fp8q::variant_serves(cfg, op) ||
      !fp8q::gemm_config_fits(cfg, M, N, K))
    return FP8Q_ERR_BAD_CONFIG;
  const size_t need = fp8q::gemm_workspace_bytes(cfg, M, N, K);
  if (need > 0) {
    if (!ws || ws_bytes < need) return FP8Q_ERR_WORKSPACE;
    if (!aligned16(ws)) return FP8Q_ERR_ALIGNMENT;
  }
  int num_cus = 0;
  rc = device_check(&num_cus);
  if (rc != FP8Q_OK) return rc;
  const int scales = op == FP8Q_OP_SCALED_MM_BLOCKWISE         ? fp8q::kScalesBlock
                     : op == FP8Q_OP_SCALED_MM_BLOCKWISE_UE8M0 ? fp8q::kScalesBlockPow2
                                                               : fp8q::kScalesPerToken;
  return launched(fp8q::launch_gemm(
      cfg, scales, static_cast<uint16_t*>(y),
      static_cast<const uint8_t*>(a), sa, static_cast<const uint8_t*>(b), sb,
      static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), ws,
      static_cast<hipStream_t>(stream)));
}

int rmsnorm_quant_any(int fmt, void* q, float* scale, const void* x, const void* w, int64_t M,
                      int64_t K, float eps, int mode, void* stream) {
  int rc = check_quant_args(q, scale, x, M, K, mode, fmt);
  if (rc != FP8Q_OK || M == 0) return rc;
  if (!w) return FP8Q_ERR_INVALID_ARG;
  if (!aligned16(w)) return FP8Q_ERR_ALIGNMENT;
  if (!(eps > 0.0f) || !std::isfinite(eps)) return FP8Q_ERR_INVALID_ARG;
  return run_quant(fp8q::kRms, fmt, q, scale, x, w, M, K, eps, mode, stream);
}

}  // namespace

extern "C" {

int fp8q_rmsnorm_quant(void* q, float* scale, const void* x, const void* w, int64_t M,
                       int64_t K, float eps, int mode, void* stream) {
  return rmsnorm_quant_any(fp8q::kFmtE4m3, q, scale, x, w, M, K, eps, mode, stream);
}

int fp8q_silu_mul_quant(void* q, float* scale, const void* gate_up, int64_t M, int64_t D,
                        int mode, void* stream) {
  int rc = check_quant_args(q, scale, gate_up, M, D, mode, fp8q::kFmtE4m3);
  if (rc != FP8Q_OK || M == 0) return rc;
  return run_quant(fp8q::kSilu, fp8q::kFmtE4m3, q, scale, gate_up, nullptr, M, D, 0.0f, mode,
                   stream);
}

int fp8q_quant(void* q, float* scale, const void* x, int64_t M, int64_t K, int mode,
               void* stream) {
  int rc = check_quant_args(q, scale, x, M, K, mode, fp8q::kFmtE4m3);
  if (rc != FP8Q_OK || M == 0) return rc;
  return run_quant(fp8q::kIdent, fp8q::kFmtE4m3, q, scale, x, nullptr, M, K, 0.0f, mode,
                   stream);
}

int fp8q_rmsnorm_quant_int8(void* q, float* scale, const void* x, const void* w, int64_t M,
                            int64_t K, float eps, int mode, void* stream) {
  return rmsnorm_quant_any(fp8q::kFmtI8, q, scale, x, w, M, K, eps, mode, stream);
}

int fp8q_silu_mul_quant_int8(void* q, float* scale, const void* gate_up, int64_t M,
                             int64_t D, int mode, void* stream) {
  int rc = check_quant_args(q, scale, gate_up, M, D, mode, fp8q::kFmtI8);
  if (rc != FP8Q_OK || M == 0) return rc;
  return run_quant(fp8q::kSilu, fp8q::kFmtI8, q, scale, gate_up, nullptr, M, D, 0.0f, mode,
                   stream);
}

int fp8q_quant_int8(void* q, float* scale, const void* x, int64_t M, int64_t K, int mode,
                    void* stream) {
  int rc = check_quant_args(q, scale, x, M, K, mode, fp8q::kFmtI8);
  if (rc != FP8Q_OK || M == 0) return rc;
  return run_quant(fp8q::kIdent, fp8q::kFmtI8, q, scale, x, nullptr, M, K, 0.0f, mode,
                   stream);
}

int fp8q_scaled_mm_int8(void* y, const void* a, const void* b, const float* sa,
                        const float* sb, int64_t M, int64_t N, int64_t K, void* ws,
                        size_t ws_bytes, void* stream) {
  return run_gemm(FP8Q_OP_SCALED_MM_INT8, y, a, sa, b, sb, M, N, K, ws, ws_bytes, -1, stream);
}

int fp8q_scaled_mm_int8_cfg(void* y, const void* a, const void* b, const float* sa,
                            const float* sb, int64_t M, int64_t N, int64_t K, void* ws,
                            size_t ws_bytes, int cfg, void* stream) {
  return run_gemm(FP8Q_OP_SCALED_MM_INT8, y, a, sa, b, sb, M, N, K, ws, ws_bytes, cfg, stream);
}

int fp8q_scaled_mm(void* y, const void* a, const void* b, const float* sa, const float* sb,
                   int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes, void* stream) {
  return run_gemm(FP8Q_OP_SCALED_MM, y, a, sa, b, sb, M, N, K, ws, ws_bytes, -1, stream);
}

int fp8q_scaled_mm_blockwise(void* y, const void* a, const void* b, const float* sa,
                             const float* sb, int64_t M, int64_t N, int64_t K, void* ws,
                             size_t ws_bytes, void* stream) {
  return run_gemm(FP8Q_OP_SCALED_MM_BLOCKWISE, y, a, sa, b, sb, M, N, K, ws, ws_bytes, -1,
                  stream);
}

int fp8q_scaled_mm_blockwise_ue8m0(void* y, const void* a, const void* b, const float* sa,
                                   const float* sb, int64_t M, int64_t N, int64_t K, void* ws,
                                   size_t ws_bytes, void* stream) {
  return run_gemm(FP8Q_OP_SCALED_MM_BLOCKWISE_UE8M0, y, a, sa, b, sb, M, N, K, ws, ws_bytes,
                  -1, stream);
}

int fp8q_scaled_mm_blockwise_silu_quant(void* q, float* scale, const void* a, const void* b,
                                        const float* sa, const float* sb, int64_t M, int64_t N,
                                        int64_t K, void* stream) {
  int rc = check_gemm_args(FP8Q_OP_SCALED_MM_BLOCKWISE, q, a, b, sa, sb, M, N, K);
  if (rc != FP8Q_OK || M == 0) return rc;
  if (!scale) return FP8Q_ERR_INVALID_ARG;
  if (!aligned16(scale)) return FP8Q_ERR_ALIGNMENT;
  if (N % 256 != 0) return FP8Q_ERR_UNSUPPORTED_SHAPE;  // N/2 whole 128-column groups
  // a tile's weight rows span its gate rows to its up rows, N/2 rows apart,
  // addressed with 32-bit byte offsets
  if ((N / 2 + 128) * K >= (static_cast<int64_t>(1) << 32)) return FP8Q_ERR_UNSUPPORTED_SHAPE;
  int num_cus = 0;
  rc = device_check(&num_cus);
  if (rc != FP8Q_OK) return rc;
  return launched(fp8q::launch_gemm_silu_quant(
      static_cast<uint8_t*>(q), scale, static_cast<const uint8_t*>(a), sa,
      static_cast<const uint8_t*>(b), sb, static_cast<int>(M), static_cast<int>(N),
      static_cast<int>(K), static_cast<hipStream_t>(stream)));
}

int fp8q_scaled_mm_blockwise_ue8m0_cfg(void* y, const void* a, const void* b, const float* sa,
                                       const float* sb, int64_t M, int64_t N, int64_t K,
                                       void* ws, size_t ws_bytes, int cfg, void* stream) {
  return run_gemm(FP8Q_OP_SCALED_MM_BLOCKWISE_UE8M0, y, a, sa, b, sb, M, N, K, ws, ws_bytes,
                  cfg, stream);
}

int fp8q_scaled_mm_cfg(void* y, const void* a, const void* b, const float* sa,
                       const float* sb, int64_t M, int64_t N, int64_t K, void* ws,
                       size_t ws_bytes, int cfg, void* stream) {
  return run_gemm(FP8Q_OP_SCALED_MM, y, a, sa, b, sb, M, N, K, ws, ws_bytes, cfg, stream);
}

int fp8q_scaled_mm_blockwise_cfg(void* y, const void* a, const void* b, const float* sa,
                                 const float* sb, int64_t M, int64_t N, int64_t K, void* ws,
                                 size_t ws_bytes, int cfg, void* stream) {
  return run_gemm(FP8Q_OP_SCALED_MM_BLOCKWISE, y, a, sa, b, sb, M, N, K, ws, ws_bytes, cfg,
                  stream);
}

int fp8q_scaled_mm_blockwise_noalloc(void* y, const void* a, const void* b, const float* sa,
                                     const float* sb, int64_t M, int64_t N, int64_t K,
                                     void* stream) {
  int rc = check_gemm_args(FP8Q_OP_SCALED_MM_BLOCKWISE, y, a, b, sa, sb, M, N, K);
  if (rc != FP8Q_OK || M == 0) return rc;
  const int cfg = fp8q::dispatch_gemm(FP8Q_OP_SCALED_MM_BLOCKWISE, M, N, K);
  if (cfg < 0 || !fp8q::gemm_config_fits(cfg, M, N, K)) return FP8Q_ERR_BAD_CONFIG;
  const size_t need = fp8q::gemm_workspace_bytes(cfg, M, N, K);
  if (need > fp8q::kScratchBytes) return FP8Q_ERR_WORKSPACE;
  int num_cus = 0;
  rc = device_check(&num_cus);
  if (rc != FP8Q_OK) return rc;
  void* ws = nullptr;
  if (need > 0) {
    rc = launched(fp8q::scratch_workspace(&ws));
    if (rc != FP8Q_OK) return rc;
  }
  return launched(fp8q::launch_gemm(cfg, fp8q::kScalesBlock, static_cast<uint16_t*>(y),
                                    static_cast<const uint8_t*>(a), sa,
                                    static_cast<const uint8_t*>(b), sb, static_cast<int>(M),
                                    static_cast<int>(N), static_cast<int>(K), ws,
                                    static_cast<hipStream_t>(stream)));
}

size_t fp8q_workspace_size(int op, int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  if (op < FP8Q_OP_SCALED_MM || op > FP8Q_OP_SCALED_MM_BLOCKWISE_UE8M0) return 0;
  const int cfg = fp8q::dispatch_gemm(op, M, N, K);
  return cfg < 0 ? 0 : fp8q::gemm_workspace_bytes(cfg, M, N, K);
}

size_t fp8q_workspace_size_cfg(int cfg, int64_t M, int64_t N, int64_t K) {
  if (cfg < 0 || cfg >= fp8q::gemm_num_configs() || M <= 0 || N <= 0 || K <= 0) return 0;
  return fp8q::gemm_workspace_bytes(cfg, M, N, K);
}

int fp8q_gemm_num_configs(void) { return fp8q::gemm_num_configs(); }

const char* fp8q_gemm_config_name(int cfg) {
  if (cfg < 0 || cfg >= fp8q::gemm_num_configs()) return nullptr;
  return fp8q::gemm_config(cfg).name;
}

int fp8q_gemm_config_for(int op, int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return -1;
  return fp8q::dispatch_gemm(op, M, N, K);
}

int fp8q_cvt_e4m3(void* q, const float* x, int64_t n, void* stream) {
  if (n < 0) return FP8Q_ERR_INVALID_ARG;
  if (n == 0) return FP8Q_OK;
  if (!q || !x) return FP8Q_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(x)) return FP8Q_ERR_ALIGNMENT;
  int num_cus = 0;
  int rc = device_check(&num_cus);
  if (rc != FP8Q_OK) return rc;
  return launched(fp8q::launch_cvt_e4m3(static_cast<uint8_t*>(q), x, static_cast<long>(n),
                                        num_cus, static_cast<hipStream_t>(stream)));
}

int fp8q_silu(float* y, const void* g, int64_t n, void* stream) {
  if (n < 0) return FP8Q_ERR_INVALID_ARG;
  if (n == 0) return FP8Q_OK;
  if (!y || !g) return FP8Q_ERR_INVALID_ARG;
  if (!aligned16(y) || !aligned16(g)) return FP8Q_ERR_ALIGNMENT;
  int num_cus = 0;
  int rc = device_check(&num_cus);
  if (rc != FP8Q_OK) return rc;
  return launched(fp8q::launch_silu(y, static_cast<const uint16_t*>(g), static_cast<long>(n),
                                    num_cus, static_cast<hipStream_t>(stream)));
}

int fp8q_quant_launch_config(int front_end, int mode, int64_t M, int64_t K, int num_cus,
                             int* tpr, int* ch, int* grid) {
  if (front_end < fp8q::kIdent || front_end > fp8q::kSilu) return FP8Q_ERR_INVALID_ARG;
  if (M <= 0 || K <= 0 || num_cus <= 0 || !tpr || !ch || !grid) return FP8Q_ERR_INVALID_ARG;
  // the same shape checks as the calls (aligned fake pointers: only sizes matter)
  const int rc = check_quant_args(reinterpret_cast<void*>(16), reinterpret_cast<float*>(16),
                                  reinterpret_cast<void*>(16), M, K, mode, fp8q::kFmtE4m3);
  if (rc != FP8Q_OK) return rc;
  fp8q::QuantLaunch lc;
  if (!fp8q::quant_launch_config(front_end, mode, static_cast<long>(M), static_cast<int>(K),
                                 num_cus, &lc))
    return FP8Q_ERR_UNSUPPORTED_SHAPE;
  *tpr = lc.tpr;
  *ch = lc.ch;
  *grid = lc.grid;
  return FP8Q_OK;
}

const char* fp8q_status_string(int status) {
  switch (status) {
    case FP8Q_OK: return "ok";
    case FP8Q_ERR_INVALID_ARG: return "invalid argument";
    case FP8Q_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case FP8Q_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
    case FP8Q_ERR_WORKSPACE: return "workspace too small";
    case FP8Q_ERR_NO_DEVICE: return "no usable HIP device";
    case FP8Q_ERR_ARCH: return "device is not gfx950";
    case FP8Q_ERR_HIP: return "HIP launch error";
    case FP8Q_ERR_BAD_MODE: return "unknown quantization mode";
    case FP8Q_ERR_BAD_CONFIG: return "unknown or inapplicable GEMM config";
    default: return "unknown status";
  }
}

int fp8q_last_hip_error(void) { return g_last_hip; }

int fp8q_version(void) { return FP8Q_VERSION; }

}  // extern "C"
