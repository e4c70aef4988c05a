// Internal launch interface of the quantization kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

enum QuantOp { kIdent = 0, kRms = 1, kSilu = 2 };
// Values equal the fp8q_quant_mode values of the C ABI.
enum QuantMode {
  kPerToken = 0,      // dynamic, one scale per row, scale = amax / 448
  kGroup128 = 1,      // dynamic, one scale per 1x128 group
  kStaticTensor = 2,  // caller-given scale[0] for the whole tensor (input)
  kPerTokenUe8 = 3,   // per row, power-of-two scale
  kGroup128Ue8 = 4    // per 1x128 group, power-of-two scale
};
// Output format: OCP e4m3 codes, or symmetric int8 (W8A8; modes kPerToken
// and kStaticTensor only).
enum QuantFormat { kFmtE4m3 = 0, kFmtI8 = 1 };
constexpr bool mode_is_row(int m) { return m == kPerToken || m == kPerTokenUe8; }
constexpr bool mode_is_group(int m) { return m == kGroup128 || m == kGroup128Ue8; }
constexpr bool mode_is_ue8(int m) { return m == kPerTokenUe8 || m == kGroup128Ue8; }

// Largest K (columns of the quantized output) a launch supports.
int quant_max_k();

// Launch shape of a quantizer call: threads per work unit (64, 128 or 256),
// 16-byte chunks per thread (the kernel instantiation's CH) and workgroups.
// Pure host logic; false if no instantiation serves K.
struct QuantLaunch {
  int tpr, ch, grid;
};
bool quant_launch_config(int op, int mode, long M, int K, int num_cus, QuantLaunch* out);

// q [M,K] e4m3, scale [M] or [M,K/128] (written) or [1] (kStaticTensor:
// read); x is [M,K] bf16 (kIdent, kRms) or
// gate_up [M,2K] bf16 (kSilu); w [K] bf16 (kRms only).
hipError_t launch_quant(int op, int mode, int fmt, uint8_t* q, float* scale,
                        const uint16_t* x, const uint16_t* w, int M, int K, float eps,
                        int num_cus, hipStream_t st);
hipError_t launch_cvt_e4m3(uint8_t* q, const float* x, long n, int num_cus, hipStream_t st);
hipError_t launch_silu(float* y, const uint16_t* g, long n, int num_cus, hipStream_t st);

}  // namespace fp8q
