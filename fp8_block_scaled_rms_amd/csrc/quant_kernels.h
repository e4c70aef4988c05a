// Internal launch interface of the quantization kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

enum QuantOp { kIdent = 0, kRms = 1, kSilu = 2 };
enum QuantMode { kPerToken = 0, kGroup128 = 1 };

// Largest K (columns of the quantized output) a launch supports.
int quant_max_k();

// q [M,K] e4m3, scale [M] or [M,K/128]; x is [M,K] bf16 (kIdent, kRms) or
// gate_up [M,2K] bf16 (kSilu); w [K] bf16 (kRms only).
hipError_t launch_quant(int op, int mode, uint8_t* q, float* scale, const uint16_t* x,
                        const uint16_t* w, int M, int K, float eps, int num_cus,
                        hipStream_t st);
hipError_t launch_cvt_e4m3(uint8_t* q, const float* x, long n, int num_cus, hipStream_t st);
hipError_t launch_silu(float* y, const uint16_t* g, long n, int num_cus, hipStream_t st);

}  // namespace fp8q
