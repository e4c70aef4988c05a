// Internal launch interface of the FP8 GEMM kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8q {

// One compiled GEMM variant.
//   kind kTiled:  LDS-staged tiles of bn weight rows x bm tokens in an
//                 ST-stage ring, wn x wm waves; optionally split along K
//                 (`split` workgroup rows, partials reduced in order).
//   kind kSkinny: weight-streaming kernel for small M: a workgroup owns
//                 rw*16 weight rows and all (<= tm*16) tokens; each of its wk
//                 waves loads `split` (= j) K blocks at once; the waves are
//                 reduced through LDS, and K longer than wk*j blocks is split
//                 across workgroups through an fp32 workspace.
//   kind kHybrid: two launches of tiled variants over column ranges of one
//                 output: the weight-row tiles that fill whole rounds of
//                 resident workgroups with variant part_a (bm x bn tiles, no
//                 split), the remaining columns with variant part_b (split
//                 along K), so the last round of part_a's tiles is not left
//                 part-empty.  bm/bn/wm/wn describe part_a; split is
//                 part_b's split-K factor.
// All keep the weight rows on the 16-row side of the 16x16x128 MFMA and the
// tokens on the 16-column side (the swap-AB orientation).
enum GemmKind { kTiled = 0, kSkinny = 1, kHybrid = 2 };

// Accumulation engine (see gemm_kernels.hip): 0 = FP8 MFMA (fast, hardware
// group-truncated sums), 1 = exact f16 MFMA on losslessly widened operands,
// 2 = int8 MFMA with exact int32 sums (W8A8 INT8 operands, per-token x
// per-channel scales only).
enum GemmEngine { kEngineFp8 = 0, kEngineExact = 1, kEngineInt8 = 2 };

struct GemmConfig {
  const char* name;
  int kind;
  int engine;
  int bm, bn, wm, wn;  // kTiled
  int tm, rw, wk;      // kSkinny
  int split;           // kSkinny: K blocks per wave (j); kTiled: split-K factor
  int part_a, part_b;  // kHybrid: the two tiled variants (registry ids)
};

int gemm_num_configs();
const GemmConfig& gemm_config(int id);
// Whether config `id` can run a problem of M tokens (the skinny kernel has a
// compile-time token limit).
bool gemm_config_fits(int id, long M, long N, long K);
size_t gemm_workspace_bytes(int id, long M, long N, long K);

// Scale layouts of a launch:
//   kScalesPerToken: per-token x per-channel (sa [M], sb [N]);
//   kScalesBlock:    sa [M, K/128], sb [N/128, K/128] (not for kEngineInt8);
//   kScalesBlockPow2: the same, expected to hold powers of two (UE8M0), which
//                    the tiled exact-engine kernels fold into the widening
//                    (other kernels, or scales that do not qualify, take the
//                    kScalesBlock path).
// The operand bytes are e4m3 codes, or int8 values for a kEngineInt8 variant.
enum GemmScales { kScalesPerToken = 0, kScalesBlock = 1, kScalesBlockPow2 = 2 };
hipError_t launch_gemm(int id, int scales, uint16_t* y, const uint8_t* a, const float* sa,
                       const uint8_t* b, const float* sb, int M, int N, int K, void* ws,
                       hipStream_t st);

// Device address of this GPU's scratch array (kScratchBytes, 256-byte
// aligned), the split-K workspace of the allocation-free entry point.
// Looked up once per device (the current one) and cached; no allocation.
constexpr size_t kScratchBytes = size_t{64} << 20;
hipError_t scratch_workspace(void** ptr);

// Blockwise GEMM (exact engine, 128x256 tiles) with SiLU-and-mul and
// group-128 e4m3 quantization in its epilogue: b holds N = 2D weight rows,
// the gate rows then the up rows; writes q [M, D] e4m3 and scale [M, D/128]
// fp32, as silu_mul_quant (group 128) of the bf16 [M, 2D] product would.
// Requires D % 128 == 0 and K % 128 == 0.
hipError_t launch_gemm_silu_quant(uint8_t* q, float* scale, const uint8_t* a, const float* sa,
                                  const uint8_t* b, const float* sb, int M, int N, int K,
                                  hipStream_t st);

}  // namespace fp8q
