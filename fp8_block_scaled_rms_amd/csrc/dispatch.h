// Per-shape GEMM variant choice.
#pragma once

namespace fp8q {

// GEMM ops (the fp8q_gemm_op values of the C ABI).
constexpr int kOpScaledMm = 0;
constexpr int kOpBlockwise = 1;
constexpr int kOpInt8 = 2;         // W8A8 INT8 scaled_mm
constexpr int kOpBlockwisePow2 = 3; // blockwise with power-of-two (UE8M0) scales

// Variant id for a GEMM call of op `op`.  Returns -1 if no variant can run
// the shape.
int dispatch_gemm(int op, long M, long N, long K);

// Whether variant `id` computes op `op` (the int8 engine serves only the
// int8 op, the FP8 engines only the FP8 ops).
bool variant_serves(int id, int op);

}  // namespace fp8q
