// Per-shape GEMM variant choice.
#pragma once

namespace fp8q {

// Variant id for a GEMM call; op 0 = scaled_mm, 1 = scaled_mm_blockwise.
// Returns -1 if no variant can run the shape.
int dispatch_gemm(int op, long M, long N, long K);

}  // namespace fp8q
