// Per-shape choice of GEMM variant.
//
// The page "Helion can accelerate vLLM LLM inference on NVIDIA GPUs"
// (aihirek.info), section "Autotuning picks the right variant", contrasts
// hand-written dispatch rules with treating the algorithm (conventional,
// split-K, swap-AB) as a tuned parameter chosen per input shape.  Here the
// choice is a compiled-in table keyed by (op, N, K, M bucket) whose rows are
// written from on-device measurements (tune_table.inc); shapes it does not
// cover fall back to a fixed rule.  The lookup is a short linear scan of
// static data: no allocation, no locks, no HIP calls.
#include <cstring>

#include "dispatch.h"
#include "gemm_kernels.h"

namespace fp8q {
namespace {

struct TableRow {
  int op;
  long n, k, m_max;
  const char* variant;
};

const TableRow kTable[] = {
#include "tune_table.inc"
    {-1, 0, 0, 0, nullptr}};

int find_variant(const char* name) {
  const int n = gemm_num_configs();
  for (int i = 0; i < n; ++i)
    if (std::strcmp(gemm_config(i).name, name) == 0) return i;
  return -1;
}

int find_skinny(int engine, int tm, int rw, int wk, int j) {
  const int n = gemm_num_configs();
  for (int i = 0; i < n; ++i) {
    const GemmConfig& c = gemm_config(i);
    if (c.kind == kSkinny && c.engine == engine && c.tm == tm && c.rw == rw && c.wk == wk &&
        c.split == j)
      return i;
  }
  return -1;
}

// Fixed rule for shapes without a measured row (exact FP8 engine, or the
// int8 engine for op 2): the weight-streaming kernel up to 128 tokens, the
// tiled kernel above.
int rule(int op, long M, long N, long K) {
  (void)K;
  const int engine = op == kOpInt8 ? kEngineInt8 : kEngineExact;
  if (M <= 128) {
    const int tm = M <= 16 ? 1 : M <= 32 ? 2 : M <= 64 ? 4 : 8;
    const int rw = (N >= 8192 && N % 32 == 0) ? 2 : 1;
    const int j = tm <= 2 ? (engine == kEngineInt8 ? 4 : 8) : tm == 4 ? 4 : 2;
    int id = find_skinny(engine, tm, rw, 4, j);
    if (id < 0) id = find_skinny(engine, tm, 1, 4, j);
    if (id < 0) id = find_skinny(engine, tm, 1, 4, 2);
    if (id >= 0) return id;
  }
  if (N % 128 == 0)
    return find_variant(engine == kEngineInt8 ? "i8_tiled_m128_n128_w2x2_st2"
                                              : "f16_tiled_m128_n128_w2x2_st2");
  return -1;
}

}  // namespace

bool variant_serves(int id, int op) {
  if (id < 0 || id >= gemm_num_configs()) return false;
  const bool i8 = gemm_config(id).engine == kEngineInt8;
  return op == kOpInt8 ? i8
                       : (op == kOpScaledMm || op == kOpBlockwise || op == kOpBlockwisePow2) && !i8;
}

int dispatch_gemm(int op, long M, long N, long K) {
  // power-of-two blockwise scales run the blockwise variants (the table is
  // measured with general scales)
  const int table_op = op == kOpBlockwisePow2 ? kOpBlockwise : op;
  for (const TableRow* r = kTable; r->variant != nullptr; ++r) {
    if (r->op == table_op && r->n == N && r->k == K && M <= r->m_max) {
      const int id = find_variant(r->variant);
      if (id >= 0 && variant_serves(id, op) && gemm_config_fits(id, M, N, K)) return id;
      break;
    }
  }
  return rule(op, M, N, K);
}

}  // namespace fp8q
