// FP8 (OCP e4m3) GEMMs with fp32 accumulation and bf16 output for gfx950.
//
//   scaled_mm            y[m,n] = sa[m] sb[n] sum_k a[m,k] b[n,k]
//   scaled_mm_blockwise  y[m,n] = sum_kb sa[m,kb] sb[n/128,kb] sum_{k in kb} a[m,k] b[n,k]
//
// (page "Helion in vLLM: FP8 inference of Qwen3", 24-ai.news, section
// "Kernels integrated into vLLM": scaled_mm and scaled_mm_blockwise).  Both
// operands are K-contiguous ("NT": a [M,K] activations, b [N,K] weights).
//
// The unit of work is one 16x16 output tile over one 128-wide K block (one
// scale block), computed by one of two matrix-core engines (see kEngineF8 /
// kEngineF16 below; the exact f16 engine is the default), so the blockwise
// scales are applied per K-block result in VALU (acc += p * sa * sb).
// Weight rows sit on the MFMA's 16-row side and tokens on its 16-column
// side, so each lane's four results share one token (one activation scale)
// and are four adjacent output columns (one 8-byte bf16 store).  This is the
// swap-AB orientation of the page "Helion can accelerate vLLM LLM inference
// on NVIDIA GPUs" (aihirek.info), section "One GEMM implementation handles
// several algorithms"; with a 16x16 instruction it costs nothing at large M.
//
// Operand fragments: lane l of a 16x128 fragment holds row (l % 16), bytes
// [32 (l / 16), 32 (l / 16) + 32) of the 128-byte K block.  Both operands use
// the same byte-to-K assignment, so the dot product is the same whatever
// K order the hardware applies inside the instruction.  The result lane l
// holds rows 4 (l / 16) + r, r = 0..3, of column l % 16.
//
// Two kernels:
//  * tiled: for large M.  A workgroup stages a BN x 128 weight tile and a
//    BM x 128 token tile per K block into LDS with direct global->LDS 16-byte
//    loads (no VGPR round trip) in an ST-stage ring, XOR-swizzled by 16-byte
//    chunk so the fragment reads do not collide in LDS banks.
//  * skinny: for small M (decode).  HBM traffic is the weight matrix; a
//    workgroup streams rw*16 weight rows straight into registers, its wk
//    waves take interleaved K blocks (split-K inside the workgroup) and are
//    summed through LDS in a fixed order.  `split` > 1 additionally splits K
//    across workgroups through an fp32 workspace and an ordered reduction
//    (page above: split K when M or N is too small to fill the GPU).
#include "fp8q_common.hpp"
#include "gemm_common.hpp"
#include "silu_table.hpp"
#include "gemm_kernels.h"

#include <atomic>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <mutex>
#include <string>
#include <type_traits>
#include <utility>
#include <vector>

namespace fp8q {
namespace {

using namespace tile;


constexpr int kBK = 128;  // K per stage = one scale block = one MFMA


// Accumulation engines for one 16x16 output tile over one 128-wide K block.
//
// kEngineF8: one v_mfma_scale_f32_16x16x128_f8f6f4 (operand formats e4m3,
//   neutral E8M0 scales 2^0).  Fastest, but the FP8 datapath adds its 128
//   products in groups of 8 consecutive K aligned to the largest product of
//   each group: every product is truncated toward zero to a multiple of
//   2^(E-13), E the exponent of that largest product, so elements whose sum
//   cancels heavily carry a relative error well above fp32 rounding.
// kEngineF16: every e4m3 byte is widened exactly to f16 (each e4m3 value is
//   representable in f16) with v_cvt_scalef32_pk_f16_fp8 and the block is
//   four v_mfma_f32_16x16x32_f16, whose sums are exact to fp32 rounding.  Half
//   the matrix-core rate of kEngineF8; the default wherever the table does not
//   choose otherwise.
// Both engines use the same 32-byte-per-lane fragments; kEngineF16 feeds
// instruction s with bytes [8s, 8s+8) of each lane's 32, identically for both
// operands, which is a fixed permutation of K inside the block.
//
// kEngineI8 (W8A8 INT8, per-token x per-channel only): the operands are int8
// and the block is two v_mfma_i32_16x16x64_i8 (bytes [0,16) and [16,32) of
// each lane's 32), accumulated exactly in int32 across all of K; the
// epilogue converts to fp32 and applies the scales.
constexpr int kEngineF8 = kEngineFp8;
constexpr int kEngineF16 = kEngineExact;
constexpr int kEngineI8 = kEngineInt8;

// Accumulator of one 16x16 tile in a lane: 4 fp32, or 4 int32 (kEngineI8).
template <int E>
struct AccT {
  typedef v4f T;
};
template <>
struct AccT<kEngineI8> {
  typedef v4i T;
};
template <int E>
__device__ __forceinline__ typename AccT<E>::T acc_zero() {
  typename AccT<E>::T z;
#pragma unroll
  for (int r = 0; r < 4; ++r) z[r] = 0;
  return z;
}
__device__ __forceinline__ v4f to_f32(v4f a) { return a; }
__device__ __forceinline__ v4f to_f32(v4i a) { return __builtin_convertvector(a, v4f); }

constexpr const char* engine_prefix(int e) {
  return e == kEngineF8 ? "f8" : e == kEngineF16 ? "f16" : "i8";
}

__device__ __forceinline__ v8h widen8(int lo, int hi) {
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  v8h r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// The same widening multiplied by a power of two `scale` (exact whenever the
// result is representable in f16, which the caller guarantees).
__device__ __forceinline__ v8h widen8_scaled(int lo, int hi, float scale) {
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, scale, false);
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, scale, true);
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, scale, false);
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, scale, true);
  v8h r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// A fragment prepared for an engine: the raw bytes (kEngineF8) or four f16
// slabs (kEngineF16).
template <int E>
struct Frag;
template <>
struct Frag<kEngineF8> {
  v8i b;
};
template <>
struct Frag<kEngineF16> {
  v8h h[4];
};
template <>
struct Frag<kEngineI8> {
  v4i lo, hi;
};

template <int E>
__device__ __forceinline__ Frag<E> prep(const v8i& raw) {
  Frag<E> f;
  if constexpr (E == kEngineF8) {
    f.b = raw;
  } else if constexpr (E == kEngineI8) {
    f.lo = v4i{raw[0], raw[1], raw[2], raw[3]};
    f.hi = v4i{raw[4], raw[5], raw[6], raw[7]};
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) f.h[s] = widen8(raw[2 * s], raw[2 * s + 1]);
  }
  return f;
}

// prep<E> with the widened values multiplied by a power of two (exact f16
// engine only; the other engines never fold scales and ignore `scale`).
template <int E>
__device__ __forceinline__ Frag<E> prep_scaled(const v8i& raw, float scale) {
  if constexpr (E == kEngineF16) {
    Frag<E> f;
#pragma unroll
    for (int s = 0; s < 4; ++s) f.h[s] = widen8_scaled(raw[2 * s], raw[2 * s + 1], scale);
    return f;
  } else {
    (void)scale;
    return prep<E>(raw);
  }
}

// 2^(biased exponent of the power of two `s` - eref) as a float, eref chosen
// so that the result lies in [2^-15, 2^7].
__device__ __forceinline__ float pow2_rebased(float s, int eref) {
  const int e = static_cast<int>((__float_as_uint(s) >> 23) & 0xFFu);
  return __uint_as_float(static_cast<uint32_t>(e - eref + 127) << 23);
}

// c + W_block * X_block^T for one tile (weights on the 16-row side).
template <int E>
__device__ __forceinline__ typename AccT<E>::T block_mma(const Frag<E>& w, const Frag<E>& x,
                                                         typename AccT<E>::T c) {
  if constexpr (E == kEngineI8) {
    c = __builtin_amdgcn_mfma_i32_16x16x64_i8(w.lo, x.lo, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(w.hi, x.hi, c, 0, 0, 0);
  } else if constexpr (E == kEngineF8) {
    // operand formats 0 = e4m3; scale 127 = E8M0 2^0 on both sides
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w.b, x.b, c, 0, 0, 0, 127, 0, 127);
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x32_f16(w.h[s], x.h[s], c, 0, 0, 0);
    return c;
  }
}

// Direct global -> LDS loads (global_load_lds_dword[x4]): the data of lane i
// lands at lds + i * size, `lds` being a wave-uniform LDS byte address (it is
// passed in M0).  They are issued from inline assembly on purpose: the
// compiler cannot tell which LDS buffer such a load writes, so for the
// intrinsic it drains every load in flight before each LDS read, which would
// serialise the multi-stage pipeline.  Completion is instead tracked
// explicitly with s_waitcnt vmcnt (wait_stage) followed by a workgroup
// barrier before the stage is read.  The instructions write no registers.
// M0 is a reserved register the compiler does not allocate; in these kernels
// nothing but the two helpers below writes or reads it (the build scans the
// generated assembly for any other M0 use and fails if it finds one).  An
// SALU write of M0 needs one wait state before an LDS-DMA load reads it,
// which the compiler's hazard pass cannot insert inside an asm block: hence
// the s_nop between the two.
// The global address is a wave-uniform 64-bit base (SGPRs, the `saddr`
// form) plus a 32-bit per-lane byte offset: one VGPR per address.
__device__ __forceinline__ void g2lds16s(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(off), "s"(base)
               : "memory");
}
__device__ __forceinline__ void g2lds4s(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds), "v"(off), "s"(base)
               : "memory");
}


__device__ __forceinline__ v8i load_frag_lds(const uint8_t* tile, int r, int g) {
  const uint8_t* row = tile + r * kBK;
  const uint4 lo = *reinterpret_cast<const uint4*>(row + (((2 * g) ^ swz(r)) << 4));
  const uint4 hi = *reinterpret_cast<const uint4*>(row + (((2 * g + 1) ^ swz(r)) << 4));
  v8i f;
  f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
  f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
  return f;
}




// ------------------------------------------------------------- tiled --

template <int BM, int BN, int WM, int WN, int ST, bool BLOCK>
struct TiledShape {
  static constexpr int kThreads = WM * WN * 64;
  static constexpr int kWaves = WM * WN;
  static constexpr int kTM = BM / WM;   // tokens per wave
  static constexpr int kTN = BN / WN;   // weight rows per wave
  static constexpr int kFT = kTM / 16;  // token fragments per wave
  static constexpr int kFW = kTN / 16;  // weight fragments per wave
  static constexpr int kXBytes = BM * kBK;
  static constexpr int kWBytes = BN * kBK;
  // blockwise: one 64-float segment per wave holding [sa column | sb row | pad]
  static constexpr int kSBytes = BLOCK ? kWaves * 256 : 0;
  static constexpr int kStage = kXBytes + kWBytes + kSBytes;
  static constexpr int kLds = ST * kStage;
  // global->LDS load instructions each wave issues per stage (all equal)
  static constexpr int kLoadsPerStage = (BM * 8 + BN * 8) / kThreads + (BLOCK ? 1 : 0);
  static_assert((BM * 8) % kThreads == 0 && (BN * 8) % kThreads == 0, "tile/threads");
  static_assert(128 % kTN == 0, "a wave's weight rows must sit in one 128-row block");
  static_assert(!BLOCK || BM + 64 <= 64 * kWaves, "scale segments");
  static_assert(ST >= 2 && kLoadsPerStage * (ST - 2) < 64, "vmcnt range");
};

template <int L, int ST>
__device__ __forceinline__ void wait_stage(int after) {
  // `after` = stages issued after the one needed, 0 <= after <= ST - 2
  if constexpr (ST >= 4) {
    if (after >= 2) { wait_vm<L * (ST - 2)>(); return; }
  }
  if constexpr (ST >= 3) {
    if (after >= 1) { wait_vm<L>(); return; }
  }
  wait_vm<0>();
}

// ST-stage ring of LDS buffers fed by direct global->LDS loads: the loads of
// K block kb+ST-1 are in flight while block kb is multiplied, which covers
// the HBM/L2 latency at the consumption rate of the matrix cores.
// P2 (blockwise, exact engine): when every scale a wave uses is a power of
// two and the exponents of its token rows and of its weight block each span
// at most 22 binades over the K range, the scales are folded exactly into
// the f16 widening (2^(e - eref), eref = largest exponent - 7, so every
// widened value stays exactly representable in f16) and the MFMAs
// accumulate across K blocks directly: no per-block scale FMA.  The wave
// multiplies by 2^(eref_a + eref_b) in the epilogue.  Waves whose scales do
// not qualify run the per-block FMA path.  UE8M0 scales (the page "Helion
// in vLLM: FP8 inference of Qwen3", section "Practical limits") qualify.
// SQ (SiLU-and-mul + group quantization fused into the epilogue; blockwise,
// exact engine, 128x256 tiles of 2x4 waves): B holds N = 2D rows, the gate
// rows [0, D) then the up rows [D, 2D), and the output is the e4m3 codes
// q [M, D] (through `y`) with fp32 scales [M, D/128] (through `ws`) that
// silu_mul_quant would produce, in group-128 mode, from the bf16 result of
// the plain kernel -- without writing that result.  Each wave's 64 weight
// rows are 32 gate rows and the 32 matching up rows, so a lane holds the
// gate and up values of the same output columns, and the 128 output columns
// of a workgroup are one quantization group.
// The bf16 output's rows are ldy elements apart (N, or the whole width when
// a launch covers a column range of a wider output); split-K partials and
// the fused epilogue's codes are laid out by N.
template <int BM, int BN, int WM, int WN, int ST, bool BLOCK, int E, int PRIO = 0,
          bool P2 = false, bool SQ = false>
__global__ __launch_bounds__(WM* WN * 64) void gemm_tiled_kernel(
    uint16_t* __restrict__ y, float* __restrict__ ws, const uint8_t* __restrict__ A,
    const float* __restrict__ sa, const uint8_t* __restrict__ B, const float* __restrict__ sb,
    int M, int N, int K, int SPLIT, int ldy) {
  using S = TiledShape<BM, BN, WM, WN, ST, BLOCK>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  // Blockwise scales on the exact engine, without folding: the rotated K
  // loop below.  Eight-wave tiles run it in two wave groups (see there).
  constexpr bool kRotate = BLOCK && E == kEngineF16 && !P2 && S::kWaves >= 4;
  constexpr bool kGroups = kRotate && S::kWaves == 8 && ST == 3 && !PRIO;
  // the same two-group schedule for the eight-wave kernels on the plain
  // block loop (power-of-two folding, per-token scales, int8): weight
  // fragments 0-1, barrier, 2-3
  constexpr bool kGroupsPlain = !kRotate && E != kEngineF8 && S::kWaves == 8 && ST == 3 && !PRIO;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % WN, wm = wave / WN;
  const int lr = lane & 15, g = lane >> 4;

  int tn, tmi;
  tile_coords(blockIdx.x, (M + BM - 1) / BM, N / BN, tn, tmi);
  const int n0 = tn * BN, m0 = tmi * BM;
  const int KB = K / kBK;
  // split-K: workgroup row blockIdx.y takes K blocks [kb_first, kb_first + nkb)
  const int per_split = (KB + SPLIT - 1) / SPLIT;
  const int kb_first = static_cast<int>(blockIdx.y) * per_split;
  const int nkb = (KB - kb_first < per_split) ? KB - kb_first : per_split;

  // per-thread, K-block-invariant parts of the load addresses: byte offsets
  // from the workgroup's first token row and first weight row (below
  // BM * K and BN * K, or (D + 128) * K for SQ; the host checks they fit
  // in 32 bits)
  // Load j of a thread covers LDS row j * kThreads / 8 + tid / 8, whose
  // swizzle does not depend on j.  Token rows past M are clamped to the
  // last one.  The eight-wave blockwise tiles, short of registers, derive
  // every token-row offset from the first (kThreads / 8 rows further per
  // load, clamped to a_lim; K is a multiple of 128, so the low 7 bits of an
  // offset are its chunk); the others keep one offset per load.
  static_assert((S::kThreads / 8) % 16 == 0, "load rows must keep their swizzle");
  constexpr bool kCompactA = kGroups || kGroupsPlain;
  constexpr int kALoads = BM * 8 / S::kThreads;
  uint32_t a_off[kCompactA ? 1 : kALoads], b_off0;
#pragma unroll
  for (int j = 0; j < (kCompactA ? 1 : kALoads); ++j) {
    const int qi = j * S::kThreads + tid;
    const int r = qi >> 3, p = qi & 7;
    const int rr = (m0 + r < M) ? r : M - 1 - m0;
    a_off[j] = static_cast<uint32_t>(kCompactA ? r : rr) * static_cast<uint32_t>(K) +
               ((p ^ swz(r)) << 4);
  }
  // last valid token row of the tile, as a byte offset (below BM * K < 2^32
  // whatever M is: the row index is clamped before the multiply)
  const int a_last = (M - 1 - m0 < BM - 1) ? M - 1 - m0 : BM - 1;
  const uint32_t a_lim = static_cast<uint32_t>(a_last) * static_cast<uint32_t>(K);
  static_assert(!SQ || (BLOCK && E == kEngineF16 && !P2 && S::kTN == 64 && WN * 32 == 128),
                "fused SiLU-and-mul quantization: blockwise exact engine, 128 output columns");
  // SQ: LDS weight row r (wave r / 64) is gate row 32 (r / 64) + r % 64 of the
  // output column tile, or the matching up row for r % 64 >= 32
  const int D = N / 2;
  const int o0 = tn * 128;  // SQ: first output column of the tile
  const int nb0 = SQ ? o0 : n0;  // first weight row of the tile's row set
  auto b_row = [&](int r) -> int {
    if constexpr (SQ) {
      const int w = r >> 6, l = r & 63;
      return (l < 32) ? o0 + 32 * w + l : D + o0 + 32 * w + (l - 32);
    } else {
      return n0 + r;
    }
  };
  // Weight rows: global row b_row of the LDS row, kBStep rows further for
  // each load (tiles hold whole weight rows: no clamp).
  constexpr int kBStep = SQ ? 32 : S::kThreads / 8;
  {
    const int r = tid >> 3, p = tid & 7;
    b_off0 = static_cast<uint32_t>(b_row(r) - nb0) * static_cast<uint32_t>(K) + ((p ^ swz(r)) << 4);
  }
  // blockwise scales: wave w fetches floats [64w, 64w+64) of [sa column | sb | pad]
  // (a wave-uniform base: the tile's first token row of sa, or for the wave
  // holding the sb entries, the tile's first weight block; byte offsets
  // from it per lane)
  const int blk0 = SQ ? o0 / 128 : n0 / 128;
  const float* s_base = (BLOCK && wave == BM / 64) ? sb + static_cast<long>(blk0) * KB
                                                   : sa + static_cast<long>(m0) * KB;
  uint32_t s_off = 0;
  if constexpr (BLOCK) {
    static_assert(BM % 64 == 0 && BN / 128 <= 64, "scale segment layout");
    const int q = wave * 64 + lane;
    if (q < BM) {
      const int rr = (m0 + q < M) ? q : M - 1 - m0;
      s_off = static_cast<uint32_t>(rr) * static_cast<uint32_t>(KB) * 4u;
    } else if (q < BM + BN / 128) {
      const int blk = SQ ? (q == BM ? o0 / 128 : (D + o0) / 128) : n0 / 128 + (q - BM);
      s_off = static_cast<uint32_t>(blk - blk0) * static_cast<uint32_t>(KB) * 4u;
    }  // else padding: offset 0 from either base is a valid address
  }

  const uint32_t lds0 = lds_address(smem);
  const uint8_t* A0 = A + static_cast<long>(m0) * K;
  const uint8_t* B0 = B + static_cast<long>(nb0) * K;
  auto load_stage = [&](int kb, int buf) {
    const uint32_t base = lds0 + buf * S::kStage + wave * 64 * 16;
    const uint8_t* Ak = A0 + static_cast<long>(kb) * kBK;
    const uint8_t* Bk = B0 + static_cast<long>(kb) * kBK;
#pragma unroll
    for (int j = 0; j < kALoads; ++j) {
      if constexpr (kCompactA) {
        const uint32_t o =
            a_off[0] + static_cast<uint32_t>(j * (S::kThreads / 8)) * static_cast<uint32_t>(K);
        const uint32_t lim = a_lim + (a_off[0] & 127u);
        g2lds16s(Ak, o < lim ? o : lim, base + j * S::kThreads * 16);
      } else {
        g2lds16s(Ak, a_off[j], base + j * S::kThreads * 16);
      }
    }
#pragma unroll
    for (int j = 0; j < BN * 8 / S::kThreads; ++j)
      g2lds16s(Bk + static_cast<long>(j * kBStep) * K, b_off0, base + S::kXBytes + j * S::kThreads * 16);
    if constexpr (BLOCK)
      g2lds4s(s_base + kb, s_off, lds0 + buf * S::kStage + S::kXBytes + S::kWBytes + wave * 256);
  };

  static_assert(!(BLOCK && E == kEngineI8), "the int8 engine is per-token x per-channel only");
  static_assert(!P2 || (BLOCK && E == kEngineF16), "scale folding: blockwise, exact engine");

  // reference exponents for folded power-of-two scales (see above)
  int ea_ref[S::kFT];
  int eb_ref = 0;
  bool fold = false;
  if constexpr (P2) {
    bool ok = true;
#pragma unroll
    for (int t = 0; t < S::kFT; ++t) {
      const int mr = m0 + wm * S::kTM + 16 * t + lr;
      const long row = (mr < M) ? mr : M - 1;
      int emax = 0, emin = 255;
      for (int kb = kb_first + g; kb < kb_first + nkb; kb += 4) {  // 4 lanes share a row
        const uint32_t u = __float_as_uint(sa[row * KB + kb]);
        const int e = static_cast<int>((u >> 23) & 0xFFu);
        ok = ok && (u & 0x807FFFFFu) == 0 && e != 0 && e != 255;
        emax = e > emax ? e : emax;
        emin = e < emin ? e : emin;
      }
#pragma unroll
      for (int o = 16; o < 64; o <<= 1) {
        const int a = __shfl_xor(emax, o), b = __shfl_xor(emin, o);
        emax = a > emax ? a : emax;
        emin = b < emin ? b : emin;
      }
      ea_ref[t] = emax - 7;
      ok = ok && emax - emin <= 22;
    }
    const long nb = (n0 + wn * S::kTN) / 128;
    int fmax = 0, fmin = 255;
    for (int kb = kb_first + lane; kb < kb_first + nkb; kb += 64) {
      const uint32_t u = __float_as_uint(sb[nb * KB + kb]);
      const int e = static_cast<int>((u >> 23) & 0xFFu);
      ok = ok && (u & 0x807FFFFFu) == 0 && e != 0 && e != 255;
      fmax = e > fmax ? e : fmax;
      fmin = e < fmin ? e : fmin;
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int a = __shfl_xor(fmax, o), b = __shfl_xor(fmin, o);
      fmax = a > fmax ? a : fmax;
      fmin = b < fmin ? b : fmin;
    }
    eb_ref = fmax - 7;
    ok = ok && fmax - fmin <= 22;
    fold = __all(ok);
  }

  typename AccT<E>::T acc[S::kFW][S::kFT];
#pragma unroll
  for (int i = 0; i < S::kFW; ++i)
#pragma unroll
    for (int t = 0; t < S::kFT; ++t) acc[i][t] = acc_zero<E>();

  // The fused kernel (SQ) scales each block's products at the end of that
  // block (after its second half) rather than in the next block's first
  // half, which also waits for that block's LDS fragments.  The plain
  // kernels keep the FMAs in the first half, where their schedule measured
  // faster.
  constexpr bool kEndFma = kGroups && SQ;

  // the grouped loop issues the same number of loads per block throughout:
  // past the last block it loads the last block again, into its own buffer
  // (the same bytes), so its waits are the same constants everywhere
  auto load_block = [&](int b) {
    const int bl = (b < nkb) ? b : nkb - 1;
    load_stage(kb_first + bl, bl % ST);
  };
#pragma unroll
  for (int p = 0; p < ST - 1; ++p) {
    if constexpr (kGroups || kGroupsPlain)
      load_block(p);
    else if (p < nkb)
      load_stage(kb_first + p, p);
  }

  // the raw fragments and block scales of block j from its LDS buffer (SQ:
  // swr_hi is the up rows' weight scale, swr the gate rows'; else equal)
  auto read_scales = [&](int j, float(&sar)[S::kFT], float& swr, float& swr_hi) {
    if constexpr (BLOCK) {
      const float* sas =
          reinterpret_cast<const float*>(smem + (j % ST) * S::kStage + S::kXBytes + S::kWBytes);
      if constexpr (SQ) {
        swr = sas[BM];
        swr_hi = sas[BM + 1];
      } else {
        swr = sas[BM + (wn * S::kTN) / 128];
        swr_hi = swr;
      }
#pragma unroll
      for (int t = 0; t < S::kFT; ++t) sar[t] = sas[wm * S::kTM + 16 * t + lr];
    }
  };
  auto read_block = [&](int j, v8i(&xr)[S::kFT], v8i(&wr)[S::kFW], float(&sar)[S::kFT],
                        float& swr, float& swr_hi) {
    const uint8_t* xs = smem + (j % ST) * S::kStage;
    const uint8_t* wsm = xs + S::kXBytes;
#pragma unroll
    for (int t = 0; t < S::kFT; ++t) xr[t] = load_frag_lds(xs, wm * S::kTM + 16 * t + lr, g);
#pragma unroll
    for (int i = 0; i < S::kFW; ++i) wr[i] = load_frag_lds(wsm, wn * S::kTN + 16 * i + lr, g);
    read_scales(j, sar, swr, swr_hi);
  };

  // one block's products from its raw fragments and scales (weight
  // fragments [I0, I1))
  auto multiply = [&](auto fold_c, const v8i(&xr)[S::kFT], const v8i(&wr)[S::kFW],
                      const float(&sar)[S::kFT], float swr, auto i0, auto i1) {
    constexpr int I0 = decltype(i0)::value, I1 = decltype(i1)::value;
    constexpr bool FOLD = decltype(fold_c)::value;
    float sab[S::kFT];
    float sxf[S::kFT];
    float swf = 1.0f;
    if constexpr (BLOCK) {
      if constexpr (FOLD) {
        swf = pow2_rebased(swr, eb_ref);
#pragma unroll
        for (int t = 0; t < S::kFT; ++t) sxf[t] = pow2_rebased(sar[t], ea_ref[t]);
      } else {
#pragma unroll
        for (int t = 0; t < S::kFT; ++t) sab[t] = sar[t] * swr;
      }
    }
    Frag<E> xf[S::kFT];
#pragma unroll
    for (int t = 0; t < S::kFT; ++t) {
      if constexpr (FOLD)
        xf[t] = prep_scaled<E>(xr[t], sxf[t]);
      else
        xf[t] = prep<E>(xr[t]);
    }
#pragma unroll
    for (int i = I0; i < I1; ++i) {
      Frag<E> wf;
      if constexpr (FOLD)
        wf = prep_scaled<E>(wr[i], swf);
      else
        wf = prep<E>(wr[i]);
#pragma unroll
      for (int t = 0; t < S::kFT; ++t) {
        if constexpr (BLOCK) {
          if constexpr (!FOLD) {
            const v4f p = block_mma<E>(wf, xf[t], acc_zero<E>());
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][t][r] = fmaf(p[r], sab[t], acc[i][t][r]);
          } else {  // scales already folded into the operands
            acc[i][t] = block_mma<E>(wf, xf[t], acc[i][t]);
          }
        } else {
          acc[i][t] = block_mma<E>(wf, xf[t], acc[i][t]);
        }
      }
    }
  };

  // Blockwise scales on the exact engine, without folding: the substeps
  // of a block are the outer loop (consecutive matrix instructions are
  // independent) and the products of block j are scaled into the
  // accumulators while block j+1's first substep is issued, when they are
  // long finished, instead of waiting at the end of block j for the last
  // instructions of each chain.  The same products are added to the
  // accumulators in the same order as in the plain loop.  (Not used where
  // it would exceed 256 VGPRs and halve the occupancy: in the folding
  // kernels, whose folded loop shares the register budget, and in two-wave
  // tiles, whose lanes hold twice the load addresses.)
  // Eight-wave tiles (two waves per SIMD) run the rotated loop with the
  // waves in two groups half a block apart: waves 4..7 pass one extra
  // barrier before the loop and waves 0..3 one after it, and every block
  // has a second barrier after its first two substeps.  Each SIMD holds one
  // wave of each group, so while one wave waits for its LDS fragments and
  // applies the previous block's scales (VALU), the other issues matrix
  // instructions.  In lock step both waves of a SIMD did those at the same
  // time and the matrix cores idled.  (The mid-block barrier is fenced with
  // sched_barrier: the compiler would otherwise hoist the second half's
  // matrix instructions above it.)

  // SQ: once the last block is in flight, the buffer after it is free for
  // good; the SiLU table (32 KiB: 4 x 1 KiB per wave) goes there while the
  // last block is multiplied
  auto prefetch_table = [&](int j) {
    if constexpr (SQ) {
      if (j == nkb - 1) {
        const uint32_t tl = lds0 + ((j + 1) % ST) * S::kStage;
        const uint8_t* tg = reinterpret_cast<const uint8_t*>(kSiluTable);
#pragma unroll
        for (int c = 0; c < 32 / S::kWaves; ++c) {
          const int chunk = wave * (32 / S::kWaves) + c;
          g2lds16s(tg + chunk * 1024, lane * 16, tl + chunk * 1024);
        }
      }
    }
  };

  // The four substeps of one block on the rotated schedule; after_s1()
  // runs between substeps 1 and 2.  sprev(i, t): the previous block's
  // scale product for weight fragment i and token fragment t, applied in
  // substep 0.  With END, the block's own products are instead scaled into
  // the accumulators after its last substep, with scur(i, t) (the same
  // products added in the same order, so the same sums).
  auto rotated_block = [&](v4f(&p)[S::kFW][S::kFT], auto sprev, const v8i(&xr)[S::kFT],
                           const v8i(&wr)[S::kFW], auto after_s1, auto end_c, auto scur) {
    constexpr bool END = decltype(end_c)::value;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v8h xh[S::kFT];
#pragma unroll
      for (int t = 0; t < S::kFT; ++t) xh[t] = widen8(xr[t][2 * s], xr[t][2 * s + 1]);
#pragma unroll
      for (int i = 0; i < S::kFW; ++i) {
        const v8h wh = widen8(wr[i][2 * s], wr[i][2 * s + 1]);
#pragma unroll
        for (int t = 0; t < S::kFT; ++t) {
          if (s == 0) {  // block j-1's products (zeros before the first block)
            if constexpr (!END) {
              const float sp = sprev(i, t);
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[i][t][r] = fmaf(p[i][t][r], sp, acc[i][t][r]);
            }
            p[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wh, xh[t], v4f{0, 0, 0, 0}, 0, 0, 0);
          } else {
            p[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wh, xh[t], p[i][t], 0, 0, 0);
          }
        }
      }
      if (s == 1) after_s1();
    }
    if constexpr (END) {
#pragma unroll
      for (int i = 0; i < S::kFW; ++i)
#pragma unroll
        for (int t = 0; t < S::kFT; ++t) {
          const float sc = scur(i, t);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][t][r] = fmaf(p[i][t][r], sc, acc[i][t][r]);
        }
    }
  };

  auto k_loop_rotated = [&]() {
    v4f p[S::kFW][S::kFT];
    float sprev[S::kFT], sprev_hi[S::kFT];
#pragma unroll
    for (int t = 0; t < S::kFT; ++t) sprev[t] = sprev_hi[t] = 0.0f;
#pragma unroll
    for (int i = 0; i < S::kFW; ++i)
#pragma unroll
      for (int t = 0; t < S::kFT; ++t) p[i][t] = v4f{0, 0, 0, 0};
    if constexpr (kGroups) {
      constexpr int L = S::kLoadsPerStage;
      const bool late = wave >= S::kWaves / 2;
      // sprev/sprev_hi: the previous block's scale products (unused with
      // kEndFma)
      auto scale_of = [&](int i, int t) {
        return (SQ && i >= S::kFW / 2) ? sprev_hi[t] : sprev[t];
      };
      // before the mid-block barrier this wave's LDS reads of block j have
      // returned (its buffer is refilled after the next barrier) and its
      // loads of block j+1 have landed (the other group reads block j+1
      // after this barrier)
      auto mid_barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        wait_vm<L>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      };
      // Every block: wait for its loads (one stage of L loads may stay in
      // flight), barrier, read it, load block j+2 (or the last block again),
      // substeps 0-1, mid-block barrier, substeps 2-3.  (nkb >= 1: a
      // split along K never leaves a workgroup row without blocks.)
      if (late) {
        wait_vm<L>();
        __builtin_amdgcn_s_barrier();
      }
      for (int j = 0; j < nkb; ++j) {
        wait_vm<L>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        float sar[S::kFT], swr = 0.0f, swr_hi = 0.0f;
        v8i xr[S::kFT], wr[S::kFW];
        read_block(j, xr, wr, sar, swr, swr_hi);
        load_block(j + ST - 1);
        prefetch_table(j);
        rotated_block(p, scale_of, xr, wr, mid_barrier, std::integral_constant<bool, kEndFma>{},
                      [&](int i, int t) {
                        return sar[t] * ((SQ && i >= S::kFW / 2) ? swr_hi : swr);
                      });
        if constexpr (!kEndFma) {
#pragma unroll
          for (int t = 0; t < S::kFT; ++t) {
            sprev[t] = sar[t] * swr;
            sprev_hi[t] = sar[t] * swr_hi;
          }
        }
      }
      if (!late) __builtin_amdgcn_s_barrier();
      wait_vm<0>();  // the repeated loads of the last block
    } else {
      v8i xr[S::kFT], wr[S::kFW];
      float sar[S::kFT], swr = 0.0f, swr_hi = 0.0f;
      for (int j = 0; j < nkb; ++j) {
        const int after = (nkb - 1 - j < ST - 2) ? nkb - 1 - j : ST - 2;
        wait_stage<S::kLoadsPerStage, ST>(after);
        __builtin_amdgcn_s_barrier();  // as in the plain loop below
        asm volatile("" ::: "memory");
        read_block(j, xr, wr, sar, swr, swr_hi);
        if (j + ST - 1 < nkb) load_stage(kb_first + j + ST - 1, (j + ST - 1) % ST);
        prefetch_table(j);
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
        rotated_block(
            p, [&](int i, int t) { return (SQ && i >= S::kFW / 2) ? sprev_hi[t] : sprev[t]; },
            xr, wr, []() {}, std::false_type{}, [](int, int) { return 0.0f; });
#pragma unroll
        for (int t = 0; t < S::kFT; ++t) {
          sprev[t] = sar[t] * swr;
          sprev_hi[t] = sar[t] * swr_hi;
        }
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
      }
    }
    if constexpr (!kEndFma) {  // the last block's products
#pragma unroll
      for (int i = 0; i < S::kFW; ++i)
#pragma unroll
        for (int t = 0; t < S::kFT; ++t) {
          const float sp = (SQ && i >= S::kFW / 2) ? sprev_hi[t] : sprev[t];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][t][r] = fmaf(p[i][t][r], sp, acc[i][t][r]);
        }
    }
  };

  auto k_loop = [&](auto fold_c) {
    if constexpr (kRotate && !decltype(fold_c)::value) {
      k_loop_rotated();
    } else if constexpr (kGroupsPlain) {
      // the two-group schedule of k_loop_rotated on the plain block loop
      constexpr int L = S::kLoadsPerStage;
      const bool late = wave >= S::kWaves / 2;
      using H0 = std::integral_constant<int, 0>;
      using H1 = std::integral_constant<int, S::kFW / 2>;
      using H2 = std::integral_constant<int, S::kFW>;
      if (late) {
        wait_vm<L>();
        __builtin_amdgcn_s_barrier();
      }
      for (int j = 0; j < nkb; ++j) {
        wait_vm<L>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        v8i xr[S::kFT], wr[S::kFW];
        float sar[S::kFT], swr = 0.0f, swr_hi = 0.0f;
        read_block(j, xr, wr, sar, swr, swr_hi);
        load_block(j + ST - 1);
        multiply(fold_c, xr, wr, sar, swr, H0{}, H1{});
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        wait_vm<L>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        multiply(fold_c, xr, wr, sar, swr, H1{}, H2{});
      }
      if (!late) __builtin_amdgcn_s_barrier();
      wait_vm<0>();  // the repeated loads of the last block
    } else {
      for (int j = 0; j < nkb; ++j) {
        const int after = (nkb - 1 - j < ST - 2) ? nkb - 1 - j : ST - 2;
        wait_stage<S::kLoadsPerStage, ST>(after);
        // Block j is in LDS (each wave waited for its own loads, whose data
        // is written before the counter drops) and every wave is done
        // reading j-1.  A bare s_barrier: __syncthreads() would also wait
        // for the loads of the later stages still in flight.
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        v8i xr[S::kFT], wr[S::kFW];
        float sar[S::kFT], swr = 0.0f, swr_hi = 0.0f;
        read_block(j, xr, wr, sar, swr, swr_hi);
        // the buffer of block j-1 is free: refill it with block j+ST-1
        if (j + ST - 1 < nkb) load_stage(kb_first + j + ST - 1, (j + ST - 1) % ST);
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
        multiply(fold_c, xr, wr, sar, swr, std::integral_constant<int, 0>{},
                 std::integral_constant<int, S::kFW>{});
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
      }
    }
  };
  if constexpr (P2) {
    if (fold)
      k_loop(std::true_type{});
    else
      k_loop(std::false_type{});
  } else {
    k_loop(std::false_type{});
  }

  if constexpr (SQ) {
    // Fused epilogue.  Lane (lr, g) holds, for token lr of fragment t, the
    // gate values of output columns 32 wn + 16 h + 4 g + r (fragments h = 0,
    // 1) and the up values of the same columns (fragments h + 2).  Each is
    // rounded to bf16 as the plain kernel stores it, then y = silu(gate) * up
    // and the group-128 quantization follow silu_mul_quant exactly.
    // The table was loaded into the buffer after the last block's (K loop
    // above); once this wave's loads have landed and every wave is past the
    // barrier, it is complete and no wave reads the staging buffers any more.
    wait_vm<0>();
    __syncthreads();
    const int jl = nkb - 1;
    const float* tab = reinterpret_cast<const float*>(smem + ((jl + 1) % ST) * S::kStage);
    float* red = reinterpret_cast<float*>(smem + (jl % ST) * S::kStage);  // [BM][WN] amax
    constexpr int kH = S::kFW / 2;
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    typedef float v2f __attribute__((ext_vector_type(2)));
    // round to bf16 (nearest even, as the plain kernel's stores) two values at a time
    auto bf16x2 = [](float lo, float hi) -> uint32_t {
      return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{lo, hi}, v2bf));
    };
    float v[S::kFT][kH][4];
#pragma unroll
    for (int t = 0; t < S::kFT; ++t) {
      float cm = 0.0f;
#pragma unroll
      for (int h = 0; h < kH; ++h)
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          const uint32_t gb = bf16x2(acc[h][t][r], acc[h][t][r + 1]);
          const uint32_t ub = bf16x2(acc[h + kH][t][r], acc[h + kH][t][r + 1]);
          v[t][h][r] = silu_bf16(gb & 0xFFFFu, tab) * __uint_as_float(ub << 16);
          v[t][h][r + 1] = silu_bf16(gb >> 16, tab) * __uint_as_float(ub & 0xFFFF0000u);
          cm = fmaxf(cm, fmaxf(fabsf(v[t][h][r]), fabsf(v[t][h][r + 1])));
        }
      // the wave's 32 columns of this token sit in lanes lr, lr + 16, lr + 32, lr + 48
      {  // non-negative: integer max of the bit patterns (no NaN-quieting moves)
        uint32_t u = __float_as_uint(cm);
        u = u32_max(u, static_cast<uint32_t>(__shfl_xor(static_cast<int>(u), 16)));
        u = u32_max(u, static_cast<uint32_t>(__shfl_xor(static_cast<int>(u), 32)));
        cm = __uint_as_float(u);
      }
      if (g == 0) red[(wm * S::kTM + 16 * t + lr) * WN + wn] = cm;
    }
    __syncthreads();
    uint8_t* q = reinterpret_cast<uint8_t*>(y);
    const int ngroups = D / 128;
#pragma unroll
    for (int t = 0; t < S::kFT; ++t) {
      const int row = wm * S::kTM + 16 * t + lr;
      const int m = m0 + row;
      float amax = red[row * WN];
#pragma unroll
      for (int w = 1; w < WN; ++w)
        amax = __uint_as_float(u32_max(__float_as_uint(amax), __float_as_uint(red[row * WN + w])));
      if (m >= M) continue;
      const GroupScale gs = make_scale(amax);
      if (wn == 0 && g == 0) ws[static_cast<long>(m) * ngroups + tn] = gs.s;
#pragma unroll
      for (int h = 0; h < kH; ++h) {
        const int col = o0 + 32 * wn + 16 * h + 4 * g;
        const uint32_t code =
            pack4_e4m3_dynamic(quotient(v[t][h][0], gs), quotient(v[t][h][1], gs),
                               quotient(v[t][h][2], gs), quotient(v[t][h][3], gs));
        *reinterpret_cast<uint32_t*>(q + static_cast<long>(m) * D + col) = code;
      }
    }
    return;
  }

  // epilogue: lane holds weight rows n..n+3 of token m
#pragma unroll
  for (int t = 0; t < S::kFT; ++t) {
    const int m = m0 + wm * S::kTM + 16 * t + lr;
    if (m >= M) continue;
    if constexpr (P2) {
      if (fold) {  // undo the folding: exact power-of-two rescale
        const int sh = ea_ref[t] + eb_ref - 254;
#pragma unroll
        for (int i = 0; i < S::kFW; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][t][r] = ldexpf(acc[i][t][r], sh);
      }
    }
    if (SPLIT > 1) {  // raw partials (fp32, or int32 bits) for splitk_reduce_kernel
#pragma unroll
      for (int i = 0; i < S::kFW; ++i) {
        const int n = n0 + wn * S::kTN + 16 * i + 4 * g;
        *reinterpret_cast<typename AccT<E>::T*>(
            ws + (static_cast<long>(blockIdx.y) * M + m) * N + n) = acc[i][t];
      }
      continue;
    }
    float sm = 1.0f;
    if constexpr (!BLOCK) sm = sa[m];
#pragma unroll
    for (int i = 0; i < S::kFW; ++i) {
      const int n = n0 + wn * S::kTN + 16 * i + 4 * g;
      v4f v = to_f32(acc[i][t]);
      if constexpr (!BLOCK) {
        const float4 s4 = *reinterpret_cast<const float4*>(sb + n);
        v[0] = v[0] * sm * s4.x;
        v[1] = v[1] * sm * s4.y;
        v[2] = v[2] * sm * s4.z;
        v[3] = v[3] * sm * s4.w;
      }
      store_bf16x4(y + static_cast<long>(m) * ldy + n, v[0], v[1], v[2], v[3]);
    }
  }
}

// ------------------------------------------------------------ skinny --
// Small M (output rows ldy elements apart, as in the tiled kernel): the
// weight matrix is the HBM traffic, so the kernel is built to
// keep enough bytes in flight.  A workgroup owns RW*16 weight rows and all
// tokens (<= TMX*16); each of its WK waves owns J K blocks (interleaved
// across the waves) and issues the loads of all of them before the first
// MFMA.  The WK partial sums are added through LDS in wave order; when K
// needs more than WK*J blocks, further workgroups along K write fp32
// partials that splitk_reduce_kernel adds in order.
template <int TMX, int RW, int WK, int J, bool BLOCK, int E>
__global__ __launch_bounds__(WK * 64) void gemm_skinny_kernel(
    uint16_t* __restrict__ y, float* __restrict__ ws, const uint8_t* __restrict__ A,
    const float* __restrict__ sa, const uint8_t* __restrict__ B, const float* __restrict__ sb,
    int M, int N, int K, int SPLIT, int ldy) {
  extern __shared__ __attribute__((aligned(16))) float red[];  // [WK][RW*TMX][64] v4f
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * RW * 16;
  const int s = blockIdx.y;
  const int KB = K / kBK;
  const int kb0 = s * (WK * J) + wave;  // this wave: kb0, kb0 + WK, ...

  // Fragments are loaded through buffer resources over this workgroup's
  // weight rows and over the M token rows (offsets below 2^32: K <= 2^22,
  // at most 64 weight rows and 128 tokens).  A token row at or beyond M, or
  // a block past K (offset kOutside), lies outside its resource and loads
  // zeros without touching memory.
  const __amdgpu_buffer_rsrc_t wres =
      buffer_rsrc(B + static_cast<long>(n0) * K, static_cast<uint32_t>(RW * 16) * K);
  const __amdgpu_buffer_rsrc_t xres = buffer_rsrc(A, static_cast<uint32_t>(M) * K);
  constexpr uint32_t kOutside = 0x80000000u;
  uint32_t woff[RW], xoff[TMX];
  bool xok[TMX];
#pragma unroll
  for (int i = 0; i < RW; ++i) woff[i] = static_cast<uint32_t>(16 * i + lr) * K + 32 * g;
#pragma unroll
  for (int t = 0; t < TMX; ++t) {
    const int m = 16 * t + lr;
    xok[t] = m < M;
    xoff[t] = static_cast<uint32_t>(m) * K + 32 * g;
  }
  const long sb_row = static_cast<long>(n0 / 128) * KB;

  // issue every load of this wave first, with no branch: where a branch
  // around a load joins, the compiler may copy the loaded register, and
  // that copy waits for every load issued before it, turning the J blocks
  // into J round trips to memory.  The buffer resources mask the fragments;
  // the block scales are loaded from clamped (valid) addresses and masked
  // afterwards.
  v8i wr[J][RW], xr[J][TMX];
  float sab[J][TMX];
  float sar[J][TMX], sbr[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int kb = kb0 + WK * j;
    const bool on = kb < KB;
    const uint32_t koff = on ? static_cast<uint32_t>(kb * kBK) : kOutside;
#pragma unroll
    for (int i = 0; i < RW; ++i) wr[j][i] = load_frag_buffer(wres, woff[i] + koff);
#pragma unroll
    for (int t = 0; t < TMX; ++t) xr[j][t] = load_frag_buffer(xres, xoff[t] + koff);
    if constexpr (BLOCK) {
      const int kbc = on ? kb : KB - 1;
      sbr[j] = sb[sb_row + kbc];
#pragma unroll
      for (int t = 0; t < TMX; ++t) {
        const long m = xok[t] ? 16 * t + lr : 0;
        sar[j][t] = sa[m * KB + kbc];
      }
    }
  }
  // keep every load above this point: the optimizer otherwise sinks each
  // block's loads into the branch that uses them (after the test for blocks
  // past K), and the scheduler toward their first use to save registers,
  // which again costs one round trip per block.  An empty asm that takes
  // the operand and scale pointers and clobbers memory stops the former
  // (with the pointers passed in, it may write what the loads read, so they
  // cannot move below it); the scheduling barrier stops the latter.
  asm volatile("" ::"s"(A), "s"(B), "s"(sa), "s"(sb) : "memory");
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (BLOCK) {
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int t = 0; t < TMX; ++t)
        sab[j][t] = (kb0 + WK * j < KB && xok[t]) ? sar[j][t] * sbr[j] : 0.0f;
  }

  static_assert(!(BLOCK && E == kEngineI8), "the int8 engine is per-token x per-channel only");
  typedef typename AccT<E>::T Acc;
  Acc acc[RW][TMX];
#pragma unroll
  for (int i = 0; i < RW; ++i)
#pragma unroll
    for (int t = 0; t < TMX; ++t) acc[i][t] = acc_zero<E>();
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (kb0 + WK * j >= KB) break;
    Frag<E> xf[TMX];
#pragma unroll
    for (int t = 0; t < TMX; ++t) xf[t] = prep<E>(xr[j][t]);
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const Frag<E> wf = prep<E>(wr[j][i]);
#pragma unroll
      for (int t = 0; t < TMX; ++t) {
        if constexpr (BLOCK) {
          const v4f p = block_mma<E>(wf, xf[t], acc_zero<E>());
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][t][r] = fmaf(p[r], sab[j][t], acc[i][t][r]);
        } else {
          acc[i][t] = block_mma<E>(wf, xf[t], acc[i][t]);
        }
      }
    }
  }

  // add the WK waves' partial sums in a fixed order (int32 sums are exact)
  constexpr int kFrags = RW * TMX;
  Acc* r4 = reinterpret_cast<Acc*>(red);
#pragma unroll
  for (int i = 0; i < RW; ++i)
#pragma unroll
    for (int t = 0; t < TMX; ++t) r4[(wave * kFrags + i * TMX + t) * 64 + lane] = acc[i][t];
  __syncthreads();
  for (int f = wave; f < kFrags; f += WK) {
    const int i = f / TMX, t = f % TMX;
    Acc va = r4[f * 64 + lane];
    for (int w = 1; w < WK; ++w) va += r4[(w * kFrags + f) * 64 + lane];
    const int m = 16 * t + lr;
    if (m >= M) continue;
    const int n = n0 + 16 * i + 4 * g;
    if (SPLIT > 1) {  // raw partial (fp32, or int32 bits for the int8 engine)
      *reinterpret_cast<Acc*>(ws + (static_cast<long>(s) * M + m) * N + n) = va;
      continue;
    }
    v4f v = to_f32(va);
    if constexpr (!BLOCK) {
      const float sm = sa[m];
      const float4 s4 = *reinterpret_cast<const float4*>(sb + n);
      v[0] = v[0] * sm * s4.x;
      v[1] = v[1] * sm * s4.y;
      v[2] = v[2] * sm * s4.z;
      v[3] = v[3] * sm * s4.w;
    }
    store_bf16x4(y + static_cast<long>(m) * ldy + n, v[0], v[1], v[2], v[3]);
  }
}

// Ordered sum of the split-K partials (fp32, or exact int32 for the int8
// engine), then (scaled_mm) the epilogue scales.  The partials of a split
// are loaded kReduceBatch at a time before any is added (clamped to the last
// split, the surplus unused), so a thread waits for one memory round trip
// per batch rather than one per split; the sum still runs in split order.
constexpr int kReduceBatch = 8;

template <bool BLOCK, bool INT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(uint16_t* __restrict__ y,
                                                            const float* __restrict__ ws,
                                                            const float* __restrict__ sa,
                                                            const float* __restrict__ sb,
                                                            int M, int N, int SPLIT,
                                                            int ldy) {
  typedef typename std::conditional<INT, int4, float4>::type V;
  const long total = static_cast<long>(M) * (N / 4);
  const long plane = static_cast<long>(M) * N;  // floats per split
  for (long idx = blockIdx.x * 256L + threadIdx.x; idx < total; idx += gridDim.x * 256L) {
    const int m = static_cast<int>(idx / (N / 4));
    const int n = static_cast<int>(idx % (N / 4)) * 4;
    const float* p = ws + static_cast<long>(m) * N + n;
    V t = *reinterpret_cast<const V*>(p);
    for (int s0 = 1; s0 < SPLIT; s0 += kReduceBatch) {
      V u[kReduceBatch];
#pragma unroll
      for (int i = 0; i < kReduceBatch; ++i) {
        const int s = s0 + i < SPLIT ? s0 + i : SPLIT - 1;
        u[i] = *reinterpret_cast<const V*>(p + s * plane);
      }
#pragma unroll
      for (int i = 0; i < kReduceBatch; ++i) {
        if (s0 + i < SPLIT) {
          t.x += u[i].x; t.y += u[i].y; t.z += u[i].z; t.w += u[i].w;
        }
      }
    }
    float4 v;
    if constexpr (INT)
      v = make_float4(static_cast<float>(t.x), static_cast<float>(t.y),
                      static_cast<float>(t.z), static_cast<float>(t.w));
    else
      v = t;
    if constexpr (!BLOCK) {
      const float sm = sa[m];
      const float4 s4 = *reinterpret_cast<const float4*>(sb + n);
      v.x = v.x * sm * s4.x;
      v.y = v.y * sm * s4.y;
      v.z = v.z * sm * s4.z;
      v.w = v.w * sm * s4.w;
    }
    store_bf16x4(y + static_cast<long>(m) * ldy + n, v.x, v.y, v.z, v.w);
  }
}

// ------------------------------------------------------- scratch --
// Split-K partials of the allocation-free entry point: one array per GPU,
// resident from the library's load on that device until the process ends.
// Host code never uses the array's name as an address (on the host it names
// a stand-in); it takes the device address from hipGetSymbolAddress, once
// per device, with that device current.
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

// ------------------------------------------------------ registry --
struct Variant {
  GemmConfig cfg;
  const void* fn[3];  // [scale kind]: per-token, blockwise, blockwise with power-of-two folding
  int threads;
  size_t lds;
};

// Variant names live as long as the process (the registry is never freed).
const char* keep_name(const std::string& n) {
  static std::mutex mu;
  static std::vector<std::unique_ptr<std::string>> names;
  std::lock_guard<std::mutex> lock(mu);
  names.push_back(std::make_unique<std::string>(n));
  return names.back()->c_str();
}

// SPLITK > 1: the K blocks are shared among SPLITK workgroup rows (fp32 or
// int32 partials in the workspace, then splitk_reduce_kernel); a run-time
// choice on the same kernel.
template <int BM, int BN, int WM, int WN, int ST, int E, int PRIO = 0, int SPLITK = 1>
Variant tiled_variant() {
  Variant v{};
  const char* name = keep_name(std::string(engine_prefix(E)) + "_tiled_m" +
                               std::to_string(BM) + "_n" + std::to_string(BN) + "_w" +
                               std::to_string(WM) + "x" + std::to_string(WN) + "_st" +
                               std::to_string(ST) + (PRIO ? "_p" : "") +
                               (SPLITK > 1 ? "_s" + std::to_string(SPLITK) : ""));
  v.cfg = GemmConfig{name, kTiled, E, BM, BN, WM, WN, 0, 0, 0, SPLITK};
  v.fn[0] =
      reinterpret_cast<const void*>(&gemm_tiled_kernel<BM, BN, WM, WN, ST, false, E, PRIO>);
  if constexpr (E != kEngineI8)
    v.fn[1] =
        reinterpret_cast<const void*>(&gemm_tiled_kernel<BM, BN, WM, WN, ST, true, E, PRIO>);
  // Power-of-two scales are folded into the widening only in the eight-wave
  // tiles, where that measured faster (the 32B prefill gate_up at M=8192:
  // 3776 us against 3997 us on the general path).  The four-wave tiles keep
  // the rotated loop, whose general path measured faster (the 32B qkv at
  // M=2048 on the 128x128 tile: 186 us against 197 us folded).
  if constexpr (E == kEngineF16 && WM * WN == 8)
    v.fn[2] = reinterpret_cast<const void*>(
        &gemm_tiled_kernel<BM, BN, WM, WN, ST, true, E, PRIO, true>);
  else
    v.fn[2] = v.fn[1];
  v.threads = WM * WN * 64;
  v.lds = TiledShape<BM, BN, WM, WN, ST, true>::kLds;  // the larger of the two
  return v;
}

template <int TMX, int RW, int WK, int J, int E>
Variant skinny_variant() {
  Variant v{};
  const char* name = keep_name(std::string(engine_prefix(E)) + "_skinny_t" +
                               std::to_string(TMX) + "_r" + std::to_string(RW) + "_k" +
                               std::to_string(WK) + "_j" + std::to_string(J));
  v.cfg = GemmConfig{name, kSkinny, E, 0, 0, 0, 0, TMX, RW, WK, J};
  v.fn[0] = reinterpret_cast<const void*>(&gemm_skinny_kernel<TMX, RW, WK, J, false, E>);
  if constexpr (E != kEngineI8)
    v.fn[1] = reinterpret_cast<const void*>(&gemm_skinny_kernel<TMX, RW, WK, J, true, E>);
  v.fn[2] = v.fn[1];  // no scale folding in the weight-streaming kernel
  v.threads = WK * 64;
  v.lds = static_cast<size_t>(WK) * RW * TMX * 64 * 16;
  return v;
}

// A kHybrid variant of two registered tiled variants: `a` unsplit over the
// columns that fill whole rounds of workgroups, `b` (split along K) over the
// rest.  Named after `a` with suffix _h<b's split>.
Variant hybrid_variant(const std::vector<Variant>& v, const char* a, const char* b) {
  int ia = -1, ib = -1;
  for (size_t i = 0; i < v.size(); ++i) {
    if (std::strcmp(v[i].cfg.name, a) == 0) ia = static_cast<int>(i);
    if (std::strcmp(v[i].cfg.name, b) == 0) ib = static_cast<int>(i);
  }
  Variant h{};
  if (ia < 0 || ib < 0) {  // not registered: a variant that fits no shape
    h.cfg = GemmConfig{keep_name(std::string(a) + "_h_unavailable"), kHybrid, kEngineF16,
                       0, 0, 0, 0, 0, 0, 0, 0, -1, -1};
    return h;
  }
  const GemmConfig& ca = v[ia].cfg;
  const GemmConfig& cb = v[ib].cfg;
  const char* name = keep_name(std::string(ca.name) + "_h" + std::to_string(cb.split));
  h.cfg = GemmConfig{name, kHybrid, ca.engine, ca.bm, ca.bn, ca.wm, ca.wn, 0, 0, 0, cb.split,
                     ia, ib};
  return h;
}

// FP8Q_NONCONFORMING_FP8_MFMA=1: also register the FP8-MFMA engine's variants.
bool nonconforming_fp8_requested() {
  const char* v = std::getenv("FP8Q_NONCONFORMING_FP8_MFMA");
  return v != nullptr && std::strcmp(v, "1") == 0;
}

std::vector<Variant>& registry() {
  static std::vector<Variant> r = [] {
    std::vector<Variant> v;
    v.push_back(tiled_variant<128, 128, 2, 2, 2, kEngineF16>());
    v.push_back(tiled_variant<128, 128, 2, 2, 3, kEngineF16>());
    v.push_back(tiled_variant<128, 128, 2, 2, 4, kEngineF16>());
    v.push_back(tiled_variant<128, 256, 2, 4, 3, kEngineF16>());
    v.push_back(tiled_variant<256, 128, 4, 2, 3, kEngineF16>());
    v.push_back(tiled_variant<64, 128, 1, 2, 3, kEngineF16>());
    v.push_back(tiled_variant<128, 128, 2, 2, 2, kEngineF16, 1>());
    v.push_back(tiled_variant<128, 256, 2, 4, 3, kEngineF16, 1>());
    v.push_back(tiled_variant<128, 128, 4, 2, 3, kEngineF16>());
    // small tiles of four waves: more workgroups for mid-size GEMMs
    v.push_back(tiled_variant<64, 64, 2, 2, 3, kEngineF16>());
    v.push_back(tiled_variant<64, 64, 2, 2, 3, kEngineF16, 0, 4>());
    v.push_back(tiled_variant<64, 64, 2, 2, 3, kEngineF16, 0, 8>());
    v.push_back(tiled_variant<64, 64, 2, 2, 3, kEngineF16, 0, 16>());
    v.push_back(tiled_variant<64, 128, 2, 2, 3, kEngineF16>());
    v.push_back(tiled_variant<64, 128, 2, 2, 3, kEngineF16, 0, 8>());
    v.push_back(tiled_variant<64, 128, 1, 2, 3, kEngineF16, 0, 4>());
    v.push_back(tiled_variant<64, 128, 1, 2, 3, kEngineF16, 0, 8>());
    v.push_back(tiled_variant<64, 128, 1, 2, 3, kEngineF16, 0, 16>());
    v.push_back(tiled_variant<128, 128, 2, 2, 2, kEngineF16, 0, 2>());
    v.push_back(tiled_variant<128, 128, 2, 2, 2, kEngineF16, 0, 4>());
    // whole rounds of unsplit 128x256 tiles, the remaining columns split 2 or
    // 4 ways on 128x128 tiles
    v.push_back(hybrid_variant(v, "f16_tiled_m128_n256_w2x4_st3", "f16_tiled_m128_n128_w2x2_st2_s2"));
    v.push_back(hybrid_variant(v, "f16_tiled_m128_n256_w2x4_st3", "f16_tiled_m128_n128_w2x2_st2_s4"));
    // the FP8-MFMA engine misses the accuracy contract (group truncation, see
    // kEngineF8): registered only on explicit request, for measurements
    if (nonconforming_fp8_requested()) {
      v.push_back(tiled_variant<128, 128, 2, 2, 2, kEngineF8>());
      v.push_back(tiled_variant<128, 128, 2, 2, 4, kEngineF8>());
      v.push_back(tiled_variant<128, 256, 2, 4, 3, kEngineF8>());
      v.push_back(tiled_variant<256, 128, 4, 2, 3, kEngineF8>());
    }
#define FP8Q_SKINNY(T, R, W, J) v.push_back(skinny_variant<T, R, W, J, kEngineF16>());
    FP8Q_SKINNY(1, 1, 4, 1)
    FP8Q_SKINNY(1, 2, 4, 1)
    FP8Q_SKINNY(1, 2, 4, 2)
    FP8Q_SKINNY(1, 4, 4, 2)
    FP8Q_SKINNY(2, 1, 4, 2)
    FP8Q_SKINNY(2, 2, 4, 2)
    FP8Q_SKINNY(2, 4, 4, 2)
    FP8Q_SKINNY(4, 1, 4, 1)
    FP8Q_SKINNY(1, 1, 4, 2)
    FP8Q_SKINNY(1, 1, 4, 4)
    FP8Q_SKINNY(1, 1, 4, 8)
    FP8Q_SKINNY(1, 2, 4, 4)
    FP8Q_SKINNY(1, 2, 4, 8)
    FP8Q_SKINNY(1, 4, 4, 4)
    FP8Q_SKINNY(1, 1, 8, 4)
    FP8Q_SKINNY(1, 2, 8, 4)
    FP8Q_SKINNY(2, 1, 4, 4)
    FP8Q_SKINNY(2, 1, 4, 8)
    FP8Q_SKINNY(2, 2, 4, 4)
    FP8Q_SKINNY(2, 2, 4, 8)
    FP8Q_SKINNY(2, 1, 8, 4)
    FP8Q_SKINNY(4, 1, 4, 2)
    FP8Q_SKINNY(4, 1, 4, 4)
    FP8Q_SKINNY(4, 2, 4, 2)
    FP8Q_SKINNY(4, 2, 4, 4)
    FP8Q_SKINNY(8, 1, 4, 2)
    FP8Q_SKINNY(8, 1, 4, 4)
    FP8Q_SKINNY(8, 2, 4, 2)
    // the whole of a long K in one launch (no split-K reduction): 8 or 16
    // waves with 6 to 12 blocks each
    FP8Q_SKINNY(1, 1, 8, 6)
    FP8Q_SKINNY(1, 1, 8, 12)
    FP8Q_SKINNY(1, 2, 8, 6)
    FP8Q_SKINNY(1, 1, 16, 6)
    FP8Q_SKINNY(2, 1, 8, 6)
#undef FP8Q_SKINNY
    // W8A8 INT8 (per-token x per-channel only)
    v.push_back(tiled_variant<128, 128, 2, 2, 2, kEngineI8>());
    v.push_back(tiled_variant<128, 128, 2, 2, 4, kEngineI8>());
    v.push_back(tiled_variant<128, 256, 2, 4, 3, kEngineI8>());
    v.push_back(tiled_variant<128, 128, 4, 2, 3, kEngineI8>());
    v.push_back(tiled_variant<64, 128, 1, 2, 3, kEngineI8>());
    v.push_back(tiled_variant<64, 64, 2, 2, 3, kEngineI8>());
    v.push_back(tiled_variant<64, 128, 2, 2, 3, kEngineI8>());
    v.push_back(tiled_variant<64, 128, 1, 2, 3, kEngineI8, 0, 4>());
    v.push_back(tiled_variant<128, 128, 2, 2, 2, kEngineI8, 0, 2>());
#define FP8Q_SKINNY_I8(T, R, W, J) v.push_back(skinny_variant<T, R, W, J, kEngineI8>());
    FP8Q_SKINNY_I8(1, 1, 4, 1)
    FP8Q_SKINNY_I8(1, 1, 4, 4)
    FP8Q_SKINNY_I8(1, 1, 4, 8)
    FP8Q_SKINNY_I8(1, 2, 4, 4)
    FP8Q_SKINNY_I8(1, 2, 4, 8)
    FP8Q_SKINNY_I8(1, 4, 4, 4)
    FP8Q_SKINNY_I8(1, 1, 8, 4)
    FP8Q_SKINNY_I8(1, 2, 8, 4)
    FP8Q_SKINNY_I8(2, 1, 4, 4)
    FP8Q_SKINNY_I8(2, 2, 4, 4)
    FP8Q_SKINNY_I8(4, 1, 4, 2)
    FP8Q_SKINNY_I8(4, 1, 4, 4)
    FP8Q_SKINNY_I8(4, 2, 4, 2)
    FP8Q_SKINNY_I8(8, 1, 4, 2)
    FP8Q_SKINNY_I8(8, 1, 4, 4)
    FP8Q_SKINNY_I8(8, 2, 4, 2)
#undef FP8Q_SKINNY_I8
    return v;
  }();
  return r;
}

// Raise the dynamic-LDS limit of each kernel once per device (above 64 KiB
// needs it).  A failure is not remembered, so the next launch retries and
// the launch itself reports the error.
void ensure_fn_lds(const void* fn, size_t lds) {
  if (lds <= 64 * 1024) return;
  static std::mutex mu;
  static std::vector<std::pair<int, const void*>> done;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& d : done)
    if (d.first == dev && d.second == fn) return;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(lds)) == hipSuccess)
    done.emplace_back(dev, fn);
}

void ensure_lds_attr(const Variant& v, int scales) { ensure_fn_lds(v.fn[scales], v.lds); }

}  // namespace

hipError_t scratch_workspace(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    ptrs[dev] = p;
  }
  *ptr = ptrs[dev];
  return hipSuccess;
}

int gemm_num_configs() { return static_cast<int>(registry().size()); }
const GemmConfig& gemm_config(int id) { return registry()[id].cfg; }

bool gemm_config_fits(int id, long M, long N, long K) {
  const GemmConfig& c = gemm_config(id);
  if (c.kind == kTiled) return N % c.bn == 0;
  if (c.kind == kHybrid) return c.part_b >= 0 && N % gemm_config(c.part_b).bn == 0;
  if (M > 16L * c.tm) return false;
  if (N % (16L * c.rw)) return false;
  return true;
}

// Workgroups along K for the skinny kernel: each covers wk*j K blocks.
int skinny_split(const GemmConfig& c, long K) {
  const long kb = K / kBK;
  const long per = static_cast<long>(c.wk) * c.split;
  return static_cast<int>((kb + per - 1) / per);
}

// Workgroup rows along K for a tiled variant: c.split, reduced so that none
// is empty.
int tiled_split(const GemmConfig& c, long K) {
  const long kb = K / kBK;
  if (c.split <= 1 || kb <= 1) return 1;
  const long per = (kb + c.split - 1) / c.split;
  return static_cast<int>((kb + per - 1) / per);
}

int split_of(const GemmConfig& c, long K) {
  return c.kind == kSkinny ? skinny_split(c, K) : tiled_split(c, K);
}

// Compute units of the current device, cached per device; 256 (an MI355X)
// where no device answers (a workspace-size query on a host without a GPU).
int device_cus() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cus[kMaxDev];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
    (void)hipGetLastError();
    return 256;
  }
  int c = cus[dev].load(std::memory_order_relaxed);
  if (c > 0) return c;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      c <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  cus[dev].store(c, std::memory_order_relaxed);
  return c;
}

// Column split of a kHybrid launch: part_a takes na columns, whole bn-wide
// tiles of every token-tile row that together fill whole rounds of resident
// workgroups; part_b the nt remaining columns (a multiple of its tile width,
// as N is).  na = 0 when the tiles do not fill one round; nt = 0 when they
// fill whole rounds exactly.
struct ColumnSplit {
  int na, nt;
};
ColumnSplit hybrid_columns(const GemmConfig& c, long M, long N) {
  const Variant& va = registry()[c.part_a];
  // part_a's workgroups per CU: bounded by its LDS ring (160 KiB per CU) and
  // by two waves per SIMD (eight per CU)
  long per_cu = (160L * 1024) / static_cast<long>(va.lds);
  const long by_waves = 8L * 64 / va.threads;
  if (by_waves < per_cu) per_cu = by_waves;
  if (per_cu < 1) per_cu = 1;
  const long slots = per_cu * device_cus();
  const long rows = (M + c.bm - 1) / c.bm, cols = N / c.bn;
  const long whole = (rows * cols / slots) * slots;
  long na_cols = whole / rows;
  if (na_cols > cols) na_cols = cols;
  const long na = na_cols * c.bn;
  return {static_cast<int>(na), static_cast<int>(N - na)};
}

size_t gemm_workspace_bytes(int id, long M, long N, long K) {
  const GemmConfig& c = gemm_config(id);
  if (c.kind == kHybrid) {
    if (c.part_a < 0 || c.part_b < 0) return 0;
    const ColumnSplit cs = hybrid_columns(c, M, N);
    return cs.nt > 0 ? gemm_workspace_bytes(c.part_b, M, cs.nt, K) : 0;
  }
  const int split = split_of(c, K);
  if (split <= 1) return 0;
  return static_cast<size_t>(split) * M * N * sizeof(float);
}

// One launch of a tiled or skinny variant over N output columns whose rows
// lie ldy elements apart in y (then the split-K reduction, if any).
hipError_t launch_one(const Variant& v, int scales, uint16_t* y, const uint8_t* a,
                      const float* sa, const uint8_t* b, const float* sb, int M, int N, int K,
                      int ldy, void* ws, hipStream_t st) {
  const int bw = scales;
  const bool blockwise = scales != kScalesPerToken;
  if (v.fn[bw] == nullptr) return hipErrorInvalidDeviceFunction;
  ensure_lds_attr(v, bw);
  int split = split_of(v.cfg, K);
  float* wsf = static_cast<float*>(ws);
  {
    void* args[] = {&y, &wsf, &a, &sa, &b, &sb, &M, &N, &K, &split, &ldy};
    const dim3 grid = v.cfg.kind == kTiled
                          ? dim3((N / v.cfg.bn) * ((M + v.cfg.bm - 1) / v.cfg.bm), split)
                          : dim3(N / (16 * v.cfg.rw), split);
    hipError_t e0 = hipLaunchKernel(v.fn[bw], grid, dim3(v.threads), args, v.lds, st);
    if (e0 != hipSuccess) return e0;
  }
  if (split <= 1) return hipSuccess;
  const long total = static_cast<long>(M) * (N / 4);
  long blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blockwise)
    hipLaunchKernelGGL((splitk_reduce_kernel<true, false>), dim3(blocks), dim3(256), 0, st, y,
                       wsf, sa, sb, M, N, split, ldy);
  else if (v.cfg.engine == kEngineI8)
    hipLaunchKernelGGL((splitk_reduce_kernel<false, true>), dim3(blocks), dim3(256), 0, st, y,
                       wsf, sa, sb, M, N, split, ldy);
  else
    hipLaunchKernelGGL((splitk_reduce_kernel<false, false>), dim3(blocks), dim3(256), 0, st, y,
                       wsf, sa, sb, M, N, split, ldy);
  return hipGetLastError();
}

hipError_t launch_gemm(int id, int scales, uint16_t* y, const uint8_t* a, const float* sa,
                       const uint8_t* b, const float* sb, int M, int N, int K, void* ws,
                       hipStream_t st) {
  const Variant& v = registry()[id];
  if (v.cfg.kind != kHybrid) return launch_one(v, scales, y, a, sa, b, sb, M, N, K, N, ws, st);
  if (v.cfg.part_a < 0 || v.cfg.part_b < 0) return hipErrorInvalidDeviceFunction;
  // part_a on columns [0, na), part_b on [na, N): the weight rows, their
  // scales and the output columns of each range, rows of y N apart
  const ColumnSplit cs = hybrid_columns(v.cfg, M, N);
  if (cs.na > 0) {
    const hipError_t e =
        launch_one(registry()[v.cfg.part_a], scales, y, a, sa, b, sb, M, cs.na, K, N, nullptr, st);
    if (e != hipSuccess || cs.nt == 0) return e;
  }
  const long kb = K / kBK;
  const float* sb_t = scales == kScalesPerToken ? sb + cs.na : sb + (cs.na / 128) * kb;
  return launch_one(registry()[v.cfg.part_b], scales, y + cs.na, a, sa,
                    b + static_cast<long>(cs.na) * K, sb_t, M, cs.nt, K, N, ws, st);
}

hipError_t launch_gemm_silu_quant(uint8_t* q, float* scale, const uint8_t* a, const float* sa,
                                  const uint8_t* b, const float* sb, int M, int N, int K,
                                  hipStream_t st) {
  constexpr int kBM = 128, kBN = 256, kWM = 2, kWN = 4, kST = 3;
  const void* fn = reinterpret_cast<const void*>(
      &gemm_tiled_kernel<kBM, kBN, kWM, kWN, kST, true, kEngineF16, 0, false, true>);
  const size_t lds = TiledShape<kBM, kBN, kWM, kWN, kST, true>::kLds;
  ensure_fn_lds(fn, lds);
  uint16_t* y = reinterpret_cast<uint16_t*>(q);
  int split = 1, ldy = N;  // (the fused epilogue writes q and scale by D)
  void* args[] = {&y, &scale, &a, &sa, &b, &sb, &M, &N, &K, &split, &ldy};
  const dim3 grid((N / kBN) * ((M + kBM - 1) / kBM), 1);
  return hipLaunchKernel(fn, grid, dim3(kWM * kWN * 64), args, lds, st);
}

}  // namespace fp8q
