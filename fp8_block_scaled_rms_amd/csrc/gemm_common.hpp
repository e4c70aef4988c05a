// Device helpers shared by the tiled GEMM kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8q_common.hpp"

namespace fp8q {
namespace tile {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_ptr)p));
}

// 16-byte-chunk swizzle of a 128-byte LDS row: rows 0..7 use distinct chunks
// and rows of equal parity within 16 also do, so a 16-lane fragment read is
// free of bank conflicts for 32 or 64 banks.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ void store_bf16x4(uint16_t* y, float a, float b, float c, float d) {
  uint2 v;
  v.x = pack_bf16x2(a, b);
  v.y = pack_bf16x2(c, d);
  *reinterpret_cast<uint2*>(y) = v;
}

// 32 bytes at byte offset `off` of a buffer as one fragment (two 16-byte
// loads); zeros where the offset is outside the buffer.
__device__ __forceinline__ v8i load_frag_buffer(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const v4u lo = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0);
  const v4u hi = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off + 16), 0, 0);
  v8i f;
  f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
  f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
  return f;
}

// Workgroup -> output tile.  Workgroups are dispatched round-robin over the
// 8 XCDs (workgroup b runs on XCD b % 8) and each XCD has its own L2, so
// first every XCD is given one contiguous range of logical tile ids; inside
// that range tiles are walked in groups of kGroupRows token-tile rows, column
// by column, so the workgroups resident at the same time share a few token
// tiles and a few weight tiles in L2 instead of streaming whole operands.
// (Cutting the tile grid into per-XCD rectangles that minimise the operand
// bytes each XCD fetches measured no faster on the Qwen3 shapes: the 256 MB
// last-level cache serves the repeated weight reads.)
constexpr int kXcds = 8;
constexpr int kGroupRows = 8;

__device__ __forceinline__ void tile_coords(int b, int tiles_m, int tiles_n, int& tn, int& tm) {
  const int ntiles = tiles_m * tiles_n;
  const int q = ntiles / kXcds, r = ntiles % kXcds;
  const int xcd = b % kXcds, local = b / kXcds;
  const int logical = xcd * q + (xcd < r ? xcd : r) + local;
  const int group_tiles = kGroupRows * tiles_n;
  const int group = logical / group_tiles;
  const int first_m = group * kGroupRows;
  const int rows = (tiles_m - first_m < kGroupRows) ? tiles_m - first_m : kGroupRows;
  const int in_group = logical - group * group_tiles;
  tm = first_m + in_group % rows;
  tn = in_group / rows;
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace tile
}  // namespace fp8q
