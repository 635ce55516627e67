// LDS staging for the bf16 chunk kernels (gfx950).
//
// Operand tiles move from global memory to LDS with global_load_lds_dwordx4:
// each lane sends 16 bytes from its own global address straight into LDS at
// base + 16 * lane, without passing through registers, so a chunk's operands
// can be fetched while the previous chunk is being computed.
//
// Row tiles (64 token rows x 128 bf16, 256 B per row) are stored with their
// 16-byte chunks XOR-swizzled by the row (physical chunk = chunk ^ (row & 15)),
// so that the 16 rows an MFMA fragment read touches fall in different banks.
#pragma once

#include "device.hpp"

namespace gdn {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// 16 bytes per lane: global src (per lane) -> LDS wave_base + 16 * lane.
// `wave_base` must be the same for every lane of the wave.
__device__ __forceinline__ void copy16_to_lds(const void *src, void *wave_base) {
  __builtin_amdgcn_global_load_lds((glb_void_t *)(src), (lds_void_t *)(wave_base), 16, 0, 0);
}
// 4 bytes per lane: global src -> LDS wave_base + 4 * lane.
__device__ __forceinline__ void copy4_to_lds(const void *src, void *wave_base) {
  __builtin_amdgcn_global_load_lds((glb_void_t *)(src), (lds_void_t *)(wave_base), 4, 0, 0);
}
// Waits for this wave's outstanding global loads (including LDS-bound ones).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0); }

// Element offset of (row, col) in a swizzled 64 x 128 bf16 row tile.
__device__ __forceinline__ int rowtile_off(int row, int col) {
  return row * 128 + 8 * ((col >> 3) ^ (row & 15)) + (col & 7);
}

// Stages rows [0, 64) of a 128-wide bf16 row-major matrix (row stride
// `stride` elements) into a swizzled row tile with 16 instructions.  Rows at
// or beyond `len` repeat row len - 1 (in-bounds, finite filler that the chunk
// algebra multiplies by exact zeros).  `inst0`/`ninst` select which of the 16
// one-KiB pieces this wave issues.
__device__ __forceinline__ void stage_rowtile(bf16_t *tile, const bf16_t *src, int64_t stride,
                                              int len, int lane, int inst0, int ninst) {
  for (int i = inst0; i < inst0 + ninst; ++i) {
    const int row = 4 * i + (lane >> 4);
    const int phys = lane & 15;
    const int logical = phys ^ (row & 15);
    const int r = row < len ? row : len - 1;
    copy16_to_lds(src + int64_t(r) * stride + 8 * logical, tile + 512 * i);
  }
}

// A (or B) fragment of rows [16 rt, 16 rt + 16), contraction columns
// [32 kk, 32 kk + 32), from a swizzled row tile, in the kappa convention.
__device__ __forceinline__ Frag<bf16_t> rowtile_frag(const bf16_t *tile, int rt, int kk,
                                                     int lane) {
  const int row = 16 * rt + (lane & 15);
  const int g = lane >> 4;
  const int c0 = 32 * kk + 4 * g;        // elements j = 0..3
  const int c1 = 32 * kk + 16 + 4 * g;   // elements j = 4..7
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  const bf16x4_t lo = *reinterpret_cast<const bf16x4_t *>(tile + rowtile_off(row, c0));
  const bf16x4_t hi = *reinterpret_cast<const bf16x4_t *>(tile + rowtile_off(row, c1));
  Frag<bf16_t> f;
  f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}

}  // namespace gdn
