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
// Waits until at most N of this wave's vector memory operations are
// outstanding (s_waitcnt vmcnt(N); expcnt and lgkmcnt untouched).  Loads
// complete in issue order, so this leaves only the N newest loads in flight.
template <int N> __device__ __forceinline__ void wait_vmem_upto() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without the memory fence of __syncthreads (whose release
// fence waits for every outstanding global load, including prefetches).  The
// caller orders LDS itself: its own LDS-bound loads by wait_vmem[_upto], and
// its LDS reads are complete because their results have been consumed.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | (0x7 << 4) | (0x0 << 8) | ((0x3F >> 4) << 14));
  __builtin_amdgcn_s_barrier();
}

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

// ---------------------------------------------------------------------------
// Raw LDS access by byte offset (address space 3, so the compiler emits ds_*
// instructions and folds constant offsets into them).
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) char lds_t;
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ lds_t *lds_ptr(void *generic_shared) {
  return (lds_t *)(generic_shared);
}
template <typename V> __device__ __forceinline__ V lds_load(const lds_t *p) {
  return *(const __attribute__((address_space(3))) V *)(p);
}
template <typename V> __device__ __forceinline__ void lds_store(lds_t *p, V v) {
  *(__attribute__((address_space(3))) V *)(p) = v;
}
// ds_read_b64_tr_b16: inside each group of 16 lanes, lane i receives for
// j = 0..3 the (i mod 4)-th 16-bit element of the 8 bytes addressed by lane
// (i / 4) + 4 j of the group.  Reads 4 rows x 16 columns of a row-major bf16
// matrix as four values of one column per lane.
__device__ __forceinline__ bf16x4_t lds_read_tr16(const lds_t *p) {
  s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(p));
  return __builtin_bit_cast(bf16x4_t, v);
}
__device__ __forceinline__ Frag<bf16_t> frag_cat(bf16x4_t lo, bf16x4_t hi) {
  Frag<bf16_t> f;
  f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}

// Transposed fragment of a swizzled row tile: lane l holds column
// m = 16 rm + (l & 15) (an A-operand row of the transpose) and elements
// j = 0..7 stand for tile rows 32 kk + kappa(l, j).  With the row swizzle the
// 64 lanes of each 2-byte read spread over 32 banks without conflicts.
__device__ __forceinline__ Frag<bf16_t> rowtile_colfrag(const bf16_t *tile, int rm, int kk,
                                                        int lane) {
  const int m = 16 * rm + (lane & 15);
  Frag<bf16_t> f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = 32 * kk + kappa(lane, j);
    f.v[j] = __builtin_bit_cast(__bf16, tile[rowtile_off(i, m)]);
  }
  return f;
}

}  // namespace gdn
