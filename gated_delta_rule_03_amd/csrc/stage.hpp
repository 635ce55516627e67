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
#include "tile_index.hpp"

namespace gdn {

typedef __attribute__((address_space(3))) char lds_t;

__device__ __forceinline__ lds_t *lds_ptr(void *generic_shared) {
  return (lds_t *)(generic_shared);
}

// 16 bytes per lane from global `base + voff` (base wave-uniform, voff per
// lane) into LDS at dst + 16 * lane (dst wave-uniform).  Issued as inline
// assembly on purpose: the compiler then adds no waits of its own for these
// copies, and every user orders them explicitly (counted vmcnt waits followed
// by a barrier) -- the compiler's own rule would wait for every in-flight
// prefetch before any LDS read it cannot prove disjoint.
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, lds_t *dst) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"((uint32_t)(uintptr_t)dst), "v"(voff), "s"(base)
               : "memory", "m0");
}
// Buffer resource (V#) for a raw byte buffer of `bytes` bytes at `base`
// (wave-uniform): stride 0, so a lane's access is out of range, and reads as
// zero, once its offset + size exceeds `bytes`.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t buffer_rsrc(const void *base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  return i32x4_t{int(uint32_t(p)), int(uint32_t(p >> 32) & 0xffff), int(bytes), 0x00020000};
}

// Bounds-checked form of dma16: 16 bytes per lane from byte offset `voff` of
// the buffer `rsrc` into LDS at dst + 16 * lane; lanes whose 16 bytes are not
// wholly inside the buffer write zeros.  Same ordering rules as dma16.
__device__ __forceinline__ void dma16_buf(i32x4_t rsrc, uint32_t voff, lds_t *dst) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"((uint32_t)(uintptr_t)dst), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// dma16_buf with the nontemporal hint, for data that is read exactly once:
// its lines leave the L2 first, ahead of tiles that other blocks still read.
__device__ __forceinline__ void dma16_buf_nt(i32x4_t rsrc, uint32_t voff, lds_t *dst) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :
               : "s"((uint32_t)(uintptr_t)dst), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// Bounds-checked 4-byte-per-lane form: lane l's 4 bytes land at dst + 4 * l.
__device__ __forceinline__ void dma4_buf(i32x4_t rsrc, uint32_t voff, lds_t *dst) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"((uint32_t)(uintptr_t)dst), "v"(voff), "s"(rsrc)
               : "memory", "m0");
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


// Stages rows [0, 64) of a 128-wide bf16 row-major matrix (row stride
// `stride` elements) into a swizzled row tile (copies as in tile_index.hpp).
// Rows at or beyond `len` repeat row len - 1.  `inst0`/`ninst` select which
// of the 16 copies this wave issues.
__device__ __forceinline__ void stage_rowtile(lds_t *tile, const bf16_t *src, int64_t stride,
                                              int len, int lane, int inst0, int ninst) {
  for (int i = inst0; i < inst0 + ninst; ++i)
    dma16(src, uint32_t(rowtile_copy_src(i, lane, len, stride)), tile + 1024 * i);
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
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

template <typename V> __device__ __forceinline__ V lds_load(const lds_t *p) {
  return *(const __attribute__((address_space(3))) V *)(p);
}
// Volatile form: never merged with a neighbouring read into a paired
// ds_read2 (whose results would then have to be moved apart again to form
// MFMA operands).
template <typename V> __device__ __forceinline__ V lds_load_single(const lds_t *p) {
  return *(const volatile __attribute__((address_space(3))) V *)(p);
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

// Inclusive prefix sum over the 64 lanes of a wave: shifts within rows of 16
// lanes, then the last lane of rows 0 and 2 into rows 1 and 3, then lane 31
// into rows 2 and 3 (DPP row_shr and row_bcast).
__device__ __forceinline__ float wave_prefix_sum(float x) {
#define GDN_ADD_DPP(ctrl, rows, bound) \
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, rows, 0xf, bound))
  GDN_ADD_DPP(0x111, 0xf, true);   // row_shr:1 (lanes without a source add 0)
  GDN_ADD_DPP(0x112, 0xf, true);   // row_shr:2
  GDN_ADD_DPP(0x114, 0xf, true);   // row_shr:4
  GDN_ADD_DPP(0x118, 0xf, true);   // row_shr:8
  GDN_ADD_DPP(0x142, 0xa, false);  // row_bcast:15 into rows 1 and 3
  GDN_ADD_DPP(0x143, 0xc, false);  // row_bcast:31 into rows 2 and 3
#undef GDN_ADD_DPP
  return x;
}

// 16 x 16 x 16 fp32 product, acc += X Y: `xr` holds X[r][4g .. 4g + 3] and
// `yt` holds Y^T[r][4g .. 4g + 3] (r = lane mod 16, g = lane / 16); the
// result is in accumulator layout (rows 4g + e, column r).  Contraction slot
// j of each of the four MFMAs is k = 4g + j.
__device__ __forceinline__ f32x4_t mm16(f32x4_t xr, f32x4_t yt, f32x4_t acc) {
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xr[j], yt[j], acc, 0, 0, 0);
  return acc;
}

// The same 16 x 16 x 16 product from bf16 MFMAs with each fp32 operand split
// as x = hi + lo (hi = bf16(x), lo = bf16(x - hi)): hi*hi + lo*hi + hi*lo
// carries about 16 significant bits (the dropped lo*lo term is ~2^-16
// relative).  One 16 x 16 x 32 MFMA takes [x_hi | x_lo] against
// [y_hi ; y_hi] (the operand's contraction index 4 g + j sits in elements
// j and 4 + j of the kappa fragment), a second [x_hi | x_lo] against
// [y_lo ; 0].
struct Split16 {
  bf16x4_t hi, lo;
};
__device__ __forceinline__ Split16 split16(f32x4_t x) {
  Split16 s;
  s.hi = __builtin_convertvector(x, bf16x4_t);
  s.lo = __builtin_convertvector(x - __builtin_convertvector(s.hi, f32x4_t), bf16x4_t);
  return s;
}
__device__ __forceinline__ f32x4_t mm16x3(const Split16 &x, const Split16 &y, f32x4_t acc) {
  const bf16x4_t z = {0, 0, 0, 0};
  const bf16x8_t a = __builtin_shufflevector(x.hi, x.lo, 0, 1, 2, 3, 4, 5, 6, 7);
  const bf16x8_t b1 = __builtin_shufflevector(y.hi, y.hi, 0, 1, 2, 3, 4, 5, 6, 7);
  const bf16x8_t b2 = __builtin_shufflevector(y.lo, z, 0, 1, 2, 3, 4, 5, 6, 7);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b1, acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b2, acc, 0, 0, 0);
}

}  // namespace gdn
