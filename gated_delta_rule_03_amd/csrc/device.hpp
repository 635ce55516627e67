// Device-side helpers shared by the libgdn kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kWave = 64;

// log2(alpha) is clamped here before the chunk-local prefix sum: alpha = 0
// stays finite in the log domain, and 2^(-288 * 64) still flushes to 0.
constexpr float kLog2Floor = -288.0f;

// ---------------------------------------------------------------------------
// Element types.  bf16 is carried as raw 16-bit patterns (uint16_t).
// ---------------------------------------------------------------------------
typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// log2 alpha, clamped below at kLog2Floor; alpha = 0 hits the floor, NaN and
// negative gates propagate as NaN.
__device__ __forceinline__ float clamped_log2(float a) {
  if (a > 0.0f) return fmaxf(log2f(a), kLog2Floor);
  if (a == 0.0f) return kLog2Floor;
  return __builtin_nanf("");
}

// 2^x with the hardware v_exp_f32 (about 1 ulp; results below the normal
// range flush to zero).  The chunk kernels only take 2^x of non-positive
// log-gate differences, where a flushed tiny factor is as good as exact.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float(uint32_t(x) << 16); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  __bf16 h = static_cast<__bf16>(x);  // round to nearest even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(bf16_t, h);
}

// Four consecutive elements starting at p, widened to float (p must be aligned
// to four elements).
__device__ __forceinline__ float4 load4_f32(const float *p) {
  return *reinterpret_cast<const float4 *>(p);
}
__device__ __forceinline__ float4 load4_f32(const bf16_t *p) {
  uint2 u = *reinterpret_cast<const uint2 *>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}

// ---------------------------------------------------------------------------
// MFMA operand fragments.
//
// A "K32 fragment" holds one 16 x 32 operand tile of a 16x16 output tile:
// each lane holds 8 elements.  For an A operand lane l holds row (l & 15); for
// a B operand lane l holds column (l & 15).  Element j of lane l stands for
// the contraction index
//     kappa(l, j) = 16 * (j >> 2) + 4 * (l >> 4) + (j & 3)
// A and B use the same kappa, so any assignment of kappa to the hardware's
// k-slots gives the same sum.  This kappa is chosen so that two vertically
// stacked 16x16 accumulator tiles (lane l holds rows 4 * (l >> 4) + i,
// i = 0..3, of column l & 15) ARE a B fragment: accumulators feed the next
// product without a trip through LDS.
//
// bf16: one v_mfma_f32_16x16x32_bf16 per fragment pair.
// f32:  eight v_mfma_f32_16x16x4_f32, element j in the j-th.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int kappa(int lane, int j) {
  return 16 * (j >> 2) + 4 * (lane >> 4) + (j & 3);
}

template <typename T> struct Frag;

template <> struct Frag<bf16_t> {
  bf16x8_t v;
  __device__ __forceinline__ void zero() {
    for (int j = 0; j < 8; ++j) v[j] = static_cast<__bf16>(0.0f);
  }
  __device__ __forceinline__ void set(int j, float x) { v[j] = static_cast<__bf16>(x); }
  __device__ __forceinline__ float get(int j) const { return static_cast<float>(v[j]); }
};

template <> struct Frag<float> {
  float v[8];
  __device__ __forceinline__ void zero() {
    for (int j = 0; j < 8; ++j) v[j] = 0.0f;
  }
  __device__ __forceinline__ void set(int j, float x) { v[j] = x; }
  __device__ __forceinline__ float get(int j) const { return v[j]; }
};

__device__ __forceinline__ f32x4_t mfma(const Frag<bf16_t> &a, const Frag<bf16_t> &b,
                                        f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma(const Frag<float> &a, const Frag<float> &b, f32x4_t c) {
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
  return c;
}

// XCD-aware block numbering for the per-(unit, column block) kernels: the
// launch hands out block ids round-robin over the 8 XCDs (bid % 8), so giving
// all column blocks of a unit the same bid % 8 puts them on one XCD, where
// they share that XCD's L2 copy of the unit's k, q and v.  Blocks come in
// groups of 8 units x n_colblk column blocks.
__device__ __forceinline__ void decode_block(int bid, int n_colblk, int &u, int &cb) {
  const int per_group = 8 * n_colblk;
  const int grp = bid / per_group, rem = bid - grp * per_group;
  cb = rem >> 3;
  u = grp * 8 + (rem & 7);
}

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}; }

// B fragment from two stacked accumulator tiles (rows 0-15 and 16-31 of a
// 32-deep contraction block).
template <typename T>
__device__ __forceinline__ Frag<T> frag_from_acc(const f32x4_t &lo, const f32x4_t &hi) {
  Frag<T> f;
  for (int i = 0; i < 4; ++i) {
    f.set(i, lo[i]);
    f.set(4 + i, hi[i]);
  }
  return f;
}

// Row fragment of a row-major matrix whose contraction index runs along the
// row: lane l reads row `row` (already including l & 15), elements
// k0 + kappa(l, j).  Rows >= n_rows and columns >= n_cols read as zero.
// `n_cols` must be a multiple of 16 (then each group of four is all in or all
// out of range).
template <typename T>
__device__ __forceinline__ Frag<T> load_row_frag(const T *base, int64_t row_stride, int row,
                                                 int n_rows, int k0, int n_cols, int lane) {
  Frag<T> f;
  const int c0 = k0 + 4 * (lane >> 4);
  const bool row_ok = row < n_rows;
  const T *p = base + int64_t(row) * row_stride;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = c0 + 16 * h;
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row_ok && c < n_cols) x = load4_f32(p + c);
    f.set(4 * h + 0, x.x);
    f.set(4 * h + 1, x.y);
    f.set(4 * h + 2, x.z);
    f.set(4 * h + 3, x.w);
  }
  return f;
}

// Whole-fragment load/store for fragments kept in workspace memory in
// fragment order: fragment f of a tile set occupies 64 lanes x 8 elements.
__device__ __forceinline__ Frag<bf16_t> load_frag(const bf16_t *p, int lane) {
  Frag<bf16_t> f;
  f.v = *reinterpret_cast<const bf16x8_t *>(p + 8 * lane);
  return f;
}
__device__ __forceinline__ Frag<float> load_frag(const float *p, int lane) {
  Frag<float> f;
  const float4 *q = reinterpret_cast<const float4 *>(p + 8 * lane);
  float4 a = q[0], b = q[1];
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
  return f;
}
__device__ __forceinline__ void store_frag(bf16_t *p, int lane, const Frag<bf16_t> &f) {
  *reinterpret_cast<bf16x8_t *>(p + 8 * lane) = f.v;
}
__device__ __forceinline__ void store_frag(float *p, int lane, const Frag<float> &f) {
  float4 *q = reinterpret_cast<float4 *>(p + 8 * lane);
  q[0] = make_float4(f.v[0], f.v[1], f.v[2], f.v[3]);
  q[1] = make_float4(f.v[4], f.v[5], f.v[6], f.v[7]);
}

// ---------------------------------------------------------------------------
// Sequence / chunk geometry.  A uniform batch (cu_seqlens == nullptr) is
// B sequences of T tokens laid end to end on the flattened B*T token axis.
// ---------------------------------------------------------------------------
struct SeqGeom {
  const int32_t *cu_seqlens;  // device; nullptr for a uniform batch
  const int32_t *chunk_off;   // device, n_seqs + 1 prefix sums of chunk counts (packed only)
  const int32_t *seq_order;   // device, sequences by chunk count, most first (packed only)
  int32_t n_seqs;
  int32_t T;                  // tokens per sequence (uniform) / total tokens (packed)
  int32_t chunk;
  int32_t chunks_per_seq;     // uniform only: ceil(T / chunk)
  int32_t n_slots;            // chunk slots in the workspace; chunks beyond are skipped

  // Offsets are clamped into [0, T] and made non-decreasing, so a malformed
  // cu_seqlens yields empty sequences rather than out-of-range accesses.
  __device__ __forceinline__ void seq_bounds(int s, int &start, int &end) const {
    if (cu_seqlens) {
      start = min(max(cu_seqlens[s], 0), T);
      end = min(max(cu_seqlens[s + 1], start), T);
    } else {
      start = s * T;
      end = start + T;
    }
  }
  // The i-th sequence in scheduling order: packed batches are walked longest
  // first, so the longest sequential scans start in the first wave of blocks.
  __device__ __forceinline__ int ordered(int i) const { return seq_order ? seq_order[i] : i; }
  __device__ __forceinline__ int first_chunk(int s) const {
    return cu_seqlens ? chunk_off[s] : s * chunks_per_seq;
  }
  __device__ __forceinline__ int total_chunks() const {
    return min(cu_seqlens ? chunk_off[n_seqs] : n_seqs * chunks_per_seq, n_slots);
  }
  // Global chunk index -> (sequence, first token, token count).  Returns false
  // for indices past the last chunk.
  __device__ __forceinline__ bool locate(int c, int &s, int &tok0, int &len) const {
    if (c >= total_chunks()) return false;
    if (cu_seqlens) {
      int lo = 0, hi = n_seqs - 1;  // largest s with chunk_off[s] <= c
      while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (chunk_off[mid] <= c) lo = mid; else hi = mid - 1;
      }
      s = lo;
      int start, end;
      seq_bounds(s, start, end);
      tok0 = start + (c - chunk_off[s]) * chunk;
      len = min(chunk, end - tok0);
    } else {
      s = c / chunks_per_seq;
      int j = c - s * chunks_per_seq;
      tok0 = s * T + j * chunk;
      len = min(chunk, T - j * chunk);
    }
    return true;
  }
};

}  // namespace gdn
