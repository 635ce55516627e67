// The GDN block's steps on either side of the recurrence, as two fused
// kernels ("Linear attention", section "A naive PyTorch implementation",
// describes the steps; projections are plain matrix products and are not
// part of this library).
//
// Prologue, from the projections q_raw, k_raw, v_raw and the gate inputs:
//   causal depthwise convolution of width 4 on every channel (tokens before
//   a sequence's start are zeros) + bias, then SiLU;
//   q and k scaled to unit length per head (q then times q_scale), v
//   RMS-normalised per head (times a weight);
//   alpha = exp(-exp(log A[h]) softplus(a)), beta = sigmoid(b).
// Epilogue, from the recurrence's output o and the output gate's
// projection g: RMS normalisation of each head's output, times a weight,
// times SiLU(g).
//
// Both are HBM-bound: each reads its inputs once and writes its outputs
// once, and keeps many loads in flight (a wave that waited for one row at a
// time would leave HBM mostly idle).  Both lay a (token, head) row over one
// DPP row of 16 lanes, d / 16 channels per lane (16 bytes for bf16 at
// d = 128), so a row's sum of squares is a DPP sum and one load instruction
// moves four rows, adjacent in memory.
// Prologue: a wave takes 64 tokens of four heads of one tensor and streams
// their raw rows through a ring of 16 register sets, loading each row 13
// tokens before it is needed; waves over value heads also form alpha and
// beta.  Epilogue: 16 rows per wave, every load issued before any
// arithmetic.
#include "launch.hpp"

namespace gdn {

template <typename T>
struct PrologueArgs {
  const T *raw[3];  // q_raw, k_raw, v_raw
  T *out[3];        // q, k, v
  const float *conv[3], *bias[3];
  const float *a_raw, *b_raw, *log_A, *norm_w;
  float *alpha, *beta;
  const int32_t *cu_seqlens;
  int64_t n_tokens;  // B * T
  int32_t seq_len, n_seqs, H_qk, H_v;  // seq_len: tokens per sequence (uniform)
  float eps, q_scale;
};

// x plus x of another lane of the same row of 16 lanes, chosen by a DPP
// control word (quad_perm or row_ror); every lane takes part.
template <int CTRL> __device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
// Sum over each row of 16 lanes, in every lane of the row: swap neighbours,
// swap pairs, then rotate the row by 4 and by 8.
__device__ __forceinline__ float row16_sum(float x) {
  x = dpp_add<0xb1>(x);   // quad_perm [1, 0, 3, 2]
  x = dpp_add<0x4e>(x);   // quad_perm [2, 3, 0, 1]
  x = dpp_add<0x124>(x);  // row_ror 4
  return dpp_add<0x128>(x);  // row_ror 8
}

// log(1 + e^a) without overflow
__device__ __forceinline__ float softplus_f(float a) { return a > 0.0f ? a + log1pf(expf(-a)) : log1pf(expf(a)); }

// SiLU with the hardware exp2 and reciprocal (about 2 ulp).
__device__ __forceinline__ float silu_fast(float y) {
  return y * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * y));
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
constexpr int kNontemporal = 2;  // buffer access cache policy: nontemporal
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// E consecutive elements of type T held as raw 32-bit words: one lane's
// share of a (token, head) row.  Loads carry the nontemporal hint (the
// block's inputs stream through once; plain stores measured faster than
// nontemporal ones).  Accesses need the row's base 16-byte aligned, which the
// entry points check.
template <typename T, int E>
struct Row {
  static constexpr int kBytes = E * int(sizeof(T));
  static constexpr int W = kBytes < 4 ? 1 : kBytes / 4;
  uint32_t w[W];

  __device__ __forceinline__ void load(const T *p) {
    if constexpr (W % 4 == 0) {
#pragma unroll
      for (int i = 0; i < W / 4; ++i) {
        const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p) + i);
        w[4 * i] = v.x, w[4 * i + 1] = v.y, w[4 * i + 2] = v.z, w[4 * i + 3] = v.w;
      }
    } else if constexpr (W == 2) {
      const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
      w[0] = v.x, w[1] = v.y;
    } else if constexpr (kBytes == 4) {
      w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
    } else {
      w[0] = *reinterpret_cast<const uint16_t *>(p);
    }
  }
  // The same through a buffer resource at byte offset voff (per lane) + soff
  // (wave-uniform).  With voff out of the resource's range, a load reads
  // zeros and a store is dropped (the range check covers voff, not soff).
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    if constexpr (W % 4 == 0) {
#pragma unroll
      for (int i = 0; i < W / 4; ++i) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16 * i, soff, kNontemporal);
        w[4 * i] = v.x, w[4 * i + 1] = v.y, w[4 * i + 2] = v.z, w[4 * i + 3] = v.w;
      }
    } else if constexpr (W == 2) {
      const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kNontemporal);
      w[0] = v.x, w[1] = v.y;
    } else if constexpr (kBytes == 4) {
      w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kNontemporal);
    } else {
      w[0] = __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
    }
  }
  __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) const {
    if constexpr (W % 4 == 0) {
#pragma unroll
      for (int i = 0; i < W / 4; ++i) {
        u32x4_t v;
        v.x = w[4 * i], v.y = w[4 * i + 1], v.z = w[4 * i + 2], v.w = w[4 * i + 3];
        __builtin_amdgcn_raw_buffer_store_b128(v, r, voff + 16 * i, soff, 0);
      }
    } else if constexpr (W == 2) {
      u32x2_t v;
      v.x = w[0], v.y = w[1];
      __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, soff, 0);
    } else if constexpr (kBytes == 4) {
      __builtin_amdgcn_raw_buffer_store_b32(w[0], r, voff, soff, 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b16(uint16_t(w[0]), r, voff, soff, 0);
    }
  }
  __device__ __forceinline__ float get(int m) const {
    if constexpr (sizeof(T) == 4) return __uint_as_float(w[m]);
    else if constexpr (E == 1) return __uint_as_float(w[0] << 16);
    else return __uint_as_float(m & 1 ? w[m >> 1] & 0xffff0000u : w[m >> 1] << 16);
  }
  // all E elements from f (rounded to nearest even for bf16, two per
  // conversion)
  __device__ __forceinline__ void set_all(const float (&f)[E]) {
    if constexpr (sizeof(T) == 4) {
#pragma unroll
      for (int m = 0; m < E; ++m) w[m] = __float_as_uint(f[m]);
    } else if constexpr (E == 1) {
      w[0] = from_f32<bf16_t>(f[0]);
    } else {
#pragma unroll
      for (int m = 0; m < E; m += 2) {
        const bf16x2_t h = __builtin_convertvector((f32x2_t){f[m], f[m + 1]}, bf16x2_t);
        w[m >> 1] = __builtin_bit_cast(uint32_t, h);
      }
    }
  }
  __device__ __forceinline__ void store(T *p) const {
    if constexpr (W % 4 == 0) {
#pragma unroll
      for (int i = 0; i < W / 4; ++i) {
        u32x4_t v;
        v.x = w[4 * i], v.y = w[4 * i + 1], v.z = w[4 * i + 2], v.w = w[4 * i + 3];
        *(reinterpret_cast<u32x4_t *>(p) + i) = v;
      }
    } else if constexpr (W == 2) {
      u32x2_t v;
      v.x = w[0], v.y = w[1];
      *reinterpret_cast<u32x2_t *>(p) = v;
    } else if constexpr (kBytes == 4) {
      *reinterpret_cast<uint32_t *>(p) = w[0];
    } else {
      *reinterpret_cast<uint16_t *>(p) = uint16_t(w[0]);
    }
  }
};

// The first token of t's sequence.  Offsets are clamped into [0, n_tokens]
// (a malformed cu_seqlens only changes where sequences start).
template <typename T> __device__ __forceinline__ int64_t seq_start(const PrologueArgs<T> &a, int64_t t) {
  if (!a.cu_seqlens) return t / a.seq_len * a.seq_len;
  auto bound = [&](int i) -> int64_t {
    const int64_t b = a.cu_seqlens[i];
    return b < 0 ? 0 : (b > a.n_tokens ? a.n_tokens : b);
  };
  int lo = 0, hi = a.n_seqs;  // the last sequence whose start is <= t (n_seqs >= 1, checked by the caller)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (bound(mid) <= t) lo = mid; else hi = mid - 1;
  }
  return bound(lo);
}

// Prologue geometry: a wave takes kPrologueRun tokens of four heads and keeps
// a ring of P raw rows in registers (a row's registers are refilled with the
// row P tokens ahead as soon as its last token is done).
constexpr int kPrologueRun = 64;
template <typename T> constexpr int prologue_ring() { return 16; }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Prologue: a wave takes kPrologueRun tokens of four heads of one tensor.
// Lanes 16 g .. 16 g + 15 hold head 4 hb + g, E = D / 16 channels each, so a
// row's norm is a DPP sum over one row of 16 lanes and one load instruction
// moves four adjacent heads' rows.  A launch covers tensors which0 .. which0
// + n_which - 1 (q, k, v) of one width D; blocks vary fastest over (tensor,
// head group), so the waves in flight at once cover whole tokens' rows,
// contiguous in memory.
//
// Rows stream through a ring of P register sets: raw row r (token t0 - 3 +
// r) sits in slot r mod P; token i reads rows i .. i + 3, after which row i
// is dead and its slot is refilled with row i + P, P - 3 tokens before that
// row is needed.  The loop body covers P tokens, so slots are compile-time.
//
// Arithmetic: the convolution runs on weights and bias pre-multiplied by
// -log2(e), giving y' = -log2(e) y, so e^-y is one exp2 and SiLU(y) =
// -ln(2) y' / (1 + 2^y'); the constant -ln(2) folds into the per-token scale.
// A tap before its token's sequence start reads zero: the halo rows before
// the first token's start are zeroed once, and at a start inside the run the
// three rows before it are zeroed (tokens are taken in order, and no later
// token of the run reaches back across that start).
template <typename T, int D, int P>
__global__ __launch_bounds__(64) void block_prologue_kernel(PrologueArgs<T> a, int which0, int n_which) {
  constexpr int E = D / 16;
  constexpr int RUN = kPrologueRun;
  static_assert(RUN % P == 0 && P % 4 == 0 && RUN % 64 == 0, "ring geometry");
  const int lane = threadIdx.x;
  const int nq = (a.H_qk + 3) >> 2, nv = (a.H_v + 3) >> 2;
  int per_run = 0;
  for (int wv = which0; wv < which0 + n_which; ++wv) per_run += wv == 2 ? nv : nq;
  const int64_t run = blockIdx.x / unsigned(per_run);
  int hb = int(blockIdx.x - run * per_run), which = which0;
  while (hb >= (which == 2 ? nv : nq)) hb -= which++ == 2 ? nv : nq;
  const int H = which == 2 ? a.H_v : a.H_qk;
  const int h = 4 * hb + (lane >> 4);
  const bool active = h < H;
  const uint32_t lane_off = uint32_t((active ? h : H - 1) * D + E * (lane & 15));  // elements
  const int64_t row_elems = int64_t(H) * D;
  const uint32_t row_bytes = uint32_t(row_elems * sizeof(T));  // the caller keeps this below 2^24
  const int64_t t0 = run * RUN;
  const int n = a.n_tokens - t0 < RUN ? int(a.n_tokens - t0) : RUN;  // tokens of this run
  const T *__restrict__ const src = which == 0 ? a.raw[0] : which == 1 ? a.raw[1] : a.raw[2];
  T *__restrict__ const dst = which == 0 ? a.out[0] : which == 1 ? a.out[1] : a.out[2];
  const float *const conv = which == 0 ? a.conv[0] : which == 1 ? a.conv[1] : a.conv[2];
  const float *const cbias = which == 0 ? a.bias[0] : which == 1 ? a.bias[1] : a.bias[2];

  // Raw row r of the run is token t0 - 3 + r.  The load resource starts at
  // token tb = max(t0 - 3, 0) and ends with the batch, so rows past the end
  // read zeros (they feed no computed token); rows before token 0 read token
  // 0's row and are zeroed below.  The store resource starts at token t0 and
  // ends with the batch, so stores of tokens past the end, and of inactive
  // lanes (offset out of range), are dropped: no memory access is
  // conditional, and the loads stay in flight across the token loop.
  const int64_t tb = t0 < 3 ? 0 : t0 - 3;
  auto range_bytes = [&](int64_t from) -> int {
    const int64_t b = (a.n_tokens - from) * int64_t(row_bytes);
    return int(b < 0x7fffffff ? b : 0x7fffffff);
  };
  const __amdgpu_buffer_rsrc_t lrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(src + tb * row_elems), 0, range_bytes(tb), 0x00020000);
  const __amdgpu_buffer_rsrc_t srs =
      __builtin_amdgcn_make_buffer_rsrc(dst + t0 * row_elems, 0, range_bytes(t0), 0x00020000);
  // (offsets go in the per-lane offset, which the range check covers; the
  // scalar offset stays 0.  Resources hold whole rows, below 2^31 bytes, and
  // every in-range offset is below (RUN + P + 3) * 2^24 < 2^31.)
  const uint32_t lvoff = lane_off * uint32_t(sizeof(T));
  const uint32_t svoff = active ? lvoff : 0x80000000u;
  auto row_voff = [&](int r) -> uint32_t {  // this lane's byte offset of raw row r
    if (r > RUN + 2) return 0x80000000u;  // needed by no token of the run: read nothing
    const int64_t t = t0 - 3 + r - tb;
    return lvoff + uint32_t(t < 0 ? 0 : t) * row_bytes;
  };
  Row<T, E> x[P];
#pragma unroll
  for (int r = 0; r < P; ++r) x[r].load(lrs, row_voff(r), 0);

  // the tokens of the run that open a sequence (bit i % 64 of word i / 64;
  // lane l looks at tokens t0 + l + 64 q), and the first token's start s0
  uint64_t starts[RUN / 64];
  int64_t s0 = 0;
#pragma unroll
  for (int q = 0; q < RUN / 64; ++q) {
    const int i = 64 * q + lane;
    const int64_t st = i < n ? seq_start(a, t0 + i) : 0;
    starts[q] = __ballot(i < n && st == t0 + i);
    if (q == 0)
      s0 = __builtin_amdgcn_readfirstlane(int32_t(st)) |
           (int64_t(__builtin_amdgcn_readfirstlane(int32_t(st >> 32))) << 32);
  }

  float w[E][4], bias[E], nw[E];
#pragma unroll
  for (int m = 0; m < E; ++m) {
    const int c = int(lane_off) + m;  // channel within the tensor's H * D
#pragma unroll
    for (int j = 0; j < 4; ++j) w[m][j] = -kLog2e * conv[4 * c + j];
    bias[m] = cbias ? -kLog2e * cbias[c] : 0.0f;
    nw[m] = which == 2 && a.norm_w ? a.norm_w[E * (lane & 15) + m] : 1.0f;  // v only
  }
  // The per-token scale from the row's sum of z^2 (z = -log2(e) SiLU), as
  // sc_mul / sqrt(max(sum * sc_ss + sc_add, sc_floor)), which includes the
  // -ln 2 that turns z back into SiLU:
  //   v:    -ln 2 / sqrt(mean of SiLU^2 + eps)
  //   q, k: -ln 2 q_scale / max(norm of SiLU, 1e-12)  (q_scale = 1 for k)
  const bool is_v = which == 2;
  const float sc_ss = is_v ? kLn2 * kLn2 / D : kLn2 * kLn2;
  const float sc_add = is_v ? a.eps : 0.0f;
  const float sc_floor = is_v ? 0.0f : 1e-24f;
  const float sc_mul = which == 0 ? -kLn2 * a.q_scale : -kLn2;

  // unpacked rows i .. i + 3 of the current token i, in slots (row mod 4)
  float xf[4][E];
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    const bool before = t0 - 3 + r < s0;  // before the first token's sequence start (or the batch)
#pragma unroll
    for (int m = 0; m < E; ++m) xf[r][m] = before ? 0.0f : x[r].get(m);
  }

  for (int k = 0; k < RUN; k += P) {
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int i = k + j;
#pragma unroll
      for (int m = 0; m < E; ++m) xf[(j + 3) & 3][m] = x[(j + 3) % P].get(m);
      if (i > 0 && ((starts[i >> 6] >> (i & 63)) & 1)) {
        // a sequence starts at token t0 + i: its taps do not reach back (a
        // real branch, taken rarely; the barrier keeps it from becoming
        // selects)
        __asm__ volatile("" ::: "memory");
#pragma unroll
        for (int r = 0; r < 3; ++r)
#pragma unroll
          for (int m = 0; m < E; ++m) xf[(j + r) & 3][m] = 0.0f;
      }
      float z[E], ss = 0.0f;
#pragma unroll
      for (int m = 0; m < E; ++m) {
        float y = fmaf(w[m][0], xf[j & 3][m], bias[m]);
        y = fmaf(w[m][1], xf[(j + 1) & 3][m], y);
        y = fmaf(w[m][2], xf[(j + 2) & 3][m], y);
        y = fmaf(w[m][3], xf[(j + 3) & 3][m], y);                          // -log2(e) * conv
        z[m] = y * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(y));  // -log2(e) * SiLU
        ss = fmaf(z[m], z[m], ss);
      }
      const float scale = sc_mul * __builtin_amdgcn_rsqf(fmaxf(fmaf(row16_sum(ss), sc_ss, sc_add), sc_floor));
#pragma unroll
      for (int m = 0; m < E; ++m) z[m] *= scale;
      if (which == 2 && a.norm_w) {  // the same on every lane; the barrier keeps the branch
        __asm__ volatile("" ::: "memory");
#pragma unroll
        for (int m = 0; m < E; ++m) z[m] *= nw[m];
      }
      Row<T, E> out;
      out.set_all(z);
      out.store(srs, svoff + uint32_t(i) * row_bytes, 0);
      // row i is dead; its slot takes row i + P (zeros past the batch or the
      // run's last row)
      x[j].load(lrs, row_voff(i + P), 0);
    }
  }

  // The gates of this wave's value heads, one (token, head) per lane and step.
  if (which == 2) {
#pragma unroll
    for (int k = lane; k < 4 * RUN; k += 64) {
      const int i = k >> 2, hv = 4 * hb + (k & 3);
      if (i < n && hv < a.H_v) {
        const int64_t idx = (t0 + i) * a.H_v + hv;
        const float A = expf(a.log_A[hv]);
        a.alpha[idx] = expf(-A * softplus_f(a.a_raw[idx]));
        a.beta[idx] = 1.0f / (1.0f + expf(-a.b_raw[idx]));
      }
    }
  }
}

template <typename T>
struct EpilogueArgs {
  const T *o, *g;
  const float *norm_w;
  T *y;
  int64_t n_rows;  // B * T * H_v
  int32_t d_v;
  float eps;
};

// Epilogue: a row (token, head) is spread over 16 lanes, d / 16 elements each
// (16 bytes per lane for bf16 at d = 128); a wave takes 4 rows per step and
// kEpilogueSteps steps, issuing every load before any arithmetic.
constexpr int kEpilogueSteps = 4;

template <typename T, int D>
__global__ __launch_bounds__(256) void block_epilogue_kernel(EpilogueArgs<T> a) {
  constexpr int E = D / 16;  // elements per lane
  constexpr int S = kEpilogueSteps;
  const int lane = threadIdx.x & 63;
  const int64_t row0 = (int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6)) * (4 * S) + (lane >> 4);
  const int e0 = E * (lane & 15);
  // rows past the end are clamped for the (unconditional) loads and not stored
  Row<T, E> ov[S], gv[S];
#pragma unroll
  for (int st = 0; st < S; ++st) {
    const int64_t row = row0 + 4 * st;
    const int64_t rc = row < a.n_rows ? row : a.n_rows - 1;
    ov[st].load(a.o + rc * D + e0);
    gv[st].load(a.g + rc * D + e0);
  }
  float wv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) wv[e] = a.norm_w ? a.norm_w[e0 + e] : 1.0f;
#pragma unroll
  for (int st = 0; st < S; ++st) {
    const int64_t row = row0 + 4 * st;
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) ss += ov[st].get(e) * ov[st].get(e);
    const float r = __builtin_amdgcn_rsqf(row16_sum(ss) * (1.0f / D) + a.eps);
    float yv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) yv[e] = ov[st].get(e) * r * wv[e] * silu_fast(gv[st].get(e));
    Row<T, E> out;
    out.set_all(yv);
    if (row < a.n_rows) out.store(a.y + row * D + e0);
  }
}

template <typename T>
static hipError_t launch_prologue_t(const BlockProblem &p, hipStream_t st) {
  PrologueArgs<T> a;
  for (int i = 0; i < 3; ++i) {
    a.raw[i] = static_cast<const T *>(p.raw[i]);
    a.out[i] = static_cast<T *>(p.out[i]);
    a.conv[i] = p.conv[i];
    a.bias[i] = p.bias[i];
  }
  a.a_raw = p.a_raw;
  a.b_raw = p.b_raw;
  a.log_A = p.log_A;
  a.norm_w = p.norm_w;
  a.alpha = p.alpha;
  a.beta = p.beta;
  a.cu_seqlens = p.cu_seqlens;
  a.n_tokens = int64_t(p.B) * p.T;
  a.seq_len = p.T;
  a.n_seqs = p.n_seqs;
  a.H_qk = p.H_qk;
  a.H_v = p.H_v;
  a.eps = p.eps;
  a.q_scale = p.q_scale;
  constexpr int P = prologue_ring<T>();
  const int64_t ranges = (a.n_tokens + kPrologueRun - 1) / kPrologueRun;
  if (ranges == 0) return hipSuccess;
  const int nq = (p.H_qk + 3) / 4, nv = (p.H_v + 3) / 4;
  // (the caller keeps the grid within 32 bits)
  auto launch = [&](int D, int which0, int n_which) {
    int per_range = 0;
    for (int w = which0; w < which0 + n_which; ++w) per_range += w == 2 ? nv : nq;
    const dim3 grid = dim3(unsigned(ranges * per_range));
    switch (D) {
      case 16: hipLaunchKernelGGL((block_prologue_kernel<T, 16, P>), grid, dim3(64), 0, st, a, which0, n_which); break;
      case 32: hipLaunchKernelGGL((block_prologue_kernel<T, 32, P>), grid, dim3(64), 0, st, a, which0, n_which); break;
      case 64: hipLaunchKernelGGL((block_prologue_kernel<T, 64, P>), grid, dim3(64), 0, st, a, which0, n_which); break;
      default: hipLaunchKernelGGL((block_prologue_kernel<T, 128, P>), grid, dim3(64), 0, st, a, which0, n_which); break;
    }
  };
  if (p.d_k == p.d_v) {
    launch(p.d_k, 0, 3);
  } else {
    launch(p.d_k, 0, 2);
    launch(p.d_v, 2, 1);
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_epilogue_t(const BlockProblem &p, hipStream_t st) {
  EpilogueArgs<T> a;
  a.o = static_cast<const T *>(p.raw[0]);
  a.g = static_cast<const T *>(p.raw[1]);
  a.norm_w = p.norm_w;
  a.y = static_cast<T *>(p.out[0]);
  a.n_rows = int64_t(p.B) * p.T * p.H_v;
  a.d_v = p.d_v;
  a.eps = p.eps;
  const int64_t rows_per_block = 4 * 4 * kEpilogueSteps;  // 4 waves x 4 rows x steps
  const int64_t blocks = (a.n_rows + rows_per_block - 1) / rows_per_block;
  if (blocks == 0) return hipSuccess;
  switch (p.d_v) {
    case 16: hipLaunchKernelGGL((block_epilogue_kernel<T, 16>), dim3(unsigned(blocks)), dim3(256), 0, st, a); break;
    case 32: hipLaunchKernelGGL((block_epilogue_kernel<T, 32>), dim3(unsigned(blocks)), dim3(256), 0, st, a); break;
    case 64: hipLaunchKernelGGL((block_epilogue_kernel<T, 64>), dim3(unsigned(blocks)), dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL((block_epilogue_kernel<T, 128>), dim3(unsigned(blocks)), dim3(256), 0, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_block_prologue(const BlockProblem &p, hipStream_t st) {
  return p.dtype == 1 ? launch_prologue_t<bf16_t>(p, st) : launch_prologue_t<float>(p, st);
}
hipError_t launch_block_epilogue(const BlockProblem &p, hipStream_t st) {
  return p.dtype == 1 ? launch_epilogue_t<bf16_t>(p, st) : launch_epilogue_t<float>(p, st);
}

}  // namespace gdn
