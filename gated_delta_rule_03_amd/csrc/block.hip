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
// once, and each wave issues all its loads before any arithmetic (a wave
// that waited for one row at a time would leave HBM mostly idle).
// Prologue: one wave per (tensor, head, 32 tokens); a lane owns one or two
// channels (d <= 64: one, d = 128: two adjacent ones, so a row of d elements
// moves in one coalesced access) and holds the raw rows of its 32 tokens and
// the 3 before them in registers; a wave sum gives each token's norm.  The v
// waves also form alpha and beta of their head, one token per lane.
// Epilogue: 16 lanes per (token, head) row, 16 rows per wave.
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
  int32_t seq_len, n_seqs, H_qk, H_v, d_k, d_v;  // seq_len: tokens per sequence (uniform)
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
// Sum over the wave, the same value in every lane (the four row sums read
// into scalar registers).
__device__ __forceinline__ float wave_sum(float x) {
  const int r = __float_as_int(row16_sum(x));
  return (__int_as_float(__builtin_amdgcn_readlane(r, 0)) + __int_as_float(__builtin_amdgcn_readlane(r, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(r, 32)) + __int_as_float(__builtin_amdgcn_readlane(r, 48)));
}

// log(1 + e^a) without overflow
__device__ __forceinline__ float softplus_f(float a) { return a > 0.0f ? a + log1pf(expf(-a)) : log1pf(expf(a)); }

// Two consecutive elements at p (p even-aligned), widened to float.
__device__ __forceinline__ void load2(const bf16_t *__restrict__ p, float &a, float &b) {
  const uint32_t u = *reinterpret_cast<const uint32_t *>(p);
  a = __uint_as_float(u << 16);
  b = __uint_as_float(u & 0xffff0000u);
}
__device__ __forceinline__ void load2(const float *__restrict__ p, float &a, float &b) {
  const float2 u = *reinterpret_cast<const float2 *>(p);
  a = u.x;
  b = u.y;
}

// Two consecutive elements stored at p (p even-aligned).
__device__ __forceinline__ void store2(bf16_t *__restrict__ p, float a, float b) {
  *reinterpret_cast<uint32_t *>(p) = uint32_t(from_f32<bf16_t>(a)) | (uint32_t(from_f32<bf16_t>(b)) << 16);
}
__device__ __forceinline__ void store2(float *__restrict__ p, float a, float b) {
  *reinterpret_cast<float2 *>(p) = make_float2(a, b);
}

// Which of the three taps before token t lie in t's sequence: bit j - 1 set
// when token t - j does (j = 1, 2, 3).  Offsets are clamped into [0, n_tokens]
// (a malformed cu_seqlens only changes which taps count).
template <typename T> __device__ __forceinline__ int tap_mask(const PrologueArgs<T> &a, int64_t t) {
  int64_t start;
  if (a.cu_seqlens) {  // the last sequence whose start is <= t (n_seqs >= 1, checked by the caller)
    auto bound = [&](int i) -> int64_t {
      const int64_t b = a.cu_seqlens[i];
      return b < 0 ? 0 : (b > a.n_tokens ? a.n_tokens : b);
    };
    int lo = 0, hi = a.n_seqs;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (bound(mid) <= t) lo = mid; else hi = mid - 1;
    }
    start = bound(lo);
  } else {
    start = t / a.seq_len * a.seq_len;
  }
  return (t - 1 >= start ? 1 : 0) | (t - 2 >= start ? 2 : 0) | (t - 3 >= start ? 4 : 0);
}

// SiLU with the hardware exp2 and reciprocal (about 2 ulp).
__device__ __forceinline__ float silu_fast(float y) {
  return y * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * y));
}

template <typename T, int D>
__global__ __launch_bounds__(64) void block_prologue_kernel(PrologueArgs<T> a, int y0, int ny) {
  constexpr int R = kPrologueTokens;
  constexpr int EPL = D == 128 ? 2 : 1;  // channels per lane
  const int lane = threadIdx.x;
  // Block b takes token range b / ny and head row y0 + b % ny of the q heads,
  // then the k heads, then the v heads (a launch covers the heads of one
  // width D).  Heads vary fastest, so the waves in flight at once read and
  // write whole tokens' rows, contiguous in memory.
  const int64_t range = blockIdx.x / unsigned(ny);
  int which = 0, h = int(blockIdx.x - range * ny) + y0;
  if (h >= a.H_qk) {
    h -= a.H_qk;
    which = 1;
    if (h >= a.H_qk) {
      h -= a.H_qk;
      which = 2;
    }
  }
  const int H = which == 2 ? a.H_v : a.H_qk;
  const bool active = lane * EPL < D;
  const int e0 = active ? lane * EPL : 0;
  const int64_t t0 = range * R;
  // (selected, not indexed: an indexed kernel-argument array would go through
  // private memory and turn every access into a flat one)
  const T *__restrict__ const src = which == 0 ? a.raw[0] : which == 1 ? a.raw[1] : a.raw[2];
  T *__restrict__ const dst = which == 0 ? a.out[0] : which == 1 ? a.out[1] : a.out[2];
  const float *const conv = which == 0 ? a.conv[0] : which == 1 ? a.conv[1] : a.conv[2];
  const float *const cbias = which == 0 ? a.bias[0] : which == 1 ? a.bias[1] : a.bias[2];

  // The raw rows of tokens t0 - 3 .. t0 + R - 1, all loads issued first.
  // Token indices are clamped into the batch so every load is unconditional;
  // a row outside the batch is never used (rows before 0 or before a
  // sequence's start fall out through the tap mask, rows past the end belong
  // to tokens that are not computed), nor is an inactive lane's value.
  float x[R + 3][2];
#pragma unroll
  for (int i = 0; i < R + 3; ++i) {
    int64_t t = t0 - 3 + i;
    t = t < 0 ? 0 : (t >= a.n_tokens ? a.n_tokens - 1 : t);
    const T *p = src + (t * H + h) * D + e0;
    if (EPL == 2) load2(p, x[i][0], x[i][1]);
    else x[i][0] = to_f32(p[0]), x[i][1] = 0.0f;
  }
  // lane i < R: the tap mask of token t0 + i
  const int mask = lane < R && t0 + lane < a.n_tokens ? tap_mask(a, t0 + lane) : 0;

  float w[2][4], bias[2], nw[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int64_t c = int64_t(h) * D + e0 + m;
    const bool on = m < EPL;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[m][j] = on ? conv[4 * c + j] : 0.0f;
    bias[m] = on && cbias ? cbias[c] : 0.0f;
    nw[m] = on && which == 2 && a.norm_w ? a.norm_w[e0 + m] : 1.0f;
  }
  const float qs = which == 0 ? a.q_scale : 1.0f;
  const int n = a.n_tokens - t0 < R ? int(a.n_tokens - t0) : R;

#pragma unroll
  for (int i = 0; i < R; ++i) {
    if (i >= n) continue;  // n is the same on every lane
    const int mk = __builtin_amdgcn_readlane(mask, i);
    float z[2];
#pragma unroll
    for (int m = 0; m < EPL; ++m) {
      float y = bias[m] + w[m][3] * x[i + 3][m];
      if (mk & 1) y += w[m][2] * x[i + 2][m];
      if (mk & 2) y += w[m][1] * x[i + 1][m];
      if (mk & 4) y += w[m][0] * x[i][m];
      z[m] = active ? silu_fast(y) : 0.0f;
    }
    if (EPL == 1) z[1] = 0.0f;
    const float ss = wave_sum(z[0] * z[0] + z[1] * z[1]);
    // v: 1 / sqrt(mean square + eps); q, k: q_scale / max(norm, 1e-12)
    const float scale = which == 2 ? __builtin_amdgcn_rsqf(ss * (1.0f / D) + a.eps)
                                   : qs * __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));
    if (active) {
      T *p = dst + ((t0 + i) * H + h) * D + e0;
      if (EPL == 2) store2(p, z[0] * scale * nw[0], z[1] * scale * nw[1]);
      else p[0] = from_f32<T>(z[0] * scale * nw[0]);
    }
  }

  if (which == 2 && lane < n) {  // the gates of head h, one token per lane
    const int64_t i = (t0 + lane) * a.H_v + h;
    const float A = expf(a.log_A[h]);
    a.alpha[i] = expf(-A * softplus_f(a.a_raw[i]));
    a.beta[i] = 1.0f / (1.0f + expf(-a.b_raw[i]));
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
  const T *__restrict__ const o = a.o;
  const T *__restrict__ const g = a.g;
  T *__restrict__ const y = a.y;
  float ov[S][E], gv[S][E];
#pragma unroll
  for (int st = 0; st < S; ++st) {
    const int64_t row = row0 + 4 * st;
#pragma unroll
    for (int e = 0; e < E; ++e) ov[st][e] = gv[st][e] = 0.0f;
    if (row < a.n_rows) {
#pragma unroll
      for (int e = 0; e < E; e += 2) {
        if (E == 1) {
          ov[st][0] = to_f32(o[row * D + e0]);
          gv[st][0] = to_f32(g[row * D + e0]);
        } else {
          load2(o + row * D + e0 + e, ov[st][e], ov[st][e + 1]);
          load2(g + row * D + e0 + e, gv[st][e], gv[st][e + 1]);
        }
      }
    }
  }
  float wv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) wv[e] = a.norm_w ? a.norm_w[e0 + e] : 1.0f;
#pragma unroll
  for (int st = 0; st < S; ++st) {
    const int64_t row = row0 + 4 * st;
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) ss += ov[st][e] * ov[st][e];
    const float r = __builtin_amdgcn_rsqf(row16_sum(ss) * (1.0f / D) + a.eps);
    if (row < a.n_rows) {
#pragma unroll
      for (int e = 0; e < E; ++e) y[row * D + e0 + e] = from_f32<T>(ov[st][e] * r * wv[e] * silu_fast(gv[st][e]));
    }
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
  a.d_k = p.d_k;
  a.d_v = p.d_v;
  a.eps = p.eps;
  a.q_scale = p.q_scale;
  const int64_t ranges = (a.n_tokens + kPrologueTokens - 1) / kPrologueTokens;
  if (ranges == 0) return hipSuccess;
  // (the caller keeps ranges * (2 H_qk + H_v) within a 32-bit grid)
  auto launch = [&](int D, int y0, int ny) {
    const dim3 grid = dim3(unsigned(ranges * ny));
    switch (D) {
      case 16: hipLaunchKernelGGL((block_prologue_kernel<T, 16>), grid, dim3(64), 0, st, a, y0, ny); break;
      case 32: hipLaunchKernelGGL((block_prologue_kernel<T, 32>), grid, dim3(64), 0, st, a, y0, ny); break;
      case 64: hipLaunchKernelGGL((block_prologue_kernel<T, 64>), grid, dim3(64), 0, st, a, y0, ny); break;
      default: hipLaunchKernelGGL((block_prologue_kernel<T, 128>), grid, dim3(64), 0, st, a, y0, ny); break;
    }
  };
  if (p.d_k == p.d_v) {
    launch(p.d_k, 0, 2 * p.H_qk + p.H_v);
  } else {
    launch(p.d_k, 0, 2 * p.H_qk);
    launch(p.d_v, 2 * p.H_qk, p.H_v);
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
