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
// once.  Prologue: one wave per (tensor, head, 64 tokens); a lane owns one or
// two channels (d <= 64: one, d = 128: two adjacent ones, so a row of d
// elements moves in one coalesced access), keeps the last three raw values
// of its channels in registers and walks the tokens in order; a wave sum
// gives each token's norm.  The v waves also form alpha and beta of their
// head, one token per lane.  Epilogue: one wave per (token, head).
#include "launch.hpp"

namespace gdn {

constexpr int kPrologueTokens = 64;

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

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

__device__ __forceinline__ float silu_f(float y) { return y / (1.0f + expf(-y)); }

// log(1 + e^a) without overflow
__device__ __forceinline__ float softplus_f(float a) { return a > 0.0f ? a + log1pf(expf(-a)) : log1pf(expf(a)); }

template <typename T>
__global__ __launch_bounds__(64) void block_prologue_kernel(PrologueArgs<T> a) {
  const int lane = threadIdx.x;
  // blockIdx.y: q heads, then k heads, then v heads
  int which = 0, h = blockIdx.y;
  if (h >= a.H_qk) {
    h -= a.H_qk;
    which = 1;
    if (h >= a.H_qk) {
      h -= a.H_qk;
      which = 2;
    }
  }
  const int H = which == 2 ? a.H_v : a.H_qk;
  const int d = which == 2 ? a.d_v : a.d_k;
  const int epl = d == 128 ? 2 : 1;  // channels per lane
  const bool active = lane * epl < d;
  const int e0 = lane * epl;
  const int64_t t0 = int64_t(blockIdx.x) * kPrologueTokens;
  const int64_t t1 = t0 + kPrologueTokens < a.n_tokens ? t0 + kPrologueTokens : a.n_tokens;
  const T *const src = a.raw[which];
  T *const dst = a.out[which];

  float w[2][4], bias[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int64_t c = int64_t(h) * d + e0 + m;
    const bool on = active && m < epl;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[m][j] = on ? a.conv[which][4 * c + j] : 0.0f;
    bias[m] = on && a.bias[which] ? a.bias[which][c] : 0.0f;
  }
  float nw[2] = {1.0f, 1.0f};
  if (which == 2 && a.norm_w && active)
    for (int m = 0; m < epl; ++m) nw[m] = a.norm_w[e0 + m];

  auto load = [&](int64_t t, float (&x)[2]) {
    x[0] = x[1] = 0.0f;
    if (t < 0 || !active) return;
    const T *p = src + (t * H + h) * d + e0;
    x[0] = to_f32(p[0]);
    if (epl == 2) x[1] = to_f32(p[1]);
  };

  // The sequence holding token t: [start, next).  Offsets are clamped into
  // [0, n_tokens] and made non-decreasing, so malformed offsets only change
  // which taps are masked.
  int s = 0;
  int64_t start = 0, next = a.n_tokens;
  auto bound = [&](int i) -> int64_t {
    const int64_t b = a.cu_seqlens[i];
    return b < 0 ? 0 : (b > a.n_tokens ? a.n_tokens : b);
  };
  if (a.cu_seqlens) {  // n_seqs >= 1 (checked by the caller)
    int lo = 0, hi = a.n_seqs - 1;  // the last sequence whose start is <= t0
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (bound(mid) <= t0) lo = mid; else hi = mid - 1;
    }
    s = lo;
    start = bound(s);
    next = bound(s + 1) > start ? bound(s + 1) : start;
  } else {
    start = t0 / a.seq_len * a.seq_len;
    next = start + a.seq_len;
  }

  float xm[3][2];  // raw values of tokens t - 1, t - 2, t - 3
#pragma unroll
  for (int j = 0; j < 3; ++j) load(t0 - 1 - j, xm[j]);
  for (int64_t t = t0; t < t1; ++t) {
    while (t >= next) {  // the next non-empty sequence
      start = next;
      if (a.cu_seqlens) {
        ++s;
        next = s + 1 <= a.n_seqs ? (bound(s + 1) > start ? bound(s + 1) : start) : a.n_tokens;
      } else {
        next = start + a.seq_len;
      }
    }
    float x[2];
    load(t, x);
    float z[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      float y = bias[m] + w[m][3] * x[m];
      if (t - 1 >= start) y += w[m][2] * xm[0][m];
      if (t - 2 >= start) y += w[m][1] * xm[1][m];
      if (t - 3 >= start) y += w[m][0] * xm[2][m];
      z[m] = m < epl && active ? silu_f(y) : 0.0f;
    }
    const float ss = wave_sum(z[0] * z[0] + z[1] * z[1]);
    const float scale = which == 2 ? 1.0f / sqrtf(ss / float(d) + a.eps)
                                   : (which == 0 ? a.q_scale : 1.0f) / fmaxf(sqrtf(ss), 1e-12f);
    if (active) {
      T *p = dst + (t * H + h) * d + e0;
      p[0] = from_f32<T>(z[0] * scale * nw[0]);
      if (epl == 2) p[1] = from_f32<T>(z[1] * scale * nw[1]);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      xm[2][m] = xm[1][m];
      xm[1][m] = xm[0][m];
      xm[0][m] = x[m];
    }
  }

  if (which == 2) {  // the gates of head h, one token per lane
    const int64_t t = t0 + lane;
    if (t < t1) {
      const int64_t i = t * a.H_v + h;
      const float A = expf(a.log_A[h]);
      a.alpha[i] = expf(-A * softplus_f(a.a_raw[i]));
      a.beta[i] = 1.0f / (1.0f + expf(-a.b_raw[i]));
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

template <typename T>
__global__ __launch_bounds__(256) void block_epilogue_kernel(EpilogueArgs<T> a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);  // (token, head)
  if (row >= a.n_rows) return;  // the whole wave
  const int d = a.d_v;
  const int epl = d == 128 ? 2 : 1;
  const bool active = lane * epl < d;
  const int e0 = lane * epl;
  const int64_t base = row * d + e0;
  float o[2] = {0.0f, 0.0f}, g[2] = {0.0f, 0.0f};
  if (active) {
    o[0] = to_f32(a.o[base]);
    g[0] = to_f32(a.g[base]);
    if (epl == 2) {
      o[1] = to_f32(a.o[base + 1]);
      g[1] = to_f32(a.g[base + 1]);
    }
  }
  const float r = 1.0f / sqrtf(wave_sum(o[0] * o[0] + o[1] * o[1]) / float(d) + a.eps);
  if (active) {
    for (int m = 0; m < epl; ++m) {
      const float wm = a.norm_w ? a.norm_w[e0 + m] : 1.0f;
      a.y[base + m] = from_f32<T>(o[m] * r * wm * silu_f(g[m]));
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
  hipLaunchKernelGGL(block_prologue_kernel<T>, dim3(unsigned(ranges), unsigned(2 * p.H_qk + p.H_v)), dim3(64), 0, st,
                     a);
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
  const int64_t blocks = (a.n_rows + 3) / 4;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(block_epilogue_kernel<T>, dim3(unsigned(blocks)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_block_prologue(const BlockProblem &p, hipStream_t st) {
  return p.dtype == 1 ? launch_prologue_t<bf16_t>(p, st) : launch_prologue_t<float>(p, st);
}
hipError_t launch_block_epilogue(const BlockProblem &p, hipStream_t st) {
  return p.dtype == 1 ? launch_epilogue_t<bf16_t>(p, st) : launch_epilogue_t<float>(p, st);
}

}  // namespace gdn
