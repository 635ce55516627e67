// Token-by-token recurrence ("Linear attention", section "How it works",
// Eqs. (1)-(4)): decay, predict from the decayed state, correct along the key,
// read after the write -- a matrix-vector read and a rank-one write per token
// ("How linear attention works", section "Why it is called linear attention").
//
// With a per-channel gate (one rate per key channel, the channels being the
// state's rows: "Attention as Matrix Algebra", section 10, names the
// variant) the decay is diag(alpha_t) instead of a scalar; each lane owns
// whole rows, so it scales its rows by their own rates.
//
// Layout: one wavefront per (sequence, value head, 16-column block).  Lane l
// owns column 16 cb + (l & 15) and the contiguous row block
// [(l >> 4) d_k/4, (l >> 4 + 1) d_k/4) of the state, in registers.  Column sums
// over d_k reduce across the four row groups with two lane swaps.  The next
// token's operands are fetched while the current token is processed.
#include "launch.hpp"

namespace gdn {

template <typename T>
struct RecArgs {
  const T *q, *k, *v;
  const float *alpha, *beta;
  const float *h0;
  T *o;
  float *hT;
  int H_qk, H_v, d_k, d_v, group, n_units, n_colblk;
  SeqGeom geo;
};

struct TokenOps {
  float k[32], q[32];
  float ar[32];  // per-channel gate: the rates of this lane's rows
  float v, al, be;
};

template <typename T, bool PER_CHANNEL>
__device__ __forceinline__ void fetch_token(const RecArgs<T> &a, int tok, int hq, int h, int col,
                                            int r0, int nrow, TokenOps &x) {
  const int64_t qk_off = (int64_t(tok) * a.H_qk + hq) * a.d_k + r0;
  const T *kp = a.k + qk_off;
  const T *qp = a.q + qk_off;
#pragma unroll
  for (int i = 0; i < 32; i += 4) {
    if (i < nrow) {
      const float4 kk = load4_f32(kp + i), qq = load4_f32(qp + i);
      x.k[i] = kk.x; x.k[i + 1] = kk.y; x.k[i + 2] = kk.z; x.k[i + 3] = kk.w;
      x.q[i] = qq.x; x.q[i + 1] = qq.y; x.q[i + 2] = qq.z; x.q[i + 3] = qq.w;
    } else {
      for (int j = 0; j < 4; ++j) { x.k[i + j] = 0.0f; x.q[i + j] = 0.0f; }
    }
  }
  const int64_t gi = int64_t(tok) * a.H_v + h;
  x.v = to_f32(a.v[gi * a.d_v + col]);
  if constexpr (PER_CHANNEL) {
    const float *ap = a.alpha + gi * a.d_k + r0;  // alpha [.., H_v, d_k]
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
      const float4 r = i < nrow ? *reinterpret_cast<const float4 *>(ap + i) : make_float4(0.f, 0.f, 0.f, 0.f);
      x.ar[i] = r.x; x.ar[i + 1] = r.y; x.ar[i + 2] = r.z; x.ar[i + 3] = r.w;
    }
    x.al = 1.0f;
  } else {
    x.al = a.alpha[gi];
  }
  x.be = a.beta[gi];
}

template <typename T, bool PER_CHANNEL>
__global__ __launch_bounds__(64) void recurrent_kernel(RecArgs<T> a) {
  const int lane = threadIdx.x;
  const int u = blockIdx.x / a.n_colblk, cb = blockIdx.x - u * a.n_colblk;
  if (u >= a.n_units) return;
  const int s = u / a.H_v, h = u - s * a.H_v, hq = h / a.group;
  const int col = 16 * cb + (lane & 15);
  const int nrow = a.d_k >> 2;            // rows per lane group (4..32)
  const int r0 = (lane >> 4) * nrow;

  float S[32];
  const int64_t st_base = (int64_t(s) * a.H_v + h) * a.d_k * a.d_v;
#pragma unroll
  for (int i = 0; i < 32; ++i)
    S[i] = (i < nrow && a.h0) ? a.h0[st_base + int64_t(r0 + i) * a.d_v + col] : 0.0f;

  int start, end;
  a.geo.seq_bounds(s, start, end);
  TokenOps cur, nxt;
  if (start < end) fetch_token<T, PER_CHANNEL>(a, start, hq, h, col, r0, nrow, cur);
  for (int tok = start; tok < end; ++tok) {
    if (tok + 1 < end) fetch_token<T, PER_CHANNEL>(a, tok + 1, hq, h, col, r0, nrow, nxt);
    // predict: vhat = (alpha S)^T k  (per-channel: (diag(a) S)^T k)
    float p = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) p += S[i] * (PER_CHANNEL ? cur.ar[i] * cur.k[i] : cur.k[i]);
    p += __shfl_xor(p, 16);
    p += __shfl_xor(p, 32);
    const float w = cur.be * (cur.v - cur.al * p);
    // decay and correct: S = alpha S + k w ; read: o = S^T q
    float r = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      S[i] = (PER_CHANNEL ? cur.ar[i] : cur.al) * S[i] + cur.k[i] * w;
      r += S[i] * cur.q[i];
    }
    r += __shfl_xor(r, 16);
    r += __shfl_xor(r, 32);
    if (lane < 16) a.o[(int64_t(tok) * a.H_v + h) * a.d_v + col] = from_f32<T>(r);
    cur = nxt;
  }
  if (a.hT) {
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if (i < nrow) a.hT[st_base + int64_t(r0 + i) * a.d_v + col] = S[i];
  }
}

template <typename T>
static hipError_t launch_recurrent_t(const Problem &p, hipStream_t st) {
  RecArgs<T> a;
  a.q = static_cast<const T *>(p.q);
  a.k = static_cast<const T *>(p.k);
  a.v = static_cast<const T *>(p.v);
  a.alpha = p.alpha;
  a.beta = p.beta;
  a.h0 = p.h0;
  a.o = static_cast<T *>(p.o);
  a.hT = p.hT;
  a.H_qk = p.H_qk;
  a.H_v = p.H_v;
  a.d_k = p.d_k;
  a.d_v = p.d_v;
  a.group = p.H_v / p.H_qk;
  a.n_units = p.n_seqs * p.H_v;
  a.n_colblk = p.d_v / 16;
  a.geo = make_geom(p, nullptr);
  const int64_t blocks = int64_t(a.n_units) * a.n_colblk;
  if (blocks == 0) return hipSuccess;
  if (p.per_channel)
    hipLaunchKernelGGL((recurrent_kernel<T, true>), dim3(unsigned(blocks)), dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL((recurrent_kernel<T, false>), dim3(unsigned(blocks)), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_recurrent(const Problem &p, hipStream_t st) {
  return p.dtype == 1 ? launch_recurrent_t<bf16_t>(p, st) : launch_recurrent_t<float>(p, st);
}

}  // namespace gdn
