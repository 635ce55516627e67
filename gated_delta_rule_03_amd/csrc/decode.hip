// Fused decode step: one new token per sequence, state updated in place.
//
// Per (sequence, value head), with S the stored d_k x d_v state and the
// token's q, k, v, alpha, beta ("Linear attention", Eqs. (1)-(4)):
//   a = S^T k,  b = S^T q          (one pass over S)
//   vhat = alpha a,  u = beta (v - vhat)
//   o = alpha b + (q^T k) u        (= S_new^T q)
//   S <- alpha S + k u^T           (written back in place)
// The step reads and writes the state once: about rd numbers each way
// ("Attention as Matrix Algebra", section 9), so it is bound by HBM bandwidth.
//
// With a per-channel gate (alpha_t a vector over the key channels, i.e. the
// state's rows) the decay is diag(alpha): a = S^T (alpha . k),
// b = S^T (alpha . q), and row r is written back as alpha_r S_r + k_r u.
//
// Layout: one 512-thread block per (sequence, value head).  Thread tid owns
// columns 4 (tid & 31) .. +3 of rows (tid >> 5) + 16 i: each wave instruction
// moves two whole 512-byte rows (coalesced 16-byte accesses).  The state is
// read and written with nontemporal accesses: it streams through once, and
// keeping it out of the caches' normal replacement path is worth about a
// quarter more achieved bandwidth here than plain loads and stores.  k and q
// are staged once in LDS.  Column sums over d_k reduce across the two row
// groups of a wave with a lane swap and across the eight waves through LDS.
#include "launch.hpp"

namespace gdn {

template <typename T>
struct DecodeArgs {
  const T *q, *k, *v;
  const float *alpha, *beta;
  float *state;
  T *o;
  int H_qk, H_v, d_k, d_v, group;
};

constexpr int kDecodeThreads = 512;
constexpr int kDecodeRowGroups = kDecodeThreads / 32;  // 16
constexpr int kDecodeRows = 128 / kDecodeRowGroups;    // rows per thread (d_k <= 128)

// (four waves per SIMD, so two blocks fit a CU: at most 128 VGPRs)
template <typename T, bool PER_CHANNEL>
__global__ __launch_bounds__(kDecodeThreads, 4) void decode_kernel(DecodeArgs<T> a) {
  const int u = blockIdx.x;  // b * H_v + h
  const int b = u / a.H_v, h = u - b * a.H_v, hq = h / a.group;
  const int tid = threadIdx.x, cg = tid & 31, rg = tid >> 5, wave = tid >> 6;
  const bool col_ok = 4 * cg < a.d_v;

  float *S = a.state + int64_t(u) * a.d_k * a.d_v;
  const T *kp = a.k + (int64_t(b) * a.H_qk + hq) * a.d_k;
  const T *qp = a.q + (int64_t(b) * a.H_qk + hq) * a.d_k;

  f32x4_t s[kDecodeRows];
#pragma unroll
  for (int i = 0; i < kDecodeRows; ++i) {
    const int r = rg + kDecodeRowGroups * i;
    s[i] = (r < a.d_k && col_ok)
               ? __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(S + int64_t(r) * a.d_v + 4 * cg))
               : zero4();
  }
  const int64_t vi = (int64_t(b) * a.H_v + h);
  // k, q and (per-channel gate) the rates, staged once in LDS
  __shared__ float skq[PER_CHANNEL ? 3 : 2][128];
  if (tid < a.d_k) skq[0][tid] = to_f32(kp[tid]);
  else if (tid >= 128 && tid - 128 < a.d_k) skq[1][tid - 128] = to_f32(qp[tid - 128]);
  else if (PER_CHANNEL && tid >= 256 && tid - 256 < a.d_k) skq[PER_CHANNEL ? 2 : 0][tid - 256] = a.alpha[vi * a.d_k + tid - 256];
  __syncthreads();

  // per-channel rate of row r (read from LDS where used, not held in registers)
  auto rate = [&](int r) -> float { return r < a.d_k ? skq[PER_CHANNEL ? 2 : 0][r] : 0.0f; };
  float kk[kDecodeRows];
  f32x4_t ak = zero4(), bq = zero4();
#pragma unroll
  for (int i = 0; i < kDecodeRows; ++i) {
    const int r = rg + kDecodeRowGroups * i;
    kk[i] = r < a.d_k ? skq[0][r] : 0.0f;
    const float qq = r < a.d_k ? skq[1][r] : 0.0f;
    if constexpr (PER_CHANNEL) {
      const float ar = rate(r);
      ak += s[i] * (ar * kk[i]);
      bq += s[i] * (ar * qq);
    } else {
      ak += s[i] * kk[i];
      bq += s[i] * qq;
    }
  }
  // q^T k over d_k, in wave 0
  float qk = 0.0f;
  if (wave == 0) {
    if (tid < a.d_k) qk = skq[0][tid] * skq[1][tid];
    if (tid + 64 < a.d_k) qk += skq[0][tid + 64] * skq[1][tid + 64];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) qk += __shfl_xor(qk, m);
  }
  // reduce the two row groups of this wave (lanes l and l ^ 32)
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ak[e] += __shfl_xor(ak[e], 32);
    bq[e] += __shfl_xor(bq[e], 32);
  }
  __shared__ f32x4_t red_a[kDecodeThreads / 64][32], red_b[kDecodeThreads / 64][32];
  __shared__ float red_qk;
  if ((tid & 32) == 0) {
    red_a[wave][cg] = ak;
    red_b[wave][cg] = bq;
  }
  if (tid == 0) red_qk = qk;
  __syncthreads();
  ak = red_a[0][cg];
  bq = red_b[0][cg];
  qk = red_qk;
#pragma unroll
  for (int w = 1; w < kDecodeThreads / 64; ++w) {
    ak += red_a[w][cg];
    bq += red_b[w][cg];
  }

  const float al = PER_CHANNEL ? 1.0f : a.alpha[vi], be = a.beta[vi];  // per-channel: rates already applied
  f32x4_t vv = zero4();
  if (col_ok) {
    const float4 x = load4_f32(a.v + vi * a.d_v + 4 * cg);
    vv = f32x4_t{x.x, x.y, x.z, x.w};
  }
  const f32x4_t uu = be * (vv - al * ak);

  if (rg == 0 && col_ok) {
    T *op = a.o + vi * a.d_v + 4 * cg;
    const f32x4_t ov = al * bq + qk * uu;
#pragma unroll
    for (int e = 0; e < 4; ++e) op[e] = from_f32<T>(ov[e]);
  }
#pragma unroll
  for (int i = 0; i < kDecodeRows; ++i) {
    const int r = rg + kDecodeRowGroups * i;
    if (r < a.d_k && col_ok)
      __builtin_nontemporal_store((PER_CHANNEL ? rate(r) : al) * s[i] + kk[i] * uu,
                                  reinterpret_cast<f32x4_t *>(S + int64_t(r) * a.d_v + 4 * cg));
  }
}

template <typename T>
static hipError_t launch_decode_t(const Problem &p, float *state, hipStream_t st) {
  DecodeArgs<T> a;
  a.q = static_cast<const T *>(p.q);
  a.k = static_cast<const T *>(p.k);
  a.v = static_cast<const T *>(p.v);
  a.alpha = p.alpha;
  a.beta = p.beta;
  a.state = state;
  a.o = static_cast<T *>(p.o);
  a.H_qk = p.H_qk;
  a.H_v = p.H_v;
  a.d_k = p.d_k;
  a.d_v = p.d_v;
  a.group = p.H_v / p.H_qk;
  const int64_t blocks = int64_t(p.B) * p.H_v;
  if (blocks == 0) return hipSuccess;
  if (p.per_channel)
    hipLaunchKernelGGL((decode_kernel<T, true>), dim3(unsigned(blocks)), dim3(kDecodeThreads), 0, st, a);
  else
    hipLaunchKernelGGL((decode_kernel<T, false>), dim3(unsigned(blocks)), dim3(kDecodeThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_decode(const Problem &p, float *state, hipStream_t st) {
  return p.dtype == 1 ? launch_decode_t<bf16_t>(p, state, st) : launch_decode_t<float>(p, state, st);
}

}  // namespace gdn
