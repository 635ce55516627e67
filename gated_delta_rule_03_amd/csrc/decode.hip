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
// Layout: one 256-thread block per (sequence, value head).  Thread tid owns
// columns 4 (tid & 31) .. +3 of rows (tid >> 5) + 8 i: each wave instruction
// moves two whole 512-byte rows (coalesced 16-byte accesses).  Column sums
// over d_k reduce across the two row groups of a wave with a lane swap and
// across the four waves through LDS.
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

template <typename T>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs<T> a) {
  const int u = blockIdx.x;  // b * H_v + h
  const int b = u / a.H_v, h = u - b * a.H_v, hq = h / a.group;
  const int tid = threadIdx.x, cg = tid & 31, rg = tid >> 5, wave = tid >> 6;
  const bool col_ok = 4 * cg < a.d_v;

  float *S = a.state + int64_t(u) * a.d_k * a.d_v;
  const T *kp = a.k + (int64_t(b) * a.H_qk + hq) * a.d_k;
  const T *qp = a.q + (int64_t(b) * a.H_qk + hq) * a.d_k;

  float4 s[16];
  float kk[16], qq[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = rg + 8 * i;
    const bool ok = r < a.d_k;
    s[i] = (ok && col_ok) ? *reinterpret_cast<const float4 *>(S + int64_t(r) * a.d_v + 4 * cg)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
    kk[i] = ok ? to_f32(kp[r]) : 0.0f;
    qq[i] = ok ? to_f32(qp[r]) : 0.0f;
  }

  float4 ak = make_float4(0.f, 0.f, 0.f, 0.f), bq = ak;
  float qk = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    ak.x += s[i].x * kk[i]; ak.y += s[i].y * kk[i]; ak.z += s[i].z * kk[i]; ak.w += s[i].w * kk[i];
    bq.x += s[i].x * qq[i]; bq.y += s[i].y * qq[i]; bq.z += s[i].z * qq[i]; bq.w += s[i].w * qq[i];
    qk += kk[i] * qq[i];
  }
  // reduce the two row groups of this wave (lanes l and l ^ 32)
  ak.x += __shfl_xor(ak.x, 32); ak.y += __shfl_xor(ak.y, 32);
  ak.z += __shfl_xor(ak.z, 32); ak.w += __shfl_xor(ak.w, 32);
  bq.x += __shfl_xor(bq.x, 32); bq.y += __shfl_xor(bq.y, 32);
  bq.z += __shfl_xor(bq.z, 32); bq.w += __shfl_xor(bq.w, 32);
  qk += __shfl_xor(qk, 32);

  __shared__ float4 red_a[4][32], red_b[4][32];
  __shared__ float red_qk[4];
  if ((tid & 32) == 0) {
    red_a[wave][cg] = ak;
    red_b[wave][cg] = bq;
  }
  if ((tid & 63) == 0) red_qk[wave] = qk;
  __syncthreads();
  ak = red_a[0][cg]; bq = red_b[0][cg]; qk = red_qk[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    const float4 x = red_a[w][cg], y = red_b[w][cg];
    ak.x += x.x; ak.y += x.y; ak.z += x.z; ak.w += x.w;
    bq.x += y.x; bq.y += y.y; bq.z += y.z; bq.w += y.w;
    qk += red_qk[w];
  }

  const int64_t vi = (int64_t(b) * a.H_v + h);
  const float al = a.alpha[vi], be = a.beta[vi];
  float4 vv = make_float4(0.f, 0.f, 0.f, 0.f);
  if (col_ok) vv = load4_f32(a.v + vi * a.d_v + 4 * cg);
  float4 uu;
  uu.x = be * (vv.x - al * ak.x);
  uu.y = be * (vv.y - al * ak.y);
  uu.z = be * (vv.z - al * ak.z);
  uu.w = be * (vv.w - al * ak.w);

  if (rg == 0 && col_ok) {
    T *op = a.o + vi * a.d_v + 4 * cg;
    op[0] = from_f32<T>(al * bq.x + qk * uu.x);
    op[1] = from_f32<T>(al * bq.y + qk * uu.y);
    op[2] = from_f32<T>(al * bq.z + qk * uu.z);
    op[3] = from_f32<T>(al * bq.w + qk * uu.w);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = rg + 8 * i;
    if (r < a.d_k && col_ok) {
      float4 n;
      n.x = al * s[i].x + kk[i] * uu.x;
      n.y = al * s[i].y + kk[i] * uu.y;
      n.z = al * s[i].z + kk[i] * uu.z;
      n.w = al * s[i].w + kk[i] * uu.w;
      *reinterpret_cast<float4 *>(S + int64_t(r) * a.d_v + 4 * cg) = n;
    }
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
  hipLaunchKernelGGL(decode_kernel<T>, dim3(unsigned(blocks)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_decode(const Problem &p, float *state, hipStream_t st) {
  return p.dtype == 1 ? launch_decode_t<bf16_t>(p, state, st) : launch_decode_t<float>(p, state, st);
}

}  // namespace gdn
