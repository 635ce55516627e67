// Backward pass of the chunked gated delta rule (gradients for training in
// chunks).
//
// The pages motivate training in chunks ("From KV Cache to a State Matrix",
// section "Chunkwise training for DeltaNet"; "Attention as Matrix Algebra",
// section 8, "Training the delta rule in chunks") but print no gradients.
// They follow from the chunk form by reverse-mode differentiation.  Inside a
// chunk of n tokens that starts from state S, with g_t = sum_{i<=t} ln alpha_i
// (chunk-local), gamma_t = e^{g_t}, Gamma_ti = e^{g_t - g_i} (i <= t),
// s_t = e^{g_n - g_t}, gamma_C = e^{g_n}:
//
//   forward:  A = strict_lower(diag(beta) (Gamma . K K^T)),  M = (I + A)^-1,
//             T = M diag(beta),  X = V - diag(gamma) K S,  U = T X,
//             P = lower(Gamma . Q K^T),  O = diag(gamma) Q S + P U,
//             S' = gamma_C S + (diag(s) K)^T U
//
//   backward, from dO and dS' (the gradient reaching the chunk's end state):
//     dU  = P^T dO + diag(s) K dS'        dY = M^T dU,  dX = diag(beta) dY,  dV = dX
//     dS  = gamma_C dS' + Q^T diag(gamma) dO - K^T diag(gamma) dX   (to the chunk before)
//     dP  = lower(dO U^T)                 dQ = diag(gamma) dO S^T + (dP . Gamma) K
//     dA  = strict_lower(-dY U^T)         dbeta_t = sum_c dY_tc X_tc + sum_i dA_ti Gamma_ti (K K^T)_ti
//     dG  = dA . diag(beta) Gamma
//     dK  = (dP . Gamma)^T Q - diag(gamma) dX S^T + diag(s) U dS'^T + (dG + dG^T) K
//     gates: dgamma_t = sum_c (dO . Q S - dX . K S)_tc,  ds_t = sum_c (K dS' . U)_tc,
//            dGamma = dA . diag(beta) K K^T + dP . Q K^T,
//            dg = gamma . dgamma + rowsum(Gamma . dGamma) - colsum(Gamma . dGamma) - s . ds,
//            dg_n += gamma_C <S, dS'> + sum_t s_t ds_t,
//            d alpha_i = (sum_{t >= i} dg_t) / alpha_i.
//
// (dA uses M^T dU (diag(beta) X)^T M^T = dY (T X)^T = dY U^T.)
//
// Kernels: the token-by-token forward writes every chunk's start state
// (recurrent.hip, states mode); then one workgroup per (sequence, value head)
// walks that unit's chunks in reverse, carrying dS, with every intermediate
// of a chunk in fp32 in the unit's own slice of the workspace; then the
// gradients of each query/key head are summed over the value heads that read
// it.  All arithmetic is fp32; the products are workgroup-cooperative loops
// over LDS (the C x C matrices) and the workspace (each output element owned
// by one thread, so the results are the same run to run).  This is the first, correctness-first GPU backward: its
// reverse chain has the forward scan's shape, and moving its products onto
// MFMA with LDS-staged operands is the next step.
#include "launch.hpp"

namespace gdn {

namespace {

constexpr int kBwdThreads = 512;

template <typename T>
struct BwdArgs {
  const T *q, *k, *v, *d_o;
  const float *alpha, *beta, *dhT;
  const float *states;      // [slots, H_v, d_k, d_v] chunk-start states
  float *dq_part, *dk_part; // [tokens, H_v, d_k]
  float *dv, *dalpha, *dbeta, *dh0;
  float *scratch;
  int64_t unit_floats;
  int H_qk, H_v, d_k, d_v, group, n_units;
  SeqGeom geo;
};

// Per-unit scratch layout in global memory, in floats, for chunk C and sizes
// DK, DV (the chunk's C x C matrices live in LDS).
struct BwdLayout {
  int64_t K, Q, V, dO, be, al, gg, ga, sc, dg, KS, QS, X, U, KdS, dU, dY, dX, dS0, dS1, dQ, dK, total;
  __host__ __device__ BwdLayout(int C, int DK, int DV) {
    int64_t o = 0;
    auto take = [&](int64_t n) { const int64_t r = o; o += (n + 63) & ~int64_t(63); return r; };
    K = take(int64_t(C) * DK); Q = take(int64_t(C) * DK); V = take(int64_t(C) * DV); dO = take(int64_t(C) * DV);
    be = take(C); al = take(C); gg = take(C); ga = take(C); sc = take(C); dg = take(C);
    KS = take(int64_t(C) * DV); QS = take(int64_t(C) * DV); X = take(int64_t(C) * DV); U = take(int64_t(C) * DV);
    KdS = take(int64_t(C) * DV); dU = take(int64_t(C) * DV); dY = take(int64_t(C) * DV); dX = take(int64_t(C) * DV);
    dS0 = take(int64_t(DK) * DV); dS1 = take(int64_t(DK) * DV);
    dQ = take(int64_t(C) * DK); dK = take(int64_t(C) * DK);
    total = o;
  }
};

// Four k steps of a thread's 1 x 4 output strip: A(i, k..k+3) and
// B(k..k+3, j0..j0+3), as 16-byte loads where the operand is contiguous
// along that index (every array here is 16-byte aligned, with row strides
// that are multiples of four floats).
template <bool A_ROW, bool B_ROW>
__device__ __forceinline__ void strip_step(const float *a, int acs, const float *b, int brs, int bcs, int kk,
                                           const float *ks, float (&sum)[4]) {
  float av[4], bv[4][4];
  if constexpr (A_ROW) {
    const float4 x = *reinterpret_cast<const float4 *>(a + kk);
    av[0] = x.x; av[1] = x.y; av[2] = x.z; av[3] = x.w;
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) av[u] = a[int64_t(kk + u) * acs];
  }
  if (ks) {
#pragma unroll
    for (int u = 0; u < 4; ++u) av[u] *= ks[kk + u];
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if constexpr (B_ROW) {
      const float4 y = *reinterpret_cast<const float4 *>(b + int64_t(kk + u) * brs);
      bv[u][0] = y.x; bv[u][1] = y.y; bv[u][2] = y.z; bv[u][3] = y.w;
    } else {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) bv[u][jj] = b[int64_t(kk + u) * brs + int64_t(jj) * bcs];
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) sum[jj] += av[u] * bv[u][jj];
}

template <bool A_ROW, bool B_ROW>
__device__ void wg_gemm_t(float *C, int ldc, const float *A, int ars, int acs, const float *B, int brs, int bcs,
                          int m, int n, int K, float alpha, const float *rs, const float *ks, bool acc) {
  const int nb = (n + 3) >> 2;
  for (int idx = threadIdx.x; idx < m * nb; idx += kBwdThreads) {
    const int i = idx / nb, j0 = 4 * (idx - i * nb);
    const int nj = min(4, n - j0);
    const float *a = A + int64_t(i) * ars;
    const float *b = B + int64_t(j0) * bcs;
    float sum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    int kk = 0;
    if (nj == 4)
      for (; kk + 4 <= K; kk += 4) strip_step<A_ROW, B_ROW>(a, acs, b, brs, bcs, kk, ks, sum);
    for (; kk < K; ++kk) {
      const float x = a[int64_t(kk) * acs] * (ks ? ks[kk] : 1.0f);
      for (int jj = 0; jj < nj; ++jj) sum[jj] += x * b[int64_t(kk) * brs + int64_t(jj) * bcs];
    }
    const float scale = alpha * (rs ? rs[i] : 1.0f);
    float *c = C + int64_t(i) * ldc + j0;
    for (int jj = 0; jj < nj; ++jj) c[jj] = acc ? c[jj] + scale * sum[jj] : scale * sum[jj];
  }
}

// C[i][j] = (acc ? C[i][j] : 0) + alpha rs[i] sum_{k<K} A(i, k) ks[k] B(k, j)
// with A(i, k) = A[i ars + k acs], B(k, j) = B[k brs + j bcs] (rs, ks: 1 when
// null).  A thread owns four adjacent outputs of a row and walks k four steps
// at a time; the operands may sit in LDS or in global memory.  Every output
// is summed in k order by one thread, so the result does not depend on the
// launch.
__device__ void wg_gemm(float *C, int ldc, const float *A, int ars, int acs, const float *B, int brs, int bcs,
                        int m, int n, int K, float alpha = 1.0f, const float *rs = nullptr,
                        const float *ks = nullptr, bool acc = false) {
  if (acs == 1 && bcs == 1)
    wg_gemm_t<true, true>(C, ldc, A, ars, acs, B, brs, bcs, m, n, K, alpha, rs, ks, acc);
  else if (acs == 1)
    wg_gemm_t<true, false>(C, ldc, A, ars, acs, B, brs, bcs, m, n, K, alpha, rs, ks, acc);
  else if (bcs == 1)
    wg_gemm_t<false, true>(C, ldc, A, ars, acs, B, brs, bcs, m, n, K, alpha, rs, ks, acc);
  else
    wg_gemm_t<false, false>(C, ldc, A, ars, acs, B, brs, bcs, m, n, K, alpha, rs, ks, acc);
}

// Sum over the block of one value per thread (red: kBwdThreads floats of LDS).
__device__ float wg_sum(float x, float *red) {
  red[threadIdx.x] = x;
  __syncthreads();
  for (int s = kBwdThreads / 2; s > 0; s >>= 1) {
    if (int(threadIdx.x) < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

}  // namespace

template <typename T>
__global__ __launch_bounds__(kBwdThreads) void chunk_bwd_kernel(BwdArgs<T> a) {
  const int u = blockIdx.x;
  if (u >= a.n_units) return;
  const int tid = threadIdx.x;
  const int s = u / a.H_v, h = u - s * a.H_v, hq = h / a.group;
  const int C = a.geo.chunk, DK = a.d_k, DV = a.d_v;
  const BwdLayout L(C, DK, DV);
  float *w = a.scratch + int64_t(u) * a.unit_floats;
  float *Kc = w + L.K, *Qc = w + L.Q, *Vc = w + L.V, *dOc = w + L.dO;
  float *be = w + L.be, *al = w + L.al, *gg = w + L.gg, *ga = w + L.ga, *sc = w + L.sc, *dg = w + L.dg;
  // the chunk's C x C matrices (C <= 64): Gamma, K K^T, Q K^T, M, T, P, dP, dA
  __shared__ __attribute__((aligned(16))) float cc[8][64 * 64];
  float *Gm = cc[0], *KK = cc[1], *QK = cc[2], *Mi = cc[3], *Tm = cc[4], *Pm = cc[5], *dP = cc[6], *dA = cc[7];
  float *KS = w + L.KS, *QS = w + L.QS, *X = w + L.X, *U = w + L.U, *KdS = w + L.KdS, *dU = w + L.dU;
  float *dY = w + L.dY, *dX = w + L.dX, *dS = w + L.dS0, *dSn = w + L.dS1, *dQ = w + L.dQ, *dK = w + L.dK;
  __shared__ float red[kBwdThreads];

  const int64_t unit_state = (int64_t(s) * a.H_v + h) * DK * DV;
  for (int idx = tid; idx < DK * DV; idx += kBwdThreads) dS[idx] = a.dhT ? a.dhT[unit_state + idx] : 0.0f;
  __syncthreads();

  int start, end;
  a.geo.seq_bounds(s, start, end);
  const int n_chunks = (end - start + C - 1) / C;
  const int c_first = a.geo.first_chunk(s);
  for (int cc = n_chunks - 1; cc >= 0; --cc) {
    const int slot = c_first + cc;
    if (slot >= a.geo.n_slots) continue;  // (never for a well-formed batch)
    const int tok0 = start + cc * C;
    const int n = min(C, end - tok0);
    const float *S = a.states + (int64_t(slot) * a.H_v + h) * DK * DV;

    // ---- the chunk's operands in fp32 ----
    for (int idx = tid; idx < n * DK; idx += kBwdThreads) {
      const int t = idx / DK, c = idx - t * DK;
      const int64_t g = (int64_t(tok0 + t) * a.H_qk + hq) * DK + c;
      Kc[idx] = to_f32(a.k[g]);
      Qc[idx] = to_f32(a.q[g]);
    }
    for (int idx = tid; idx < n * DV; idx += kBwdThreads) {
      const int t = idx / DV, c = idx - t * DV;
      const int64_t g = (int64_t(tok0 + t) * a.H_v + h) * DV + c;
      Vc[idx] = to_f32(a.v[g]);
      dOc[idx] = to_f32(a.d_o[g]);
    }
    if (tid < n) {
      const int64_t g = int64_t(tok0 + tid) * a.H_v + h;
      be[tid] = a.beta[g];
      al[tid] = a.alpha[g];
    }
    __syncthreads();
    // chunk-local cumulative log gate (ln alpha clamped at -200, as in the
    // forward: e^-200 is zero in fp32)
    if (tid == 0) {
      float g = 0.0f;
      for (int t = 0; t < n; ++t) {
        g += fmaxf(logf(al[t]), -200.0f);
        gg[t] = g;
      }
    }
    __syncthreads();
    const float g_last = gg[n - 1];
    const float gC = expf(g_last);
    if (tid < n) {
      ga[tid] = expf(gg[tid]);
      sc[tid] = expf(g_last - gg[tid]);
    }
    for (int idx = tid; idx < n * C; idx += kBwdThreads) {
      const int t = idx / C, i = idx - t * C;
      Gm[idx] = i <= t && i < n ? expf(gg[t] - gg[i]) : 0.0f;
    }
    wg_gemm(KK, C, Kc, DK, 1, Kc, 1, DK, n, n, DK);  // K K^T
    wg_gemm(QK, C, Qc, DK, 1, Kc, 1, DK, n, n, DK);  // Q K^T
    __syncthreads();
    // A (strictly lower) into dA's slot, then M = (I + A)^-1 by forward
    // substitution, one thread per column
    for (int idx = tid; idx < n * C; idx += kBwdThreads) {
      const int t = idx / C, i = idx - t * C;
      dA[idx] = i < t ? be[t] * Gm[idx] * KK[t * C + i] : 0.0f;
    }
    __syncthreads();
    if (tid < n) {
      const int j = tid;
      for (int t = 0; t < n; ++t) {
        float m = t == j ? 1.0f : 0.0f;
        if (t > j) {
          for (int i = j; i < t; ++i) m -= dA[t * C + i] * Mi[i * C + j];
        }
        Mi[t * C + j] = m;
      }
    }
    __syncthreads();
    for (int idx = tid; idx < n * C; idx += kBwdThreads) {
      const int t = idx / C, i = idx - t * C;
      Tm[idx] = i < n ? Mi[idx] * be[i] : 0.0f;
      Pm[idx] = i <= t ? QK[idx] * Gm[idx] : 0.0f;
    }
    wg_gemm(KS, DV, Kc, DK, 1, S, DV, 1, n, DV, DK);    // K S
    wg_gemm(QS, DV, Qc, DK, 1, S, DV, 1, n, DV, DK);    // Q S
    wg_gemm(KdS, DV, Kc, DK, 1, dS, DV, 1, n, DV, DK);  // K dS'
    __syncthreads();
    for (int idx = tid; idx < n * DV; idx += kBwdThreads) X[idx] = Vc[idx] - ga[idx / DV] * KS[idx];
    __syncthreads();
    wg_gemm(U, DV, Tm, C, 1, X, DV, 1, n, DV, n);   // U = T X
    wg_gemm(dU, DV, Pm, 1, C, dOc, DV, 1, n, DV, n);  // P^T dO
    __syncthreads();
    for (int idx = tid; idx < n * DV; idx += kBwdThreads) dU[idx] += sc[idx / DV] * KdS[idx];
    __syncthreads();
    wg_gemm(dY, DV, Mi, 1, C, dU, DV, 1, n, DV, n);  // M^T dU
    __syncthreads();
    for (int idx = tid; idx < n * DV; idx += kBwdThreads) {
      const int t = idx / DV, c = idx - t * DV;
      const float x = be[t] * dY[idx];
      dX[idx] = x;
      a.dv[(int64_t(tok0 + t) * a.H_v + h) * DV + c] = x;
    }
    __syncthreads();
    // dS to the chunk before: gamma_C dS' + Q^T diag(gamma) dO - K^T diag(gamma) dX
    wg_gemm(dSn, DV, Qc, 1, DK, dOc, DV, 1, DK, DV, n, 1.0f, nullptr, ga);
    wg_gemm(dSn, DV, Kc, 1, DK, dX, DV, 1, DK, DV, n, -1.0f, nullptr, ga, true);
    wg_gemm(dP, C, dOc, DV, 1, U, 1, DV, n, n, DV);          // dO U^T (masked below)
    wg_gemm(dA, C, dY, DV, 1, U, 1, DV, n, n, DV, -1.0f);    // -dY U^T (masked below)
    wg_gemm(dQ, DK, dOc, DV, 1, S, 1, DV, n, DK, DV, 1.0f, ga);  // diag(gamma) dO S^T
    __syncthreads();
    for (int idx = tid; idx < DK * DV; idx += kBwdThreads) dSn[idx] += gC * dS[idx];
    for (int idx = tid; idx < n * C; idx += kBwdThreads) {
      const int t = idx / C, i = idx - t * C;
      const float p = i <= t ? dP[idx] : 0.0f;
      const float d = i < t ? dA[idx] : 0.0f;
      dP[idx] = p;
      dA[idx] = d;
      Pm[idx] = p * Gm[idx];           // dP . Gamma
      Tm[idx] = d * be[t] * Gm[idx];   // dG
    }
    __syncthreads();
    wg_gemm(dQ, DK, Pm, C, 1, Kc, DK, 1, n, DK, n, 1.0f, nullptr, nullptr, true);  // + (dP . Gamma) K
    wg_gemm(dK, DK, Pm, 1, C, Qc, DK, 1, n, DK, n);                                 // (dP . Gamma)^T Q
    __syncthreads();
    wg_gemm(dK, DK, dX, DV, 1, S, 1, DV, n, DK, DV, -1.0f, ga, nullptr, true);      // - diag(gamma) dX S^T
    __syncthreads();
    wg_gemm(dK, DK, U, DV, 1, dS, 1, DV, n, DK, DV, 1.0f, sc, nullptr, true);       // + diag(s) U dS'^T
    __syncthreads();
    wg_gemm(dK, DK, Tm, C, 1, Kc, DK, 1, n, DK, n, 1.0f, nullptr, nullptr, true);   // + dG K
    __syncthreads();
    wg_gemm(dK, DK, Tm, 1, C, Kc, DK, 1, n, DK, n, 1.0f, nullptr, nullptr, true);   // + dG^T K
    // Gamma . dGamma into Mi's slot (M is no longer needed)
    for (int idx = tid; idx < n * C; idx += kBwdThreads) {
      const int t = idx / C, i = idx - t * C;
      Mi[idx] = i <= t ? Gm[idx] * (dA[idx] * be[t] * KK[idx] + dP[idx] * QK[idx]) : 0.0f;
    }
    __syncthreads();
    // per-token sums: dbeta, dgamma, ds
    float ds_t = 0.0f;
    if (tid < n) {
      const int t = tid;
      float db = 0.0f, dgam = 0.0f, dss = 0.0f;
      for (int c = 0; c < DV; ++c) {
        db += dY[t * DV + c] * X[t * DV + c];
        dgam += dOc[t * DV + c] * QS[t * DV + c] - dX[t * DV + c] * KS[t * DV + c];
        dss += KdS[t * DV + c] * U[t * DV + c];
      }
      float row = 0.0f, col = 0.0f;
      for (int i = 0; i < n; ++i) {
        db += dA[t * C + i] * Gm[t * C + i] * KK[t * C + i];
        row += Mi[t * C + i];
        col += Mi[i * C + t];
      }
      a.dbeta[int64_t(tok0 + t) * a.H_v + h] = db;
      dg[t] = ga[t] * dgam + row - col - sc[t] * dss;
      ds_t = sc[t] * dss;
    }
    // gamma_C <S, dS'> + sum_t s_t ds_t joins the last slot's dg
    float part = 0.0f;
    for (int idx = tid; idx < DK * DV; idx += kBwdThreads) part += S[idx] * dS[idx];
    const float sd = wg_sum(part, red);
    const float sds = wg_sum(ds_t, red);
    if (tid == 0) {
      dg[n - 1] += gC * sd + sds;
      float acc = 0.0f;
      for (int t = n - 1; t >= 0; --t) {
        acc += dg[t];
        a.dalpha[int64_t(tok0 + t) * a.H_v + h] = acc / al[t];
      }
    }
    for (int idx = tid; idx < n * DK; idx += kBwdThreads) {
      const int t = idx / DK, c = idx - t * DK;
      const int64_t g = (int64_t(tok0 + t) * a.H_v + h) * DK + c;
      a.dq_part[g] = dQ[idx];
      a.dk_part[g] = dK[idx];
    }
    __syncthreads();
    float *tmp = dS;
    dS = dSn;
    dSn = tmp;
  }
  if (a.dh0)
    for (int idx = tid; idx < DK * DV; idx += kBwdThreads) a.dh0[unit_state + idx] = dS[idx];
}

// dq (and dk) of a query/key head: the sum over the value heads that read it.
__global__ __launch_bounds__(256) void group_sum_kernel(const float *part, float *out, int64_t tokens, int H_qk,
                                                        int group, int d) {
  const int64_t total = tokens * H_qk * d;
  for (int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x; idx < total; idx += int64_t(gridDim.x) * 256) {
    const int64_t tok = idx / (int64_t(H_qk) * d);
    const int rem = int(idx - tok * H_qk * d);
    const int hq = rem / d, c = rem - hq * d;
    float sum = 0.0f;
    for (int j = 0; j < group; ++j) sum += part[(tok * (int64_t(H_qk) * group) + hq * group + j) * d + c];
    out[idx] = sum;
  }
}

size_t bwd_unit_floats(int chunk, int d_k, int d_v) { return size_t(BwdLayout(chunk, d_k, d_v).total); }

template <typename T>
static hipError_t launch_chunk_bwd_t(const BwdProblem &b, hipStream_t st) {
  const Problem &p = b.p;
  BwdArgs<T> a;
  a.q = static_cast<const T *>(p.q);
  a.k = static_cast<const T *>(p.k);
  a.v = static_cast<const T *>(p.v);
  a.d_o = static_cast<const T *>(b.d_o);
  a.alpha = p.alpha;
  a.beta = p.beta;
  a.dhT = b.dhT;
  a.states = b.states;
  a.dq_part = b.dq_part;
  a.dk_part = b.dk_part;
  a.dv = b.dv;
  a.dalpha = b.dalpha;
  a.dbeta = b.dbeta;
  a.dh0 = b.dh0;
  a.scratch = b.scratch;
  a.unit_floats = int64_t(bwd_unit_floats(p.chunk, p.d_k, p.d_v));
  a.H_qk = p.H_qk;
  a.H_v = p.H_v;
  a.d_k = p.d_k;
  a.d_v = p.d_v;
  a.group = p.H_v / p.H_qk;
  a.n_units = p.n_seqs * p.H_v;
  a.geo = make_geom(p, &b.ws);
  if (a.n_units == 0) return hipSuccess;
  hipLaunchKernelGGL(chunk_bwd_kernel<T>, dim3(unsigned(a.n_units)), dim3(kBwdThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t tokens = p.n_tokens();
  const int64_t total = tokens * p.H_qk * p.d_k;
  if (total == 0) return hipSuccess;
  const unsigned blocks = unsigned(std::min<int64_t>((total + 255) / 256, 1 << 16));
  hipLaunchKernelGGL(group_sum_kernel, dim3(blocks), dim3(256), 0, st, b.dq_part, b.dq, tokens, p.H_qk, a.group,
                     p.d_k);
  hipLaunchKernelGGL(group_sum_kernel, dim3(blocks), dim3(256), 0, st, b.dk_part, b.dk, tokens, p.H_qk, a.group,
                     p.d_k);
  return hipGetLastError();
}

hipError_t launch_chunk_bwd(const BwdProblem &b, hipStream_t st) {
  return b.p.dtype == 1 ? launch_chunk_bwd_t<bf16_t>(b, st) : launch_chunk_bwd_t<float>(b, st);
}

}  // namespace gdn
