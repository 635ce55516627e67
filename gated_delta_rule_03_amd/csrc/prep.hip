// Intra-chunk kernel: the WY / UT form of one chunk.
//
// Inside a chunk the delta rule's pseudo-values solve one unit lower
// triangular system ("Attention as Matrix Algebra: From Softmax to the Delta
// Rule", section 8; "From KV Cache to a State Matrix", section "Chunkwise
// training for DeltaNet" -- the compact WY / UT transform).  With the decay
// gate of "Linear attention" Eq. (1) carried as chunk-local log gates g
// (Gamma_ti = 2^(g_t - g_i), i <= t), the chunk equations are
//
//   A_ti = beta_t Gamma_ti k_t^T k_i   (i < t),      T = (I + A)^-1 diag(beta)
//   U    = T (V - diag(gamma) K S)                    (pseudo-values)
//   O    = diag(gamma) Q S + P U,       P_ti = Gamma_ti q_t^T k_i  (i <= t)
//   S   <- gamma_C S + Ktilde^T U,      Ktilde_i = 2^(g_C - g_i) k_i
//
// This kernel computes everything that does not depend on the incoming state:
// T, P and Ktilde^T for one (chunk, value head).  It writes them to the
// workspace in MFMA fragment order, ready for the sequential state scan.
// A chunk is padded to 64 token slots.  Padded slots carry beta = 0 and the
// chunk's last gate; their k and q rows (zero, or a copy of the chunk's last
// row when staged) only ever meet exact zeros: rows and columns of A and T
// vanish with beta, Ktilde^T columns are written as zeros, and P rows of
// padded tokens only reach outputs that are never stored.
//
// MFMA: k k^T and k q^T are dense 64 x 64 x d_k contractions (bf16 MFMA for
// bf16 inputs, fp32 MFMA for fp32 inputs).  The triangular inverse is fp32:
// four 16 x 16 diagonal blocks by forward substitution (one lane per column),
// then block forward substitution for the off-diagonal blocks.
#include "launch.hpp"
#include "stage.hpp"

namespace gdn {

template <typename T>
struct PrepArgs {
  const T *q, *k;
  const float *g, *beta;
  T *entries;
  int H_qk, H_v, d_k, group;
  SeqGeom geo;
};

// kStaged (bf16, d_k = 128): the chunk's k and q rows are first copied into
// swizzled LDS row tiles with every load in flight at once, and all fragment
// reads come from LDS.  Otherwise fragments are read from global memory.
template <typename T, bool kStaged>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs<T> a) {
  const int c = blockIdx.x;
  const int h = blockIdx.y;
  int s, tok0, len;
  if (!a.geo.locate(c, s, tok0, len)) return;
  const int hq = h / a.group;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  __shared__ float sg[64], sb[64];
  __shared__ float sA[64][65];
  __shared__ float sM[64][65];
  __shared__ float sY[3][16][17];
  __shared__ __attribute__((aligned(16))) bf16_t sK[kStaged ? 64 * 128 : 1];
  __shared__ __attribute__((aligned(16))) bf16_t sQ[kStaged ? 64 * 128 : 1];

  const int64_t stride = int64_t(a.H_qk) * a.d_k;
  const T *kb = a.k + int64_t(tok0) * stride + int64_t(hq) * a.d_k;
  const T *qb = a.q + int64_t(tok0) * stride + int64_t(hq) * a.d_k;
  if constexpr (kStaged) {
    // 16 one-KiB pieces per tile; each wave issues 4 of each.
    stage_rowtile(sK, kb, stride, len, lane, 4 * wave, 4);
    stage_rowtile(sQ, qb, stride, len, lane, 4 * wave, 4);
  }
  if (tid < 64) {
    const int t = tid < len ? tid : len - 1;
    const int64_t idx = int64_t(tok0 + t) * a.H_v + h;
    sg[tid] = a.g[idx];
    sb[tid] = tid < len ? a.beta[idx] : 0.0f;
  }
  if constexpr (kStaged) wait_vmem();
  __syncthreads();

  // Row fragment of k (src 0) or q (src 1): rows 16 r + (lane & 15),
  // contraction block kk.  Staged rows past the chunk repeat its last row;
  // those rows and columns meet beta = 0 or are never stored.
  auto frag = [&](int src, int r, int kk) -> Frag<T> {
    if constexpr (kStaged) {
      return rowtile_frag(src == 0 ? sK : sQ, r, kk, lane);
    } else {
      return load_row_frag(src == 0 ? kb : qb, stride, 16 * r + (lane & 15), len, 32 * kk,
                           a.d_k, lane);
    }
  };
  T *entry = a.entries + (int64_t(c) * a.H_v + h) * kEntryElems;
  T *fragT = entry;
  T *fragP = entry + 8 * kFragElems;
  T *fragK = entry + 16 * kFragElems;
  const int nkb = (a.d_k + 31) / 32;

  // ---- 20 tiles: 10 of A = K K^T (rt >= ct), 10 of P^T = K Q^T (ri <= ct) ----
  for (int tile = wave; tile < 20; tile += 4) {
    const bool isA = tile < 10;
    int r, cc;
    {
      // enumerate lower-triangular pairs (r >= cc) for A, upper (r <= cc) for P^T
      int idx = isA ? tile : tile - 10, rr = 0;
      while (idx > rr) { idx -= rr + 1; ++rr; }
      if (isA) { r = rr; cc = idx; } else { r = idx; cc = rr; }
    }
    f32x4_t acc = zero4();
    for (int kk = 0; kk < nkb; ++kk) acc = mfma(frag(0, r, kk), frag(isA ? 0 : 1, cc, kk), acc);
    const int col = 16 * cc + (lane & 15);
    if (isA) {
      // rows t, column i: A_ti for i < t
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * r + 4 * (lane >> 4) + e;
        const float gam = exp2f(sg[t] - sg[col <= t ? col : t]);
        sA[t][col] = col < t ? sb[t] * gam * acc[e] : 0.0f;
      }
    } else {
      // P^T tile: rows i = 16r + ..., column t = col.  Lane layout equals the
      // A-fragment layout of P (row t, contraction i): write 4 elements.
      Frag<T> half;
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * r + 4 * (lane >> 4) + e;
        const int t = col;
        const float gam = exp2f(sg[t] - sg[i <= t ? i : t]);
        half.set(e, i <= t ? gam * acc[e] : 0.0f);
      }
      T *dst = fragP + (cc * 2 + (r >> 1)) * kFragElems + 8 * lane + 4 * (r & 1);
      for (int e = 0; e < 4; ++e) dst[e] = from_f32<T>(half.get(e));
    }
  }
  // zero halves of P fragments whose P^T tile lies below the diagonal (ri > ct)
  for (int z = wave; z < 6; z += 4) {
    int idx = z, rr = 1;
    while (idx >= rr) { idx -= rr; ++rr; }
    const int ri = rr, ct = idx;  // ri > ct
    T *dst = fragP + (ct * 2 + (ri >> 1)) * kFragElems + 8 * lane + 4 * (ri & 1);
    for (int e = 0; e < 4; ++e) dst[e] = from_f32<T>(0.0f);
  }
  __syncthreads();

  // ---- M = (I + A)^-1: diagonal 16 x 16 blocks, one lane per column ----
  if (wave == 0) {
    const int b = lane >> 4, col = lane & 15;
    float x[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float acc = (t == col) ? 1.0f : 0.0f;
#pragma unroll
      for (int i = 0; i < t; ++i) acc -= sA[16 * b + t][16 * b + i] * x[i];
      x[t] = acc;
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) sM[16 * b + t][16 * b + col] = x[t];
  }
  __syncthreads();
  // ---- off-diagonal blocks: M_bc = -M_bb sum_{j=c}^{b-1} A_bj M_jc ----
  {
    const int t = tid >> 4, col = tid & 15;
    for (int br = 1; br < 4; ++br) {
      for (int cb = 0; cb < br; ++cb) {
        float y = 0.0f;
        for (int j = cb; j < br; ++j)
#pragma unroll
          for (int i = 0; i < 16; ++i) y += sA[16 * br + t][16 * j + i] * sM[16 * j + i][16 * cb + col];
        sY[cb][t][col] = y;
      }
      __syncthreads();
      for (int cb = 0; cb < br; ++cb) {
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) m -= sM[16 * br + t][16 * br + i] * sY[cb][i][col];
        sM[16 * br + t][16 * cb + col] = m;
      }
      __syncthreads();
    }
  }

  // ---- T = M diag(beta) as A fragments (row t, contraction i) ----
  for (int f = wave; f < 8; f += 4) {
    const int rt = f >> 1, kk = f & 1;
    const int t = 16 * rt + (lane & 15);
    Frag<T> fr;
    for (int j = 0; j < 8; ++j) {
      const int i = 32 * kk + kappa(lane, j);
      fr.set(j, (i >> 4) <= (t >> 4) ? sM[t][i] * sb[i] : 0.0f);
    }
    store_frag(fragT + f * kFragElems, lane, fr);
  }

  // ---- Ktilde^T as A fragments (row m of d_k, contraction over tokens i) ----
  const float g_last = sg[63];
  for (int f = wave; f < 16; f += 4) {
    const int rm = f >> 1, kk = f & 1;
    const int m = 16 * rm + (lane & 15);
    Frag<T> fr;
    for (int j = 0; j < 8; ++j) {
      const int i = 32 * kk + kappa(lane, j);
      float x = 0.0f;
      if (i < len && m < a.d_k) {
        float kv;
        if constexpr (kStaged) kv = to_f32(sK[rowtile_off(i, m)]);
        else kv = to_f32(kb[int64_t(i) * stride + m]);
        x = exp2f(g_last - sg[i]) * kv;
      }
      fr.set(j, x);
    }
    store_frag(fragK + f * kFragElems, lane, fr);
  }
}

template <typename T, bool kStaged>
static hipError_t launch_prep_t(const Problem &p, const Workspace &ws, hipStream_t st) {
  PrepArgs<T> a;
  a.q = static_cast<const T *>(p.q);
  a.k = static_cast<const T *>(p.k);
  a.g = ws.g;
  a.beta = p.beta;
  a.entries = static_cast<T *>(ws.entries);
  a.H_qk = p.H_qk;
  a.H_v = p.H_v;
  a.d_k = p.d_k;
  a.group = p.H_v / p.H_qk;
  a.geo = make_geom(p, &ws);
  const int64_t slots = chunk_slots(p);
  hipLaunchKernelGGL((prep_kernel<T, kStaged>), dim3(unsigned(slots), unsigned(p.H_v)), dim3(256),
                     0, st, a);
  return hipGetLastError();
}

hipError_t launch_prep(const Problem &p, const Workspace &ws, hipStream_t st) {
  if (chunk_slots(p) == 0) return hipSuccess;
  if (p.dtype == 1)
    return p.d_k == 128 ? launch_prep_t<bf16_t, true>(p, ws, st)
                        : launch_prep_t<bf16_t, false>(p, ws, st);
  return launch_prep_t<float, false>(p, ws, st);
}

}  // namespace gdn
