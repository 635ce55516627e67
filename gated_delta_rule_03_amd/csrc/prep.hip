// Intra-chunk kernel: the cumulative gate and the WY / UT form of one chunk.
//
// Gate.  The decay of "Linear attention" Eq. (1) compounds inside a chunk:
// the state reaching token t from the chunk start has been scaled by
// prod_{i<=t} alpha_i.  It is kept in the log domain as the chunk-local
// prefix sum g_t = sum_{i<=t} log2 alpha_i (a wave-level inclusive scan), so
// every factor below is exp2 of a difference g_t - g_i <= 0 (the
// prefix-product structure of "From KV Cache to a State Matrix", section
// "Chunkwise training for DeltaNet").  log2 alpha is clamped at -288, so
// alpha = 0 stays finite and still flushes every product through it to 0.
//
// WY / UT form.  Inside a chunk the delta rule's pseudo-values solve one
// unit lower triangular system ("Attention as Matrix Algebra: From Softmax to
// the Delta Rule", section 8; "From KV Cache to a State Matrix", section
// "Chunkwise training for DeltaNet").  With Gamma_ti = 2^(g_t - g_i):
//
//   A_ti = beta_t Gamma_ti k_t^T k_i   (i < t),      T = (I + A)^-1 diag(beta)
//   U    = T (V - diag(gamma) K S)                    (pseudo-values)
//   O    = diag(gamma) Q S + P U,       P_ti = Gamma_ti q_t^T k_i  (i <= t)
//   S   <- gamma_C S + K^T diag(2^(g_C - g)) U
//
// This kernel computes what does not depend on the incoming state -- T, P and
// the gate factors gamma_t = 2^g_t and s_t = 2^(g_C - g_t) for one (chunk,
// value head) -- and writes them to the workspace entry (T and P in MFMA
// fragment order, then the gate block).
//
// MFMA: k k^T and k q^T are dense 64 x 64 x d_k contractions (bf16 MFMA for
// bf16 inputs, fp32 MFMA for fp32 inputs).  The triangular inverse is fp32:
// four 16 x 16 diagonal blocks by forward substitution (one lane per column),
// then block forward substitution for the off-diagonal blocks.
//
// Padding: a chunk is padded to 64 token slots.  Padded slots carry beta = 0
// and the last token's gate; their k and q rows (zero, or a copy of the
// chunk's last row when staged) only ever meet exact zeros: their rows and
// columns of A and T vanish with beta, and their rows of P only reach outputs
// that are never stored.
#include "launch.hpp"
#include "stage.hpp"

namespace gdn {

template <typename T>
struct PrepArgs {
  const T *q, *k;
  const float *alpha, *beta;
  char *entries;
  int H_qk, H_v, d_k, group;
  SeqGeom geo;
};

// kStaged (bf16, d_k = 128): the chunk's k and q rows are first copied into
// swizzled LDS row tiles with every load in flight at once, and fragment reads
// come from LDS.  Otherwise fragments are read from global memory.
template <typename T, bool kStaged>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs<T> a) {
  const int c = blockIdx.x;
  const int h = blockIdx.y;
  int s, tok0, len;
  if (!a.geo.locate(c, s, tok0, len)) return;
  const int hq = h / a.group;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // LDS: the staged k/q tiles (32 KiB) are dead once the tiles are in
  // registers; A and M = (I + A)^-1 then reuse the same bytes.
  constexpr int kLdsMain = 2 * 64 * 65 * 4;
  __shared__ __attribute__((aligned(16))) char smem[kLdsMain];
  __shared__ float sY[3][16][17];
  __shared__ float sg[64], sb[64];
  bf16_t *sK = reinterpret_cast<bf16_t *>(smem);
  bf16_t *sQ = sK + 64 * 128;
  float(*sA)[65] = reinterpret_cast<float(*)[65]>(smem);
  float(*sM)[65] = reinterpret_cast<float(*)[65]>(smem + 64 * 65 * 4);

  const int64_t stride = int64_t(a.H_qk) * a.d_k;
  const T *kb = a.k + int64_t(tok0) * stride + int64_t(hq) * a.d_k;
  const T *qb = a.q + int64_t(tok0) * stride + int64_t(hq) * a.d_k;
  if constexpr (kStaged) {
    static_assert(sizeof(T) == 2, "staged path is bf16");
    stage_rowtile(lds_ptr(sK), reinterpret_cast<const bf16_t *>(kb), stride, len, lane, 4 * wave, 4);
    stage_rowtile(lds_ptr(sQ), reinterpret_cast<const bf16_t *>(qb), stride, len, lane, 4 * wave, 4);
  }
  char *entry = a.entries + (int64_t(c) * a.H_v + h) * entry_bytes<T>();
  T *fragT = reinterpret_cast<T *>(entry);
  T *fragP = fragT + 8 * kFragElems;
  float *gate_out = reinterpret_cast<float *>(fragT + 16 * kFragElems);

  // ---- cumulative gate (wave 0): g_t for slot t, padded slots hold g_last ----
  if (wave == 0) {
    const int t = lane;
    const int64_t idx = int64_t(tok0 + min(t, len - 1)) * a.H_v + h;
    float x = t < len ? clamped_log2(a.alpha[idx]) : 0.0f;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float y = __shfl_up(x, d);
      if (lane >= d) x += y;
    }
    sg[t] = x;
    sb[t] = t < len ? a.beta[idx] : 0.0f;
    const float g_last = __shfl(x, 63);
    gate_out[t] = exp2f(x);             // gamma_t
    gate_out[64 + t] = exp2f(g_last - x);  // s_t
  }
  if constexpr (kStaged) wait_vmem();
  lds_barrier();

  auto frag = [&](int src, int r, int kk) -> Frag<T> {
    if constexpr (kStaged) {
      return rowtile_frag(src == 0 ? sK : sQ, r, kk, lane);
    } else {
      return load_row_frag(src == 0 ? kb : qb, stride, 16 * r + (lane & 15), len, 32 * kk,
                           a.d_k, lane);
    }
  };
  const int nkb = (a.d_k + 31) / 32;

  // ---- 20 tiles: 10 of A = K K^T (r >= cc), 10 of P^T = K Q^T (r <= cc) ----
  // This wave's tiles are wave + 4 n (n = 0..4), kept in registers.
  f32x4_t acc[5];
  int tr[5], tc[5];
#pragma unroll
  for (int n = 0; n < 5; ++n) {
    const int tile = wave + 4 * n;
    const bool isA = tile < 10;
    int idx = isA ? tile : tile - 10, rr = 0;
    while (idx > rr) { idx -= rr + 1; ++rr; }
    tr[n] = isA ? rr : idx;
    tc[n] = isA ? idx : rr;
    acc[n] = zero4();
    for (int kk = 0; kk < nkb; ++kk)
      acc[n] = mfma(frag(0, tr[n], kk), frag(isA ? 0 : 1, tc[n], kk), acc[n]);
  }
  lds_barrier();  // the k/q tiles are dead from here on

#pragma unroll
  for (int n = 0; n < 5; ++n) {
    const int tile = wave + 4 * n;
    const int r = tr[n], cc = tc[n];
    const int col = 16 * cc + (lane & 15);
    if (tile < 10) {
      // rows t, column i: A_ti for i < t
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * r + 4 * (lane >> 4) + e;
        const float gam = fast_exp2(sg[t] - sg[col <= t ? col : t]);
        sA[t][col] = col < t ? sb[t] * gam * acc[n][e] : 0.0f;
      }
    } else {
      // P^T tile (rows i = 16 r + ..., column t): its lane layout is the
      // A-fragment layout of P (row t, contraction i), so its 4 elements go
      // straight into half of fragment (t-tile, i-block).
      T *dst = fragP + (cc * 2 + (r >> 1)) * kFragElems + 8 * lane + 4 * (r & 1);
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * r + 4 * (lane >> 4) + e;
        const int t = col;
        const float gam = fast_exp2(sg[t] - sg[i <= t ? i : t]);
        dst[e] = from_f32<T>(i <= t ? gam * acc[n][e] : 0.0f);
      }
    }
  }
  // zero halves of P fragments whose P^T tile lies below the diagonal (ri > ct)
  for (int z = wave; z < 6; z += 4) {
    int idx = z, rr = 1;
    while (idx >= rr) { idx -= rr; ++rr; }
    const int ri = rr, ct = idx;
    T *dst = fragP + (ct * 2 + (ri >> 1)) * kFragElems + 8 * lane + 4 * (ri & 1);
    for (int e = 0; e < 4; ++e) dst[e] = from_f32<T>(0.0f);
  }
  lds_barrier();

  // ---- M = (I + A)^-1: diagonal 16 x 16 blocks, one lane per column ----
  if (wave == 0) {
    const int b = lane >> 4, col = lane & 15;
    float x[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float v = (t == col) ? 1.0f : 0.0f;
#pragma unroll
      for (int i = 0; i < t; ++i) v -= sA[16 * b + t][16 * b + i] * x[i];
      x[t] = v;
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) sM[16 * b + t][16 * b + col] = x[t];
  }
  lds_barrier();
  // ---- off-diagonal blocks: M_bc = -M_bb sum_{j=c}^{b-1} A_bj M_jc ----
  {
    const int t = tid >> 4, col = tid & 15;
    for (int br = 1; br < 4; ++br) {
      for (int cb = 0; cb < br; ++cb) {
        float y = 0.0f;
        for (int j = cb; j < br; ++j)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            y += sA[16 * br + t][16 * j + i] * sM[16 * j + i][16 * cb + col];
        sY[cb][t][col] = y;
      }
      lds_barrier();
      for (int cb = 0; cb < br; ++cb) {
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) m -= sM[16 * br + t][16 * br + i] * sY[cb][i][col];
        sM[16 * br + t][16 * cb + col] = m;
      }
      lds_barrier();
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
}

template <typename T, bool kStaged>
static hipError_t launch_prep_t(const Problem &p, const Workspace &ws, hipStream_t st) {
  PrepArgs<T> a;
  a.q = static_cast<const T *>(p.q);
  a.k = static_cast<const T *>(p.k);
  a.alpha = p.alpha;
  a.beta = p.beta;
  a.entries = static_cast<char *>(ws.entries);
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
