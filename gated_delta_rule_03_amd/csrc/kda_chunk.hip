// Chunked form of the delta rule with one decay rate per key channel.
//
// "Attention as Matrix Algebra: From Softmax to the Delta Rule", section 10,
// names Kimi Delta Attention: the gated delta rule with its own forget rate
// for each feature channel.  The channels are the key features (the rows of
// the keys x values state), so step t decays the state by diag(alpha_t).  The
// chunk algebra of section 8 of the same page ("Training the delta rule in
// chunks") carries over with the scalar cumulative gate replaced by a vector
// one.  Inside a chunk that starts from state S, with G_t = sum_{i<=t}
// log2 alpha_i (chunk-local, per channel) and Gamma_t = 2^G_t:
//
//   A_ti = beta_t sum_c k_tc k_ic 2^(G_tc - G_ic)   (i < t),  T = (I + A)^-1 diag(beta)
//   P_ti = sum_c q_tc k_ic 2^(G_tc - G_ic)          (i <= t)
//   Khat_t = Gamma_t . k_t,  Qhat_t = Gamma_t . q_t,  Ktil_i = 2^(G_C - G_i) . k_i
//   U  = T (V - Khat S)          pseudo-values
//   O  = Qhat S + P U            the chunk's outputs
//   S <- diag(Gamma_C) S + Ktil^T U
//
// (unrolling u_t = beta_t (v_t - (diag(alpha_t) S_{t-1})^T k_t) through the
// chunk exactly as for the scalar gate, with every scalar decay product
// replaced by its diagonal matrix).  Every exponent is a difference G_t - G_i
// <= 0 for i <= t, or G_t <= 0, so no factor exceeds one.  The exponent of
// A and P differs per channel, so it cannot be pulled out of the channel sum
// as the scalar gate's can; the prep kernel evaluates those sums with the
// exact per-channel factors in fp32.
//
// The prep kernel writes, per (chunk slot, value head), T and P and the
// pre-scaled operands Khat, Qhat (A-operand fragments, rows = tokens) and
// Ktil^T (A-operand fragments, rows = key channels) in MFMA fragment order,
// then Gamma_C; the scan walks each unit's chunks in order with the state in
// accumulator registers, one wave per 16 state columns.
#include <type_traits>

#include "launch.hpp"
#include "stage.hpp"

namespace gdn {

// Entry of one (chunk slot, value head), kda_entry_bytes (launch.hpp):
// fragments of 64 lanes x 8 elements of the operand type -- T (8), P (8),
// Khat (16: 4 token tiles x 4 contraction blocks of d_k), Qhat (16), Ktil^T
// (16: 8 channel tiles x 2 token blocks) -- then Gamma_C (128 fp32).
constexpr int kKdaFragT = 0, kKdaFragP = 8, kKdaFragKh = 16, kKdaFragQh = 32, kKdaFragKt = 48;

template <typename T>
struct KdaArgs {
  const T *q, *k, *v;
  const float *alpha, *beta;  // alpha [tokens, H_v, d_k], beta [tokens, H_v]
  char *entries;
  const float *h0;
  T *o;
  float *hT;
  int H_qk, H_v, d_k, d_v, group, n_units, n_colblk;
  SeqGeom geo;
};

constexpr int kKRow = 129;  // fp32 row stride of the LDS token x channel tiles (odd: column walks hit every bank)

// ---------------------------------------------------------------------------
// Prep: one block of 512 threads per (chunk slot, value head).
//
// LDS holds k and q rows in the input type and G in fp32; the scaled operands
// 2^G k, 2^G q and 2^-G k of the A and P products are formed as they are
// read.  P is formed first, so that A can take q's space and M then k's
// (bf16 inputs: 66 KiB, two blocks per CU).
// ---------------------------------------------------------------------------
template <typename T> struct KdaRows;
template <> struct KdaRows<bf16_t> { static constexpr int LD = 132; };  // 264-byte rows: 8-byte aligned stores
template <> struct KdaRows<float> { static constexpr int LD = kKRow; };

template <typename T>
__global__ __launch_bounds__(512, (sizeof(T) == 2 ? 4 : 2)) void kda_prep_kernel(KdaArgs<T> a) {
  constexpr int LDT = KdaRows<T>::LD;
  static_assert(64 * LDT * sizeof(T) >= 64 * 65 * 4, "A and M fit in a row tile's space");
  const int c = blockIdx.x, h = blockIdx.y;
  int s, tok0, len;
  if (!a.geo.locate(c, s, tok0, len)) return;
  const int hq = h / a.group;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int dk = a.d_k;

  __shared__ float sG[64 * kKRow];                                 // G_t per channel (log2)
  __shared__ __attribute__((aligned(16))) T sK[64 * LDT];          // k rows, zero past the chunk's end
  __shared__ __attribute__((aligned(16))) T sQ[64 * LDT];          // q rows
  __shared__ float sb[64];
  float(*sA)[65] = reinterpret_cast<float(*)[65]>(sQ);             // A (strictly lower), once P is formed
  float(*sM)[65] = reinterpret_cast<float(*)[65]>(sK);             // M = (I + A)^-1, once A is formed
  float(*sY)[16][17] = reinterpret_cast<float(*)[16][17]>(sG);     // the inverse's block products

  const int64_t qk_stride = int64_t(a.H_qk) * dk;
  const T *kb = a.k + int64_t(tok0) * qk_stride + int64_t(hq) * dk;
  const T *qb = a.q + int64_t(tok0) * qk_stride + int64_t(hq) * dk;
  const float *ab = a.alpha + (int64_t(tok0) * a.H_v + h) * dk;
  const int64_t a_stride = int64_t(a.H_v) * dk;

  // ---- rows of k, q and the clamped log2 rates (zero past the chunk's end),
  // four channels per load.  Every load is issued before any is used: rows
  // past the chunk's end and pieces past d_k are clamped onto valid ones
  // (the latter rewrite the same values), then zeroed ----
  {
    constexpr int kPieces = (16 * 128 + 511) / 512;
    using Piece = typename std::conditional<sizeof(T) == 2, uint2, uint4>::type;  // four elements of T
    const int np = 16 * dk;
    Piece kv[kPieces], qv[kPieces];
    float4 av[kPieces];
#pragma unroll
    for (int m = 0; m < kPieces; ++m) {
      const int idx = min(tid + 512 * m, np - 1);
      const int t = idx / (dk / 4), ch = 4 * (idx - t * (dk / 4));
      const int64_t tc = min(t, len - 1);
      kv[m] = *reinterpret_cast<const Piece *>(kb + tc * qk_stride + ch);
      qv[m] = *reinterpret_cast<const Piece *>(qb + tc * qk_stride + ch);
      av[m] = *reinterpret_cast<const float4 *>(ab + tc * a_stride + ch);
    }
#pragma unroll
    for (int m = 0; m < kPieces; ++m) {
      const int idx = min(tid + 512 * m, np - 1);
      const int t = idx / (dk / 4), ch = 4 * (idx - t * (dk / 4));
      const bool in = t < len;
      const Piece zero{};
      const Piece kp = in ? kv[m] : zero, qp = in ? qv[m] : zero;
      if constexpr (sizeof(T) == 2) {  // 8-byte aligned: LDT is a multiple of 4
        *reinterpret_cast<Piece *>(sK + t * LDT + ch) = kp;
        *reinterpret_cast<Piece *>(sQ + t * LDT + ch) = qp;
      } else {  // the odd fp32 row stride allows 4-byte stores only
        const float *kf = reinterpret_cast<const float *>(&kp), *qf = reinterpret_cast<const float *>(&qp);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sK[t * LDT + ch + e] = kf[e];
          sQ[t * LDT + ch + e] = qf[e];
        }
      }
      float *pg = sG + t * kKRow + ch;
      pg[0] = in ? clamped_log2(av[m].x) : 0.0f;
      pg[1] = in ? clamped_log2(av[m].y) : 0.0f;
      pg[2] = in ? clamped_log2(av[m].z) : 0.0f;
      pg[3] = in ? clamped_log2(av[m].w) : 0.0f;
    }
  }
  if (tid < 64) {
    const float bv = a.beta[int64_t(tok0 + min(tid, len - 1)) * a.H_v + h];
    sb[tid] = tid < len ? bv : 0.0f;
  }
  lds_barrier();
  // ---- chunk-local cumulative log gate: a wave per channel, lane = token ----
  // (several channels at a time, so their reads are in flight together;
  // d_k >= 16, so channels ch and ch + 8 always exist)
  for (int ch = wave; ch < dk; ch += 32) {
    float *pg = sG + lane * kKRow + ch;
    if (ch + 16 < dk) {
      float x0 = pg[0], x1 = pg[8], x2 = pg[16], x3 = pg[24];
      x0 = wave_prefix_sum(x0);
      x1 = wave_prefix_sum(x1);
      x2 = wave_prefix_sum(x2);
      x3 = wave_prefix_sum(x3);
      pg[0] = x0;
      pg[8] = x1;
      pg[16] = x2;
      pg[24] = x3;
    } else {
      float x0 = pg[0], x1 = pg[8];
      x0 = wave_prefix_sum(x0);
      x1 = wave_prefix_sum(x1);
      pg[0] = x0;
      pg[8] = x1;
    }
  }
  lds_barrier();

  char *entry = a.entries + (int64_t(c) * a.H_v + h) * kda_entry_bytes<T>();
  T *frag = reinterpret_cast<T *>(entry);
  float *gamma_C = reinterpret_cast<float *>(frag + kKdaFrags * kFragElems);
  auto kval = [&](int t, int ch) { return to_f32(sK[t * LDT + ch]); };
  auto qval = [&](int t, int ch) { return to_f32(sQ[t * LDT + ch]); };

  // ---- pre-scaled operands, A-operand fragments in the kappa convention ----
  // Khat, Qhat: fragment (rt, kk) holds rows 16 rt + lane mod 16, channels 32 kk + kappa.
  for (int f = wave; f < 32; f += 8) {
    const bool isq = f >= 16;
    const int ff = f & 15, rt = ff >> 2, kk = ff & 3;
    const int t = 16 * rt + (lane & 15);
    Frag<T> fr;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int ch = 32 * kk + kappa(lane, j);
      float x = 0.0f;
      if (ch < dk) x = fast_exp2(sG[t * kKRow + ch]) * (isq ? qval(t, ch) : kval(t, ch));
      fr.set(j, x);
    }
    store_frag(frag + ((isq ? kKdaFragQh : kKdaFragKh) + ff) * kFragElems, lane, fr);
  }
  // Ktil^T: fragment (rm, kk) holds channel 16 rm + lane mod 16, tokens 32 kk + kappa.
  for (int f = wave; f < 16; f += 8) {
    const int rm = f >> 1, kk = f & 1;
    const int ch = 16 * rm + (lane & 15);
    Frag<T> fr;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = 32 * kk + kappa(lane, j);
      float x = 0.0f;
      if (ch < dk) x = fast_exp2(sG[63 * kKRow + ch] - sG[i * kKRow + ch]) * kval(i, ch);
      fr.set(j, x);
    }
    store_frag(frag + (kKdaFragKt + f) * kFragElems, lane, fr);
  }
  if (tid < 128) gamma_C[tid] = tid < dk ? fast_exp2(sG[63 * kKRow + tid]) : 0.0f;

  // ---- P, then A ----
  // When every cumulative log gate of the chunk lies within [-60, 60], the
  // exponent of the channel sums factors without overflow:
  // 2^(G_tc - G_ic) = 2^(G_tc) 2^(-G_ic), both factors in [2^-60, 2^60], so
  //   A_ti = beta_t (Khat Kinv^T)_ti,  P_ti = (Qhat Kinv^T)_ti,
  // Khat = 2^G . k, Qhat = 2^G . q, Kinv = 2^-G . k, each a 64 x 64 x d_k
  // product (fp32 MFMA, the lower tiles only, operands scaled as they are
  // read).  Otherwise (a chunk that decays by more than 2^60, e.g. through
  // alpha = 0) every pair i <= t is summed with one exact exponent per
  // channel.  P goes first: A then takes q's space.
  T *fragP = frag + kKdaFragP * kFragElems;
  auto put_p = [&](int t, int i, float x) {
    const int ii = i & 31, kk = i >> 5;
    const int ln = 16 * ((ii & 15) >> 2) + (t & 15), el = 4 * (ii >> 4) + (ii & 3);
    fragP[((t >> 4) * 2 + kk) * kFragElems + 8 * ln + el] = from_f32<T>(x);
  };
  // the upper tiles of P's fragments are zero
  for (int idx = tid; idx < 6 * 256; idx += 512) {
    const int tile = idx >> 8, e = idx & 255;
    const int rt = tile < 3 ? 0 : (tile < 5 ? 1 : 2), ct = tile < 3 ? tile + 1 : (tile < 5 ? tile - 1 : 3);
    put_p(16 * rt + (e >> 4), 16 * ct + (e & 15), 0.0f);
  }
  bool far = false;
  for (int idx = tid; idx < 64 * dk; idx += 512) {
    const int t = idx / dk, ch = idx - t * dk;
    far |= fabsf(sG[t * kKRow + ch]) > 60.0f;
  }
  far = __syncthreads_or(far);  // (also: every fragment above has read sK, sQ and sG)
  const int r0 = lane & 15, kq = lane >> 4;
  for (int pass = 0; pass < 2; ++pass) {
    const bool isP = pass == 0;
    if (!isP) lds_barrier();  // q is dead: A takes its space
    if (!far) {
      // 10 lower 16 x 16 tiles over the 8 waves
      for (int job = wave; job < 10; job += 8) {
        int idx = job, rt = 0;
        while (idx > rt) { idx -= rt + 1; ++rt; }
        const int ct = idx;  // tile (rt, ct), ct <= rt
        const T *xa = (isP ? sQ : sK) + (16 * rt + r0) * LDT;
        const float *ga = sG + (16 * rt + r0) * kKRow;
        const T *xb = sK + (16 * ct + r0) * LDT;
        const float *gb = sG + (16 * ct + r0) * kKRow;
        f32x4_t acc = zero4();
        // channels in groups of cgw = min(64, d_k): k-slot kq of a product
        // takes channel cg + (cgw / 4) kq + u, so that the 16 rows x 4 slots
        // of a G read fall in distinct banks (odd row stride); each step
        // issues its four products' LDS reads together
        const int cgw = min(64, dk), per = cgw >> 2;
        for (int cg = 0; cg < dk; cg += cgw) {
          const int cb = cg + per * kq;
#pragma unroll 2
          for (int u0 = 0; u0 < per; u0 += 4) {
            float xs[4], ys[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int ch = cb + u0 + v;
              xs[v] = fast_exp2(ga[ch]) * to_f32(xa[ch]);
              ys[v] = fast_exp2(-gb[ch]) * to_f32(xb[ch]);
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xs[v], ys[v], acc, 0, 0, 0);
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * rt + 4 * kq + e, i = 16 * ct + r0;
          if (isP) put_p(t, i, i <= t ? acc[e] : 0.0f);
          else sA[t][i] = i < t ? sb[t] * acc[e] : 0.0f;
        }
      }
    } else {
      for (int p = tid; p < 64 * 64; p += 512) {
        const int t = p >> 6, i = p & 63;
        if ((i >> 4) > (t >> 4)) continue;  // upper tiles: zero above (P) / never read (A)
        float acc = 0.0f;
        if (i <= t) {
          const float *gt = sG + t * kKRow, *gi = sG + i * kKRow;
          for (int ch = 0; ch < dk; ++ch)
            acc += (isP ? qval(t, ch) : kval(t, ch)) * (fast_exp2(gt[ch] - gi[ch]) * kval(i, ch));
        }
        if (isP) put_p(t, i, acc);
        else sA[t][i] = i < t ? sb[t] * acc : 0.0f;
      }
    }
  }
  lds_barrier();  // k and G are dead: M and the inverse's block products take their space

  // ---- M = (I + A)^-1: diagonal 16 x 16 blocks by forward substitution ----
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
    const int t = (tid >> 4) & 15, col = tid & 15;
    const bool active = tid < 256;
    for (int br = 1; br < 4; ++br) {
      if (active)
        for (int cb = 0; cb < br; ++cb) {
          float y = 0.0f;
          for (int j = cb; j < br; ++j)
#pragma unroll
            for (int i = 0; i < 16; ++i) y += sA[16 * br + t][16 * j + i] * sM[16 * j + i][16 * cb + col];
          sY[cb][t][col] = y;
        }
      lds_barrier();
      if (active)
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
  for (int f = wave; f < 8; f += 8) {
    const int rt = f >> 1, kk = f & 1;
    const int t = 16 * rt + (lane & 15);
    Frag<T> fr;
    for (int j = 0; j < 8; ++j) {
      const int i = 32 * kk + kappa(lane, j);
      fr.set(j, (i >> 4) <= (t >> 4) ? sM[t][i] * sb[i] : 0.0f);
    }
    store_frag(frag + (kKdaFragT + f) * kFragElems, lane, fr);
  }
}

// ---------------------------------------------------------------------------
// Scan: one wave per (unit, 16 state columns), chunks in order.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(64) void kda_scan_kernel(KdaArgs<T> a) {
  const int lane = threadIdx.x;
  int u, cb;
  decode_block(blockIdx.x, a.n_colblk, u, cb);
  if (u >= a.n_units) return;
  const int s = a.geo.ordered(u / a.H_v), h = u % a.H_v;
  const int g = lane >> 4;
  const int col = 16 * cb + (lane & 15);
  const int nkt = a.d_k >> 4;        // 16-row tiles of the state
  const int nkb = (a.d_k + 31) >> 5; // 32-deep contraction blocks over d_k

  f32x4_t S[8];
  const int64_t st_base = (int64_t(s) * a.H_v + h) * a.d_k * a.d_v;
#pragma unroll
  for (int rt = 0; rt < 8; ++rt) {
    S[rt] = zero4();
    if (rt < nkt && a.h0)
      for (int e = 0; e < 4; ++e) S[rt][e] = a.h0[st_base + int64_t(16 * rt + 4 * g + e) * a.d_v + col];
  }
  int start, end;
  a.geo.seq_bounds(s, start, end);
  const int n_chunks = (end - start + a.geo.chunk - 1) / a.geo.chunk;
  const int c_first = a.geo.first_chunk(s);
  const int64_t v_stride = int64_t(a.H_v) * a.d_v;

  for (int cc = 0; cc < n_chunks; ++cc) {
    const int c = c_first + cc;
    if (c >= a.geo.n_slots) break;
    const int tok0 = start + cc * a.geo.chunk;
    const int len = min(a.geo.chunk, end - tok0);
    const T *frag = reinterpret_cast<const T *>(a.entries + (int64_t(c) * a.H_v + h) * kda_entry_bytes<T>());
    const float *gamma_C = reinterpret_cast<const float *>(frag + kKdaFrags * kFragElems);
    const T *vb = a.v + int64_t(tok0) * v_stride + int64_t(h) * a.d_v + col;

    Frag<T> Sf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) Sf[kk] = frag_from_acc<T>(S[2 * kk], S[2 * kk + 1]);
    // Y = Khat S, OQ = Qhat S
    f32x4_t Y[4], OQ[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      Y[rt] = zero4();
      OQ[rt] = zero4();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        if (kk < nkb) {
          Y[rt] = mfma(load_frag(frag + (kKdaFragKh + 4 * rt + kk) * kFragElems, lane), Sf[kk], Y[rt]);
          OQ[rt] = mfma(load_frag(frag + (kKdaFragQh + 4 * rt + kk) * kFragElems, lane), Sf[kk], OQ[rt]);
        }
    }
    // X = V - Y, U = T X
    f32x4_t X[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * rt + 4 * g + e;
        X[rt][e] = (t < len ? to_f32(vb[int64_t(t) * v_stride]) : 0.0f) - Y[rt][e];
      }
    Frag<T> Xf[2] = {frag_from_acc<T>(X[0], X[1]), frag_from_acc<T>(X[2], X[3])};
    f32x4_t Ua[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      Ua[rt] = zero4();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        Ua[rt] = mfma(load_frag(frag + (kKdaFragT + rt * 2 + kk) * kFragElems, lane), Xf[kk], Ua[rt]);
    }
    Frag<T> Uf[2] = {frag_from_acc<T>(Ua[0], Ua[1]), frag_from_acc<T>(Ua[2], Ua[3])};
    // O = Qhat S + P U
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f32x4_t acc = OQ[rt];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        acc = mfma(load_frag(frag + (kKdaFragP + rt * 2 + kk) * kFragElems, lane), Uf[kk], acc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * rt + 4 * g + e;
        if (t < len) a.o[int64_t(tok0 + t) * v_stride + int64_t(h) * a.d_v + col] = from_f32<T>(acc[e]);
      }
    }
    // S <- diag(Gamma_C) S + Ktil^T U
#pragma unroll
    for (int rm = 0; rm < 8; ++rm) {
      if (rm < nkt) {
        const f32x4_t gc = *reinterpret_cast<const f32x4_t *>(gamma_C + 16 * rm + 4 * g);
        f32x4_t acc = gc * S[rm];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          acc = mfma(load_frag(frag + (kKdaFragKt + rm * 2 + kk) * kFragElems, lane), Uf[kk], acc);
        S[rm] = acc;
      }
    }
  }
  if (a.hT) {
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
      if (rt < nkt)
        for (int e = 0; e < 4; ++e) a.hT[st_base + int64_t(16 * rt + 4 * g + e) * a.d_v + col] = S[rt][e];
  }
}

// ---------------------------------------------------------------------------
// Staged scan (bf16): one block per (sequence, value head) with one wave per
// 16 state columns.  A chunk's entry (the fragments and Gamma_C) is the same
// for every column, so it is copied once per block into one of two LDS
// stages, one chunk ahead of the chunk being computed, by all waves together
// (16 bytes per lane, straight to LDS).  The chunk's v rows come along into
// the stage's row area.  A wave reads its 16 columns of v there and writes
// its outputs back into the same place; once the block has passed the
// chunk's closing barrier, the rows leave for o with 16-byte stores, before
// the stage is refilled.  The fragments of T and P above their diagonal
// blocks (rows 0-31, columns 32-63: fragments 1, 3, 9 and 11) are zero and
// are neither copied nor multiplied.  Rows past a partial chunk read as zero
// and are not stored.
// ---------------------------------------------------------------------------
constexpr int kKdaStagedFrags = kKdaFrags - 4;           // fragments copied
constexpr int kKdaStGamma = kKdaStagedFrags * 1024;      // Gamma_C (512 bytes of a 1 KiB slot)
constexpr int kKdaStRows = kKdaStGamma + 1024;           // 64 rows of v / o, d_v bf16 each (<= 16 KiB)
constexpr int kKdaStageBytes = kKdaStRows + 64 * 128 * 2;
__host__ __device__ constexpr int kda_slot(int f) {  // LDS slot of entry fragment f (not 1, 3, 9, 11)
  return f - (f > 1) - (f > 3) - (f > 9) - (f > 11);
}

__global__ __launch_bounds__(512) void kda_scan_staged_kernel(KdaArgs<bf16_t> a) {
  __shared__ __attribute__((aligned(16))) char kda_stage0[kKdaStageBytes];
  __shared__ __attribute__((aligned(16))) char kda_stage1[kKdaStageBytes];
  const int u = blockIdx.x;
  if (u >= a.n_units) return;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = a.d_v >> 4;  // waves (16 columns each)
  const int s = a.geo.ordered(u / a.H_v), h = u % a.H_v;
  const int g = lane >> 4, r0 = lane & 15;
  const int col = 16 * w + r0;
  const int nkt = a.d_k >> 4;         // 16-row tiles of the state
  const int nkb = (a.d_k + 31) >> 5;  // 32-deep contraction blocks over d_k

  f32x4_t S[8];
  const int64_t st_base = (int64_t(s) * a.H_v + h) * a.d_k * a.d_v;
#pragma unroll
  for (int rt = 0; rt < 8; ++rt) {
    S[rt] = zero4();
    if (rt < nkt && a.h0)
      for (int e = 0; e < 4; ++e) S[rt][e] = a.h0[st_base + int64_t(16 * rt + 4 * g + e) * a.d_v + col];
  }
  int start, end;
  a.geo.seq_bounds(s, start, end);
  const int C = a.geo.chunk;
  const int c_first = a.geo.first_chunk(s);
  const int n_chunks = max(0, min((end - start + C - 1) / C, a.geo.n_slots - c_first));
  const uint32_t row_bytes = uint32_t(2 * a.d_v);                  // one token's v (or o) of this head
  const uint32_t tok_bytes = uint32_t(2 * int64_t(a.H_v) * a.d_v);  // token stride of v and o
  const int row_copies = a.d_v / 8;  // row bytes / 1 KiB per copy x 64 rows
  constexpr int64_t kEntry = kda_entry_bytes<bf16_t>();
  // this lane's piece of a row copy: rows of row_bytes, 16 bytes per lane
  const int lanes_per_row = int(row_bytes / 16);
  const int row_of_lane = lane / lanes_per_row, piece = lane - row_of_lane * lanes_per_row;
  const int rows_per_copy = 64 / lanes_per_row;

  auto copy_stage = [&](int cc, char *buf) {
    lds_t *st = lds_ptr(buf);
    const char *entry = a.entries + (int64_t(c_first + cc) * a.H_v + h) * kEntry;
    const i32x4_t res = buffer_rsrc(entry, uint32_t(kEntry));
    for (int i = w; i <= kKdaStagedFrags; i += nw) {
      if (i < kKdaStagedFrags) {
        const int f = i + (i >= 1) + (i >= 2) + (i >= 7) + (i >= 8);  // entry fragment of slot i
        dma16_buf(res, uint32_t(1024 * f + 16 * lane), st + 1024 * i);
      } else {
        dma16_buf(res, uint32_t(1024 * kKdaFrags + 16 * lane), st + kKdaStGamma);  // lanes 32-63: zeros
      }
    }
    // row copy j is issued by the wave that stores row piece j (store_rows),
    // so that its own wait orders the read of the previous rows before it
    const int tok0 = start + cc * C;
    const int len = min(C, end - tok0);
    const char *vb = reinterpret_cast<const char *>(a.v) + int64_t(tok0) * tok_bytes + int64_t(h) * row_bytes;
    const i32x4_t vres = buffer_rsrc(vb, uint32_t(len - 1) * tok_bytes + row_bytes);
    for (int j = w; j < row_copies; j += nw) {
      const int row = j * rows_per_copy + row_of_lane;
      dma16_buf(vres, uint32_t(row) * tok_bytes + 16 * piece, st + kKdaStRows + 1024 * j);
    }
  };
  // the rows of chunk cc's outputs, from the stage's row area, to o
  auto store_rows = [&](int cc, char *buf) {
    const lds_t *st = lds_ptr(buf);
    const int tok0 = start + cc * C;
    const int len = min(C, end - tok0);
    char *ob = reinterpret_cast<char *>(a.o) + int64_t(tok0) * tok_bytes + int64_t(h) * row_bytes;
    const __amdgpu_buffer_rsrc_t ores =
        __builtin_amdgcn_make_buffer_rsrc(ob, 0, int((len - 1) * tok_bytes + row_bytes), 0x00020000);
    for (int j = w; j < row_copies; j += nw) {
      const u32x4_t x = lds_load<u32x4_t>(st + kKdaStRows + 1024 * j + 16 * lane);
      const int row = j * rows_per_copy + row_of_lane;
      __builtin_amdgcn_raw_buffer_store_b128(x, ores, uint32_t(row) * tok_bytes + 16 * piece, 0, 0);
    }
  };

  if (n_chunks > 0) copy_stage(0, kda_stage0);
  wait_vmem();
  lds_barrier();
  for (int cc = 0; cc < n_chunks; ++cc) {
    char *cur = (cc & 1) ? kda_stage1 : kda_stage0;
    char *nxt = (cc & 1) ? kda_stage0 : kda_stage1;
    // the previous chunk's outputs leave the other stage before it is
    // refilled: each wave waits for its own reads of the row pieces it then
    // refills (lgkmcnt(0))
    if (cc > 0) store_rows(cc - 1, nxt);
    if (cc + 1 < n_chunks) {
      __builtin_amdgcn_s_waitcnt((0xF) | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
      copy_stage(cc + 1, nxt);
    }
    lds_t *st = lds_ptr(cur);
    auto frag = [&](int f) {
      Frag<bf16_t> x;
      x.v = lds_load<bf16x8_t>(st + 1024 * kda_slot(f) + 16 * lane);
      return x;
    };
    // this wave's column of v and o in the row area: row t at t * row_bytes
    lds_t *rows = st + kKdaStRows + 2 * col;

    Frag<bf16_t> Sf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) Sf[kk] = frag_from_acc<bf16_t>(S[2 * kk], S[2 * kk + 1]);
    // Y = Khat S, OQ = Qhat S
    f32x4_t Y[4], OQ[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      Y[rt] = zero4();
      OQ[rt] = zero4();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        if (kk < nkb) {
          Y[rt] = mfma(frag(kKdaFragKh + 4 * rt + kk), Sf[kk], Y[rt]);
          OQ[rt] = mfma(frag(kKdaFragQh + 4 * rt + kk), Sf[kk], OQ[rt]);
        }
    }
    // X = V - Y, U = T X
    f32x4_t X[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * rt + 4 * g + e;
        X[rt][e] = float(lds_load<__bf16>(rows + t * row_bytes)) - Y[rt][e];
      }
    const Frag<bf16_t> Xf[2] = {frag_from_acc<bf16_t>(X[0], X[1]), frag_from_acc<bf16_t>(X[2], X[3])};
    f32x4_t Ua[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      Ua[rt] = mfma(frag(kKdaFragT + rt * 2), Xf[0], zero4());
      if (rt >= 2) Ua[rt] = mfma(frag(kKdaFragT + rt * 2 + 1), Xf[1], Ua[rt]);
    }
    const Frag<bf16_t> Uf[2] = {frag_from_acc<bf16_t>(Ua[0], Ua[1]), frag_from_acc<bf16_t>(Ua[2], Ua[3])};
    // O = Qhat S + P U, into the row area (this wave's own column)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f32x4_t acc = mfma(frag(kKdaFragP + rt * 2), Uf[0], OQ[rt]);
      if (rt >= 2) acc = mfma(frag(kKdaFragP + rt * 2 + 1), Uf[1], acc);
#pragma unroll
      for (int e = 0; e < 4; ++e) lds_store<__bf16>(rows + (16 * rt + 4 * g + e) * row_bytes, __bf16(acc[e]));
    }
    // S <- diag(Gamma_C) S + Ktil^T U
#pragma unroll
    for (int rm = 0; rm < 8; ++rm) {
      if (rm < nkt) {
        const f32x4_t gc = lds_load<f32x4_t>(st + kKdaStGamma + 4 * (16 * rm + 4 * g));
        f32x4_t acc = gc * S[rm];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) acc = mfma(frag(kKdaFragKt + rm * 2 + kk), Uf[kk], acc);
        S[rm] = acc;
      }
    }
    // the next stage has landed; every wave's outputs are in the row area
    wait_vmem();
    lds_barrier();
  }
  if (n_chunks > 0) {
    store_rows(n_chunks - 1, ((n_chunks - 1) & 1) ? kda_stage1 : kda_stage0);
    wait_vmem();
  }
  if (a.hT) {
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
      if (rt < nkt)
        for (int e = 0; e < 4; ++e) a.hT[st_base + int64_t(16 * rt + 4 * g + e) * a.d_v + col] = S[rt][e];
  }
}

template <typename T>
static hipError_t launch_kda_chunk_t(const Problem &p, const Workspace &ws, hipStream_t st) {
  KdaArgs<T> a;
  a.q = static_cast<const T *>(p.q);
  a.k = static_cast<const T *>(p.k);
  a.v = static_cast<const T *>(p.v);
  a.alpha = p.alpha;
  a.beta = p.beta;
  a.entries = static_cast<char *>(ws.entries);
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
  a.geo = make_geom(p, &ws);
  const int64_t slots = chunk_slots(p);
  if (slots > 0) {
    hipLaunchKernelGGL(kda_prep_kernel<T>, dim3(unsigned(slots), unsigned(p.H_v)), dim3(512), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if constexpr (sizeof(T) == 2) {
    // bf16: the staged scan, one block per unit
    if (a.n_units == 0) return hipSuccess;
    hipLaunchKernelGGL(kda_scan_staged_kernel, dim3(unsigned(a.n_units)), dim3(64 * (p.d_v / 16)), 0, st, a);
    return hipGetLastError();
  }
  const int64_t blocks = (int64_t(p.n_seqs) * p.H_v + 7) / 8 * 8 * (p.d_v / 16);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(kda_scan_kernel<T>, dim3(unsigned(blocks)), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_kda_chunk(const Problem &p, const Workspace &ws, hipStream_t st) {
  if (p.dtype == 1) return launch_kda_chunk_t<bf16_t>(p, ws, st);
  return launch_kda_chunk_t<float>(p, ws, st);
}

}  // namespace gdn
