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
// (dA uses M^T dU (diag(beta) X)^T M^T = dY (T X)^T = dY U^T.)  The row sums
// over d_v are taken through d_k-sized products that the gradients need
// anyway: sum_c dO_tc (Q S)_tc = sum_k Q_tk (dO S^T)_tk, and likewise for
// dX . K S (through dY S^T) and K dS' . U (through U dS'^T).
//
// Only the two state recurrences are sequential: S forward and dS backward.
// Everything else is independent per chunk.  Three launches:
//   1. bwd_factor_kernel, one block per (chunk, value head): gates, M by a
//      blocked triangular inverse, P and Gamma . K K^T, into the chunk's entry.
//   2. bwd_chain_kernel: per (unit, column block of d_v) one block walks the
//      chunks forward keeping S (writing each chunk's start state and U)
//      and another walks them backward keeping dS (writing each chunk's end
//      gradient, dY and dv).  The state sits in MFMA accumulators, and the
//      next chunk's operands are loaded while the current one is computed.
//   3. bwd_grad_kernel, one block per (chunk, value head): the products over
//      d_v (dO S^T, dY S^T, U dS'^T, dO U^T, dY U^T), then dq, dk, dbeta and
//      dalpha.
// Under grouped heads a last pass sums dq and dk over the value heads that
// read each query/key head.  The products run on fp32 MFMA
// (v_mfma_f32_16x16x4f32), except two groups that need no fp32 operand
// rounding beyond a split: K K^T and Q K^T of bf16 inputs (exact products)
// on the bf16 MFMA, and for bf16 inputs the backward chain's state update
// Q^T diag(gamma) dO - K^T diag(gamma) dX, whose fp32 factors are split as
// x = hi + lo in bf16 (about 16 significant bits).  Every sum has a fixed
// order, so results repeat bit for bit from run to run.
#include "launch.hpp"
#include "stage.hpp"

namespace gdn {

namespace {

// Floats of one entry (one chunk of one value head) in the workspace.
struct BwdEntry {
  int64_t M, P, G, gate, S, dS, U, dY, total;
  __host__ __device__ BwdEntry(int C, int DK, int DV) {
    int64_t o = 0;
    M = o;    o += int64_t(C) * C;    // (I + A)^-1, row-major C x C
    P = o;    o += int64_t(C) * C;    // lower(Gamma . Q K^T)
    gate = o; o += 256;               // gamma_t, s_t, log2 cumulative gate, beta_t (64 each)
    G = o;    o += int64_t(C) * C;    // strict_lower(Gamma . K K^T); the forward's entries end here
    S = o;    o += int64_t(DK) * DV;  // state entering the chunk
    dS = o;   o += int64_t(DK) * DV;  // gradient reaching the chunk's end state
    U = o;    o += int64_t(C) * DV;   // T X, X = V - diag(gamma) K S
    dY = o;   o += int64_t(C) * DV;   // M^T dU
    total = o;
  }
};
constexpr int kGateGamma = 0, kGateS = 64, kGateLog2 = 128, kGateBeta = 192;

template <typename T>
struct BwdArgs {
  const T *q, *k, *v, *d_o;
  const float *alpha, *beta, *h0, *dhT;
  float *ent;             // [n_slots * H_v] entries of ent_floats
  int64_t ent_floats;
  float *dq, *dk;         // [tokens, H_v, d_k]: the gradients themselves when every
                          // query/key head has one value head, else per-value-head parts
  float *dv, *dalpha, *dbeta, *dh0;
  T *o;                   // the forward: outputs [tokens, H_v, d_v] and final states (or null)
  float *hT;
  float *mb;              // the transition pass: [units, d_k, d_v + d_k] segment maps (B, then M)
  bool want_g;            // the backward: the factor kernel also writes Gamma . K K^T
  int cols;               // columns of d_v per forward-chain block: 16 or 32 (d_v >= 32), else d_v
  int H_qk, H_v, d_k, d_v, group, n_units;
  SeqGeom geo;
};

// ---- 16 x 16 fp32 MFMA tiles ----------------------------------------------
// Lane roles: r = lane & 15, g = lane >> 4.  An accumulator holds D[4g + e][r]
// (e = 0..3); mm16(xr, yt, acc) adds X Y over a 16-deep slice with
// xr = X[r][4g .. 4g + 3] and yt = Y[4g .. 4g + 3][r], so an accumulator is
// itself a valid yt for the next product.
template <typename P> __device__ __forceinline__ f32x4_t row4(const P *p) {
  const float4 x = load4_f32(p);
  return f32x4_t{x.x, x.y, x.z, x.w};
}
template <typename P> __device__ __forceinline__ f32x4_t col4(const P *p, int ld) {
  return f32x4_t{to_f32(p[0]), to_f32(p[ld]), to_f32(p[2 * ld]), to_f32(p[3 * ld])};
}

// Sum of x over aligned groups of w lanes (w a power of two <= 64), fixed order.
__device__ __forceinline__ float group_sum(float x, int w) {
  for (int o = 1; o < w; o <<= 1) x += __shfl_xor(x, o);
  return x;
}

// Workgroup barrier for LDS traffic: waits for this wave's LDS operations but
// not for its outstanding global loads, so the next chunk's operands stay in
// flight across it (__syncthreads would wait for them).  The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_sync() {
  asm volatile("" ::: "memory");
  lds_barrier();
  asm volatile("" ::: "memory");
}

// The k-th lower 16 x 16 tile (row tile >= column tile), row by row.
__device__ __forceinline__ void lower_tile(int k, int &rt, int &ct) {
  rt = 0;
  while (k > rt) {
    k -= rt + 1;
    ++rt;
  }
  ct = k;
}

constexpr int kChainThreads = 256;

// One chunk's token-row tile (K or Q: C rows x d_k of T) as 16-byte pieces in
// the registers of NTH threads, then in LDS.  Rows at or past n read as zero.  Branch-free (an
// index past the tile is clamped onto its last piece, which then is loaded
// and stored twice with the same value), so that the compiler can count the
// loads still in flight exactly and wait only for these.
template <typename T, int C, int NTH = kChainThreads> struct TileLoader {
  static constexpr int EPP = 16 / sizeof(T);
  static constexpr int MAXP = (C * 128 / EPP + NTH - 1) / NTH;
  uint4 v[MAXP];
  __device__ __forceinline__ void load(const T *base, int64_t row_stride, int n, int DK) {
    const int ppr = DK / EPP, np = C * ppr;
#pragma unroll
    for (int m = 0; m < MAXP; ++m) {
      const int p = min(int(threadIdx.x % NTH) + NTH * m, np - 1);
      const int t = p / ppr, c = (p - t * ppr) * EPP;
      const uint4 x = *reinterpret_cast<const uint4 *>(base + int64_t(min(t, n - 1)) * row_stride + c);
      v[m] = t < n ? x : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(T *lds, int ldk, int DK) const {
    const int ppr = DK / EPP, np = C * ppr;
#pragma unroll
    for (int m = 0; m < MAXP; ++m) {
      const int p = min(int(threadIdx.x % NTH) + NTH * m, np - 1);
      const int t = p / ppr, c = (p - t * ppr) * EPP;
      *reinterpret_cast<uint4 *>(lds + t * ldk + c) = v[m];
    }
  }
};

}  // namespace

// ---------------------------------------------------------------------------
// 1. Per (chunk, value head): gates, M = (I + A)^-1, P, Gamma . K K^T.
// ---------------------------------------------------------------------------
template <typename T, int C>
__global__ __launch_bounds__(256) void bwd_factor_kernel(BwdArgs<T> a) {
  constexpr int NB = C / 16, LD = C + 4, NL = NB * (NB + 1) / 2;
  const int e = blockIdx.x;
  const int slot = e / a.H_v, h = e - slot * a.H_v;
  int s, tok0, n;
  if (!a.geo.locate(slot, s, tok0, n)) return;
  const int hq = h / a.group, DK = a.d_k;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
  // LDS: the chunk's K and Q rows.  A takes Q's space once P is formed, and
  // M takes K's once A is (fp32 inputs: two blocks per CU, bf16: four).
  // Rows 32 bytes past a multiple of 128: LDS bank conflicts 2-3 % of
  // LDS-active cycles instead of 26-32 % at 16 bytes past (measured).
  constexpr int LDK = 128 + 32 / sizeof(T);
  constexpr int kTileBytes = C * LDK * sizeof(T);
  static_assert(kTileBytes >= C * LD * 4, "A and M each fit in a row tile's space");
  __shared__ __attribute__((aligned(16))) char sBuf[2 * kTileBytes];
  __shared__ float sg[64], sb[64];
  T *sK = reinterpret_cast<T *>(sBuf), *sQ = reinterpret_cast<T *>(sBuf + kTileBytes);
  float *sA = reinterpret_cast<float *>(sBuf + kTileBytes);
  float *sM = reinterpret_cast<float *>(sBuf);
  float *ent = a.ent + int64_t(e) * a.ent_floats;
  const BwdEntry L(C, DK, a.d_v);
  const int64_t krow = int64_t(a.H_qk) * DK;

  {
    TileLoader<T, C> kl, ql;
    kl.load(a.k + int64_t(tok0) * krow + int64_t(hq) * DK, krow, n, DK);
    ql.load(a.q + int64_t(tok0) * krow + int64_t(hq) * DK, krow, n, DK);
    if (w == 0) {  // chunk-local cumulative log2 gate; padded slots add 0
      const bool in = lane < n;
      const int64_t gi = int64_t(tok0 + min(lane, n - 1)) * a.H_v + h;
      const float al = a.alpha[gi], be = a.beta[gi];
      const float g2 = wave_prefix_sum(in ? clamped_log2(al) : 0.0f);
      if (lane < C) {
        sg[lane] = g2;
        sb[lane] = in ? be : 0.0f;
      }
    }
    // P and Gamma . K K^T are zero above the diagonal tiles, for the gradient
    // kernel (the forward chain reads only the lower tiles of P)
    if (a.want_g) {
      for (int idx = tid; idx < C * C; idx += 256) {
        const int t = idx / C, i = idx - t * C;
        if ((i >> 4) > (t >> 4)) {
          ent[L.P + idx] = 0.0f;
          ent[L.G + idx] = 0.0f;
        }
      }
    }
    kl.store(sK, LDK, DK);
    ql.store(sQ, LDK, DK);
  }
  __syncthreads();
  // lower tiles of Q K^T and then of K K^T (contraction over d_k); each
  // leaves as P = Gamma . Q K^T (lower) or as Gamma . K K^T (strict lower;
  // A = diag(beta) times it into LDS).  Every tile of A that the inverse
  // reads is written here (the diagonal tiles' upper halves as zeros).
  for (int pass = 0; pass < 2; ++pass) {
    const bool mat_q = pass == 0;
    if (!mat_q) __syncthreads();  // Q is dead: A takes its space
    for (int job = w; job < NL; job += 4) {
      int rt, ct;
      lower_tile(job, rt, ct);
      f32x4_t acc = zero4();
      if constexpr (sizeof(T) == 2) {
        // bf16 inputs: their products are exact in fp32, so the bf16 MFMA
        // (32 channels a step, lane group g taking channels 8g .. 8g + 7)
        // gives the same sums; groups past d_k (d_k = 16) read as zero
        const T *pa = (mat_q ? sQ : sK) + (16 * rt + r) * LDK + 8 * g;
        const T *pb = sK + (16 * ct + r) * LDK + 8 * g;
        for (int k0 = 0; k0 < DK; k0 += 32) {
          const bool in = k0 + 8 * g < DK;
          const bf16x8_t x = *reinterpret_cast<const bf16x8_t *>(pa + k0);
          const bf16x8_t y = *reinterpret_cast<const bf16x8_t *>(pb + k0);
          const bf16x8_t z = {};
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(in ? x : z, in ? y : z, acc, 0, 0, 0);
        }
      } else {
        const T *pa = (mat_q ? sQ : sK) + (16 * rt + r) * LDK + 4 * g;
        const T *pb = sK + (16 * ct + r) * LDK + 4 * g;
        for (int k0 = 0; k0 < DK; k0 += 16) acc = mm16(row4(pa + k0), row4(pb + k0), acc);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = 16 * rt + 4 * g + q, i = 16 * ct + r;
        const float gam = i <= t ? fast_exp2(sg[t] - sg[i]) : 0.0f;
        if (mat_q) {
          ent[L.P + t * C + i] = gam * acc[q];
        } else {
          const float gkk = i < t ? gam * acc[q] : 0.0f;
          if (a.want_g) ent[L.G + t * C + i] = gkk;
          sA[t * LD + i] = sb[t] * gkk;
        }
      }
    }
  }
  if (tid < C) {
    const float gl = sg[C - 1];
    ent[L.gate + kGateGamma + tid] = fast_exp2(sg[tid]);
    ent[L.gate + kGateS + tid] = fast_exp2(gl - sg[tid]);
    ent[L.gate + kGateLog2 + tid] = sg[tid];
    ent[L.gate + kGateBeta + tid] = sb[tid];
  }
  __syncthreads();  // K is dead: M takes its space
  for (int i = tid; i < C * LD; i += 256) sM[i] = 0.0f;
  __syncthreads();
  // (I + A)^-1 by 16 x 16 blocks: the diagonal blocks by forward substitution
  // (lane group g inverts block g, lane r owns column r) ...
  if (w == 0 && g < NB) {
    const int o = 16 * g;
    float m[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float x = t == r ? 1.0f : 0.0f;
#pragma unroll
      for (int kk = 0; kk < t; ++kk) x -= sA[(o + t) * LD + o + kk] * m[kk];
      m[t] = x;
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) sM[(o + t) * LD + o + r] = m[t];
  }
  __syncthreads();
  // ... then the blocks d below the diagonal, one wave per block:
  // M_ij = -M_ii sum_{j <= k < i} A_ik M_kj
  for (int d = 1; d < NB; ++d) {
    const int j = w, i = w + d;
    if (i < NB) {
      f32x4_t z = zero4();
      for (int kb = j; kb < i; ++kb)
        z = mm16(row4(&sA[(16 * i + r) * LD + 16 * kb + 4 * g]), col4(&sM[(16 * kb + 4 * g) * LD + 16 * j + r], LD),
                 z);
      const f32x4_t m = mm16(row4(&sM[(16 * i + r) * LD + 16 * i + 4 * g]), z, zero4());
#pragma unroll
      for (int q = 0; q < 4; ++q) sM[(16 * i + 4 * g + q) * LD + 16 * j + r] = -m[q];
    }
    __syncthreads();
  }
  for (int idx = tid; idx < C * C; idx += 256) {
    const int t = idx / C, i = idx - t * C;
    ent[L.M + idx] = sM[t * LD + i];
  }
}

// ---------------------------------------------------------------------------
// 2. The two chains, each on four waves over a column block of
// CB = min(32, d_v) columns of one unit; the kernel below puts a chain of
// each direction in one block where LDS allows, and the forward pass's own
// chain also runs 16-column blocks when there are few units.  With w the wave within its
// four: tiles of a C x CB product are i = w + 4m, row tile i % (C/16), column
// tile i / (C/16), so a wave keeps one row tile; tiles of the d_k x CB state
// are i = w + 4m, row tile i % (d_k/16), column tile i / (d_k/16).
// ---------------------------------------------------------------------------
namespace {

template <typename T, int C> struct ChainLds {
  // Row strides of the K / Q tiles, the transposed operands and the token
  // splits are 32 bytes past a multiple of 128: measured on the chains, that
  // leaves a quarter fewer LDS bank conflicts than 16 bytes past.
  static constexpr int LDK = 128 + 32 / sizeof(T);  // K / Q rows (elements of T), d_k <= 128
  static constexpr int LDT = 128 + 8;               // transposed state: [column][d_k] floats
  static constexpr int LDC = C + 8;                 // transposed C x CB operands: [column][token] floats
  static constexpr int kTile = C * LDK * sizeof(T);
  static constexpr int kState = 32 * LDT * 4;
  static constexpr int kCol = 32 * LDC * 4;
  static constexpr int kGate = 3 * 64 * 4;
  // bf16 inputs: the backward chain's state update runs on the bf16 MFMA
  // with its fp32 operands diag(gamma) dO and -diag(gamma) dX split into
  // bf16 hi + lo, stored per column as [hi x4 | lo x4] per 4 tokens
  static constexpr bool kSplitB = sizeof(T) == 2;
  static constexpr int LDP = 2 * C + 16;            // split rows over tokens: bf16 elements
  static constexpr int LDSS = 2 * 128 + 8;          // split rows over d_k (a split state^T, within kState bytes)
  static constexpr int kSplit = 32 * LDP * 2;
  static_assert(32 * LDSS * 2 <= kState, "a split state^T fits in the state's space");
  // forward: K, S^T, Y^T, (diag(s) U)^T, gates; backward: K, Q, dS^T, dO^T,
  // dU^T, (-diag(gamma) dX)^T (bf16: its split, and the split of
  // diag(gamma) dO), gates
  static constexpr int kFwd = kTile + kState + 2 * kCol + kGate;
  static constexpr int kRev = kSplitB ? 2 * kTile + kState + 2 * kCol + 2 * kSplit + kGate
                                      : 2 * kTile + kState + 3 * kCol + kGate;
  static constexpr int kBytes = kFwd > kRev ? kFwd : kRev;
  // one block runs a chain of each direction when both fit in a CU's LDS
  static constexpr bool kPaired = kFwd + kRev <= 160 * 1024;
  // the forward pass itself: K, Q, S^T, Y^T, U^T, gates
  static constexpr int kOut = 2 * kTile + kState + 2 * kCol + kGate;
};

// A fragment of K^T (or Q^T) from a row-major token-row tile in LDS: lane
// (r, g) gets tile[t0 + 4g + j][col0 + r], j = 0..3.  For bf16 one
// ds_read_b64_tr_b16: lane L of each 16-lane group addresses row
// t0 + 4g + L / 4, columns col0 + 4 (L % 4) .. + 3, and lane r then holds
// column col0 + r of the four rows.
template <typename T>
__device__ __forceinline__ f32x4_t tile_colfrag(const T *tile, int ld, int t0, int col0, int r, int g);
template <>
__device__ __forceinline__ f32x4_t tile_colfrag<bf16_t>(const bf16_t *tile, int ld, int t0, int col0, int r, int g) {
  const bf16_t *p = tile + (t0 + 4 * g + (r >> 2)) * ld + col0 + 4 * (r & 3);
  return __builtin_convertvector(lds_read_tr16(lds_ptr((void *)p)), f32x4_t);
}
template <>
__device__ __forceinline__ f32x4_t tile_colfrag<float>(const float *tile, int ld, int t0, int col0, int r, int g) {
  return col4(tile + (t0 + 4 * g) * ld + col0 + r, ld);
}
// The same four bf16 values of a bf16 tile, unconverted.
__device__ __forceinline__ bf16x4_t tile_colfrag_raw(const bf16_t *tile, int ld, int t0, int col0, int r, int g) {
  const bf16_t *p = tile + (t0 + 4 * g + (r >> 2)) * ld + col0 + 4 * (r & 3);
  return lds_read_tr16(lds_ptr((void *)p));
}
// x = hi + lo in bf16 (hi = bf16(x), lo = bf16(x - hi): about 16 significant
// bits), as the 8 elements [hi x4 | lo x4].
__device__ __forceinline__ bf16x8_t split_hi_lo(f32x4_t x) {
  const bf16x4_t hi = __builtin_convertvector(x, bf16x4_t);
  const bf16x4_t lo = __builtin_convertvector(x - __builtin_convertvector(hi, f32x4_t), bf16x4_t);
  return __builtin_shufflevector(hi, lo, 0, 1, 2, 3, 4, 5, 6, 7);
}
// The 16 x 16 x 16 step of mm16 (xr, yt as there) on the bf16 MFMA when one
// factor is exact in bf16: the other split as hi + lo, [x_hi | x_lo] against
// [y ; y] (mm16_sx: yt exact) or [x ; x] against [y_hi ; y_lo] (mm16_sy:
// xr exact).
__device__ __forceinline__ f32x4_t mm16_sx(f32x4_t xr, f32x4_t yt, f32x4_t acc) {
  const bf16x4_t y = __builtin_convertvector(yt, bf16x4_t);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(split_hi_lo(xr), __builtin_shufflevector(y, y, 0, 1, 2, 3, 0, 1, 2, 3),
                                                 acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mm16_sy(f32x4_t xr, bf16x8_t ys, f32x4_t acc) {
  const bf16x4_t x = __builtin_convertvector(xr, bf16x4_t);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_shufflevector(x, x, 0, 1, 2, 3, 0, 1, 2, 3), ys, acc, 0, 0, 0);
}

// One chunk's gamma, s and beta: thread t holds token (t mod 64)'s.
struct GateLoader {
  float gam = 0.0f, sc = 0.0f, be = 0.0f;
  __device__ __forceinline__ void load(const float *gate) {
    const int t = threadIdx.x & 63;
    gam = gate[kGateGamma + t];
    sc = gate[kGateS + t];
    be = gate[kGateBeta + t];
  }
  __device__ __forceinline__ void store(float *sgate) const {
    const int t = threadIdx.x & 63;
    sgate[t] = gam;
    sgate[64 + t] = sc;
    sgate[128 + t] = be;
  }
};

// Unit u's sequence, value head, token range, first chunk slot and chunk count.
__device__ __forceinline__ void unit_of(const SeqGeom &geo, int H_v, int u, int &s, int &h, int &start, int &end,
                                        int &c_first, int &n_chunks) {
  s = geo.ordered(u / H_v);
  h = u - (u / H_v) * H_v;
  geo.seq_bounds(s, start, end);
  n_chunks = (end - start + geo.chunk - 1) / geo.chunk;
  c_first = geo.first_chunk(s);
  n_chunks = max(0, min(n_chunks, geo.n_slots - c_first));
}

// The forward chain over one column block of one unit.  For the backward
// (OUT = false) it stores each chunk's start state, X and U in the chunk's
// entry.  For the forward pass itself (OUT = true) it stores nothing in the
// entries: it also stages the chunk's Q rows, forms
// O = diag(gamma) Q S + P U, and writes O and the last state.
template <typename T, int C, bool OUT, int NW = 4, bool TRANS = false>
__device__ void fwd_chain(const BwdArgs<T> &a, int u, int cb, char *smem) {
  using Lds = ChainLds<T, C>;
  constexpr int NRT = C / 16, LDK = Lds::LDK, LDT = Lds::LDT, LDC = Lds::LDC;
  // NW waves; a wave's C x CB tiles (at most 8 in all) and d_k x CB state
  // tiles (at most 16) are i = w + NW m
  constexpr int NTH = 64 * NW, MT = (8 + NW - 1) / NW, MS = (16 + NW - 1) / NW;
  static_assert(NW % NRT == 0, "a wave keeps one row tile");
  const int DK = a.d_k, DV = a.d_v, CB = a.cols, c0 = cb * CB;
  const int NKT = DK / 16, NCT = CB / 16;
  const int tid = threadIdx.x % NTH, w = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
  T *sK = reinterpret_cast<T *>(smem);
  T *sQ = reinterpret_cast<T *>(smem + Lds::kTile);                           // OUT only
  float *sSt = reinterpret_cast<float *>(smem + (OUT ? 2 : 1) * Lds::kTile);  // S^T
  float *sYt = sSt + 32 * LDT;                                                // (diag(beta) X)^T
  float *sUt = sYt + 32 * LDC;        // (diag(s) U)^T; U^T when OUT (scaled where it is read)
  float *sgate = sUt + 32 * LDC;      // gamma[64], s[64], beta[64]
  // the backward's forward chain with bf16 inputs: K S and the state update
  // on the bf16 MFMA, with S^T and (diag(s) U)^T stored split as hi + lo
  // ([hi x4 | lo x4] per 4 rows of the contraction) in the same space
  constexpr bool SPL = Lds::kSplitB && !OUT;
  bf16_t *sSs = reinterpret_cast<bf16_t *>(sSt);
  bf16_t *sUs = reinterpret_cast<bf16_t *>(sUt);
  int s, h, start, end, c_first, n_chunks;
  unit_of(a.geo, a.H_v, u, s, h, start, end, c_first, n_chunks);
  const int hq = h / a.group;
  const BwdEntry L(C, DK, DV);
  const int64_t krow = int64_t(a.H_qk) * DK, vrow = int64_t(a.H_v) * DV;

  // this wave's C x CB tiles (one row tile) and state tiles
  const int rt = w % NRT;
  const int nmine = (w < NRT * NCT) ? ((MT > 1 && w + NW < NRT * NCT) ? 2 : 1) : 0;
  const int nst = NKT * NCT;
  f32x4_t accS[MS];
#pragma unroll
  for (int m = 0; m < MS; ++m) {
    accS[m] = zero4();
    const int i = w + NW * m;
    if constexpr (TRANS) {
      // the transition pass: B's columns start from zero, M's from the identity
      const int kt = i % NKT, ct = i / NKT;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        accS[m][q] = (i < nst && c0 >= DV && 16 * kt + 4 * g + q == c0 - DV + 16 * ct + r) ? 1.0f : 0.0f;
    } else if (i < nst && a.h0) {
      const int kt = i % NKT, ct = i / NKT;
      const float *h0 = a.h0 + (int64_t(s) * a.H_v + h) * DK * DV;
#pragma unroll
      for (int q = 0; q < 4; ++q) accS[m][q] = h0[int64_t(16 * kt + 4 * g + q) * DV + c0 + 16 * ct + r];
    }
  }
  // the state after the last chunk (the entry state for an empty sequence);
  // the transition pass writes it as the segment's map
  auto store_final = [&]() {
    if constexpr (TRANS) {
      const int ldm = DV + DK;
      float *mb = a.mb + (int64_t(s) * a.H_v + h) * DK * ldm;
#pragma unroll
      for (int m = 0; m < MS; ++m) {
        const int i = w + NW * m;
        if (i < nst) {
          const int kt = i % NKT, ct = i / NKT;
#pragma unroll
          for (int q = 0; q < 4; ++q) mb[int64_t(16 * kt + 4 * g + q) * ldm + c0 + 16 * ct + r] = accS[m][q];
        }
      }
      return;
    }
    if (!OUT || !a.hT) return;
    float *hT = a.hT + (int64_t(s) * a.H_v + h) * DK * DV;
#pragma unroll
    for (int m = 0; m < MS; ++m) {
      const int i = w + NW * m;
      if (i < nst) {
        const int kt = i % NKT, ct = i / NKT;
#pragma unroll
        for (int q = 0; q < 4; ++q) hT[int64_t(16 * kt + 4 * g + q) * DV + c0 + 16 * ct + r] = accS[m][q];
      }
    }
  };
  if (n_chunks == 0) {
    store_final();
    return;
  }

  TileLoader<T, C, NTH> kl, ql;
  GateLoader gl;
  // V at this wave's accumulator positions and the A fragments of M (and for
  // OUT of P, lower tiles only) for its row tile: loaded a chunk ahead, right
  // after their last use
  f32x4_t vcur[MT], mcur[NRT], pcur[NRT];
  auto load_v = [&](int cc) {
    const int tok0 = start + cc * C, n = min(C, end - tok0);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int ct = min((w + NW * m) / NRT, NCT - 1);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = 16 * rt + 4 * g + q;
        // (the transition pass's M columns have no values: read a valid column, use zero)
        const int col = TRANS ? min(c0 + 16 * ct + r, DV - 1) : c0 + 16 * ct + r;
        const float x = to_f32(a.v[int64_t(tok0 + min(t, n - 1)) * vrow + int64_t(h) * DV + col]);
        vcur[m][q] = (t < n && (!TRANS || c0 < DV)) ? x : 0.0f;
      }
    }
  };
  auto load_m = [&](int cc) {
    const float *ent = a.ent + (int64_t(c_first + cc) * a.H_v + h) * a.ent_floats;
#pragma unroll
    for (int kb = 0; kb < NRT; ++kb) mcur[kb] = row4(ent + L.M + (16 * rt + r) * C + 16 * kb + 4 * g);
  };
  auto load_p = [&](int cc) {  // tiles right of the diagonal are not used (nor written): re-read a used one
    const float *ent = a.ent + (int64_t(c_first + cc) * a.H_v + h) * a.ent_floats;
#pragma unroll
    for (int kb = 0; kb < NRT; ++kb) pcur[kb] = row4(ent + L.P + (16 * rt + r) * C + 16 * min(kb, rt) + 4 * g);
  };
  auto load_tiles = [&](int cc) {
    const int tok0 = start + cc * C, n = min(C, end - tok0);
    kl.load(a.k + int64_t(tok0) * krow + int64_t(hq) * DK, krow, n, DK);
    if constexpr (OUT) ql.load(a.q + int64_t(tok0) * krow + int64_t(hq) * DK, krow, n, DK);
    gl.load(a.ent + (int64_t(c_first + cc) * a.H_v + h) * a.ent_floats + L.gate);
  };
  load_tiles(0);
  load_v(0);
  load_m(0);
  if constexpr (OUT) load_p(0);
  kl.store(sK, LDK, DK);
  if constexpr (OUT) ql.store(sQ, LDK, DK);
  gl.store(sgate);

  for (int cc = 0; cc < n_chunks; ++cc) {
    float *ent = a.ent + (int64_t(c_first + cc) * a.H_v + h) * a.ent_floats;
    // the state entering this chunk: to LDS, transposed (operand of K S and Q S), and to the entry
#pragma unroll
    for (int m = 0; m < MS; ++m) {
      const int i = w + NW * m;
      if (i < nst) {
        const int kt = i % NKT, ct = i / NKT;
        if constexpr (SPL)
          *reinterpret_cast<bf16x8_t *>(sSs + (16 * ct + r) * Lds::LDSS + 32 * kt + 8 * g) = split_hi_lo(accS[m]);
        else
          *reinterpret_cast<f32x4_t *>(sSt + (16 * ct + r) * LDT + 16 * kt + 4 * g) = accS[m];
        if constexpr (!OUT && !TRANS) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            ent[L.S + (16 * kt + 4 * g) * DV + c0 + 16 * ct + r + q * DV] = accS[m][q];
        }
      }
    }
    const int nx = min(cc + 1, n_chunks - 1);  // the next chunk (the last one reloads itself)
    load_tiles(nx);
    lds_sync();
    // X = V - diag(gamma) K S;  Y = diag(beta) X;  for OUT also diag(gamma) Q S
    f32x4_t oacc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) oacc[m] = zero4();
    if (nmine > 0) {
      f32x4_t acc[MT], qacc[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m] = qacc[m] = zero4();
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        if (16 * kk < DK) {
          if constexpr (SPL) {
            // [K | K] against [S_hi ; S_lo], 16 channels a step
            const bf16x4_t kr = *reinterpret_cast<const bf16x4_t *>(sK + (16 * rt + r) * LDK + 16 * kk + 4 * g);
            const bf16x8_t k8 = __builtin_shufflevector(kr, kr, 0, 1, 2, 3, 0, 1, 2, 3);
#pragma unroll
            for (int m = 0; m < MT; ++m)
              if (m < nmine)
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    k8, *reinterpret_cast<const bf16x8_t *>(sSs + (16 * ((w + NW * m) / NRT) + r) * Lds::LDSS + 32 * kk + 8 * g),
                    acc[m], 0, 0, 0);
          } else {
            const f32x4_t xr = row4(sK + (16 * rt + r) * LDK + 16 * kk + 4 * g);
            f32x4_t qr = zero4();
            if constexpr (OUT) qr = row4(sQ + (16 * rt + r) * LDK + 16 * kk + 4 * g);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              if (m < nmine) {
                const f32x4_t st = row4(sSt + (16 * ((w + NW * m) / NRT) + r) * LDT + 16 * kk + 4 * g);
                acc[m] = mm16(xr, st, acc[m]);
                if constexpr (OUT) qacc[m] = mm16(qr, st, qacc[m]);
              }
            }
          }
        }
      }
      const f32x4_t gam = row4(sgate + 16 * rt + 4 * g), be = row4(sgate + 128 + 16 * rt + 4 * g);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < nmine) {
          const int col = 16 * ((w + NW * m) / NRT) + r;
          const f32x4_t x = vcur[m] - gam * acc[m];
          if constexpr (OUT) oacc[m] = gam * qacc[m];
          *reinterpret_cast<f32x4_t *>(sYt + col * LDC + 16 * rt + 4 * g) = be * x;
        }
      }
    }
    load_v(nx);
    lds_sync();
    // U = M Y;  diag(s) U for the state update (for OUT, U itself: O needs it too)
    if (nmine > 0) {
      const f32x4_t sc = row4(sgate + 64 + 16 * rt + 4 * g);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < nmine) {
          const int col = 16 * ((w + NW * m) / NRT) + r;
          f32x4_t acc = zero4();
#pragma unroll
          for (int kb = 0; kb < NRT; ++kb) acc = mm16(mcur[kb], row4(sYt + col * LDC + 16 * kb + 4 * g), acc);
          if constexpr (!OUT) {
            if constexpr (!TRANS) {
#pragma unroll
              for (int q = 0; q < 4; ++q) ent[L.U + (16 * rt + 4 * g) * DV + c0 + col + q * DV] = acc[q];
            }
            if constexpr (SPL)
              *reinterpret_cast<bf16x8_t *>(sUs + col * Lds::LDP + 32 * rt + 8 * g) = split_hi_lo(sc * acc);
            else
              *reinterpret_cast<f32x4_t *>(sUt + col * LDC + 16 * rt + 4 * g) = sc * acc;
          } else {
            *reinterpret_cast<f32x4_t *>(sUt + col * LDC + 16 * rt + 4 * g) = acc;
          }
        }
      }
    }
    load_m(nx);
    lds_sync();
    // S <- gamma_C S + K^T diag(s) U
    const float gC = sgate[C - 1];
#pragma unroll
    for (int m = 0; m < MS; ++m) {
      const int i = w + NW * m;
      if (i < nst) {
        const int kt = i % NKT, ct = i / NKT;
        f32x4_t acc = accS[m] * gC;
        if constexpr (SPL) {
          // [K^T | K^T] against [(sU)_hi ; (sU)_lo], 16 tokens a step
#pragma unroll
          for (int kb = 0; kb < NRT; ++kb) {
            const bf16x4_t ak = tile_colfrag_raw(sK, LDK, 16 * kb, 16 * kt, r, g);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_shufflevector(ak, ak, 0, 1, 2, 3, 0, 1, 2, 3),
                *reinterpret_cast<const bf16x8_t *>(sUs + (16 * ct + r) * Lds::LDP + 32 * kb + 8 * g), acc, 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int kb = 0; kb < NRT; ++kb) {
            f32x4_t ut = row4(sUt + (16 * ct + r) * LDC + 16 * kb + 4 * g);
            if constexpr (OUT) ut = ut * row4(sgate + 64 + 16 * kb + 4 * g);
            acc = mm16(tile_colfrag(sK, LDK, 16 * kb, 16 * kt, r, g), ut, acc);
          }
        }
        accS[m] = acc;
      }
    }
    if constexpr (OUT) {
      // O = diag(gamma) Q S + P U, over the lower tiles of P's row tile
      if (nmine > 0) {
        const int tok0 = start + cc * C, n = min(C, end - tok0);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m < nmine) {
            const int col = 16 * ((w + NW * m) / NRT) + r;
            f32x4_t acc = oacc[m];
#pragma unroll
            for (int kb = 0; kb < NRT; ++kb)
              if (kb <= rt) acc = mm16(pcur[kb], row4(sUt + col * LDC + 16 * kb + 4 * g), acc);
            T *o = a.o + int64_t(tok0) * vrow + int64_t(h) * DV + c0 + col;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int t = 16 * rt + 4 * g + q;
              if (t < n) o[int64_t(t) * vrow] = from_f32<T>(acc[q]);
            }
          }
        }
      }
      load_p(nx);
    }
    lds_sync();
    kl.store(sK, LDK, DK);
    if constexpr (OUT) ql.store(sQ, LDK, DK);
    gl.store(sgate);
  }
  store_final();
}

template <typename T, int C>
__device__ void rev_chain(const BwdArgs<T> &a, int u, int cb, char *smem) {
  using Lds = ChainLds<T, C>;
  constexpr int NRT = C / 16, LDK = Lds::LDK, LDT = Lds::LDT, LDC = Lds::LDC;
  const int DK = a.d_k, DV = a.d_v, CB = min(32, DV), c0 = cb * CB;
  const int NKT = DK / 16, NCT = CB / 16;
  const int tid = threadIdx.x % kChainThreads, w = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
  T *sK = reinterpret_cast<T *>(smem);
  T *sQ = reinterpret_cast<T *>(smem + Lds::kTile);
  float *sdSt = reinterpret_cast<float *>(smem + 2 * Lds::kTile);  // dS'^T
  float *sdOt = sdSt + 32 * LDT;                                     // dO^T
  float *sdUt = sdOt + 32 * LDC;                                     // dU^T
  float *sdXt = sdUt + 32 * LDC;                                     // (-diag(gamma) dX)^T (fp32 inputs)
  // bf16 inputs: the splits of -diag(gamma) dX and of diag(gamma) dO, per
  // column: tokens 16 b + 4 g + j (j < 4) at 32 b + 8 g + j (hi) and + 4 (lo)
  bf16_t *sXs = reinterpret_cast<bf16_t *>(sdXt);
  bf16_t *sOs = sXs + 32 * Lds::LDP;
  bf16_t *sdSs = reinterpret_cast<bf16_t *>(sdSt);  // bf16 inputs: dS'^T split as hi + lo
  float *sgate = Lds::kSplitB ? reinterpret_cast<float *>(sOs + 32 * Lds::LDP) : sdXt + 32 * LDC;
  int s, h, start, end, c_first, n_chunks;
  unit_of(a.geo, a.H_v, u, s, h, start, end, c_first, n_chunks);
  const int hq = h / a.group;
  const BwdEntry L(C, DK, DV);
  const int64_t krow = int64_t(a.H_qk) * DK, vrow = int64_t(a.H_v) * DV;
  const int64_t unit_state = (int64_t(s) * a.H_v + h) * DK * DV;

  const int rt = w % NRT;
  const int nmine = (w < NRT * NCT) ? ((w + 4 < NRT * NCT) ? 2 : 1) : 0;
  const int nst = NKT * NCT;
  f32x4_t accS[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    accS[m] = zero4();
    const int i = w + 4 * m;
    if (i < nst && a.dhT) {
      const int kt = i % NKT, ct = i / NKT;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        accS[m][q] = a.dhT[unit_state + int64_t(16 * kt + 4 * g + q) * DV + c0 + 16 * ct + r];
    }
  }

  if (n_chunks > 0) {
    TileLoader<T, C> kl, ql;
    GateLoader gl;
    // dO column block: C rows x CB columns of T in 16-byte pieces
    constexpr int EPP = 16 / sizeof(T);
    constexpr int MAXO = (C * 32 / EPP + kChainThreads - 1) / kChainThreads;
    const int oppr = CB / EPP;
    uint4 ocur[MAXO];
    f32x4_t pcur[NRT], mcur[NRT];  // A fragments of P^T and M^T for this wave's row tile
    auto load_tiles = [&](int cc) {
      const int tok0 = start + cc * C, n = min(C, end - tok0);
      kl.load(a.k + int64_t(tok0) * krow + int64_t(hq) * DK, krow, n, DK);
      ql.load(a.q + int64_t(tok0) * krow + int64_t(hq) * DK, krow, n, DK);
      gl.load(a.ent + (int64_t(c_first + cc) * a.H_v + h) * a.ent_floats + L.gate);
#pragma unroll
      for (int m = 0; m < MAXO; ++m) {
        const int p = min(tid + kChainThreads * m, C * oppr - 1);
        const int t = p / oppr, c = (p - t * oppr) * EPP;
        const uint4 x =
            *reinterpret_cast<const uint4 *>(a.d_o + int64_t(tok0 + min(t, n - 1)) * vrow + int64_t(h) * DV + c0 + c);
        ocur[m] = t < n ? x : make_uint4(0, 0, 0, 0);
      }
    };
    // loaded a chunk ahead, right after their last use
    auto load_p = [&](int cc) {
      const float *ent = a.ent + (int64_t(c_first + cc) * a.H_v + h) * a.ent_floats;
#pragma unroll
      for (int kb = 0; kb < NRT; ++kb) pcur[kb] = col4(ent + L.P + (16 * kb + 4 * g) * C + 16 * rt + r, C);
    };
    auto load_m = [&](int cc) {
      const float *ent = a.ent + (int64_t(c_first + cc) * a.H_v + h) * a.ent_floats;
#pragma unroll
      for (int kb = 0; kb < NRT; ++kb) mcur[kb] = col4(ent + L.M + (16 * kb + 4 * g) * C + 16 * rt + r, C);
    };
    auto store_do = [&]() {  // transposed: dO^T[column][token]
#pragma unroll
      for (int m = 0; m < MAXO; ++m) {
        const int p = min(tid + kChainThreads * m, C * oppr - 1);
        const int t = p / oppr, c = (p - t * oppr) * EPP;
        const T *x = reinterpret_cast<const T *>(&ocur[m]);
#pragma unroll
        for (int j = 0; j < EPP; ++j) sdOt[(c + j) * LDC + t] = to_f32(x[j]);
      }
    };
    load_tiles(n_chunks - 1);
    load_p(n_chunks - 1);
    load_m(n_chunks - 1);
    kl.store(sK, LDK, DK);
    ql.store(sQ, LDK, DK);
    gl.store(sgate);
    store_do();

    for (int cc = n_chunks - 1; cc >= 0; --cc) {
      const int tok0 = start + cc * C, n = min(C, end - tok0);
      float *ent = a.ent + (int64_t(c_first + cc) * a.H_v + h) * a.ent_floats;
      // the gradient at this chunk's end state: to LDS, transposed, and to the entry
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int i = w + 4 * m;
        if (i < nst) {
          const int kt = i % NKT, ct = i / NKT;
          if constexpr (Lds::kSplitB)
            *reinterpret_cast<bf16x8_t *>(sdSs + (16 * ct + r) * Lds::LDSS + 32 * kt + 8 * g) = split_hi_lo(accS[m]);
          else
            *reinterpret_cast<f32x4_t *>(sdSt + (16 * ct + r) * LDT + 16 * kt + 4 * g) = accS[m];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            ent[L.dS + (16 * kt + 4 * g) * DV + c0 + 16 * ct + r + q * DV] = accS[m][q];
        }
      }
      const int nx = max(cc - 1, 0);  // the next chunk back (the first one reloads itself)
      load_tiles(nx);
      lds_sync();
      // dU = P^T dO + diag(s) K dS'
      if (nmine > 0) {
        f32x4_t kds[2] = {zero4(), zero4()}, pdo[2] = {zero4(), zero4()};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          if (16 * kk < DK) {
            if constexpr (Lds::kSplitB) {
              // [K | K] against [dS'_hi ; dS'_lo], 16 channels a step
              const bf16x4_t kr = *reinterpret_cast<const bf16x4_t *>(sK + (16 * rt + r) * LDK + 16 * kk + 4 * g);
              const bf16x8_t k8 = __builtin_shufflevector(kr, kr, 0, 1, 2, 3, 0, 1, 2, 3);
#pragma unroll
              for (int m = 0; m < 2; ++m)
                if (m < nmine)
                  kds[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                      k8,
                      *reinterpret_cast<const bf16x8_t *>(sdSs + (16 * ((w + 4 * m) / NRT) + r) * Lds::LDSS + 32 * kk +
                                                          8 * g),
                      kds[m], 0, 0, 0);
            } else {
              const f32x4_t xr = row4(sK + (16 * rt + r) * LDK + 16 * kk + 4 * g);
#pragma unroll
              for (int m = 0; m < 2; ++m)
                if (m < nmine)
                  kds[m] = mm16(xr, row4(sdSt + (16 * ((w + 4 * m) / NRT) + r) * LDT + 16 * kk + 4 * g), kds[m]);
            }
          }
        }
#pragma unroll
        for (int kb = 0; kb < NRT; ++kb)
#pragma unroll
          for (int m = 0; m < 2; ++m)
            if (m < nmine)
              pdo[m] = mm16(pcur[kb], row4(sdOt + (16 * ((w + 4 * m) / NRT) + r) * LDC + 16 * kb + 4 * g), pdo[m]);
        const f32x4_t sc = row4(sgate + 64 + 16 * rt + 4 * g);
#pragma unroll
        for (int m = 0; m < 2; ++m)
          if (m < nmine)
            *reinterpret_cast<f32x4_t *>(sdUt + (16 * ((w + 4 * m) / NRT) + r) * LDC + 16 * rt + 4 * g) =
                pdo[m] + sc * kds[m];
      }
      if constexpr (Lds::kSplitB) {
        // diag(gamma) dO, split, for the state update
        for (int it = tid; it < CB * (C / 4); it += kChainThreads) {
          const int col = it / (C / 4), tq = it - col * (C / 4);
          const f32x4_t x = row4(sdOt + col * LDC + 4 * tq) * row4(sgate + 4 * tq);
          *reinterpret_cast<bf16x8_t *>(sOs + col * Lds::LDP + 32 * (tq >> 2) + 8 * (tq & 3)) = split_hi_lo(x);
        }
      }
      load_p(nx);
      lds_sync();
      // dY = M^T dU;  dv = dX = diag(beta) dY
      if (nmine > 0) {
        const f32x4_t gam = row4(sgate + 16 * rt + 4 * g), be = row4(sgate + 128 + 16 * rt + 4 * g);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          if (m < nmine) {
            const int col = 16 * ((w + 4 * m) / NRT) + r;
            f32x4_t acc = zero4();
#pragma unroll
            for (int kb = 0; kb < NRT; ++kb) acc = mm16(mcur[kb], row4(sdUt + col * LDC + 16 * kb + 4 * g), acc);
            const f32x4_t dx = be * acc;
            // dY to the entry; dv = dX to the output (rows past the chunk's end are not stored)
            float *dvp = a.dv + (int64_t(tok0) + 16 * rt + 4 * g) * vrow + int64_t(h) * DV + c0 + col;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              ent[L.dY + (16 * rt + 4 * g) * DV + c0 + col + q * DV] = acc[q];
              if (16 * rt + 4 * g + q < n) dvp[q * vrow] = dx[q];
            }
            if constexpr (Lds::kSplitB)
              *reinterpret_cast<bf16x8_t *>(sXs + col * Lds::LDP + 32 * rt + 8 * g) = split_hi_lo(-(gam * dx));
            else
              *reinterpret_cast<f32x4_t *>(sdXt + col * LDC + 16 * rt + 4 * g) = -(gam * dx);
          }
        }
      }
      load_m(nx);
      lds_sync();
      // dS <- gamma_C dS' + Q^T diag(gamma) dO - K^T diag(gamma) dX
      const float gC = sgate[C - 1];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int i = w + 4 * m;
        if (i < nst) {
          const int kt = i % NKT, ct = i / NKT;
          f32x4_t acc = accS[m] * gC;
          if constexpr (Lds::kSplitB) {
            // bf16 MFMA, 16 tokens a step: [Q^T | Q^T] against [hi ; lo]
#pragma unroll
            for (int kb = 0; kb < NRT; ++kb) {
              const bf16x4_t aq = tile_colfrag_raw(sQ, LDK, 16 * kb, 16 * kt, r, g);
              const bf16x4_t ak = tile_colfrag_raw(sK, LDK, 16 * kb, 16 * kt, r, g);
              const int o = (16 * ct + r) * Lds::LDP + 32 * kb + 8 * g;
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_shufflevector(aq, aq, 0, 1, 2, 3, 0, 1, 2, 3),
                                                            *reinterpret_cast<const bf16x8_t *>(sOs + o), acc, 0, 0, 0);
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_shufflevector(ak, ak, 0, 1, 2, 3, 0, 1, 2, 3),
                                                            *reinterpret_cast<const bf16x8_t *>(sXs + o), acc, 0, 0, 0);
            }
          } else {
#pragma unroll
            for (int kb = 0; kb < NRT; ++kb) {
              const f32x4_t xq = tile_colfrag(sQ, LDK, 16 * kb, 16 * kt, r, g) * row4(sgate + 16 * kb + 4 * g);
              acc = mm16(xq, row4(sdOt + (16 * ct + r) * LDC + 16 * kb + 4 * g), acc);
              acc = mm16(tile_colfrag(sK, LDK, 16 * kb, 16 * kt, r, g),
                         row4(sdXt + (16 * ct + r) * LDC + 16 * kb + 4 * g), acc);
            }
          }
          accS[m] = acc;
        }
      }
      lds_sync();
      kl.store(sK, LDK, DK);
      ql.store(sQ, LDK, DK);
      gl.store(sgate);
      store_do();
    }
  }
  if (a.dh0) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int i = w + 4 * m;
      if (i < nst) {
        const int kt = i % NKT, ct = i / NKT;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          a.dh0[unit_state + int64_t(16 * kt + 4 * g + q) * DV + c0 + 16 * ct + r] = accS[m][q];
      }
    }
  }
}

}  // namespace

// One block per (unit, column block): waves 0-3 walk the chunks forward and
// waves 4-7 walk them backward, each on its own LDS region.  Both take the
// same barriers (four per chunk, over the same chunks), so each CU runs one
// chain of each direction and the two share its matrix units (the backward
// chain has 1.6 times the forward's products).  Where the two regions do not
// fit together (fp32 inputs in chunks of 64), a block of four waves runs one
// direction: even slots of a unit forward, odd ones backward.  Blocks come in
// groups of 8 units x column blocks: the blocks of a unit have the same block
// id mod 8, so they share one XCD's L2 copy of its k and q.
template <typename T, int C>
__global__ __launch_bounds__((ChainLds<T, C>::kPaired ? 2 * kChainThreads : kChainThreads)) void bwd_chain_kernel(
    BwdArgs<T> a) {
  using Lds = ChainLds<T, C>;
  const int n_cb = a.d_v / min(32, a.d_v);
  int u, x;
  if constexpr (Lds::kPaired) {
    __shared__ __attribute__((aligned(16))) char smem_f[Lds::kFwd];
    __shared__ __attribute__((aligned(16))) char smem_r[Lds::kRev];
    decode_block(blockIdx.x, n_cb, u, x);
    if (u >= a.n_units) return;
    if (threadIdx.x >= kChainThreads)
      rev_chain<T, C>(a, u, x, smem_r);
    else
      fwd_chain<T, C, false>(a, u, x, smem_f);
  } else {
    __shared__ __attribute__((aligned(16))) char smem[Lds::kBytes];
    decode_block(blockIdx.x, 2 * n_cb, u, x);
    if (u >= a.n_units) return;
    if (x & 1)
      rev_chain<T, C>(a, u, x >> 1, smem);
    else
      fwd_chain<T, C, false>(a, u, x >> 1, smem);
  }
}

// The forward pass on the chained form: one block of four waves per (unit,
// column block), in the same XCD-aware order, running the forward chain with
// outputs.
template <typename T, int C, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void chain_fwd_kernel(BwdArgs<T> a) {
  using Lds = ChainLds<T, C>;
  __shared__ __attribute__((aligned(16))) char smem[Lds::kOut];
  const int n_cb = a.d_v / a.cols;
  int u, x;
  decode_block(blockIdx.x, n_cb, u, x);
  if (u >= a.n_units) return;
  fwd_chain<T, C, true, NW>(a, u, x, smem);
}
// The transition pass of the segment-parallel form on the chained form: one
// block per (segment unit, column block of the d_v + d_k state columns of
// [B | M]), no outputs; each segment's final [B | M] goes to the map buffer.
template <typename T, int C, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void chain_trans_kernel(BwdArgs<T> a) {
  using Lds = ChainLds<T, C>;
  __shared__ __attribute__((aligned(16))) char smem[Lds::kFwd];
  const int n_cb = (a.d_v + a.d_k) / a.cols;
  int u, x;
  decode_block(blockIdx.x, n_cb, u, x);
  if (u >= a.n_units) return;
  fwd_chain<T, C, false, NW, true>(a, u, x, smem);
}
// Waves per forward-pass chain block: fp32 operands fill enough LDS that a CU
// holds one block, so it gets eight waves (two per SIMD) to hide LDS and
// barrier waits; a bf16 block has four, and a CU holds two.
template <typename T> constexpr int chain_fwd_waves() { return sizeof(T) == 4 ? 8 : 4; }

// ---------------------------------------------------------------------------
// 3. Per (chunk, value head): the gradients.  16 waves.
//
// Phase 1 runs over d_v in slabs of DVS columns staged in LDS (dO, dY, U).
// The C x d_k products W1 = dO S^T, W2 = dY S^T, W3 = U dS'^T are tiled
// 16 x 16: wave w owns d_k column tile w % (d_k/16) and the row tiles i with
// i % (16 / (d_k/16)) == w / (d_k/16), and reads its S and dS' rows straight
// from the entry.  Each lower tile of dO U^T and dY U^T has a wave of its
// own.  Phase 2 forms dP . Gamma, dG and
// Gamma . dGamma in LDS and finishes dq and dk with the products against K and
// Q (contraction over the chunk).
// ---------------------------------------------------------------------------
namespace {
constexpr int kGradThreads = 1024;
constexpr int kGradWaves = kGradThreads / 64;
}

template <typename T, int C, int DVS>
__global__ __launch_bounds__(kGradThreads) void bwd_grad_kernel(BwdArgs<T> a) {
  // slab rows 32 bytes past a multiple of 128 (LDV): half the LDS bank
  // conflicts of 16 bytes past, measured
  constexpr int NRT = C / 16, LD = C + 4, LDV = DVS + 8, NL = NRT * (NRT + 1) / 2;
  constexpr int kSlabFloats = 3 * C * LDV, kPh2Floats = 3 * C * LD;
  constexpr int kBig = kSlabFloats > kPh2Floats ? kSlabFloats : kPh2Floats;
  constexpr int NK = DVS / 16;                                        // 16-deep steps per slab
  constexpr int WPR = DVS / 4;                                        // float4 pieces per slab row
  constexpr int NPC = (C * WPR + kGradThreads - 1) / kGradThreads;    // pieces per thread
  constexpr bool SPLG = sizeof(T) == 2;  // bf16 inputs: products with dO, k or q on the bf16 MFMA
  __shared__ __attribute__((aligned(16))) float big[kBig];
  __shared__ float sPartG[64 * 8], sPartS[64 * 8], sPartK[64 * 8];
  __shared__ float sR1[64], sRowE[64], sRowF[64], sColE[64], sSd[kGradWaves];
  __shared__ float sGam[64], sSc[64], sG2[64], sBe[64];
  // the chunk's K and Q rows (operands of the products over the chunk in
  // phase 2), staged once at the start
  constexpr int LDKG = 128 + 16 / sizeof(T);
  __shared__ __attribute__((aligned(16))) T sKg[C * LDKG];
  __shared__ __attribute__((aligned(16))) T sQg[C * LDKG];

  const int e = blockIdx.x;
  const int slot = e / a.H_v, h = e - slot * a.H_v;
  int s, tok0, n;
  if (!a.geo.locate(slot, s, tok0, n)) return;
  const int hq = h / a.group, DK = a.d_k, DV = a.d_v;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
  const BwdEntry L(C, DK, DV);
  const float *ent = a.ent + int64_t(e) * a.ent_floats;
  const int64_t krow = int64_t(a.H_qk) * DK, vrow = int64_t(a.H_v) * DV;
  {
    TileLoader<T, C, kGradThreads> kl, ql;
    kl.load(a.k + int64_t(tok0) * krow + int64_t(hq) * DK, krow, n, DK);
    ql.load(a.q + int64_t(tok0) * krow + int64_t(hq) * DK, krow, n, DK);
    kl.store(sKg, LDKG, DK);
    ql.store(sQg, LDKG, DK);
  }

  if (tid < C) {
    sGam[tid] = ent[L.gate + kGateGamma + tid];
    sSc[tid] = ent[L.gate + kGateS + tid];
    sG2[tid] = ent[L.gate + kGateLog2 + tid];
    sBe[tid] = ent[L.gate + kGateBeta + tid];
  }

  // ---- tile ownership ----
  const int NKT = DK / 16, wpc = kGradWaves / NKT;  // waves per d_k column tile
  const int ct = w % NKT, rsel = w / NKT;  // d_k column tile, row-tile residue
  const bool has_rows = rsel < NRT;
  // lower C x C tile of this wave (at most 10 of them: C <= 64)
  static_assert(NL <= kGradWaves, "one lower tile per wave");
  const int np = w < NL;
  int prt[1], pct[1];
  lower_tile(min(w, NL - 1), prt[0], pct[0]);
  // this wave's row tiles: i = rsel + m wpc (wpc >= 2, so at most RPW of them)
  constexpr int RPW = (NRT + 1) / 2;
  f32x4_t W1[RPW], W2[RPW], W3[RPW], aP[1], aA[1];
#pragma unroll
  for (int m = 0; m < RPW; ++m) W1[m] = W2[m] = W3[m] = zero4();
  aP[0] = aA[0] = zero4();
  float sd = 0.0f;  // <S, dS'> partial (one wave per d_k column tile)
  float r1acc[NPC];
#pragma unroll
  for (int m = 0; m < NPC; ++m) r1acc[m] = 0.0f;

  float *sdO = big, *sdY = big + C * LDV, *sU = big + 2 * C * LDV;
  const float *Sg = ent + L.S + int64_t(16 * ct + r) * DV + 4 * g;
  const float *dSg = ent + L.dS + int64_t(16 * ct + r) * DV + 4 * g;
  for (int dv0 = 0; dv0 < DV; dv0 += DVS) {
    f32x4_t yS[NK], ydS[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      yS[kk] = has_rows ? row4(Sg + dv0 + 16 * kk) : zero4();
      ydS[kk] = has_rows ? row4(dSg + dv0 + 16 * kk) : zero4();
    }
    // stage dO, dY, U; sum dY . V on the way (the dY . X row sums of dbeta
    // are dY . V - gamma K . (dY S^T), and dY S^T is formed here anyway)
#pragma unroll
    for (int m = 0; m < NPC; ++m) {
      const int p = tid + kGradThreads * m;
      float part = 0.0f;
      if (p < C * WPR) {
        const int t = p / WPR, c = (p - t * WPR) * 4;
        const f32x4_t od = row4(a.d_o + int64_t(tok0 + min(t, n - 1)) * vrow + int64_t(h) * DV + dv0 + c);
        const f32x4_t o = t < n ? od : zero4();
        const f32x4_t y = row4(ent + L.dY + int64_t(t) * DV + dv0 + c);
        const f32x4_t uu = row4(ent + L.U + int64_t(t) * DV + dv0 + c);
        const f32x4_t vx = row4(a.v + int64_t(tok0 + min(t, n - 1)) * vrow + int64_t(h) * DV + dv0 + c);
        const f32x4_t x = t < n ? vx : zero4();
        *reinterpret_cast<f32x4_t *>(sdO + t * LDV + c) = o;
        *reinterpret_cast<f32x4_t *>(sdY + t * LDV + c) = y;
        *reinterpret_cast<f32x4_t *>(sU + t * LDV + c) = uu;
        part = y[0] * x[0] + y[1] * x[1] + y[2] * x[2] + y[3] * x[3];
      }
      r1acc[m] += group_sum(part, WPR);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const int k0 = 16 * kk + 4 * g;
      if (has_rows) {
        // bf16 inputs: dO is exact in bf16, so dO S^T runs on the bf16 MFMA
        // with S split hi + lo
        bf16x8_t ySs{};
        if constexpr (SPLG) ySs = split_hi_lo(yS[kk]);
#pragma unroll
        for (int m = 0; m < RPW; ++m) {
          const int i = rsel + m * wpc;
          if (i >= NRT) continue;
          const int row = (16 * i + r) * LDV + k0;
          if constexpr (SPLG)
            W1[m] = mm16_sy(row4(sdO + row), ySs, W1[m]);
          else
            W1[m] = mm16(row4(sdO + row), yS[kk], W1[m]);
          W2[m] = mm16(row4(sdY + row), yS[kk], W2[m]);
          W3[m] = mm16(row4(sU + row), ydS[kk], W3[m]);
        }
        if (rsel == 0) {
          const f32x4_t pr = yS[kk] * ydS[kk];
          sd += (pr[0] + pr[1]) + (pr[2] + pr[3]);
        }
      }
#pragma unroll
      for (int j = 0; j < 1; ++j) {
        if (j < np) {
          const f32x4_t yu = row4(sU + (16 * pct[j] + r) * LDV + k0);
          if constexpr (SPLG)
            aP[j] = mm16_sy(row4(sdO + (16 * prt[j] + r) * LDV + k0), split_hi_lo(yu), aP[j]);
          else
            aP[j] = mm16(row4(sdO + (16 * prt[j] + r) * LDV + k0), yu, aP[j]);
          aA[j] = mm16(row4(sdY + (16 * prt[j] + r) * LDV + k0), yu, aA[j]);
        }
      }
    }
    __syncthreads();
  }
  // row sums of dY . V: the first thread of each row's group holds them
#pragma unroll
  for (int m = 0; m < NPC; ++m) {
    const int p = tid + kGradThreads * m;
    if (p < C * WPR && (p % WPR) == 0) sR1[p / WPR] = r1acc[m];
  }
  {
    const float sdw = group_sum(sd, 64);
    if (lane == 0) sSd[w] = sdw;
  }

  // ---- phase 2: C x C matrices in LDS (the slab area is free) ----
  float *sdP = big, *sdA = big + C * LD, *sE = big + 2 * C * LD;
  // tiles above the diagonal are zero; the computed lower tiles carry their masks
  for (int idx = tid; idx < C * C; idx += kGradThreads) {
    const int t = idx / C, i = idx - t * C;
    if ((i >> 4) > (t >> 4)) {
      sdP[t * LD + i] = 0.0f;
      sdA[t * LD + i] = 0.0f;
    }
  }
#pragma unroll
  for (int j = 0; j < 1; ++j) {
    if (j < np) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = 16 * prt[j] + 4 * g + q, i = 16 * pct[j] + r;
        sdP[t * LD + i] = i <= t ? aP[j][q] : 0.0f;
        sdA[t * LD + i] = i < t ? -aA[j][q] : 0.0f;
      }
    }
  }
  // K and Q values of this wave's d_k column tile, from LDS:
  // kf(i)[j] = K[16 i + 4g + j][16 ct + r] (rows past the chunk's end are zero)
  auto kf = [&](int i) { return tile_colfrag(sKg, LDKG, 16 * i, 16 * ct, r, g); };
  auto qf = [&](int i) { return tile_colfrag(sQg, LDKG, 16 * i, 16 * ct, r, g); };
  __syncthreads();
  // elementwise, 8 threads per row: dP . Gamma, dG = dA . diag(beta) Gamma,
  // E = Gamma . dGamma = diag(beta) dA . (Gamma . KK^T) + dP . P
  {
    const int t = tid >> 3, part = tid & 7;
    float rowE = 0.0f, rowF = 0.0f;
    if (t < C) {
      for (int i = part; i < C; i += 8) {
        const float dp = sdP[t * LD + i], da = sdA[t * LD + i];
        const float gam = i <= t ? fast_exp2(sG2[t] - sG2[i]) : 0.0f;
        const float f = da * ent[L.G + t * C + i];
        const float ev = sBe[t] * f + dp * ent[L.P + t * C + i];
        rowE += ev;
        rowF += f;
        sdP[t * LD + i] = dp * gam;
        sdA[t * LD + i] = da * sBe[t] * gam;
        sE[t * LD + i] = ev;
      }
    }
    rowE = group_sum(rowE, 8);
    rowF = group_sum(rowF, 8);
    if (t < C && part == 0) {
      sRowE[t] = rowE;
      sRowF[t] = rowF;
    }
  }
  __syncthreads();
  if (tid < C) {
    float c = 0.0f;
    for (int i = 0; i < C; ++i) c += sE[i * LD + tid];
    sColE[tid] = c;
  }
  __syncthreads();
  // H = dG + dG^T, into E's place
  for (int idx = tid; idx < C * C; idx += kGradThreads) {
    const int t = idx / C, i = idx - t * C;
    sE[t * LD + i] = sdA[t * LD + i] + sdA[i * LD + t];
  }
  __syncthreads();
  // dq, dk and the d_k row sums of this wave's tiles
  if (has_rows) {
#pragma unroll
    for (int m = 0; m < RPW; ++m) {
      const int i = rsel + m * wpc;
      if (i >= NRT) continue;
      const f32x4_t kfi = kf(i), qfi = qf(i);  // K and Q values of row tile i
      f32x4_t aq = zero4(), ak = zero4();
#pragma unroll
      for (int kb = 0; kb < NRT; ++kb) {
        const f32x4_t kk = kf(kb), qq = qf(kb);
        if constexpr (SPLG) {  // k and q exact in bf16: the C x C factors split
          aq = mm16_sx(row4(sdP + (16 * i + r) * LD + 16 * kb + 4 * g), kk, aq);
          ak = mm16_sx(col4(sdP + (16 * kb + 4 * g) * LD + 16 * i + r, LD), qq, ak);
          ak = mm16_sx(row4(sE + (16 * i + r) * LD + 16 * kb + 4 * g), kk, ak);
        } else {
          aq = mm16(row4(sdP + (16 * i + r) * LD + 16 * kb + 4 * g), kk, aq);
          ak = mm16(col4(sdP + (16 * kb + 4 * g) * LD + 16 * i + r, LD), qq, ak);
          ak = mm16(row4(sE + (16 * i + r) * LD + 16 * kb + 4 * g), kk, ak);
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = 16 * i + 4 * g + q, col = 16 * ct + r;
        const float dqv = sGam[t] * W1[m][q] + aq[q];
        const float dkv = ak[q] - sGam[t] * sBe[t] * W2[m][q] + sSc[t] * W3[m][q];
        const float pg = group_sum(qfi[q] * W1[m][q] - sBe[t] * kfi[q] * W2[m][q], 16);
        const float ps = group_sum(kfi[q] * W3[m][q], 16);
        const float pk = group_sum(kfi[q] * W2[m][q], 16);
        if (r == 0) {
          sPartG[t * 8 + ct] = pg;
          sPartS[t * 8 + ct] = ps;
          sPartK[t * 8 + ct] = pk;
        }
        if (t < n) {
          const int64_t o = (int64_t(tok0 + t) * a.H_v + h) * DK + col;
          a.dq[o] = dqv;
          a.dk[o] = dkv;
        }
      }
    }
  }
  __syncthreads();
  // per-token scalars, lane t of wave 0
  if (w == 0) {
    const int t = lane;
    float dg = 0.0f, sds = 0.0f;
    if (t < n) {
      float pg = 0.0f, ps = 0.0f, pk = 0.0f;
      for (int c = 0; c < NKT; ++c) {
        pg += sPartG[t * 8 + c];
        ps += sPartS[t * 8 + c];
        pk += sPartK[t * 8 + c];
      }
      sds = sSc[t] * ps;
      dg = sGam[t] * pg + sRowE[t] - sColE[t] - sds;
      a.dbeta[int64_t(tok0 + t) * a.H_v + h] = (sR1[t] - sGam[t] * pk) + sRowF[t];
    }
    const float tot_sds = group_sum(sds, 64);
    float sdsum = 0.0f;
    for (int i = 0; i < kGradWaves; ++i) sdsum += sSd[i];
    if (t == n - 1) dg += sGam[C - 1] * sdsum + tot_sds;
    // suffix sums over t' >= t: a prefix sum over the reversed lanes
    const float rev = __shfl(dg, max(n - 1 - lane, 0));
    const float pre = wave_prefix_sum(lane < n ? rev : 0.0f);
    const float suf = __shfl(pre, max(n - 1 - lane, 0));
    if (t < n) {
      const int64_t gi = int64_t(tok0 + t) * a.H_v + h;
      a.dalpha[gi] = suf / a.alpha[gi];
    }
  }
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

size_t bwd_entry_floats(int chunk, int d_k, int d_v) { return size_t(BwdEntry(chunk, d_k, d_v).total); }

template <typename T, int C>
static hipError_t launch_bwd_c(const BwdProblem &b, const BwdArgs<T> &a, hipStream_t st) {
  const Problem &p = b.p;
  const unsigned n_ent = unsigned(int64_t(a.geo.n_slots) * p.H_v);
  if (n_ent > 0) {
    hipLaunchKernelGGL((bwd_factor_kernel<T, C>), dim3(n_ent), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int n_cb = p.d_v / std::min(32, p.d_v);
  const int64_t groups = (int64_t(a.n_units) + 7) / 8;
  if (ChainLds<T, C>::kPaired)
    hipLaunchKernelGGL((bwd_chain_kernel<T, C>), dim3(unsigned(groups * 8 * n_cb)), dim3(2 * kChainThreads), 0, st, a);
  else
    hipLaunchKernelGGL((bwd_chain_kernel<T, C>), dim3(unsigned(groups * 8 * 2 * n_cb)), dim3(kChainThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_ent == 0) return e;
  if (p.d_v >= 32)
    hipLaunchKernelGGL((bwd_grad_kernel<T, C, 32>), dim3(n_ent), dim3(kGradThreads), 0, st, a);
  else
    hipLaunchKernelGGL((bwd_grad_kernel<T, C, 16>), dim3(n_ent), dim3(kGradThreads), 0, st, a);
  return hipGetLastError();
}

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
  a.h0 = p.h0;
  a.dhT = b.dhT;
  a.ent = b.entries;
  a.ent_floats = int64_t(bwd_entry_floats(p.chunk, p.d_k, p.d_v));
  const int group = p.H_v / p.H_qk;
  a.dq = group == 1 ? b.dq : b.dq_part;
  a.dk = group == 1 ? b.dk : b.dk_part;
  a.dv = b.dv;
  a.dalpha = b.dalpha;
  a.dbeta = b.dbeta;
  a.dh0 = b.dh0;
  a.o = nullptr;
  a.hT = nullptr;
  a.want_g = true;
  a.cols = std::min(32, p.d_v);
  a.H_qk = p.H_qk;
  a.H_v = p.H_v;
  a.d_k = p.d_k;
  a.d_v = p.d_v;
  a.group = group;
  a.n_units = p.n_seqs * p.H_v;
  a.geo = make_geom(p, &b.ws);
  if (a.n_units == 0) return hipSuccess;
  hipError_t e = p.chunk == 16   ? launch_bwd_c<T, 16>(b, a, st)
                 : p.chunk == 32 ? launch_bwd_c<T, 32>(b, a, st)
                                 : launch_bwd_c<T, 64>(b, a, st);
  if (e != hipSuccess || group == 1) return e;
  const int64_t tokens = p.n_tokens();
  const int64_t total = tokens * p.H_qk * p.d_k;
  if (total == 0) return hipSuccess;
  const unsigned blocks = unsigned(std::min<int64_t>((total + 255) / 256, 1 << 16));
  hipLaunchKernelGGL(group_sum_kernel, dim3(blocks), dim3(256), 0, st, b.dq_part, b.dq, tokens, p.H_qk, group,
                     p.d_k);
  hipLaunchKernelGGL(group_sum_kernel, dim3(blocks), dim3(256), 0, st, b.dk_part, b.dk, tokens, p.H_qk, group,
                     p.d_k);
  return hipGetLastError();
}

hipError_t launch_chunk_bwd(const BwdProblem &b, hipStream_t st) {
  return b.p.dtype == 1 ? launch_chunk_bwd_t<bf16_t>(b, st) : launch_chunk_bwd_t<float>(b, st);
}

// ---------------------------------------------------------------------------
// The chained forward: the factor kernel (M, P and the gates only), then the
// forward chain with outputs; in the segment-parallel form the factor kernel,
// the transition pass (each segment's map), the fold, and the forward chain
// from the folded states.  Its entries are the first BwdEntry::G floats of a
// backward entry.
// ---------------------------------------------------------------------------
template <typename T>
static BwdArgs<T> chain_args(const Problem &p, const Workspace &ws, float *mb) {
  BwdArgs<T> a{};
  a.q = static_cast<const T *>(p.q);
  a.k = static_cast<const T *>(p.k);
  a.v = static_cast<const T *>(p.v);
  a.alpha = p.alpha;
  a.beta = p.beta;
  a.h0 = p.h0;
  a.ent = static_cast<float *>(ws.entries);
  a.ent_floats = BwdEntry(p.chunk, 0, 0).G;
  a.o = static_cast<T *>(p.o);
  a.hT = p.hT;
  a.mb = mb;
  a.want_g = false;
  a.H_qk = p.H_qk;
  a.H_v = p.H_v;
  a.d_k = p.d_k;
  a.d_v = p.d_v;
  a.group = p.H_v / p.H_qk;
  a.n_units = p.n_seqs * p.H_v;
  // 16-column blocks where 32-column ones would leave CUs without a chain (or,
  // in the transition pass, where a 32-column block would straddle B and M)
  const int cols = p.d_v + (mb ? p.d_k : 0);
  a.cols = std::min(32, p.d_v);
  if (a.cols == 32 && (int64_t(a.n_units) * (cols / 32) < 256 || (mb && p.d_k % 32 != 0))) a.cols = 16;
  a.geo = make_geom(p, &ws);
  return a;
}

template <typename T, int C>
static hipError_t launch_chain_c(const BwdArgs<T> &a, bool factors, hipStream_t st) {
  const unsigned n_ent = unsigned(int64_t(a.geo.n_slots) * a.H_v);
  if (factors && n_ent > 0) {
    hipLaunchKernelGGL((bwd_factor_kernel<T, C>), dim3(n_ent), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.n_units == 0) return hipSuccess;
  const int64_t groups = (int64_t(a.n_units) + 7) / 8;
  constexpr int NW = chain_fwd_waves<T>();
  if (a.mb) {
    const int n_cb = (a.d_v + a.d_k) / a.cols;
    hipLaunchKernelGGL((chain_trans_kernel<T, C, NW>), dim3(unsigned(groups * 8 * n_cb)), dim3(64 * NW), 0, st, a);
  } else {
    const int n_cb = a.d_v / a.cols;
    hipLaunchKernelGGL((chain_fwd_kernel<T, C, NW>), dim3(unsigned(groups * 8 * n_cb)), dim3(64 * NW), 0, st, a);
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_chain_t(const Problem &p, const Workspace &ws, float *mb, bool factors, hipStream_t st) {
  const BwdArgs<T> a = chain_args<T>(p, ws, mb);
  return p.chunk == 16   ? launch_chain_c<T, 16>(a, factors, st)
         : p.chunk == 32 ? launch_chain_c<T, 32>(a, factors, st)
                         : launch_chain_c<T, 64>(a, factors, st);
}

hipError_t launch_chain_fwd(const Problem &p, const Workspace &ws, hipStream_t st, float *mb, bool factors) {
  if (int64_t(entry_stride(p)) != BwdEntry(p.chunk, 0, 0).G * int64_t(sizeof(float))) return hipErrorInvalidValue;
  return p.dtype == 1 ? launch_chain_t<bf16_t>(p, ws, mb, factors, st) : launch_chain_t<float>(p, ws, mb, factors, st);
}

}  // namespace gdn
