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

// General path (fp32, or d_k != 128): fragments are read from global memory,
// A and M = (I + A)^-1 live in LDS.
template <typename T>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs<T> a) {
  const int c = blockIdx.x;
  const int h = blockIdx.y;
  int s, tok0, len;
  if (!a.geo.locate(c, s, tok0, len)) return;
  const int hq = h / a.group;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  constexpr int kLdsMain = 2 * 64 * 65 * 4;
  __shared__ __attribute__((aligned(16))) char smem[kLdsMain];
  __shared__ float sY[3][16][17];
  __shared__ float sg[64], sb[64];
  float(*sA)[65] = reinterpret_cast<float(*)[65]>(smem);
  float(*sM)[65] = reinterpret_cast<float(*)[65]>(smem + 64 * 65 * 4);

  const int64_t stride = int64_t(a.H_qk) * a.d_k;
  const T *kb = a.k + int64_t(tok0) * stride + int64_t(hq) * a.d_k;
  const T *qb = a.q + int64_t(tok0) * stride + int64_t(hq) * a.d_k;
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
  lds_barrier();

  auto frag = [&](int src, int r, int kk) -> Frag<T> {
    return load_row_frag(src == 0 ? kb : qb, stride, 16 * r + (lane & 15), len, 32 * kk, a.d_k,
                         lane);
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

// ---------------------------------------------------------------------------
// bf16, d_k = 128: the factor kernel.  One workgroup per (chunk slot, value
// head); its k and q rows and gates are copied into LDS with bounds-checked
// buffer loads (rows past the chunk's end read as zeros, padded slots get
// beta = 0 and add nothing to the gate).
//
// M = (I + A)^-1 in 16 x 16 blocks: D_b = (I + A_bb)^-1 by forward
// substitution and M_bc = -D_b sum_{j=c}^{b-1} A_bj M_jc for b > c, the
// products on fp32 MFMA.  The block columns of M are independent: wave 0
// forms column 0 (9 products), wave 1 columns 1-3 (7); the part both need (gates,
// A, the D_b) runs as one code path in both, so their shared LDS writes carry
// identical values.  A stays in registers: by the symmetry of K K^T the tile
// K_j K_b^T holds row t = 16 b + r of A_bj in lane (r, g) (columns
// 16 j + 4 g .. + 3), the left-operand layout of the block products.  Waves 2
// and 3 form P (t-blocks 0-2 and 3) and the gate factors, which go out
// directly.  T stays in registers until P is formed; it is then assembled
// over the dead q tile and leaves in 16-byte stores (48 KiB of LDS: three
// workgroups per CU).
// ---------------------------------------------------------------------------
namespace {
constexpr int kXK = 0;          // k rows, 64 x 128 bf16 row tile
constexpr int kXQ = 16384;      // q rows; once P is formed, T is assembled here
constexpr int kXAlpha = 32768;  // alpha, 64 fp32
constexpr int kXBeta = 33024;   // beta, 64 fp32
// fp32 16 x 16 blocks (1 KiB, row-major) and gate vectors
constexpr int kXAd = 33280;     // A_bb, b = 0..3
constexpr int kXD = 37376;      // D_b
constexpr int kXDt = 41472;     // D_b^T
constexpr int kXM10 = 45568;    // M_10^T (wave 0)
constexpr int kXM20 = 46592;    // M_20^T (wave 0)
constexpr int kXM21 = 47616;    // M_21^T (wave 1)
constexpr int kXG = 48640;      // g_t, 64 fp32
constexpr int kXB = 48896;      // beta_t, 64 fp32 (0 past the chunk's end)
constexpr int kXBytes = 49152;  // three workgroups per CU
}  // namespace

__global__ __launch_bounds__(256) void factors_kernel(PrepArgs<bf16_t> a) {
  const int c = blockIdx.x, h = blockIdx.y;
  int s, tok0, len;
  if (!a.geo.locate(c, s, tok0, len)) return;
  const int hq = h / a.group;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r0 = lane & 15, g = lane >> 4;
  __shared__ __attribute__((aligned(16))) char factors_smem[kXBytes];
  lds_t *const sm = lds_ptr(factors_smem);

  // ---- copies: wave 0 the k rows, wave 1 the q rows, wave 2 alpha and beta ----
  const uint32_t row_bytes = uint32_t(a.H_qk) * 256;
  if (wave < 2) {
    const char *src = reinterpret_cast<const char *>(wave == 0 ? a.k : a.q) +
                      (int64_t(tok0) * a.H_qk + hq) * 256;
    const i32x4_t res = buffer_rsrc(src, rowtile_valid_bytes(len, row_bytes));
    lds_t *const tile = sm + (wave == 0 ? kXK : kXQ);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      dma16_buf(res, uint32_t(rowtile_copy_src(i, lane, 64, int64_t(a.H_qk) * 128)), tile + 1024 * i);
  } else if (wave == 2) {
    const uint32_t gate_bytes = uint32_t(len - 1) * uint32_t(a.H_v) * 4 + 4;
    const int64_t first = int64_t(tok0) * a.H_v + h;
    const uint32_t voff = uint32_t(lane) * uint32_t(a.H_v) * 4;
    dma4_buf(buffer_rsrc(a.alpha + first, gate_bytes), voff, sm + kXAlpha);
    dma4_buf(buffer_rsrc(a.beta + first, gate_bytes), voff, sm + kXBeta);
  }
  wait_vmem();
  lds_barrier();

  char *const entry = a.entries + (int64_t(c) * a.H_v + h) * entry_bytes<bf16_t>();
  // chunk-local cumulative log2 gate of slot `lane` (slots past len add 0)
  const float gl =
      wave_prefix_sum(lane < len ? clamped_log2(lds_load<float>(sm + kXAlpha + 4 * lane)) : 0.0f);
  int kq_off[4][2];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) kq_off[kk][hf] = 2 * rowtile_off(r0, 32 * kk + 16 * hf + 4 * g);
  auto row_frag = [&](int tile, int rt, int kk) -> Frag<bf16_t> {
    const lds_t *p = sm + tile + 4096 * rt;
    return frag_cat(lds_load_single<bf16x4_t>(p + kq_off[kk][0]),
                    lds_load_single<bf16x4_t>(p + kq_off[kk][1]));
  };

  // T results kept in registers until the q tile is dead: this lane's column
  // of its diagonal block (x, scaled by beta of slot `lane`) and up to four
  // off-diagonal blocks in accumulator layout
  float x[16];
  f32x4_t mt[4];
  float bl = 0.0f;
  if (wave < 2) {
    // ---- T: gates and betas of all slots for broadcast reads ----
    bl = lane < len ? lds_load<float>(sm + kXBeta + 4 * lane) : 0.0f;
    lds_store<float>(sm + kXG + 4 * lane, gl);
    lds_store<float>(sm + kXB + 4 * lane, bl);
    Frag<bf16_t> kf[4][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) kf[rt][kk] = row_frag(kXK, rt, kk);
    // A_bj rows (wave 1 does not need A_b0, b > 0)
    f32x4_t At[4][4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int j = 0; j <= b; ++j) {
        if (wave == 1 && j == 0 && b > 0) continue;
        f32x4_t acc = zero4();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) acc = mfma(kf[j][kk], kf[b][kk], acc);
        const int t = 16 * b + r0;
        const float gt = lds_load<float>(sm + kXG + 4 * t), bt = lds_load<float>(sm + kXB + 4 * t);
        const f32x4_t gi = lds_load<f32x4_t>(sm + kXG + 4 * (16 * j + 4 * g));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * j + 4 * g + e;
          At[b][j][e] = i < t ? bt * fast_exp2(gt - gi[e]) * acc[e] : 0.0f;
        }
        if (j == b) lds_store<f32x4_t>(sm + kXAd + 1024 * b + 64 * r0 + 16 * g, At[b][b]);
      }
    // D_b by forward substitution: lane (b = g, column r0) solves for column
    // r0 of D_b; then D_b row-major and D_b^T (this lane's column as a row)
    {
      const lds_t *ab = sm + kXAd + 1024 * g;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        float v = t == r0 ? 1.0f : 0.0f;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          if (4 * q4 < t) {
            const f32x4_t arow = lds_load<f32x4_t>(ab + 64 * t + 16 * q4);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (4 * q4 + e < t) v -= arow[e] * x[4 * q4 + e];
          }
        }
        x[t] = v;
      }
#pragma unroll
      for (int t = 0; t < 16; ++t) lds_store<float>(sm + kXD + 1024 * g + 64 * t + 4 * r0, x[t]);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        lds_store<f32x4_t>(sm + kXDt + 1024 * g + 64 * r0 + 16 * q4,
                           f32x4_t{x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]});
    }
    auto rowv = [&](int off) { return lds_load<f32x4_t>(sm + off + 64 * r0 + 16 * g); };
    if (wave == 0) {
      // block column 0 (the longest dependency chain): M10, M20, M30
      mt[0] = -mm16(rowv(kXD + 1024 * 1), mm16(At[1][0], rowv(kXDt + 1024 * 0), zero4()), zero4());
      lds_store<f32x4_t>(sm + kXM10 + 64 * r0 + 16 * g, mt[0]);
      const f32x4_t Y20 = mm16(At[2][1], rowv(kXM10), mm16(At[2][0], rowv(kXDt + 1024 * 0), zero4()));
      mt[1] = -mm16(rowv(kXD + 1024 * 2), Y20, zero4());
      lds_store<f32x4_t>(sm + kXM20 + 64 * r0 + 16 * g, mt[1]);
      const f32x4_t Y30 =
          mm16(At[3][2], rowv(kXM20), mm16(At[3][1], rowv(kXM10), mm16(At[3][0], rowv(kXDt + 1024 * 0), zero4())));
      mt[2] = -mm16(rowv(kXD + 1024 * 3), Y30, zero4());
    } else {
      // block columns 1 to 3: M21, M31, M32
      mt[0] = -mm16(rowv(kXD + 1024 * 2), mm16(At[2][1], rowv(kXDt + 1024 * 1), zero4()), zero4());
      lds_store<f32x4_t>(sm + kXM21 + 64 * r0 + 16 * g, mt[0]);
      mt[2] = -mm16(rowv(kXD + 1024 * 3), mm16(At[3][2], rowv(kXDt + 1024 * 2), zero4()), zero4());
      const f32x4_t Y31 = mm16(At[3][2], rowv(kXM21), mm16(At[3][1], rowv(kXDt + 1024 * 1), zero4()));
      mt[1] = -mm16(rowv(kXD + 1024 * 3), Y31, zero4());
    }
  } else {
    // ---- P and the gate factors: wave 2 t-blocks 0-2, wave 3 t-block 3 ----
    // P^T tile (i-block r, t-block cb), r <= cb: its lane layout is the A
    // fragment layout of P (row t, contraction i), so its four values are half
    // of fragment (cb, r / 2).
    bf16_t *const fragP = reinterpret_cast<bf16_t *>(entry) + 8 * kFragElems;
    auto p_tile = [&](int r, int cb) {
      f32x4_t acc = zero4();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) acc = mfma(row_frag(kXK, r, kk), row_frag(kXQ, cb, kk), acc);
      const int t = 16 * cb + r0;
      const float gt = __shfl(gl, t);
      f32x4_t pv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * r + 4 * g + e;
        const float gi = __shfl(gl, i);  // every lane takes part in the shuffle
        pv[e] = i <= t ? fast_exp2(gt - gi) * acc[e] : 0.0f;
      }
      *reinterpret_cast<bf16x4_t *>(fragP + kFragElems * (2 * cb + (r >> 1)) + 8 * lane + 4 * (r & 1)) =
          __builtin_convertvector(pv, bf16x4_t);
    };
    if (wave == 2) {
#pragma unroll
      for (int cb = 0; cb < 3; ++cb)
#pragma unroll
        for (int r = 0; r <= cb; ++r) p_tile(r, cb);
      // halves above the diagonal in t-blocks 0-2
      *reinterpret_cast<uint64_t *>(fragP + kFragElems * 0 + 8 * lane + 4) = 0;
      *reinterpret_cast<u32x4_t *>(fragP + kFragElems * 1 + 8 * lane) = u32x4_t{0, 0, 0, 0};
      *reinterpret_cast<u32x4_t *>(fragP + kFragElems * 3 + 8 * lane) = u32x4_t{0, 0, 0, 0};
      *reinterpret_cast<uint64_t *>(fragP + kFragElems * 5 + 8 * lane + 4) = 0;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) p_tile(r, 3);
      // gate factors: gamma_t = 2^g_t, s_t = 2^(g_C - g_t)
      float *gate_out = reinterpret_cast<float *>(entry + 16 * kFragElems * sizeof(bf16_t));
      const float g_last = __shfl(gl, 63);
      gate_out[lane] = exp2f(gl);
      gate_out[64 + lane] = exp2f(g_last - gl);
    }
  }
  lds_barrier();  // every factor is formed: the q tile is dead
  if (wave < 2) {
    lds_t *const tf = sm + kXQ;
    // T entries of an off-diagonal block from its accumulator (rows 4 g + e,
    // column r0): T[16 b + 4 g + e][16 c + r0] = M beta_(16 c + r0), in
    // fragment (b, c / 2), lane 4 g + e + 16 (r0 / 4), element 4 (c mod 2) + r0 mod 4
    auto put_t = [&](int b, int cb, f32x4_t m) {
      const float bc = lds_load<float>(sm + kXB + 4 * (16 * cb + r0));
      const int f = 2 * b + (cb >> 1);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        lds_store<bf16_t>(tf + 1024 * f + 16 * ((4 * g + e) + 16 * (r0 >> 2)) + 2 * (4 * (cb & 1) + (r0 & 3)),
                          from_f32<bf16_t>(m[e] * bc));
    };
    // T entries of this lane's column of its diagonal block (b = g):
    // T[16 b + t][16 b + r0] = x[t] beta_(16 b + r0), fragment (b, b / 2),
    // lane t + 16 (r0 / 4), element 4 (b mod 2) + r0 mod 4
    auto put_diag = [&]() {
      const int b = g, f = 2 * b + (b >> 1);
#pragma unroll
      for (int t = 0; t < 16; ++t)
        lds_store<bf16_t>(tf + 1024 * f + 16 * (t + 16 * (r0 >> 2)) + 2 * (4 * (b & 1) + (r0 & 3)),
                          from_f32<bf16_t>(x[t] * bl));
    };
    if (wave == 0) {
      if (g == 0) put_diag();
      put_t(1, 0, mt[0]);
      put_t(2, 0, mt[1]);
      put_t(3, 0, mt[2]);
      // blocks above the diagonal: fragments (0, 1) and (1, 1) whole, the
      // upper halves of (0, 0) and (2, 1)
      lds_store<u32x4_t>(tf + 1024 * 1 + 16 * lane, u32x4_t{0, 0, 0, 0});
      lds_store<u32x4_t>(tf + 1024 * 3 + 16 * lane, u32x4_t{0, 0, 0, 0});
      lds_store<uint64_t>(tf + 1024 * 0 + 16 * lane + 8, uint64_t(0));
      lds_store<uint64_t>(tf + 1024 * 5 + 16 * lane + 8, uint64_t(0));
    } else {
      if (g > 0) put_diag();
      put_t(2, 1, mt[0]);
      put_t(3, 1, mt[1]);
      put_t(3, 2, mt[2]);
    }
  }
  lds_barrier();
  // ---- T leaves in 16-byte stores (8 KiB, 32 bytes per thread) ----
#pragma unroll
  for (int q2 = 0; q2 < 2; ++q2) {
    const int off = 16 * (tid + 256 * q2);
    *reinterpret_cast<u32x4_t *>(entry + off) = lds_load<u32x4_t>(sm + kXQ + off);
  }
}

template <typename T>
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
  if constexpr (sizeof(T) == 2) {
    if (p.d_k == 128) {
      hipLaunchKernelGGL(factors_kernel, dim3(unsigned(slots), unsigned(p.H_v)), dim3(256), 0, st, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((prep_kernel<T>), dim3(unsigned(slots), unsigned(p.H_v)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_prep(const Problem &p, const Workspace &ws, hipStream_t st) {
  if (chunk_slots(p) == 0) return hipSuccess;
  if (p.dtype == 1) return launch_prep_t<bf16_t>(p, ws, st);
  return launch_prep_t<float>(p, ws, st);
}

}  // namespace gdn
