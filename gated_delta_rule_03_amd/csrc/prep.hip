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
// The factor kernel below computes, for the staged path (bf16 inputs,
// d_k = 128, d_v a multiple of 32), what does not depend on the incoming
// state -- T and the gate factors gamma_t = 2^g_t and s_t = 2^(g_C - g_t) for
// one (chunk, value head) -- and writes them to the workspace entry (T in MFMA
// fragment order, then the gate block); the staged scan forms P itself.  Every
// other shape runs the chained form (bwd.hip), whose factor kernel writes M
// and P in fp32.
//
// Padding: a chunk is padded to 64 token slots.  Padded slots carry beta = 0
// and the last token's gate; their k rows (zero) only ever meet exact zeros:
// their rows and columns of A and T vanish with beta.
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

// ---------------------------------------------------------------------------
// Staged path (bf16, d_k = 128, d_v % 32 = 0): the factor kernel.  One
// workgroup of two waves per (chunk slot, value head); its k rows and gates
// are copied into LDS with bounds-checked buffer loads (rows past the chunk's
// end read as zeros, padded slots get beta = 0 and add nothing to the gate).
// It writes T and the gate block into a 6 KiB entry (launch.hpp); the staged
// scan forms P from the q and k rows it stages anyway.
//
// M = (I + A)^-1 in 16 x 16 blocks.  Wave 1 forms the diagonal blocks A_bb
// and solves D_b = (I + A_bb)^-1 for all four b at once (lane 16 b + c owns
// column c of D_b) by right-looking substitution: once x_j is final it is
// subtracted from every later row, so the dependent chain is one FMA per step.
// Wave 0 forms the six off-diagonal A_bj.  The off-diagonal blocks of M then
// follow in two levels from 2 x 2 block inversion of the two 32 x 32 halves:
//   M10 = -D1 A10 D0,  M32 = -D3 A32 D2,
//   X20 = A20 D0 + A21 M10,  X21 = A21 D1,  X30 = A30 D0 + A31 M10,  X31 = A31 D1,
//   M20 = -D2 X20,  M21 = -D2 X21,  M30 = -(D3 X30 + M32 X20),  M31 = -(D3 X31 + M32 X21)
// (wave 0: M10, M20, M30; wave 1: M21, M31, M32), on fp32 MFMA.  A product
// is formed in either orientation: with X in row layout (lane (r, g) holds
// X[r][4g..4g+3]) and Y in column layout (lane (c, g) holds Y[4g..4g+3][c]),
// one MFMA sequence gives XY in column layout and the same operands swapped
// give XY in row layout -- the layout of a T fragment, so each block of T
// leaves in one 8-byte store (two blocks side by side in one 16-byte store).
// A stays in registers: the tile K_j K_b^T holds row 16 b + c of A_bj in lane
// (c, g) (columns 16 j + 4 g .. + 3), i.e. A_bj in row layout; a diagonal tile
// is symmetric, so the same tile read as A_bb in column layout stores the
// transposed block the substitution reads.  Every factor goes straight from
// registers to the workspace entry.
//
// LDS: fp32 16 x 16 blocks use 80-byte rows, and the block strides are chosen
// so that the broadcast row reads of the substitution (one address per block)
// and its column stores fall in distinct banks.
// ---------------------------------------------------------------------------
namespace {
constexpr int kXK = 0;          // k rows, 64 x 128 bf16 row tile (dead once in registers)
constexpr int kXAlpha = 16384;  // alpha, 64 fp32
constexpr int kXBeta = 16640;   // beta, 64 fp32
constexpr int kXG = 16896;      // g_t, 64 fp32
constexpr int kXB = 17152;      // beta_t, 64 fp32 (0 past the chunk's end)
constexpr int kXRow = 80;       // row stride of an fp32 16 x 16 block
// The inverse's blocks reuse the k tile's bytes (both waves hold their k
// fragments in registers before either writes them).
constexpr int kXAdT = 0;        // A_bb^T (row j = column j of A_bb)
constexpr int kXAdTBlk = 1296;  // 324 dwords: 4 mod 32
constexpr int kXD = kXAdT + 4 * kXAdTBlk;  // D_b, row-major
constexpr int kXDBlk = 1344;               // 336 dwords: 16 mod 32
constexpr int kXDt = kXD + 4 * kXDBlk;     // D_b^T
constexpr int kXDtBlk = 1296;
static_assert(kXDt + 4 * kXDtBlk <= kXAlpha, "the inverse's blocks fit in the k tile");
constexpr int kXBytes = 17408;
}  // namespace

__global__ __launch_bounds__(128, 4) void factors_kernel(PrepArgs<bf16_t> a) {
  // Block b runs on XCD b % 8.  XCD x takes chunks x, x + 8, x + 16, ..., and
  // each chunk's heads one after another: heads vary fastest in time (the
  // blocks in flight read whole tokens' k rows, contiguous in memory), and a
  // chunk's alpha and beta lines are fetched into one XCD's L2 only.
  const unsigned j = blockIdx.x >> 3;
  const int c = int(8u * (j / unsigned(a.H_v)) + (blockIdx.x & 7u)), h = int(j % unsigned(a.H_v));
  int s, tok0, len;
  if (!a.geo.locate(c, s, tok0, len)) return;
  const int hq = h / a.group;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r0 = lane & 15, g = lane >> 4;
  __shared__ __attribute__((aligned(16))) char factors_smem[kXBytes];
  lds_t *const sm = lds_ptr(factors_smem);

  // ---- copies: wave 0 the k rows, wave 1 alpha and beta ----
  const uint32_t row_bytes = uint32_t(a.H_qk) * 256;
  if (wave == 0) {
    const char *src = reinterpret_cast<const char *>(a.k) + (int64_t(tok0) * a.H_qk + hq) * 256;
    const i32x4_t res = buffer_rsrc(src, rowtile_valid_bytes(len, row_bytes));
#pragma unroll
    for (int i = 0; i < 16; ++i)
      dma16_buf(res, uint32_t(rowtile_copy_src(i, lane, 64, int64_t(a.H_qk) * 128)), sm + kXK + 1024 * i);
  } else {
    const uint32_t gate_bytes = uint32_t(len - 1) * uint32_t(a.H_v) * 4 + 4;
    const int64_t first = int64_t(tok0) * a.H_v + h;
    const uint32_t voff = uint32_t(lane) * uint32_t(a.H_v) * 4;
    dma4_buf(buffer_rsrc(a.alpha + first, gate_bytes), voff, sm + kXAlpha);
    dma4_buf(buffer_rsrc(a.beta + first, gate_bytes), voff, sm + kXBeta);
  }
  wait_vmem();
  lds_barrier();

  char *const entry = a.entries + (int64_t(c) * a.H_v + h) * kStagedEntryBytes;
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

  // fp32 16 x 16 block operands from LDS: row layout of a row-major block
  // (lane (r, g) reads row r, columns 4 g .. + 3)
  auto rowv = [&](int off) { return lds_load<f32x4_t>(sm + off + kXRow * r0 + 16 * g); };
  // T block (b, cb) in row layout leaves as one half of fragment (b, cb / 2),
  // scaled by beta of its columns 16 cb + 4 g .. + 3
  bf16_t *const fragT = reinterpret_cast<bf16_t *>(entry);
  auto t_half = [&](int cb, f32x4_t m) -> bf16x4_t {
    const f32x4_t bc = lds_load<f32x4_t>(sm + kXB + 4 * (16 * cb + 4 * g));
    return __builtin_convertvector(m * bc, bf16x4_t);
  };
  // (fragments 0 and 5 keep elements 0-3 only: their upper halves are zero)
  auto put_frag = [&](int f, bf16x4_t lo, bf16x4_t hi) {
    if (t_compact(f))
      *reinterpret_cast<bf16x4_t *>(fragT + t_entry_byte(f) / 2 + 4 * lane) = lo;
    else
      *reinterpret_cast<bf16x8_t *>(fragT + t_entry_byte(f) / 2 + 8 * lane) = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto put_half = [&](int f, int hf, bf16x4_t v) {
    *reinterpret_cast<bf16x4_t *>(fragT + t_entry_byte(f) / 2 + 8 * lane + 4 * hf) = v;
  };
  const bf16x4_t zero_h = {0, 0, 0, 0};  // the zero half of fragments 0 and 5 (not stored)

  {
    // gates and betas of all slots for broadcast reads (both waves write the
    // same values and read only after their own writes)
    const float bl = lane < len ? lds_load<float>(sm + kXBeta + 4 * lane) : 0.0f;
    lds_store<float>(sm + kXG + 4 * lane, gl);
    lds_store<float>(sm + kXB + 4 * lane, bl);
    // k row fragments of the four 16-row blocks, read once; then the k tile's
    // bytes are free for the inverse's blocks
    Frag<bf16_t> kfr[4][4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) kfr[b][kk] = row_frag(kXK, b, kk);
    lds_barrier();
    // gated tile: (K_j K_b^T)[4 g + e][c] read as row 16 b + c of A_bj, or, for
    // j == b, as row 16 b + 4 g + e, column 16 b + c of A_bb (column layout)
    auto k_tile = [&](int j, int b) {
      f32x4_t acc = zero4();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) acc = mfma(kfr[j][kk], kfr[b][kk], acc);
      return acc;
    };
    if (wave == 0) {
      // ---- off-diagonal A_bj (j < b) in row layout: row t = 16 b + r0 ----
      f32x4_t At[4][3];
#pragma unroll
      for (int b = 1; b < 4; ++b)
#pragma unroll
        for (int j = 0; j < b; ++j) {
          const f32x4_t acc = k_tile(j, b);
          const int t = 16 * b + r0;
          const float gt = lds_load<float>(sm + kXG + 4 * t), bt = lds_load<float>(sm + kXB + 4 * t);
          const f32x4_t gi = lds_load<f32x4_t>(sm + kXG + 4 * (16 * j + 4 * g));
#pragma unroll
          for (int e = 0; e < 4; ++e) At[b][j][e] = bt * fast_exp2(gt - gi[e]) * acc[e];
        }
      Split16 As[4][3];
#pragma unroll
      for (int b = 1; b < 4; ++b)
#pragma unroll
        for (int j = 0; j < b; ++j) As[b][j] = split16(At[b][j]);
      lds_barrier();  // D_b and D_b^T are in LDS
      f32x4_t D[4];  // D_b, row layout
      Split16 Drs[4], Dcs[3];
#pragma unroll
      for (int b = 0; b < 4; ++b) D[b] = rowv(kXD + kXDBlk * b);
#pragma unroll
      for (int b = 0; b < 3; ++b) Dcs[b] = split16(rowv(kXDt + kXDtBlk * b));  // column layout
#pragma unroll
      for (int b = 1; b < 4; ++b) Drs[b] = split16(D[b]);
      const Split16 Y10c = split16(mm16x3(As[1][0], Dcs[0], zero4()));
      const Split16 M10c = split16(-mm16x3(Drs[1], Y10c, zero4()));
      const f32x4_t M10r = -mm16x3(Y10c, Drs[1], zero4());
      const Split16 M32r = split16(-mm16x3(split16(mm16x3(As[3][2], Dcs[2], zero4())), Drs[3], zero4()));
      const Split16 X20c = split16(mm16x3(As[2][1], M10c, mm16x3(As[2][0], Dcs[0], zero4())));
      const Split16 X30c = split16(mm16x3(As[3][1], M10c, mm16x3(As[3][0], Dcs[0], zero4())));
      const f32x4_t M20r = -mm16x3(X20c, Drs[2], zero4());
      const f32x4_t M30r = -mm16x3(X20c, M32r, mm16x3(X30c, Drs[3], zero4()));
      auto Dr = [&](int b) { return D[b]; };
      // fragments (0, 0) = [D0 | 0], (1, 0) = [M10 | D1] and the left halves of
      // (2, 0) and (3, 0); (0, 1) and (1, 1) are zero and not stored
      put_frag(0, t_half(0, Dr(0)), zero_h);
      put_frag(2, t_half(0, M10r), t_half(1, Dr(1)));
      put_half(4, 0, t_half(0, M20r));
      put_half(6, 0, t_half(0, M30r));
    } else {
      // gate block: gamma_t = 2^g_t, s_t = 2^(g_C - g_t), g_t
      float *gate_out = reinterpret_cast<float *>(entry + kStagedGateOffset);
      const float g_last = __shfl(gl, 63);
      gate_out[lane] = exp2f(gl);
      gate_out[64 + lane] = exp2f(g_last - gl);
      gate_out[128 + lane] = gl;
      // ---- diagonal blocks, stored transposed: A_bb^T[c][4 g + e] ----
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const f32x4_t acc = k_tile(b, b);
        const int i = 16 * b + r0;  // column of A (the tile's c)
        const float gi = lds_load<float>(sm + kXG + 4 * i);
        const f32x4_t gt = lds_load<f32x4_t>(sm + kXG + 4 * (16 * b + 4 * g));
        const f32x4_t bt = lds_load<f32x4_t>(sm + kXB + 4 * (16 * b + 4 * g));
        f32x4_t v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = 4 * g + e > r0 ? bt[e] * fast_exp2(gt[e] - gi) * acc[e] : 0.0f;
        lds_store<f32x4_t>(sm + kXAdT + kXAdTBlk * b + kXRow * r0 + 16 * g, v);
      }
      // ---- D_b = (I + A_bb)^-1: lane (b = g, column r0), right-looking ----
      {
        const lds_t *ab = sm + kXAdT + kXAdTBlk * g;
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) x[t] = t == r0 ? 1.0f : 0.0f;
        // column j of A_bb (rows t > j) is row j of A_bb^T; rows are read
        // two steps ahead of their use
        f32x4_t col[3][4];
        auto read_col = [&](int j, f32x4_t *dst) {
#pragma unroll
          for (int q4 = (j + 1) / 4; q4 < 4; ++q4) dst[q4] = lds_load<f32x4_t>(ab + kXRow * j + 16 * q4);
        };
        read_col(0, col[0]);
        read_col(1, col[1]);
#pragma unroll
        for (int j = 0; j < 15; ++j) {
          if (j + 2 < 15) read_col(j + 2, col[(j + 2) % 3]);
#pragma unroll
          for (int q4 = (j + 1) / 4; q4 < 4; ++q4)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (4 * q4 + e > j) x[4 * q4 + e] -= col[j % 3][q4][e] * x[j];
        }
        // D_b row-major (this lane's column) and D_b^T (this lane's column as a row)
#pragma unroll
        for (int t = 0; t < 16; ++t) lds_store<float>(sm + kXD + kXDBlk * g + kXRow * t + 4 * r0, x[t]);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          lds_store<f32x4_t>(sm + kXDt + kXDtBlk * g + kXRow * r0 + 16 * q4,
                             f32x4_t{x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]});
      }
      // ---- A21, A31, A32 in row layout ----
      f32x4_t At[4][3];
#pragma unroll
      for (int b = 2; b < 4; ++b)
#pragma unroll
        for (int j = 1; j < b; ++j) {
          const f32x4_t acc = k_tile(j, b);
          const int t = 16 * b + r0;
          const float gt = lds_load<float>(sm + kXG + 4 * t), bt = lds_load<float>(sm + kXB + 4 * t);
          const f32x4_t gi = lds_load<f32x4_t>(sm + kXG + 4 * (16 * j + 4 * g));
#pragma unroll
          for (int e = 0; e < 4; ++e) At[b][j][e] = bt * fast_exp2(gt - gi[e]) * acc[e];
        }
      const Split16 A21 = split16(At[2][1]), A31 = split16(At[3][1]), A32 = split16(At[3][2]);
      lds_barrier();  // D_b and D_b^T are in LDS
      f32x4_t D[4];  // D_b, row layout (b >= 1)
      Split16 Drs[4], Dcs[3];
#pragma unroll
      for (int b = 1; b < 4; ++b) D[b] = rowv(kXD + kXDBlk * b);
#pragma unroll
      for (int b = 1; b < 3; ++b) Dcs[b] = split16(rowv(kXDt + kXDtBlk * b));  // column layout
#pragma unroll
      for (int b = 2; b < 4; ++b) Drs[b] = split16(D[b]);
      const f32x4_t M32 = -mm16x3(split16(mm16x3(A32, Dcs[2], zero4())), Drs[3], zero4());
      const Split16 M32r = split16(M32);
      const Split16 X21c = split16(mm16x3(A21, Dcs[1], zero4()));
      const f32x4_t M21r = -mm16x3(X21c, Drs[2], zero4());
      const Split16 X31c = split16(mm16x3(A31, Dcs[1], zero4()));
      const f32x4_t M31r = -mm16x3(X21c, M32r, mm16x3(X31c, Drs[3], zero4()));
      auto Dr = [&](int b) { return D[b]; };
      // the right halves of (2, 0) and (3, 0); (2, 1) = [D2 | 0], (3, 1) = [M32 | D3]
      put_half(4, 1, t_half(1, M21r));
      put_half(6, 1, t_half(1, M31r));
      put_frag(5, t_half(2, Dr(2)), zero_h);
      put_frag(7, t_half(2, M32), t_half(3, Dr(3)));
    }
  }
}

// The staged path's factor kernel; other shapes run the chained form.
hipError_t launch_prep(const Problem &p, const Workspace &ws, hipStream_t st) {
  if (chunk_slots(p) == 0) return hipSuccess;
  if (!staged_path(p)) return hipErrorInvalidValue;
  using T = bf16_t;
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
  const int64_t blocks = 8 * ((slots + 7) / 8) * p.H_v;  // chunk slots rounded up to the XCD count
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(factors_kernel, dim3(unsigned(blocks)), dim3(128), 0, st, a);
  return hipGetLastError();
}



}  // namespace gdn
