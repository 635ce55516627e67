// Inter-chunk state scan with the chunk output fused in.
//
// Only the boundary state passes from one chunk to the next ("From KV Cache
// to a State Matrix", section "Chunkwise training for DeltaNet"; "Attention
// as Matrix Algebra", sections 5.1 and 8).  For each chunk, from the state S
// at its start, the intra-chunk factors T and P and the chunk-local gates g
// (gamma_t = 2^g_t, s_t = 2^(g_C - g_t)):
//
//   Y = K S                      (d_k contraction)
//   U = T (V - diag(gamma) Y)    pseudo-values
//   O = diag(gamma) (Q S) + P U  the chunk's outputs
//   S <- gamma_C S + K^T (diag(s) U)
//
// A wavefront owns 16 columns of the state (a d_k x 16 slice, fp32, in MFMA
// accumulator registers) for one (sequence, value head) and walks that
// sequence's chunks in order.  The delta-rule update acts on each value
// column separately ("Attention as Matrix Algebra", section 7.2: each write
// moves a column along the key only), so column slices are independent.  The
// accumulator layout of two stacked 16 x 16 tiles is the B-fragment layout,
// so Y, U and S feed the next product from registers.
//
// Blocks of one unit are numbered so that they share blockIdx mod 8: they land
// on the same XCD and share its L2 for the chunk's k, q, T and P.
#include "launch.hpp"
#include "stage.hpp"

namespace gdn {

template <typename T>
struct ScanArgs {
  const T *q, *k, *v;
  const char *entries;
  const float *h0;
  T *o;
  float *hT;
  int H_qk, H_v, d_k, d_v, group, n_units, n_colblk;
  SeqGeom geo;
};


// ---------------------------------------------------------------------------
// General path: any supported d_k / d_v, fp32 or bf16.  One 64-lane block per
// (unit, 16 columns); operands are read from global memory as needed.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(64) void scan_kernel(ScanArgs<T> a) {
  const int lane = threadIdx.x;
  int u, cb;
  decode_block(blockIdx.x, a.n_colblk, u, cb);
  if (u >= a.n_units) return;
  const int s = u / a.H_v, h = u - s * a.H_v, hq = h / a.group;
  const int col = 16 * cb + (lane & 15);  // this lane's state column
  const int nkt = a.d_k >> 4;             // 16-row tiles of the state
  const int nkb = (a.d_k + 31) >> 5;      // 32-deep contraction blocks over d_k

  // S[rt] holds state rows 16 rt + 4 (lane >> 4) + e of column col
  f32x4_t S[8];
  const int64_t st_base = (int64_t(s) * a.H_v + h) * a.d_k * a.d_v;
#pragma unroll
  for (int rt = 0; rt < 8; ++rt) {
    S[rt] = zero4();
    if (rt < nkt && a.h0)
      for (int e = 0; e < 4; ++e)
        S[rt][e] = a.h0[st_base + int64_t(16 * rt + 4 * (lane >> 4) + e) * a.d_v + col];
  }

  int start, end;
  a.geo.seq_bounds(s, start, end);
  const int n_chunks = (end - start + a.geo.chunk - 1) / a.geo.chunk;
  const int c_first = a.geo.first_chunk(s);
  const int64_t qk_stride = int64_t(a.H_qk) * a.d_k;
  const int64_t v_stride = int64_t(a.H_v) * a.d_v;

  for (int cc = 0; cc < n_chunks; ++cc) {
    const int c = c_first + cc;
    if (c >= a.geo.n_slots) break;
    const int tok0 = start + cc * a.geo.chunk;
    const int len = min(a.geo.chunk, end - tok0);
    const T *kb = a.k + int64_t(tok0) * qk_stride + int64_t(hq) * a.d_k;
    const T *qb = a.q + int64_t(tok0) * qk_stride + int64_t(hq) * a.d_k;
    const T *vb = a.v + int64_t(tok0) * v_stride + int64_t(h) * a.d_v + col;
    const T *entry = reinterpret_cast<const T *>(a.entries + (int64_t(c) * a.H_v + h) *
                                                                 entry_bytes<T>());
    const float *gent = reinterpret_cast<const float *>(entry + 16 * kFragElems);

    const float gam_l = gent[lane], sc_l = gent[64 + lane];  // this lane's slot
    const float gamma_C = __shfl(gam_l, 63);
    float gam[4][4], sc[4][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gam[rt][e] = __shfl(gam_l, 16 * rt + 4 * (lane >> 4) + e);
        sc[rt][e] = __shfl(sc_l, 16 * rt + 4 * (lane >> 4) + e);
      }

    Frag<T> Sf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) Sf[kk] = frag_from_acc<T>(S[2 * kk], S[2 * kk + 1]);

    // Y = K S, OQ = Q S
    f32x4_t Y[4], OQ[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      Y[rt] = zero4();
      OQ[rt] = zero4();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (kk < nkb) {
          const int row = 16 * rt + (lane & 15);
          Y[rt] = mfma(load_row_frag(kb, qk_stride, row, len, 32 * kk, a.d_k, lane), Sf[kk], Y[rt]);
          OQ[rt] = mfma(load_row_frag(qb, qk_stride, row, len, 32 * kk, a.d_k, lane), Sf[kk],
                        OQ[rt]);
        }
      }
    }
    // X = V - gamma Y
    f32x4_t X[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * rt + 4 * (lane >> 4) + e;
        const float vv = t < len ? to_f32(vb[int64_t(t) * v_stride]) : 0.0f;
        X[rt][e] = vv - gam[rt][e] * Y[rt][e];
      }
    // U = T X
    Frag<T> Xf[2] = {frag_from_acc<T>(X[0], X[1]), frag_from_acc<T>(X[2], X[3])};
    f32x4_t Ua[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      Ua[rt] = zero4();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        Ua[rt] = mfma(load_frag(entry + (rt * 2 + kk) * kFragElems, lane), Xf[kk], Ua[rt]);
    }
    Frag<T> Uf[2] = {frag_from_acc<T>(Ua[0], Ua[1]), frag_from_acc<T>(Ua[2], Ua[3])};
    // O = gamma (Q S) + P U
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f32x4_t acc;
      for (int e = 0; e < 4; ++e) acc[e] = gam[rt][e] * OQ[rt][e];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        acc = mfma(load_frag(entry + (8 + rt * 2 + kk) * kFragElems, lane), Uf[kk], acc);
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * rt + 4 * (lane >> 4) + e;
        if (t < len)
          a.o[int64_t(tok0 + t) * v_stride + int64_t(h) * a.d_v + col] = from_f32<T>(acc[e]);
      }
    }
    // S <- gamma_C S + K^T (s U); K^T fragments gathered from k
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
      for (int e = 0; e < 4; ++e) Ua[rt][e] *= sc[rt][e];
    Frag<T> Usf[2] = {frag_from_acc<T>(Ua[0], Ua[1]), frag_from_acc<T>(Ua[2], Ua[3])};
#pragma unroll
    for (int rm = 0; rm < 8; ++rm) {
      if (rm < nkt) {
        const int m = 16 * rm + (lane & 15);
        f32x4_t acc;
        for (int e = 0; e < 4; ++e) acc[e] = gamma_C * S[rm][e];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          Frag<T> kt;
          for (int j = 0; j < 8; ++j) {
            const int i = 32 * kk + kappa(lane, j);
            kt.set(j, i < len ? to_f32(kb[int64_t(i) * qk_stride + m]) : 0.0f);
          }
          acc = mfma(kt, Usf[kk], acc);
        }
        S[rm] = acc;
      }
    }
  }

  if (a.hT) {
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
      if (rt < nkt)
        for (int e = 0; e < 4; ++e)
          a.hT[st_base + int64_t(16 * rt + 4 * (lane >> 4) + e) * a.d_v + col] = S[rt][e];
  }
}

// ---------------------------------------------------------------------------
// Pipelined path: bf16, d_k = 128, d_v a multiple of 32.
//
// A block of four waves owns 32 state columns of one unit.  Waves 0 and 1
// compute (16 columns each); waves 2 and 3 copy and form P.  A chunk's
// operands -- its k and q rows (swizzled row tiles), the T fragments and gates
// of its workspace entry, and its 64 x 32 block of v -- are copied into one
// of three LDS stages with global_load_lds, two chunks ahead of the chunk
// being computed.  A copy moves 1 KiB and the memory pipeline accepts one
// from a wave only every few dozen cycles, so the copies are issued by the
// two copy waves, on SIMDs the compute waves leave idle, and the compute
// waves' instruction streams hold only LDS reads, MFMAs and their output
// stores.  While the compute waves run chunk c, the copy waves also form P
// of chunk c (P_ti = 2^(g_t - g_i) q_t . k_i, i <= t) from its staged q and
// k rows into one of two P buffers; the compute waves read it after the next
// barrier, for chunk c's outputs.  One barrier per chunk keeps the roles in
// step.  T and P are lower triangular: their two all-zero fragments (rows
// 0-31, columns 32-63) are neither copied nor formed nor multiplied.  K^T fragments for the state
// update and the v block come from the staged tiles through transposed reads
// (ds_read_b64_tr_b16).  Every LDS and global offset a lane uses is computed
// once; per chunk only wave-uniform bases change.  The k / q and v copies are
// bounds-checked buffer loads: rows past a partial chunk read as zeros.
// ---------------------------------------------------------------------------
constexpr int kStK = 0;        // 64 x 128 bf16 row tile
constexpr int kStQ = 16384;    // 64 x 128 bf16 row tile
constexpr int kStT = 32768;    // T fragments, 1 KiB each (1 and 3 unused)
constexpr int kStG = 40960;    // gate block: gamma, s, g (64 fp32 each), padding
constexpr int kStV = 41984;    // 64 x 32 bf16 v block
constexpr int kStBytes = 46080;
constexpr int kPBytes = 8192;  // P fragments, 1 KiB each (1 and 3 unused)
// Copies one copy wave issues per stage (wave 2: k tile, T fragments 0, 2, 4,
// gates, v columns 0-15; wave 3: q tile, T fragments 5, 6, 7, v columns
// 16-31).  A copy wave issues no other vector-memory operation, and loads
// complete in issue order, so waiting until only the newest stage's copies
// are outstanding completes every older stage.
constexpr int kStageLoadsW2 = 22;
constexpr int kStageLoadsW3 = 21;

// Three stages and two P buffers as distinct LDS objects: with the chunk loop
// unrolled by three, every stage access names its stage at compile time.
__shared__ __attribute__((aligned(16))) char scan_stage0[kStBytes];
__shared__ __attribute__((aligned(16))) char scan_stage1[kStBytes];
__shared__ __attribute__((aligned(16))) char scan_stage2[kStBytes];
__shared__ __attribute__((aligned(16))) char scan_p0[kPBytes];
__shared__ __attribute__((aligned(16))) char scan_p1[kPBytes];

// P of one chunk from its staged q and k rows and gate block, by one copy
// wave: tiles (i-block r, t-block cb), r <= cb, five per wave (wave CW = 0:
// (0,0) (0,1) (1,1) (0,2) (1,2); CW = 1: (2,2) (0,3) (1,3) (2,3) (3,3)).  The
// P^T tile K_r Q_cb^T has the A-fragment layout of P (row t, contraction i),
// so its four values per lane are half of fragment (cb, r / 2).  All operand
// reads are issued first and the five tiles' MFMAs interleave.
template <int CW>
__device__ __forceinline__ void scan_p_tiles(const lds_t *st, lds_t *pb, const int (&kq_off)[4][2], int lane) {
  constexpr int R[2][5] = {{0, 0, 1, 0, 1}, {2, 0, 1, 2, 3}};
  constexpr int CB[2][5] = {{0, 1, 1, 2, 2}, {2, 3, 3, 3, 3}};
  constexpr int KLO = CW == 0 ? 0 : 0, KHI = CW == 0 ? 2 : 4;  // k blocks used
  constexpr int QLO = CW == 0 ? 0 : 2, QHI = CW == 0 ? 3 : 4;  // q blocks used
  const int r0 = lane & 15, g = lane >> 4;
  auto frag = [&](int tile, int rt, int kk) -> Frag<bf16_t> {
    const lds_t *p = st + tile + 4096 * rt;
    return frag_cat(lds_load_single<bf16x4_t>(p + kq_off[kk][0]), lds_load_single<bf16x4_t>(p + kq_off[kk][1]));
  };
  Frag<bf16_t> kf[4][4], qf[4][4];
#pragma unroll
  for (int b = KLO; b < KHI; ++b)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) kf[b][kk] = frag(kStK, b, kk);
#pragma unroll
  for (int b = QLO; b < QHI; ++b)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[b][kk] = frag(kStQ, b, kk);
  f32x4_t acc[5];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int n = 0; n < 5; ++n) acc[n] = mfma(kf[R[CW][n]][kk], qf[CB[CW][n]][kk], kk == 0 ? zero4() : acc[n]);
#pragma unroll
  for (int n = 0; n < 5; ++n) {
    const int r = R[CW][n], cb = CB[CW][n];
    const int t = 16 * cb + r0;
    const float gt = lds_load<float>(st + kStG + 512 + 4 * t);
    const f32x4_t gi = lds_load<f32x4_t>(st + kStG + 512 + 4 * (16 * r + 4 * g));
    f32x4_t pv;
#pragma unroll
    for (int e = 0; e < 4; ++e) pv[e] = 16 * r + 4 * g + e <= t ? fast_exp2(gt - gi[e]) * acc[n][e] : 0.0f;
    lds_store<bf16x4_t>(pb + 1024 * (2 * cb + (r >> 1)) + 16 * lane + 8 * (r & 1), __builtin_convertvector(pv, bf16x4_t));
  }
}

// NG = 16-column groups per compute wave: 2 compute waves of one group, or
// one compute wave of two groups (which reads each k, q, T and P fragment
// once for both).  The copy waves follow the compute waves.
template <int NG>
__global__ __launch_bounds__(64 * (2 / NG + 2)) void scan_kernel_staged(ScanArgs<bf16_t> a) {
  constexpr int kCompute = 2 / NG;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r0 = lane & 15, g = lane >> 4;
  int u, cb;
  decode_block(blockIdx.x, a.n_colblk, u, cb);  // n_colblk = d_v / 32
  if (u >= a.n_units) return;  // the whole block
  const int s = u / a.H_v, h = u - s * a.H_v, hq = h / a.group;

  int start, end;
  a.geo.seq_bounds(s, start, end);
  const int C = a.geo.chunk;
  const int c_first = a.geo.first_chunk(s);
  const int n_chunks = max(0, min((end - start + C - 1) / C, a.geo.n_slots - c_first));
  const int64_t qk_stride = int64_t(a.H_qk) * 128;
  const int64_t v_stride = int64_t(a.H_v) * a.d_v;

  if (wave >= kCompute) {
    // ---- copy waves ----
    const int cw = wave - kCompute;  // 0: k tile, T, gates; 1: q tile, P
    const uint32_t kq_row_bytes = uint32_t(2 * qk_stride), v_row_bytes = uint32_t(2 * v_stride);
    const int64_t ebytes = entry_bytes<bf16_t>();
    const char *kq_src = reinterpret_cast<const char *>(cw == 0 ? a.k : a.q) + int64_t(hq) * 256;
    const char *v_src = reinterpret_cast<const char *>(a.v) + (int64_t(h) * a.d_v + 32 * cb) * 2;
    // Per-lane byte offsets of every copy of a full chunk (tile_index.hpp),
    // relative to the chunk's first row.  The k / q and v copies go through a
    // buffer resource whose size ends at the chunk's last row, so rows past a
    // partial chunk read as zeros (exact zeros that the chunk algebra only
    // multiplies by zero) and no copy can leave the sequence.
    uint32_t kq_voff[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) kq_voff[i] = uint32_t(rowtile_copy_src(i, lane, 64, qk_stride));
    uint32_t v_voff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) v_voff[i] = uint32_t(vblock_copy_src(2 * cw + i, lane, 64, v_stride));

    auto stage = [&](int cc, char *base_mem) {
      const int tok0 = start + cc * C;
      const int len = min(C, end - tok0);
      lds_t *const base = lds_ptr(base_mem);
      const i32x4_t kq_res = buffer_rsrc(kq_src + int64_t(tok0) * kq_row_bytes,
                                         rowtile_valid_bytes(len, kq_row_bytes));
      lds_t *const tile = base + (cw == 0 ? kStK : kStQ);
#pragma unroll
      for (int i = 0; i < 16; ++i) dma16_buf(kq_res, kq_voff[i], tile + 1024 * i);
      const char *entry = a.entries + (int64_t(c_first + cc) * a.H_v + h) * ebytes;
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const int f = cw == 0 ? 2 * i : 5 + i;  // T fragments 0, 2, 4 / 5, 6, 7
        dma16(entry + 1024 * f, 16 * lane, base + kStT + 1024 * f);
      }
      if (cw == 0) dma16(entry + 16384, 16 * lane, base + kStG);
      const i32x4_t v_res = buffer_rsrc(v_src + int64_t(tok0) * v_row_bytes,
                                        vblock_valid_bytes(len, v_row_bytes));
#pragma unroll
      for (int i = 0; i < 2; ++i) dma16_buf(v_res, v_voff[i], base + kStV + 2048 * cw + 1024 * i);
    };
    auto wait_all_but_newest_stage = [&]() {
      if (cw == 0)
        wait_vmem_upto<kStageLoadsW2>();
      else
        wait_vmem_upto<kStageLoadsW3>();
    };
    // P of the chunk in stage `stage_mem` into `p_mem`.
    int kq_off[4][2];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) kq_off[kk][hf] = 2 * rowtile_off(r0, 32 * kk + 16 * hf + 4 * g);
    auto p_tiles = [&](const char *stage_mem, char *p_mem) {
      if (cw == 0)
        scan_p_tiles<0>(lds_ptr(const_cast<char *>(stage_mem)), lds_ptr(p_mem), kq_off, lane);
      else
        scan_p_tiles<1>(lds_ptr(const_cast<char *>(stage_mem)), lds_ptr(p_mem), kq_off, lane);
    };
    // the zero halves of fragments 0 and 5 (tiles r = 1, cb = 0 and r = 3,
    // cb = 2) never change
    if (cw == 0) {
      const bf16x4_t z = {0, 0, 0, 0};
      lds_store<bf16x4_t>(lds_ptr(scan_p0) + 1024 * 0 + 16 * lane + 8, z);
      lds_store<bf16x4_t>(lds_ptr(scan_p0) + 1024 * 5 + 16 * lane + 8, z);
      lds_store<bf16x4_t>(lds_ptr(scan_p1) + 1024 * 0 + 16 * lane + 8, z);
      lds_store<bf16x4_t>(lds_ptr(scan_p1) + 1024 * 5 + 16 * lane + 8, z);
    }
    if (n_chunks > 0) {
      stage(0, scan_stage0);
      stage(min(1, n_chunks - 1), scan_stage1);
      wait_all_but_newest_stage();
    }
    lds_barrier();
    // In the phase of chunk cc (between the barriers that open chunks cc and
    // cc + 1) the stage of chunk cc - 1 is free: the compute waves read it
    // before the barrier that opened chunk cc.  Chunk cc + 2 goes there (past
    // the end the last chunk is copied again, so every phase issues the same
    // loads); P of chunk cc is formed from its stage into P buffer cc mod 2
    // (read by the compute waves in the next phase, and free again by the
    // phase after); then chunk cc + 1's stage must be complete.
    auto phase = [&](int cc, char *dst, const char *cur, char *p_mem) {
      stage(min(cc + 2, n_chunks - 1), dst);
      p_tiles(cur, p_mem);
      wait_all_but_newest_stage();
      lds_barrier();
    };
    for (int cc = 0; cc < n_chunks; cc += 6) {
      phase(cc, scan_stage2, scan_stage0, scan_p0);
      if (cc + 1 < n_chunks) phase(cc + 1, scan_stage0, scan_stage1, scan_p1);
      if (cc + 2 < n_chunks) phase(cc + 2, scan_stage1, scan_stage2, scan_p0);
      if (cc + 3 < n_chunks) phase(cc + 3, scan_stage2, scan_stage0, scan_p1);
      if (cc + 4 < n_chunks) phase(cc + 4, scan_stage0, scan_stage1, scan_p0);
      if (cc + 5 < n_chunks) phase(cc + 5, scan_stage1, scan_stage2, scan_p1);
    }
    wait_vmem();  // the trailing copies
    return;
  }

  // ---- compute waves: 16-column groups grp = NG wave + cg of the block ----
  // ---- lane-invariant LDS byte offsets (relative to a stage) ----
  // A fragments of k / q rows 16 rt + r0, columns 32 kk + 16 half + 4 g:
  // offset = 4096 rt + kq_off[kk][half].
  int kq_off[4][2];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      kq_off[kk][hf] = 2 * rowtile_off(r0, 32 * kk + 16 * hf + 4 * g);
  // transposed K^T fragments: lane a = r0 addresses token
  // 32 kk + 16 half + 4 g + a / 4, columns 16 rm + 4 (a mod 4) .. + 3:
  // offset = 8192 kk + 4096 half + kt_off[rm].
  int kt_off[8];
#pragma unroll
  for (int rm = 0; rm < 8; ++rm) kt_off[rm] = 2 * rowtile_off(4 * g + (r0 >> 2), 16 * rm + 4 * (r0 & 3));
  // transposed v tile rt of group grp (rows 16 rt + 4 g + a / 4, columns
  // 16 grp + 4 (a mod 4)): offset = 1024 rt + v_off[cg].
  int v_off[NG];
  // outputs as computed (transposed tiles): token row 16 rt + r0, columns
  // 16 grp + 4 g .. + 3 of the block, one 8-byte store per tile
  bf16_t *o_lane[NG];
  int col[NG];  // this lane's state column in each group
#pragma unroll
  for (int cg = 0; cg < NG; ++cg) {
    const int grp = NG * wave + cg;
    v_off[cg] = vtile_byte(4 * g + (r0 >> 2), 16 * grp + 4 * (r0 & 3));
    o_lane[cg] = a.o + int64_t(start + out_acc_row(0, lane)) * v_stride + int64_t(h) * a.d_v + 32 * cb +
                 out_acc_col(grp, lane);
    col[cg] = 32 * cb + 16 * grp + r0;
  }

  // ---- state ----
  f32x4_t S[NG][8];
  const int64_t st_base = (int64_t(s) * a.H_v + h) * 128 * a.d_v;
#pragma unroll
  for (int cg = 0; cg < NG; ++cg)
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) {
      S[cg][rt] = zero4();
      if (a.h0)
        for (int e = 0; e < 4; ++e)
          S[cg][rt][e] = a.h0[st_base + int64_t(16 * rt + 4 * g + e) * a.d_v + col[cg]];
    }

  // Operands of the chunk about to run, read from its stage right after the
  // barrier that completes it: gate factors (rows 16 rt + 4 g + e of this
  // lane's column, the token of this lane's transposed output tiles, the
  // chunk's last slot), k row fragments, v transposed, T fragments.  Row
  // fragments are two 8-byte reads each, kept single (not paired across
  // tiles) so that they land in the fragment's registers directly.
  float gamma_C;
  f32x4_t gam[4], sc[4];
  float gam_tok[4];
  Frag<bf16_t> kf[4][4];  // k rows: [contraction block][row tile]
  bf16x4_t vt[NG][4];     // v, transposed: four rows of this lane's column
  Frag<bf16_t> tf[8];
  auto read_operands = [&](const char *stage_mem) {
    const lds_t *st = lds_ptr(const_cast<char *>(stage_mem));
    gamma_C = lds_load<float>(st + kStG + 252);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      gam[rt] = lds_load<f32x4_t>(st + kStG + 64 * rt + 16 * g);
      sc[rt] = lds_load<f32x4_t>(st + kStG + 256 + 64 * rt + 16 * g);
      gam_tok[rt] = lds_load<float>(st + kStG + 4 * out_acc_row(rt, lane));
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const lds_t *pk = st + kStK + 4096 * rt;
        kf[kk][rt] = frag_cat(lds_load_single<bf16x4_t>(pk + kq_off[kk][0]),
                              lds_load_single<bf16x4_t>(pk + kq_off[kk][1]));
      }
#pragma unroll
    for (int cg = 0; cg < NG; ++cg)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) vt[cg][rt] = lds_read_tr16(st + kStV + 1024 * rt + v_off[cg]);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i != 1 && i != 3) tf[i].v = lds_load<bf16x8_t>(st + kStT + 1024 * i + 16 * lane);
  };

  lds_barrier();  // the first two stages are complete
  if (n_chunks > 0) read_operands(scan_stage0);

  // Chunk c's output products run inside chunk c + 1's state chain, where the
  // MFMA pipe would otherwise wait on the chain's VALU work: they need the
  // chunk-start state and U of chunk c (o_Sf, o_Uf), its q rows (read during
  // chunk c) and its P (read after the barrier that follows chunk c).  The
  // outputs leave at the end of the next chain, when the copy waves' burst
  // of copies after the barrier has drained from the memory pipeline.
  Frag<bf16_t> o_Sf[NG][4], o_Uf[NG][2], o_qf[4][4], o_pf[8];
  float o_gt[4];
  bf16x4_t o_pend[NG][4];
#pragma unroll
  for (int i = 0; i < 8; ++i) o_pf[i].zero();
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) o_qf[kk][rt].zero();
#pragma unroll
  for (int cg = 0; cg < NG; ++cg) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) o_Sf[cg][kk].zero();
    o_Uf[cg][0].zero();
    o_Uf[cg][1].zero();
  }
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) o_gt[rt] = 0.0f;

  // O = gamma (Q S) + P U with the chunk-start state, computed as
  // O^T = S^T (gamma Q^T) + U^T P^T: with the kappa fragment convention Sf
  // and Uf serve as A operands and the q rows and P fragments as B operands
  // unchanged, and each lane ends with four consecutive columns of one token
  // row, one 8-byte piece of the output.  (T and P rows 0-31 end at column 31.)
  f32x4_t oq[NG][4];
  auto out_qs = [&]() {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int cg = 0; cg < NG; ++cg)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) oq[cg][rt] = mfma(o_Sf[cg][kk], o_qf[kk][rt], kk == 0 ? zero4() : oq[cg][rt]);
  };
  auto out_pu = [&]() {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int cg = 0; cg < NG; ++cg) {
        f32x4_t acc = o_gt[rt] * oq[cg][rt];
#pragma unroll
        for (int kk = 0; kk < (rt < 2 ? 1 : 2); ++kk) acc = mfma(o_Uf[cg][kk], o_pf[rt * 2 + kk], acc);
        o_pend[cg][rt] = __builtin_convertvector(acc, bf16x4_t);
      }
  };
  auto store_out = [&](int oc) {
    const int len = min(C, end - (start + oc * C));
#pragma unroll
    for (int cg = 0; cg < NG; ++cg) {
      bf16_t *const o_chunk = o_lane[cg] + int64_t(oc) * C * v_stride;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
        if (out_acc_row(rt, lane) < len)
          *reinterpret_cast<bf16x4_t *>(o_chunk + int64_t(16 * rt) * v_stride) = o_pend[cg][rt];
    }
  };

  // One chunk, software-pipelined: the state chain runs from the operands
  // read after the previous barrier, with the previous chunk's output
  // products interleaved; the q rows and K^T are read from the stage during
  // the chain.  The barrier follows the state update (after it the copy
  // waves may reuse the previous chunk's stage); then the next chunk's
  // operands and this chunk's P are read.  With two groups each operand
  // fragment serves both.
  auto chunk_step = [&](int cc, char *cur_mem, char *next_mem, const char *p_mem) {
    const lds_t *const st = lds_ptr(cur_mem);

    Frag<bf16_t> Sf[NG][4];
#pragma unroll
    for (int cg = 0; cg < NG; ++cg)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) Sf[cg][kk] = frag_from_acc<bf16_t>(S[cg][2 * kk], S[cg][2 * kk + 1]);

    // Y = K S
    f32x4_t Y[NG][4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int cg = 0; cg < NG; ++cg)
          Y[cg][rt] = mfma(kf[kk][rt], Sf[cg][kk], kk == 0 ? zero4() : Y[cg][rt]);
    out_qs();  // previous chunk: S^T (Q^T)

    // K^T fragments for the state update (transposed reads of the k tile),
    // issued early so that they have landed when the update starts
    Frag<bf16_t> ktf[8][2];
#pragma unroll
    for (int rm = 0; rm < 8; ++rm)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const lds_t *p = st + kStK + 8192 * kk + kt_off[rm];
        ktf[rm][kk] = frag_cat(lds_read_tr16(p), lds_read_tr16(p + 4096));
      }

    // X = V - gamma Y, then U = T X
    Frag<bf16_t> Xf[NG][2];
#pragma unroll
    for (int cg = 0; cg < NG; ++cg) {
      f32x4_t X[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) X[rt] = __builtin_convertvector(vt[cg][rt], f32x4_t) - gam[rt] * Y[cg][rt];
      Xf[cg][0] = frag_from_acc<bf16_t>(X[0], X[1]);
      Xf[cg][1] = frag_from_acc<bf16_t>(X[2], X[3]);
    }
    f32x4_t Ua[NG][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int kk = 0; kk < (rt < 2 ? 1 : 2); ++kk)  // T rows 0-31 end at column 31
#pragma unroll
        for (int cg = 0; cg < NG; ++cg)
          Ua[cg][rt] = mfma(tf[rt * 2 + kk], Xf[cg][kk], kk == 0 ? zero4() : Ua[cg][rt]);
    out_pu();  // previous chunk: + U^T P^T

    // this chunk's q rows, for its output products in the next chunk
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const lds_t *pq = st + kStQ + 4096 * rt;
        o_qf[kk][rt] = frag_cat(lds_load_single<bf16x4_t>(pq + kq_off[kk][0]),
                                lds_load_single<bf16x4_t>(pq + kq_off[kk][1]));
      }

    Frag<bf16_t> Usf[NG][2];
#pragma unroll
    for (int cg = 0; cg < NG; ++cg) {
      o_Uf[cg][0] = frag_from_acc<bf16_t>(Ua[cg][0], Ua[cg][1]);
      o_Uf[cg][1] = frag_from_acc<bf16_t>(Ua[cg][2], Ua[cg][3]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) Ua[cg][rt] *= sc[rt];
      Usf[cg][0] = frag_from_acc<bf16_t>(Ua[cg][0], Ua[cg][1]);
      Usf[cg][1] = frag_from_acc<bf16_t>(Ua[cg][2], Ua[cg][3]);
    }

    // S <- gamma_C S + K^T (s U)
#pragma unroll
    for (int rm = 0; rm < 8; ++rm)
#pragma unroll
      for (int cg = 0; cg < NG; ++cg) {
        f32x4_t acc = gamma_C * S[cg][rm];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) acc = mfma(ktf[rm][kk], Usf[cg][kk], acc);
        S[cg][rm] = acc;
      }
    if (cc > 0) store_out(cc - 1);
#pragma unroll
    for (int cg = 0; cg < NG; ++cg)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) o_Sf[cg][kk] = Sf[cg][kk];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) o_gt[rt] = gam_tok[rt];

    // this chunk's stage reads are done (the copy waves may now refill the
    // previous chunk's stage) and the next chunk's stage is complete
    lds_barrier();
    if (cc + 1 < n_chunks) read_operands(next_mem);
    {  // P of this chunk, formed by the copy waves
      const lds_t *pb = lds_ptr(const_cast<char *>(p_mem));
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i != 1 && i != 3) o_pf[i].v = lds_load<bf16x8_t>(pb + 1024 * i + 16 * lane);
    }
  };
  for (int cc = 0; cc < n_chunks; cc += 6) {
    chunk_step(cc, scan_stage0, scan_stage1, scan_p0);
    if (cc + 1 < n_chunks) chunk_step(cc + 1, scan_stage1, scan_stage2, scan_p1);
    if (cc + 2 < n_chunks) chunk_step(cc + 2, scan_stage2, scan_stage0, scan_p0);
    if (cc + 3 < n_chunks) chunk_step(cc + 3, scan_stage0, scan_stage1, scan_p1);
    if (cc + 4 < n_chunks) chunk_step(cc + 4, scan_stage1, scan_stage2, scan_p0);
    if (cc + 5 < n_chunks) chunk_step(cc + 5, scan_stage2, scan_stage0, scan_p1);
  }
  if (n_chunks > 0) {  // the last chunk's outputs
    out_qs();
    out_pu();
    store_out(n_chunks - 1);
  }

  if (a.hT) {
#pragma unroll
    for (int cg = 0; cg < NG; ++cg)
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
        for (int e = 0; e < 4; ++e)
          a.hT[st_base + int64_t(16 * rt + 4 * g + e) * a.d_v + col[cg]] = S[cg][rt][e];
  }
}

#ifndef SCAN_GROUPS
#define SCAN_GROUPS 1
#endif

template <typename T>
static ScanArgs<T> scan_args(const Problem &p, const Workspace &ws, int colblk_width) {
  ScanArgs<T> a;
  a.q = static_cast<const T *>(p.q);
  a.k = static_cast<const T *>(p.k);
  a.v = static_cast<const T *>(p.v);
  a.entries = static_cast<const char *>(ws.entries);
  a.h0 = p.h0;
  a.o = static_cast<T *>(p.o);
  a.hT = p.hT;
  a.H_qk = p.H_qk;
  a.H_v = p.H_v;
  a.d_k = p.d_k;
  a.d_v = p.d_v;
  a.group = p.H_v / p.H_qk;
  a.n_units = p.n_seqs * p.H_v;
  a.n_colblk = p.d_v / colblk_width;
  a.geo = make_geom(p, &ws);
  return a;
}

hipError_t launch_scan(const Problem &p, const Workspace &ws, hipStream_t st) {
  const bool staged = staged_path(p);
  const int width = staged ? 32 : 16;
  const int64_t blocks = (int64_t(p.n_seqs) * p.H_v + 7) / 8 * 8 * (p.d_v / width);
  if (blocks == 0) return hipSuccess;
  if (staged) {
    hipLaunchKernelGGL(scan_kernel_staged<SCAN_GROUPS>, dim3(unsigned(blocks)), dim3(64 * (2 / SCAN_GROUPS + 2)), 0, st,
                       scan_args<bf16_t>(p, ws, width));
  } else if (p.dtype == 1) {
    hipLaunchKernelGGL(scan_kernel<bf16_t>, dim3(unsigned(blocks)), dim3(64), 0, st,
                       scan_args<bf16_t>(p, ws, width));
  } else {
    hipLaunchKernelGGL(scan_kernel<float>, dim3(unsigned(blocks)), dim3(64), 0, st,
                       scan_args<float>(p, ws, width));
  }
  return hipGetLastError();
}

}  // namespace gdn
