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
// This scan serves the staged path (bf16 inputs, d_k = 128, d_v a multiple
// of 32); every other shape runs the chained form (bwd.hip).  A chain
// wavefront owns 16 columns of the state (a d_k x 16 slice, fp32, in MFMA
// accumulator registers) for one (sequence, value head) and walks that
// sequence's chunks in order.  The delta-rule update acts on each value
// column separately ("Attention as Matrix Algebra", section 7.2: each write
// moves a column along the key only), so column slices are independent.  The
// accumulator layout of two stacked 16 x 16 tiles is the B-fragment layout,
// so Y, U and S feed the next product from registers.
//
// Blocks of one unit are numbered so that they share blockIdx mod 8: they land
// on the same XCD and share its L2 for the chunk's k, q, T and P.
//
// Transition mode (mode 1) serves the segment-parallel path: a sequence is cut
// into segments that are scanned as independent units, and each segment's
// effect on the state is the affine map S_out = M S_in + B.  The delta rule is
// linear in (S, v) ("From KV Cache to a State Matrix", section "Chunkwise
// training for DeltaNet": the chunk updates compose), so B is the segment's
// final state from S_in = 0, and M (d_k x d_k) is the final state of the same
// scan over d_k extra columns started from the identity with v = 0.  Mode 1
// computes both, as d_v + d_k state columns, and writes no outputs.
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
  // transition mode: column blocks cb >= n_colblk_v carry M; the result goes
  // to mb [n_seqs, H_v, d_k, d_v + d_k] (B in columns 0 .. d_v - 1, M after)
  int mode, n_colblk_v;
  float *mb;
};

// Initial state of column `col` of a block: h0 (mode 0), zero (mode 1, the
// columns of B) or the identity (mode 1, the columns of M).
__device__ __forceinline__ float initial_state(const float *h0, int64_t st_base, int row, int col,
                                               int d_v, int mode, bool is_m) {
  if (mode == 1) return is_m && row == col ? 1.0f : 0.0f;
  return h0 ? h0[st_base + int64_t(row) * d_v + col] : 0.0f;
}


// ---------------------------------------------------------------------------
// Pipelined path: bf16, d_k = 128, d_v a multiple of 32.
//
// A block of NCH + 6 waves owns 16 NCH state columns of one unit.  Waves
// 0 .. NCH - 1 run the state chain (16 columns each); waves NCH and NCH + 1
// form P and compute the outputs; waves NCH + 2 .. NCH + 5 copy operands.
// A chunk's operands -- its k and q rows (swizzled row tiles), the T
// fragments and gates of its workspace entry, and its 64 x 16 NCH block of v
// -- are copied into one of three LDS stages with buffer/global loads
// straight to LDS, two chunks ahead of the chunk being computed.  The copy
// waves issue every copy: each half of the k or q tile, and copy wave 0 T
// fragments 0, 2, 4, the gate block and half the v block, copy wave 1 T
// fragments 5, 6, 7 and the other half (v with the nontemporal hint: it is
// read once, and its lines should leave the L2 before the k and q lines that
// the unit's other column blocks still read).  A copy moves 1 KiB and
// one wave gets one accepted only every few dozen cycles, so four waves
// issue them; they share SIMDs with the other waves but issue no
// arithmetic, so no wave that computes waits to issue a copy.
//
// The chain waves run the state chain only (Y = K S, U = T (V - gamma Y), the
// state update) and issue no memory instruction.  Each chain wave leaves the
// chunk-start state (as the bf16 fragments it multiplies anyway) and U in one
// of two exchange buffers.  In the next phase each output wave computes the
// outputs of two of the chunk's four 16-token row blocks for every column
// group, O^T = S^T (gamma Q^T) + U^T P^T, from that exchange, the q rows and
// the rows of P it formed itself in the previous phase (kept in registers),
// and stores them.
//
// One barrier per chunk keeps the roles in step.  T and P are lower
// triangular: their all-zero fragments (rows 0-31, columns 32-63) are neither
// copied nor formed nor multiplied.  K^T fragments for the state update and
// the v block come from the staged tiles through transposed reads
// (ds_read_b64_tr_b16).  Every LDS and global offset a lane uses is computed
// once; per chunk only wave-uniform bases change.  The k / q and v copies are
// bounds-checked buffer loads: rows past a partial chunk read as zeros.
// ---------------------------------------------------------------------------
constexpr int kStK = 0;        // 64 x 128 bf16 row tile
constexpr int kStQ = 16384;    // 64 x 128 bf16 row tile
constexpr int kStT = 32768;    // T's six non-zero fragments, a 1 KiB slot each (t_slot, tile_index.hpp)
constexpr int kStG = 38912;    // gate block: gamma, s, g (64 fp32 each), padding
constexpr int kStV = 39936;    // 64 x 16 NCH bf16 v block (4 KiB)
constexpr int kStBytes = 44032;

// Exchange buffer: per chain wave w, at 6144 w, the chunk-start state as four
// bf16 A fragments of S^T (fragment kk: state rows 32 kk + kappa) and then U
// as two fragments (tokens 32 kk + kappa), 1 KiB each in fragment order.
constexpr int kExS = 0, kExU = 4096, kExWave = 6144;
constexpr int kExBytes = 2 * kExWave;
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
// k (or q) tile copies per stage and copy wave.  A copy wave issues nothing
// but copies, and loads complete in issue order, so waiting until at most
// one stage's copies are outstanding completes every earlier stage.
constexpr int kStageLoadsCopy = 8;

// Three stages and two exchange buffers as distinct LDS objects: with the
// chunk loop unrolled by six, every access names its buffer at compile time.
__shared__ __attribute__((aligned(16))) char scan_stage0[kStBytes];
__shared__ __attribute__((aligned(16))) char scan_stage1[kStBytes];
__shared__ __attribute__((aligned(16))) char scan_stage2[kStBytes];
__shared__ __attribute__((aligned(16))) char scan_ex0[kExBytes];
__shared__ __attribute__((aligned(16))) char scan_ex1[kExBytes];
// A chunk's outputs on their way out (64 token rows x 32 bf16, out_stage_byte
// in tile_index.hpp): each output wave writes and reads back only its own
// rows, so that every store covers whole rows of the block.
__shared__ __attribute__((aligned(16))) char scan_ostage[4096];
// s_sleep units (64 cycles each) the copy waves wait after a barrier, so that
// the output waves' stores enter the memory pipeline ahead of the copies.
#ifndef SCAN_COPY_DELAY
#define SCAN_COPY_DELAY 2
#endif

// Token row blocks of P and of the outputs that output wave CW owns:
// copy_rows(CW, 0..1) (tile_index.hpp), five 16 x 16 tiles of P each.
template <int CW> __device__ constexpr int own_rt(int a) { return copy_rows(CW, a); }

// What an output wave keeps from one phase to the next for a chunk's outputs.
struct OutOperands {
  Frag<bf16_t> q[2][4];  // q rows of its two row blocks, [block][contraction block]
  Frag<bf16_t> p[2][2];  // P fragments of those rows (row t, contraction i)
  float gam[2];          // gamma_t of this lane's token (16 rt + lane mod 16) in each block
};

// Output wave CW's rows of P = Gamma . (Q K^T) (i <= t) for the chunk staged at
// `st`.  The tile K_r Q_rt^T leaves, in accumulator layout, the values
// P[16 rt + lane mod 16][16 r + 4 (lane / 16) + e] -- half of the P fragment
// (rt, r / 2) -- so P stays in registers.  `between` runs after the operand
// reads are issued.
template <int CW, typename Between>
__device__ __forceinline__ void scan_form_p(const lds_t *st, const int (&kq_off)[4][2], int lane, OutOperands &op,
                                            Between &&between) {
  constexpr int KB = CW == 0 ? 4 : 3;  // k row blocks used (up to the largest own row block)
  const int r0 = lane & 15, g = lane >> 4;
  auto frag = [&](int tile, int rt, int kk) -> Frag<bf16_t> {
    const lds_t *p = st + tile + 4096 * rt;
    return frag_cat(lds_load_single<bf16x4_t>(p + kq_off[kk][0]), lds_load_single<bf16x4_t>(p + kq_off[kk][1]));
  };
  Frag<bf16_t> kf[4][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) op.q[a][kk] = frag(kStQ, own_rt<CW>(a), kk);
#pragma unroll
  for (int b = 0; b < KB; ++b)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) kf[b][kk] = frag(kStK, b, kk);
  between();
  f32x4_t acc[2][4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int r = 0; r <= own_rt<CW>(a); ++r) acc[a][r] = mfma(kf[r][kk], op.q[a][kk], kk == 0 ? zero4() : acc[a][r]);
  const bf16x4_t z = {0, 0, 0, 0};
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int rt = own_rt<CW>(a), t = 16 * rt + r0;
    const float gt = lds_load<float>(st + kStG + 512 + 4 * t);
    op.gam[a] = lds_load<float>(st + kStG + 4 * t);
    bf16x4_t pv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r > rt) {
        pv[r] = z;
        continue;
      }
      const f32x4_t gi = lds_load<f32x4_t>(st + kStG + 512 + 4 * (16 * r + 4 * g));
      f32x4_t x;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float val = fast_exp2(gt - gi[e]) * acc[a][r][e];
        x[e] = (r < rt || 4 * g + e <= r0) ? val : 0.0f;
      }
      pv[r] = __builtin_convertvector(x, bf16x4_t);
    }
    op.p[a][0] = frag_cat(pv[0], pv[1]);
    op.p[a][1] = frag_cat(pv[2], pv[3]);
  }
}

// ROLE 1: output wave CW (0, 1) forms its rows of P and computes their
// outputs for the block's NCH column groups; ROLE 2: copy wave CW (0 .. 3)
// issues half the k (CW even) or q (CW odd) tile copies of each stage; copy
// waves 0 and 1 also half the T fragments and half the v block each, and copy
// wave 0 the gate block.  In transition mode (MODE 1) nothing reads q or the
// outputs: the output waves only keep step at the barriers and the q copies
// are not issued.  `cbv` is the column block whose v is staged.
template <int CW, int ROLE, int NCH, int MODE>
__device__ __forceinline__ void scan_copy_waves(const ScanArgs<bf16_t> &a, int lane, int h, int hq, int cb,
                                                int cbv, int start, int end, int c_first, int n_chunks) {
  constexpr bool kCopies = ROLE == 2, kOutputs = ROLE == 1 && MODE == 0;
  constexpr bool kTileCopies = kCopies && !(MODE == 1 && (CW & 1));
  constexpr int W = 16 * NCH;  // columns of the block
  const int r0 = lane & 15, g = lane >> 4;
  const int C = a.geo.chunk;
  const int64_t qk_stride = int64_t(a.H_qk) * 128;
  const int64_t v_stride = int64_t(a.H_v) * a.d_v;
  const uint32_t kq_row_bytes = uint32_t(2 * qk_stride);
  const char *kq_src = reinterpret_cast<const char *>((CW & 1) == 0 ? a.k : a.q) + int64_t(hq) * 256;
  // Per-lane byte offsets of every copy of a full chunk (tile_index.hpp),
  // relative to the chunk's first row.  The k / q and v copies go through a
  // buffer resource whose size ends at the chunk's last row, so rows past a
  // partial chunk read as zeros (exact zeros that the chunk algebra only
  // multiplies by zero) and no copy can leave the sequence.
  uint32_t kq_voff[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) kq_voff[i] = uint32_t(rowtile_copy_src(i, lane, 64, qk_stride));

  // A copy wave's share of a stage's k (or q) tile, 32 rows (copies
  // 8 (CW / 2) .. + 7), in two halves of four copies.
  auto stage_part = [&](int part, int cc, char *base_mem) {
    if (!kTileCopies) return;
    const int tok0 = start + cc * C;
    const int len = min(C, end - tok0);
    const i32x4_t kq_res = buffer_rsrc(kq_src + int64_t(tok0) * kq_row_bytes, rowtile_valid_bytes(len, kq_row_bytes));
    lds_t *const tile = lds_ptr(base_mem) + ((CW & 1) == 0 ? kStK : kStQ);
#pragma unroll
    for (int i = 8 * (CW >> 1) + 4 * part; i < 8 * (CW >> 1) + 4 * part + 4; ++i)
      dma16_buf(kq_res, kq_voff[i], tile + 1024 * i);
  };
  // The rest of a stage: copy wave 0 T fragments 0, 2, 4, the gate block
  // and v rows of the first half, copy wave 1 T fragments 5, 6, 7 and the
  // second half (copy waves 2 and 3 issue tile copies only).
  const int64_t ebytes = kStagedEntryBytes;
  const char *const v_src = reinterpret_cast<const char *>(a.v) + (int64_t(h) * a.d_v + W * cbv) * 2;
  const uint32_t v_row_bytes = uint32_t(2 * v_stride);
  constexpr int kVCopies = NCH == 2 ? 2 : 1;
  uint32_t v_voff[kVCopies];
#pragma unroll
  for (int i = 0; i < kVCopies; ++i)
    v_voff[i] = CW >= 2 ? 0u
                        : uint32_t(NCH == 2 ? vblock_copy_src(2 * CW + i, lane, 64, v_stride)
                                            : vblock16_copy_src(CW, lane, 64, v_stride));
  auto stage_rest = [&](int cc, char *base_mem) {
    const int tok0 = start + cc * C;
    const int len = min(C, end - tok0);
    lds_t *const base = lds_ptr(base_mem);
    if (CW >= 2) return;
    const char *entry = a.entries + (int64_t(c_first + cc) * a.H_v + h) * ebytes;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int f = CW == 0 ? 2 * i : 5 + i;  // 0, 2, 4 / 5, 6, 7
      // (fragments 0 and 5 are 512 bytes in the entry: lanes 0-31 bring them
      // to the first half of their slot, lanes 32-63 the start of the next
      // fragment, which the chain does not read)
      dma16(entry + t_entry_byte(f), 16 * lane, base + kStT + 1024 * t_slot(f));
    }
    // the gate block is 768 bytes: lanes 48-63 fall out of the resource's
    // range and write zeros into the slot's padding
    if (CW == 0) dma16_buf(buffer_rsrc(entry + kStagedGateOffset, kStagedGateBytes), 16 * lane, base + kStG);
    const i32x4_t v_res = buffer_rsrc(v_src + int64_t(tok0) * v_row_bytes,
                                      NCH == 2 ? vblock_valid_bytes(len, v_row_bytes)
                                               : vblock16_valid_bytes(len, v_row_bytes));
#pragma unroll
    for (int i = 0; i < kVCopies; ++i)
      dma16_buf_nt(v_res, v_voff[i], base + kStV + (NCH == 2 ? 2048 * CW + 1024 * i : 1024 * CW));
  };
  auto stage = [&](int cc, char *base_mem) {
    stage_rest(cc, base_mem);
    stage_part(0, cc, base_mem);
    stage_part(1, cc, base_mem);
  };
  constexpr int kLoads = (kTileCopies ? kStageLoadsCopy : 0) + (CW >= 2 ? 0 : 3 + (CW == 0 ? 1 : 0) + kVCopies);
  auto wait_all_but_newest_stage = [&]() { wait_vmem_upto<kLoads>(); };
  int kq_off[4][2];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) kq_off[kk][hf] = 2 * rowtile_off(r0, 32 * kk + 16 * hf + 4 * g);

  // Outputs of chunk oc from exchange buffer `ex_mem` and the operands kept
  // from its phase: transposed tiles, lane = token row 16 rt + lane mod 16,
  // columns 16 cg + 4 (lane / 16) .. + 3 of the block.  The four tiles'
  // products are independent and issue interleaved.  The tiles pass through
  // the output staging buffer so that each store writes whole 64-byte rows
  // (16 bytes per lane); the stores go through a buffer resource that ends at
  // the chunk's last row, so rows past a partial chunk are dropped without a
  // branch.
  OutOperands op;
  const uint32_t o_row_bytes = uint32_t(2 * v_stride);
  const char *const o_base = reinterpret_cast<const char *>(a.o + int64_t(h) * a.d_v + W * cb);
  // this lane's output pieces: written as the MFMA leaves them (row block b,
  // column group cg), read back as 16-byte row pieces -- one per row block
  // for 32-column blocks, one for both row blocks for 16-column blocks
  constexpr int kPieces = NCH == 2 ? 2 : 1;
  int os_w[2][NCH], os_r[kPieces];
  uint32_t o_voff[kPieces];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int rt = own_rt<CW>(b);
#pragma unroll
    for (int cg = 0; cg < NCH; ++cg)
      os_w[b][cg] = NCH == 2 ? out_stage_byte(out_acc_row(rt, lane), out_acc_col(cg, lane))
                             : out_stage16_byte(out_acc_row(rt, lane), out_acc_col(cg, lane));
  }
#pragma unroll
  for (int b = 0; b < kPieces; ++b) {
    const int row = NCH == 2 ? out_piece_row(own_rt<CW>(b), lane) : out_piece16_row(own_rt<CW>(lane >> 5), lane);
    const int col = NCH == 2 ? out_piece_col(lane) : out_piece16_col(lane);
    os_r[b] = NCH == 2 ? out_stage_byte(row, col) : out_stage16_byte(row, col);
    o_voff[b] = uint32_t(row) * o_row_bytes + 2 * col;
  }
  u32x4_t o_pend[kPieces];
  int o_pend_chunk = -1;
  auto outputs = [&](int oc, const char *ex_mem) {
    const lds_t *ex = lds_ptr(const_cast<char *>(ex_mem));
    Frag<bf16_t> sx[NCH][4], ux[NCH][2];
#pragma unroll
    for (int cg = 0; cg < NCH; ++cg) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) sx[cg][kk].v = lds_load<bf16x8_t>(ex + kExWave * cg + kExS + 1024 * kk + 16 * lane);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) ux[cg][kk].v = lds_load<bf16x8_t>(ex + kExWave * cg + kExU + 1024 * kk + 16 * lane);
    }
    f32x4_t acc[2][NCH];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int cg = 0; cg < NCH; ++cg) acc[b][cg] = mfma(sx[cg][kk], op.q[b][kk], kk == 0 ? zero4() : acc[b][cg]);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int cg = 0; cg < NCH; ++cg) acc[b][cg] = op.gam[b] * acc[b][cg];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int cg = 0; cg < NCH; ++cg)
          if (kk < (own_rt<CW>(b) < 2 ? 1 : 2)) acc[b][cg] = mfma(ux[cg][kk], op.p[b][kk], acc[b][cg]);
    lds_t *const os = lds_ptr(scan_ostage);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int cg = 0; cg < NCH; ++cg) lds_store<bf16x4_t>(os + os_w[b][cg], __builtin_convertvector(acc[b][cg], bf16x4_t));
#pragma unroll
    for (int b = 0; b < kPieces; ++b) o_pend[b] = lds_load<u32x4_t>(os + os_r[b]);
    o_pend_chunk = oc;
  };
  // The stores of the outputs computed in the previous phase, issued first
  // thing in a phase, before the copy waves' burst of copies fills the
  // memory pipeline (stores issued behind it wait for it to drain).
  auto store_pending = [&]() {
    if (o_pend_chunk < 0) return;
    const int tok0 = start + o_pend_chunk * C;
    const int len = min(C, end - tok0);
    const __amdgpu_buffer_rsrc_t o_res = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(o_base + int64_t(tok0) * o_row_bytes), 0, int((len - 1) * o_row_bytes + 2 * W), 0x00020000);
#pragma unroll
    for (int b = 0; b < kPieces; ++b) __builtin_amdgcn_raw_buffer_store_b128(o_pend[b], o_res, o_voff[b], 0, 0);
    o_pend_chunk = -1;
  };

  if (kCopies && n_chunks > 0) {
    stage(0, scan_stage0);
    stage(min(1, n_chunks - 1), scan_stage1);
    wait_all_but_newest_stage();
  }
  lds_barrier();
  // In the phase of chunk cc (between the barriers that open chunks cc and
  // cc + 1): the outputs of chunk cc - 1 (its exchange buffer was written
  // before this phase's barrier); the stage of chunk cc - 1 is free (the chain
  // waves read it before that barrier), and chunk cc + 2 goes there (past the
  // end the last chunk is copied again, so every phase issues the same
  // loads); the rows of P of chunk cc from its stage; then chunk cc + 1's
  // stage must be complete.
  auto phase = [&](int cc, char *dst, const char *cur, const char *ex_prev) {
    const int pf = min(cc + 2, n_chunks - 1);
    if (kOutputs) store_pending();
    if (ROLE == 2) __builtin_amdgcn_s_sleep(SCAN_COPY_DELAY);
    if (kCopies) {
      stage_rest(pf, dst);
      stage_part(0, pf, dst);
    }
    if (kOutputs && cc > 0) outputs(cc - 1, ex_prev);
    if (kOutputs)
      scan_form_p<CW>(lds_ptr(const_cast<char *>(cur)), kq_off, lane, op, [&]() {});
    if (kCopies) stage_part(1, pf, dst);
    if (kCopies) wait_all_but_newest_stage();
    lds_barrier();
  };
  for (int cc = 0; cc < n_chunks; cc += 6) {
    phase(cc, scan_stage2, scan_stage0, scan_ex1);
    if (cc + 1 < n_chunks) phase(cc + 1, scan_stage0, scan_stage1, scan_ex0);
    if (cc + 2 < n_chunks) phase(cc + 2, scan_stage1, scan_stage2, scan_ex1);
    if (cc + 3 < n_chunks) phase(cc + 3, scan_stage2, scan_stage0, scan_ex0);
    if (cc + 4 < n_chunks) phase(cc + 4, scan_stage0, scan_stage1, scan_ex1);
    if (cc + 5 < n_chunks) phase(cc + 5, scan_stage1, scan_stage2, scan_ex0);
  }
  // the last chunk's exchange was written before the last barrier
  if (kOutputs && n_chunks > 0) {
    store_pending();
    outputs(n_chunks - 1, (n_chunks - 1) % 2 == 0 ? scan_ex0 : scan_ex1);
    store_pending();
  }
  wait_vmem();  // the trailing copies and stores
}

// NCH chain waves (one per 16-column group; a block of 16 NCH columns), then
// two output waves, which form P and the outputs, and four copy waves, which
// issue every copy of a stage.  One chain wave per block doubles the blocks
// of a problem with few units (a long single sequence) at the same per-block
// traffic.
template <int NCH, int MODE>
__global__ __launch_bounds__(64 * (NCH + 6)) void scan_kernel_staged(ScanArgs<bf16_t> a) {
  constexpr int W = 16 * NCH;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r0 = lane & 15, g = lane >> 4;
  int u, cb;
  decode_block(blockIdx.x, a.n_colblk, u, cb);  // n_colblk = d_v / W
  if (u >= a.n_units) return;  // the whole block
  // The block's unit runs on XCD u mod 8.  Heads rotate by three per
  // sequence, so that an XCD serves eight different heads rather than the two
  // with h = u mod 8 (when H_v is a multiple of 8): the slices of some heads
  // in every k, q, v and o row are served more slowly than others, and
  // spread over all XCDs they delay the last blocks less.
  const int s_idx = u / a.H_v;
  const int s = a.geo.ordered(s_idx), h = (u + 3 * s_idx) % a.H_v, hq = h / a.group;

  int start, end;
  a.geo.seq_bounds(s, start, end);
  const int C = a.geo.chunk;
  const int c_first = a.geo.first_chunk(s);
  const int n_chunks = max(0, min((end - start + C - 1) / C, a.geo.n_slots - c_first));
  // transition mode: blocks past the value columns carry M (v = 0; the v of
  // column block 0 is staged so that every copy stays inside v)
  const bool is_m = MODE == 1 && cb >= a.n_colblk_v;
  const int cbv = is_m ? 0 : cb;
  const int cbs = is_m ? cb - a.n_colblk_v : cb;  // column block within B or M

  if (wave == NCH) {
    scan_copy_waves<0, 1, NCH, MODE>(a, lane, h, hq, cb, cbv, start, end, c_first, n_chunks);
    return;
  }
  if (wave == NCH + 1) {
    scan_copy_waves<1, 1, NCH, MODE>(a, lane, h, hq, cb, cbv, start, end, c_first, n_chunks);
    return;
  }
  if (wave == NCH + 2) {
    scan_copy_waves<0, 2, NCH, MODE>(a, lane, h, hq, cb, cbv, start, end, c_first, n_chunks);
    return;
  }
  if (wave == NCH + 3) {
    scan_copy_waves<1, 2, NCH, MODE>(a, lane, h, hq, cb, cbv, start, end, c_first, n_chunks);
    return;
  }
  if (wave == NCH + 4) {
    scan_copy_waves<2, 2, NCH, MODE>(a, lane, h, hq, cb, cbv, start, end, c_first, n_chunks);
    return;
  }
  if (wave == NCH + 5) {
    scan_copy_waves<3, 2, NCH, MODE>(a, lane, h, hq, cb, cbv, start, end, c_first, n_chunks);
    return;
  }

  // ---- chain waves: wave w owns columns W cb + 16 w .. + 15 ----
  // ---- lane-invariant LDS byte offsets (relative to a stage) ----
  // A fragments of k rows 16 rt + r0, columns 32 kk + 16 half + 4 g:
  // offset = 4096 rt + kq_off[kk][half].
  int kq_off[4][2];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) kq_off[kk][hf] = 2 * rowtile_off(r0, 32 * kk + 16 * hf + 4 * g);
  // transposed K^T fragments: lane a = r0 addresses token
  // 32 kk + 16 half + 4 g + a / 4, columns 16 rm + 4 (a mod 4) .. + 3:
  // offset = 8192 kk + 4096 half + kt_off[rm].
  int kt_off[8];
#pragma unroll
  for (int rm = 0; rm < 8; ++rm) kt_off[rm] = 2 * rowtile_off(4 * g + (r0 >> 2), 16 * rm + 4 * (r0 & 3));
  // transposed v tile rt of this wave's columns (rows 16 rt + 4 g + a / 4,
  // columns 16 w + 4 (a mod 4)): offset = kVTile rt + v_off (32- or
  // 16-column v block).
  constexpr int kVTile = NCH == 2 ? 1024 : 512;
  const int v_off = NCH == 2 ? vtile_byte(4 * g + (r0 >> 2), 16 * wave + 4 * (r0 & 3))
                             : vtile16_byte(4 * g + (r0 >> 2), 4 * (r0 & 3));
  const int col = W * cbs + 16 * wave + r0;  // this lane's state column
  const int ex_off = kExWave * wave + 16 * lane;

  // ---- state ----
  f32x4_t S[8];
  const int64_t st_base = (int64_t(s) * a.H_v + h) * 128 * a.d_v;
#pragma unroll
  for (int rt = 0; rt < 8; ++rt)
#pragma unroll
    for (int e = 0; e < 4; ++e) S[rt][e] = initial_state(a.h0, st_base, 16 * rt + 4 * g + e, col, a.d_v, MODE, is_m);

  // Operands of the chunk about to run, read from its stage right after the
  // barrier that completes it: gate factors (rows 16 rt + 4 g + e of this
  // lane's column, the chunk's last slot), k row fragments, v transposed, T
  // fragments.  Row fragments are two 8-byte reads each, kept single (not
  // paired across tiles) so that they land in the fragment's registers
  // directly.
  float gamma_C;
  f32x4_t gam[4], sc[4];
  Frag<bf16_t> kf[4][4];  // k rows: [contraction block][row tile]
  bf16x4_t vt[4];         // v, transposed: four rows of this lane's column
  Frag<bf16_t> tf[8];
  auto read_operands = [&](const char *stage_mem) {
    const lds_t *st = lds_ptr(const_cast<char *>(stage_mem));
    gamma_C = lds_load<float>(st + kStG + 252);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      gam[rt] = lds_load<f32x4_t>(st + kStG + 64 * rt + 16 * g);
      sc[rt] = lds_load<f32x4_t>(st + kStG + 256 + 64 * rt + 16 * g);
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
    for (int rt = 0; rt < 4; ++rt) vt[rt] = is_m ? bf16x4_t{0, 0, 0, 0} : lds_read_tr16(st + kStV + kVTile * rt + v_off);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (t_compact(i)) {  // elements 0-3 staged, 4-7 zero
        const bf16x4_t lo = lds_load<bf16x4_t>(st + kStT + 1024 * t_slot(i) + 8 * lane);
        tf[i].v = __builtin_shufflevector(lo, bf16x4_t{0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7);
      } else if (i != 1 && i != 3) {
        tf[i].v = lds_load<bf16x8_t>(st + kStT + 1024 * t_slot(i) + 16 * lane);
      }
  };

  lds_barrier();  // the first two stages are complete
  if (n_chunks > 0) read_operands(scan_stage0);

  // One chunk: the state chain from the operands read after the previous
  // barrier, the chunk-start state and U handed to the output waves through
  // exchange buffer `ex_mem`, K^T read from the stage during the chain.  The
  // barrier follows the state update (after it the copy waves may reuse this
  // chunk's stage); then the next chunk's operands are read.
  auto chunk_step = [&](int cc, char *cur_mem, char *next_mem, char *prev_mem, char *ex_mem) {
    const lds_t *const st = lds_ptr(cur_mem);
    lds_t *const ex = lds_ptr(ex_mem) + ex_off;

    Frag<bf16_t> Sf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) Sf[kk] = frag_from_acc<bf16_t>(S[2 * kk], S[2 * kk + 1]);

    // Y = K S
    f32x4_t Y[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) Y[rt] = mfma(kf[kk][rt], Sf[kk], kk == 0 ? zero4() : Y[rt]);
    if (MODE == 0)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) lds_store<bf16x8_t>(ex + kExS + 1024 * kk, Sf[kk].v);

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
    Frag<bf16_t> Xf[2];
    {
      f32x4_t X[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) X[rt] = __builtin_convertvector(vt[rt], f32x4_t) - gam[rt] * Y[rt];
      Xf[0] = frag_from_acc<bf16_t>(X[0], X[1]);
      Xf[1] = frag_from_acc<bf16_t>(X[2], X[3]);
    }
    f32x4_t Ua[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int kk = 0; kk < (rt < 2 ? 1 : 2); ++kk)  // T rows 0-31 end at column 31
        Ua[rt] = mfma(tf[rt * 2 + kk], Xf[kk], kk == 0 ? zero4() : Ua[rt]);

    Frag<bf16_t> Usf[2];
    if (MODE == 0)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        lds_store<bf16x8_t>(ex + kExU + 1024 * kk, frag_from_acc<bf16_t>(Ua[2 * kk], Ua[2 * kk + 1]).v);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) Ua[rt] *= sc[rt];
    Usf[0] = frag_from_acc<bf16_t>(Ua[0], Ua[1]);
    Usf[1] = frag_from_acc<bf16_t>(Ua[2], Ua[3]);

    // S <- gamma_C S + K^T (s U)
#pragma unroll
    for (int rm = 0; rm < 8; ++rm) {
      f32x4_t acc = gamma_C * S[rm];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) acc = mfma(ktf[rm][kk], Usf[kk], acc);
      S[rm] = acc;
    }

    // this chunk's stage reads are done (the copy waves may now refill the
    // previous chunk's stage), the exchange is written, and the next chunk's
    // stage is complete
    lds_barrier();
    if (cc + 1 < n_chunks) read_operands(next_mem);
  };
  for (int cc = 0; cc < n_chunks; cc += 6) {
    chunk_step(cc, scan_stage0, scan_stage1, scan_stage2, scan_ex0);
    if (cc + 1 < n_chunks) chunk_step(cc + 1, scan_stage1, scan_stage2, scan_stage0, scan_ex1);
    if (cc + 2 < n_chunks) chunk_step(cc + 2, scan_stage2, scan_stage0, scan_stage1, scan_ex0);
    if (cc + 3 < n_chunks) chunk_step(cc + 3, scan_stage0, scan_stage1, scan_stage2, scan_ex1);
    if (cc + 4 < n_chunks) chunk_step(cc + 4, scan_stage1, scan_stage2, scan_stage0, scan_ex0);
    if (cc + 5 < n_chunks) chunk_step(cc + 5, scan_stage2, scan_stage0, scan_stage1, scan_ex1);
  }
  wait_vmem();  // the trailing copies

  if (MODE == 1) {
    const int ld = a.d_v + 128;
    float *dst = a.mb + (int64_t(s) * a.H_v + h) * 128 * ld + (is_m ? a.d_v : 0) + col;
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
      for (int e = 0; e < 4; ++e) dst[int64_t(16 * rt + 4 * g + e) * ld] = S[rt][e];
  } else if (a.hT) {
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
      for (int e = 0; e < 4; ++e) a.hT[st_base + int64_t(16 * rt + 4 * g + e) * a.d_v + col] = S[rt][e];
  }
}

// Below this many 32-column blocks (half the CUs of an MI355X) the staged
// scan uses 16-column blocks, one chain wave each, so that a problem with few
// (sequence, head) units spreads over twice as many CUs.
constexpr int64_t kNarrowBelowBlocks = 128;

template <typename T>
static ScanArgs<T> scan_args(const Problem &p, const Workspace &ws, int colblk_width, float *mb) {
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
  a.n_colblk_v = p.d_v / colblk_width;
  a.mode = mb ? 1 : 0;
  a.mb = mb;
  a.n_colblk = a.n_colblk_v + (mb ? p.d_k / colblk_width : 0);
  a.geo = make_geom(p, &ws);
  return a;
}

hipError_t launch_scan(const Problem &p, const Workspace &ws, hipStream_t st, float *mb) {
  if (!staged_path(p)) return hipErrorInvalidValue;  // other shapes run the chained form
  const int64_t units8 = (int64_t(p.n_seqs) * p.H_v + 7) / 8 * 8;
  const int cols = p.d_v + (mb ? p.d_k : 0);  // state columns per unit (transition mode: B and M)
  const bool narrow = units8 * (cols / 32) < kNarrowBelowBlocks;
  const int width = narrow ? 16 : 32;
  const int64_t blocks = units8 * (cols / width);
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid = dim3(static_cast<unsigned>(blocks));
  const ScanArgs<bf16_t> a = scan_args<bf16_t>(p, ws, width, mb);
  if (narrow && mb) hipLaunchKernelGGL((scan_kernel_staged<1, 1>), grid, dim3(64 * 7), 0, st, a);
  else if (narrow) hipLaunchKernelGGL((scan_kernel_staged<1, 0>), grid, dim3(64 * 7), 0, st, a);
  else if (mb) hipLaunchKernelGGL((scan_kernel_staged<2, 1>), grid, dim3(64 * 8), 0, st, a);
  else hipLaunchKernelGGL((scan_kernel_staged<2, 0>), grid, dim3(64 * 8), 0, st, a);
  return hipGetLastError();
}

}  // namespace gdn
