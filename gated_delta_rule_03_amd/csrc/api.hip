// libgdn C ABI: argument checks, workspace layout and launch order.
// The operation and the contract of every entry point are in include/gdn.h.
#include "../../include/gdn.h"

#include <cmath>
#include <limits>

#include "launch.hpp"

namespace gdn {

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int64_t chunk_slots(const Problem &p) {
  if (p.chunk <= 0) return 0;  // the token-by-token path has no chunks
  if (p.cu_seqlens) return ceil_div(p.T, p.chunk) + p.n_seqs;
  return int64_t(p.B) * ceil_div(p.T, p.chunk);
}

SeqGeom make_geom(const Problem &p, const Workspace *ws) {
  SeqGeom g;
  g.cu_seqlens = p.cu_seqlens;
  g.chunk_off = ws ? ws->chunk_off : nullptr;
  g.seq_order = ws && p.cu_seqlens ? ws->seq_order : nullptr;
  g.n_seqs = p.n_seqs;
  g.T = p.T;
  g.chunk = p.chunk > 0 ? p.chunk : 64;
  g.chunks_per_seq = int32_t(ceil_div(p.T, g.chunk));
  g.n_slots = int32_t(std::min<int64_t>(chunk_slots(p), std::numeric_limits<int32_t>::max()));
  return g;
}

size_t workspace_layout(const Problem &p, void *base, Workspace *ws) {
  const int64_t entry = entry_stride(p);
  const size_t off_bytes = align256(size_t(2 * int64_t(p.n_seqs) + 1) * sizeof(int32_t));
  const size_t ent_bytes = align256(size_t(chunk_slots(p)) * p.H_v * size_t(entry));
  if (ws) {
    char *b = static_cast<char *>(base);
    ws->chunk_off = reinterpret_cast<int32_t *>(b);
    ws->seq_order = ws->chunk_off + p.n_seqs + 1;
    ws->entries = b + off_bytes;
  }
  return off_bytes + ent_bytes;
}

static bool dim_ok(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// Shape and dtype checks.  Returns GDN_SUCCESS or the error status.
static int32_t check_shapes(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k,
                            int32_t d_v, int32_t dtype) {
  if (B < 0 || T < 0 || H_qk <= 0 || H_v <= 0 || d_k <= 0 || d_v <= 0)
    return GDN_ERROR_INVALID_VALUE;
  if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERROR_NOT_SUPPORTED;
  if (!dim_ok(d_k) || !dim_ok(d_v)) return GDN_ERROR_NOT_SUPPORTED;
  if (H_v % H_qk != 0) return GDN_ERROR_NOT_SUPPORTED;
  // Token and chunk indices are 32-bit in the kernels.
  const int64_t tokens = int64_t(B) * T;
  if (tokens > std::numeric_limits<int32_t>::max()) return GDN_ERROR_NOT_SUPPORTED;
  if (tokens * std::max<int64_t>(H_v, H_qk) * std::max(d_k, d_v) > (int64_t(1) << 40))
    return GDN_ERROR_NOT_SUPPORTED;
  return GDN_SUCCESS;
}

// Token-major tensors are read and written 16 bytes per lane.
static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Shape checks plus the tensor pointers every non-empty call needs.
static int32_t check_common(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k,
                            int32_t d_v, int32_t dtype, const void *q, const void *k,
                            const void *v, const float *alpha, const float *beta, const void *o) {
  const int32_t st = check_shapes(B, T, H_qk, H_v, d_k, d_v, dtype);
  if (st != GDN_SUCCESS) return st;
  if (int64_t(B) * T > 0 && (!q || !k || !v || !alpha || !beta || !o))
    return GDN_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return GDN_ERROR_INVALID_VALUE;
  return GDN_SUCCESS;
}

int32_t make_problem(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k,
                            int32_t d_v, int32_t dtype, const void *q, const void *k,
                            const void *v, const float *alpha, const float *beta,
                            const int32_t *cu_seqlens, int32_t n_seqs, const float *h0,
                            void *o, float *hT, Problem *p) {
  int32_t st = check_common(B, T, H_qk, H_v, d_k, d_v, dtype, q, k, v, alpha, beta, o);
  if (st != GDN_SUCCESS) return st;
  if (cu_seqlens) {
    // a packed batch with tokens must hold at least one sequence
    if (B != 1 || n_seqs < 0 || (n_seqs == 0 && T > 0)) return GDN_ERROR_INVALID_VALUE;
  } else {
    if (n_seqs != 0 && n_seqs != B) return GDN_ERROR_INVALID_VALUE;
    n_seqs = B;
  }
  if (!aligned16(h0) || !aligned16(hT)) return GDN_ERROR_INVALID_VALUE;
  *p = Problem{B, T, H_qk, H_v, d_k, d_v, dtype, q, k, v, alpha, beta,
               cu_seqlens, n_seqs, h0, o, hT, 0};
  return GDN_SUCCESS;
}

static int32_t status_of(hipError_t e) { return e == hipSuccess ? GDN_SUCCESS : GDN_ERROR_LAUNCH; }

// ---------------------------------------------------------------------------
// Segment-parallel chunked forward.  A sequence scan visits its chunks in
// order, so a problem with few (sequence, value head) units leaves most of the
// GPU idle however long the sequences are.  Cutting every sequence into
// segments of seg_chunks chunks gives more, shorter units: one transition-mode
// scan over the segments (each segment's affine map), a fold of the maps in
// sequence order (the state entering every segment, and the final state), and
// the ordinary scan over the segments from those states (the outputs).
// ---------------------------------------------------------------------------

// Chunks per segment for a problem (0: one pass).  Segments pay off when the
// one-pass scan has fewer than 128 blocks of 32 value columns (then it runs
// 16-column blocks, and still leaves CUs idle or waits on one long chain).
// The segment count aims at about two full rounds of transition-pass blocks
// (512 blocks of 32 of its d_v + d_k columns), with the segment length kept
// between 64 and 128 chunks: shorter segments pay more per-segment start-up
// and fold steps, longer ones leave the passes with too few blocks.
// Measured on MI355X, long context T = 65536, d = 128, one pass vs segments
// of 16 / 32 / 64 / 128 / 256 chunks: 16 heads 1,123 vs
// 1,150 / 957 / 886 / 844 / 921 us; 2 heads 863 vs 319 / 221 / 200 / 271 / 459 us.
//
// Shapes off the staged path run both passes on the chained kernels, whose
// chunk step is longer; there the aim is about four rounds (1,024 blocks)
// and segments of 32 to 128 chunks.  Measured, T = 65536, chunk 64, one pass
// vs segments of 32 / 64 / 128 chunks: fp32 d = 128, 2 heads 4,219 vs
// 715 / 711 / 1,010 us, 4 heads 4,475 vs 1,254 / 1,183 / 1,260, 8 heads
// 4,669 vs 2,339 / 2,176 / 2,119, 16 heads 4,839 vs 4,317 / 4,172 / 4,114;
// bf16 d = 64, 2 heads 3,225 vs 291 / 400 / 689, 4 heads 3,238 vs
// 401 / 482 / 730, 16 heads 3,479 vs 1,208 / 1,185 / 1,294.
int32_t plan_segment_chunks(const Problem &p) {
  const int64_t units = int64_t(p.n_seqs) * p.H_v;
  const int64_t max_chunks = ceil_div(p.T, p.chunk);  // the longest sequence's chunks, at most
  if (units == 0 || units * std::max(1, p.d_v / 32) >= 128) return 0;
  const bool staged = staged_path(p);
  const int64_t blocks1 = units * std::max(1, (p.d_v + p.d_k) / 32);
  const int64_t segs = ceil_div(staged ? 512 : 1024, blocks1);
  const int64_t seg = std::min<int64_t>(128, std::max<int64_t>(staged ? 64 : 32, ceil_div(max_chunks, segs)));
  return seg >= max_chunks ? 0 : int32_t(seg);
}

struct SegWorkspace {
  int32_t *seg_cu, *seg_first;
  void *base;          // the segment batch's own workspace
  float *mb, *s_in;
};

// The segment batch: one packed batch over the whole token axis, one
// sequence per segment, started from the fold's states.
static int32_t n_seg_bound(const Problem &p, int32_t seg_chunks) {
  const int64_t seg_tokens = int64_t(seg_chunks) * p.chunk;
  if (p.cu_seqlens) return int32_t(ceil_div(p.T, seg_tokens) + p.n_seqs);
  return int32_t(int64_t(p.B) * ceil_div(p.T, seg_tokens));
}
static Problem segment_problem(const Problem &p, int32_t seg_chunks, const SegWorkspace *sw) {
  Problem ps = p;
  ps.B = 1;
  ps.T = int32_t(p.n_tokens());
  ps.n_seqs = n_seg_bound(p, seg_chunks);
  static const int32_t kLayoutOnly = 0;
  ps.cu_seqlens = sw ? sw->seg_cu : &kLayoutOnly;  // selects the packed layout
  ps.h0 = sw ? sw->s_in : nullptr;
  ps.hT = nullptr;  // the fold writes the final states
  return ps;
}
static size_t seg_workspace_layout(const Problem &p, int32_t seg_chunks, void *base, SegWorkspace *sw) {
  const Problem ps = segment_problem(p, seg_chunks, nullptr);
  const int64_t nseg = ps.n_seqs;
  const size_t cu_bytes = align256(size_t(nseg + 1) * sizeof(int32_t));
  const size_t first_bytes = align256(size_t(p.n_seqs + 1) * sizeof(int32_t));
  const size_t ws_bytes = workspace_layout(ps, nullptr, nullptr);
  const size_t mb_bytes = align256(size_t(nseg) * p.H_v * p.d_k * (p.d_k + p.d_v) * sizeof(float));
  const size_t sin_bytes = align256(size_t(nseg) * p.H_v * p.d_k * p.d_v * sizeof(float));
  if (sw) {
    char *b = static_cast<char *>(base);
    sw->seg_cu = reinterpret_cast<int32_t *>(b);
    sw->seg_first = reinterpret_cast<int32_t *>(b + cu_bytes);
    sw->base = b + cu_bytes + first_bytes;
    sw->mb = reinterpret_cast<float *>(b + cu_bytes + first_bytes + ws_bytes);
    sw->s_in = reinterpret_cast<float *>(b + cu_bytes + first_bytes + ws_bytes + mb_bytes);
  }
  return cu_bytes + first_bytes + ws_bytes + mb_bytes + sin_bytes;
}

size_t chunk_workspace_bytes(const Problem &p, int32_t seg_chunks) {
  return seg_chunks > 0 ? seg_workspace_layout(p, seg_chunks, nullptr, nullptr)
                        : workspace_layout(p, nullptr, nullptr);
}

// Problem for the workspace queries (no tensors).
static Problem query_problem(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k, int32_t d_v,
                             int32_t dtype, int32_t chunk, int32_t n_seqs) {
  Problem p{};
  p.B = B;
  p.T = T;
  p.H_qk = H_qk;
  p.H_v = H_v;
  p.d_k = d_k;
  p.d_v = d_v;
  p.dtype = dtype;
  // A packed batch (B == 1, n_seqs > 0) reserves ceil(T / chunk) + n_seqs
  // chunk slots, which also covers a single uniform sequence.
  const bool packed = B == 1 && n_seqs > 0;
  p.n_seqs = packed ? n_seqs : B;
  static const int32_t kLayoutOnly = 0;
  p.cu_seqlens = packed ? &kLayoutOnly : nullptr;  // selects the packed layout; never read
  p.chunk = chunk;
  return p;
}

static bool query_ok(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k, int32_t d_v, int32_t dtype,
                     int32_t chunk, int32_t n_seqs) {
  return check_shapes(B, T, H_qk, H_v, d_k, d_v, dtype) == GDN_SUCCESS &&
         (chunk == 16 || chunk == 32 || chunk == 64) && n_seqs >= 0;
}

// Segment lengths that keep every index in range: segments of at most 2^31
// tokens, a segment count that fits a 32-bit sequence count.
static bool seg_chunks_ok(const Problem &p, int32_t seg_chunks) {
  if (seg_chunks < 0) return false;
  if (seg_chunks == 0) return true;
  if (int64_t(seg_chunks) * p.chunk > std::numeric_limits<int32_t>::max()) return false;
  const int64_t seg_tokens = int64_t(seg_chunks) * p.chunk;
  const int64_t bound = p.cu_seqlens ? ceil_div(p.T, seg_tokens) + p.n_seqs
                                     : int64_t(p.B) * ceil_div(p.T, seg_tokens);
  return bound < (int64_t(1) << 30) && bound * p.H_v * std::max(p.d_v, 32) / 16 < 0x7fffffff;
}

int32_t run_chunk_fwd(Problem p, int32_t seg_chunks, void *workspace, size_t workspace_bytes,
                      hipStream_t s) {
  const size_t need = chunk_workspace_bytes(p, seg_chunks);
  if (!workspace || workspace_bytes < need) return GDN_ERROR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return GDN_ERROR_WORKSPACE;
  if (seg_chunks == 0) {
    Workspace ws;
    workspace_layout(p, workspace, &ws);
    hipError_t e = launch_chunk_offsets(p, ws, s);
    if (chain_path(p)) {
      if (e == hipSuccess) e = launch_chain_fwd(p, ws, s);
    } else {
      if (e == hipSuccess) e = launch_prep(p, ws, s);
      if (e == hipSuccess) e = launch_scan(p, ws, s);
    }
    return status_of(e);
  }
  SegWorkspace sw;
  seg_workspace_layout(p, seg_chunks, workspace, &sw);
  const Problem ps = segment_problem(p, seg_chunks, &sw);
  Workspace ws;
  workspace_layout(ps, sw.base, &ws);
  hipError_t e = launch_segment_map(p, seg_chunks * p.chunk, ps.n_seqs, sw.seg_cu, sw.seg_first, s);
  if (e == hipSuccess) e = launch_chunk_offsets(ps, ws, s);
  const bool chained = chain_path(ps);
  if (chained) {  // factors once; the transition pass reads them, and so does the output pass
    if (e == hipSuccess) e = launch_chain_fwd(ps, ws, s, sw.mb, true);
  } else {
    if (e == hipSuccess) e = launch_prep(ps, ws, s);
    if (e == hipSuccess) e = launch_scan(ps, ws, s, sw.mb);
  }
  if (e == hipSuccess) e = launch_fold(sw.mb, p.h0, sw.s_in, p.hT, sw.seg_first, p.n_seqs, ps.n_seqs, p.H_v, p.d_k,
                                       p.d_v, s);
  if (chained) {
    if (e == hipSuccess) e = launch_chain_fwd(ps, ws, s, nullptr, false);
  } else {
    if (e == hipSuccess) e = launch_scan(ps, ws, s);
  }
  return status_of(e);
}

// Workspace of the backward pass: chunk offsets, one entry of fp32
// intermediates per (chunk slot, value head), and under grouped heads the
// per-value-head dq and dk.
size_t bwd_workspace_layout(const Problem &p, void *base, BwdProblem *b) {
  const int64_t tokens = p.n_tokens();
  const size_t off_bytes = align256(size_t(2 * int64_t(p.n_seqs) + 1) * sizeof(int32_t));
  const size_t ent_bytes =
      align256(size_t(chunk_slots(p)) * p.H_v * bwd_entry_floats(p.chunk, p.d_k, p.d_v) * sizeof(float));
  const size_t part_bytes = p.H_v > p.H_qk ? align256(size_t(tokens) * p.H_v * p.d_k * sizeof(float)) : 0;
  if (b) {
    char *c = static_cast<char *>(base);
    b->ws.chunk_off = reinterpret_cast<int32_t *>(c);
    b->ws.seq_order = b->ws.chunk_off + p.n_seqs + 1;
    b->ws.entries = nullptr;
    c += off_bytes;
    b->entries = reinterpret_cast<float *>(c);
    c += ent_bytes;
    b->dq_part = part_bytes ? reinterpret_cast<float *>(c) : nullptr;
    c += part_bytes;
    b->dk_part = part_bytes ? reinterpret_cast<float *>(c) : nullptr;
  }
  return off_bytes + ent_bytes + 2 * part_bytes;
}

}  // namespace gdn

using namespace gdn;

extern "C" {

int32_t gdn_version(void) { return 200; }  // 0.2.0: block prologue/epilogue, per-channel gate

const char *gdn_status_string(int32_t status) {
  switch (status) {
    case GDN_SUCCESS: return "success";
    case GDN_ERROR_INVALID_VALUE: return "invalid value (null pointer or inconsistent size)";
    case GDN_ERROR_NOT_SUPPORTED: return "not supported (size or dtype outside the supported set)";
    case GDN_ERROR_WORKSPACE: return "workspace missing or too small";
    case GDN_ERROR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int32_t gdn_recurrent_fwd(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k,
                          int32_t d_v, int32_t dtype, const void *q, const void *k, const void *v,
                          const float *alpha, const float *beta, const int32_t *cu_seqlens,
                          int32_t n_seqs, const float *h0, void *o, float *hT, void *stream) {
  Problem p;
  int32_t st = make_problem(B, T, H_qk, H_v, d_k, d_v, dtype, q, k, v, alpha, beta, cu_seqlens,
                            n_seqs, h0, o, hT, &p);
  if (st != GDN_SUCCESS) return st;
  return status_of(launch_recurrent(p, static_cast<hipStream_t>(stream)));
}

size_t gdn_chunk_fwd_workspace_bytes(int32_t B, int32_t T, int32_t H_qk, int32_t H_v,
                                     int32_t d_k, int32_t d_v, int32_t dtype, int32_t chunk,
                                     int32_t n_seqs) {
  if (!query_ok(B, T, H_qk, H_v, d_k, d_v, dtype, chunk, n_seqs)) return 0;
  const Problem p = query_problem(B, T, H_qk, H_v, d_k, d_v, dtype, chunk, n_seqs);
  return chunk_workspace_bytes(p, plan_segment_chunks(p));
}

int32_t gdn_chunk_fwd_plan_segments(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k,
                                    int32_t d_v, int32_t dtype, int32_t chunk, int32_t n_seqs) {
  if (!query_ok(B, T, H_qk, H_v, d_k, d_v, dtype, chunk, n_seqs)) return -1;
  return plan_segment_chunks(query_problem(B, T, H_qk, H_v, d_k, d_v, dtype, chunk, n_seqs));
}

size_t gdn_chunk_fwd_segmented_workspace_bytes(int32_t B, int32_t T, int32_t H_qk, int32_t H_v,
                                               int32_t d_k, int32_t d_v, int32_t dtype, int32_t chunk,
                                               int32_t n_seqs, int32_t seg_chunks) {
  if (!query_ok(B, T, H_qk, H_v, d_k, d_v, dtype, chunk, n_seqs)) return 0;
  const Problem p = query_problem(B, T, H_qk, H_v, d_k, d_v, dtype, chunk, n_seqs);
  if (!seg_chunks_ok(p, seg_chunks)) return 0;
  return chunk_workspace_bytes(p, seg_chunks);
}

int32_t gdn_chunk_fwd(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k, int32_t d_v,
                      int32_t dtype, const void *q, const void *k, const void *v,
                      const float *alpha, const float *beta, const int32_t *cu_seqlens,
                      int32_t n_seqs, const float *h0, void *o, float *hT, int32_t chunk,
                      void *workspace, size_t workspace_bytes, void *stream) {
  Problem p;
  int32_t st = make_problem(B, T, H_qk, H_v, d_k, d_v, dtype, q, k, v, alpha, beta, cu_seqlens,
                            n_seqs, h0, o, hT, &p);
  if (st != GDN_SUCCESS) return st;
  if (chunk != 16 && chunk != 32 && chunk != 64) return GDN_ERROR_NOT_SUPPORTED;
  p.chunk = chunk;
  return run_chunk_fwd(p, plan_segment_chunks(p), workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

int32_t gdn_chunk_fwd_segmented(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k, int32_t d_v,
                                int32_t dtype, const void *q, const void *k, const void *v,
                                const float *alpha, const float *beta, const int32_t *cu_seqlens,
                                int32_t n_seqs, const float *h0, void *o, float *hT, int32_t chunk,
                                int32_t seg_chunks, void *workspace, size_t workspace_bytes, void *stream) {
  Problem p;
  int32_t st = make_problem(B, T, H_qk, H_v, d_k, d_v, dtype, q, k, v, alpha, beta, cu_seqlens,
                            n_seqs, h0, o, hT, &p);
  if (st != GDN_SUCCESS) return st;
  if (chunk != 16 && chunk != 32 && chunk != 64) return GDN_ERROR_NOT_SUPPORTED;
  p.chunk = chunk;
  if (seg_chunks < 0) return GDN_ERROR_INVALID_VALUE;
  if (!seg_chunks_ok(p, seg_chunks)) return GDN_ERROR_NOT_SUPPORTED;
  return run_chunk_fwd(p, seg_chunks, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

size_t gdn_chunk_bwd_workspace_bytes(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k,
                                     int32_t d_v, int32_t dtype, int32_t chunk, int32_t n_seqs) {
  if (!query_ok(B, T, H_qk, H_v, d_k, d_v, dtype, chunk, n_seqs)) return 0;
  const Problem p = query_problem(B, T, H_qk, H_v, d_k, d_v, dtype, chunk, n_seqs);
  return bwd_workspace_layout(p, nullptr, nullptr);
}

int32_t gdn_chunk_bwd(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k, int32_t d_v, int32_t dtype,
                      const void *q, const void *k, const void *v, const float *alpha, const float *beta,
                      const int32_t *cu_seqlens, int32_t n_seqs, const float *h0, const void *d_o,
                      const float *dhT, float *dq, float *dk, float *dv, float *dalpha, float *dbeta, float *dh0,
                      int32_t chunk, void *workspace, size_t workspace_bytes, void *stream) {
  Problem p;
  // d_o takes the place of o in the forward's checks (required, 16-byte aligned)
  int32_t st = make_problem(B, T, H_qk, H_v, d_k, d_v, dtype, q, k, v, alpha, beta, cu_seqlens, n_seqs, h0,
                            const_cast<void *>(d_o), nullptr, &p);
  if (st != GDN_SUCCESS) return st;
  if (chunk != 16 && chunk != 32 && chunk != 64) return GDN_ERROR_NOT_SUPPORTED;
  if (p.n_tokens() > 0 && (!dq || !dk || !dv || !dalpha || !dbeta)) return GDN_ERROR_INVALID_VALUE;
  if (!aligned16(dhT) || !aligned16(dh0)) return GDN_ERROR_INVALID_VALUE;
  p.chunk = chunk;
  p.o = nullptr;
  const size_t need = bwd_workspace_layout(p, nullptr, nullptr);
  if (!workspace || workspace_bytes < need) return GDN_ERROR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return GDN_ERROR_WORKSPACE;
  BwdProblem b;
  b.p = p;
  bwd_workspace_layout(p, workspace, &b);
  b.d_o = d_o;
  b.dhT = dhT;
  b.dq = dq;
  b.dk = dk;
  b.dv = dv;
  b.dalpha = dalpha;
  b.dbeta = dbeta;
  b.dh0 = dh0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_chunk_offsets(p, b.ws, s);
  if (e == hipSuccess) e = launch_chunk_bwd(b, s);
  return status_of(e);
}

int32_t gdn_decode_step(int32_t B, int32_t H_qk, int32_t H_v, int32_t d_k, int32_t d_v,
                        int32_t dtype, const void *q, const void *k, const void *v,
                        const float *alpha, const float *beta, float *state, void *o,
                        void *stream) {
  int32_t st = check_common(B, 1, H_qk, H_v, d_k, d_v, dtype, q, k, v, alpha, beta, o);
  if (st != GDN_SUCCESS) return st;
  if ((B > 0 && !state) || !aligned16(state)) return GDN_ERROR_INVALID_VALUE;
  Problem p{};
  p.B = B;
  p.T = 1;
  p.H_qk = H_qk;
  p.H_v = H_v;
  p.d_k = d_k;
  p.d_v = d_v;
  p.dtype = dtype;
  p.q = q;
  p.k = k;
  p.v = v;
  p.alpha = alpha;
  p.beta = beta;
  p.o = o;
  p.n_seqs = B;
  return status_of(launch_decode(p, state, static_cast<hipStream_t>(stream)));
}

int32_t gdn_kda_recurrent_fwd(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k,
                              int32_t d_v, int32_t dtype, const void *q, const void *k, const void *v,
                              const float *alpha, const float *beta, const int32_t *cu_seqlens,
                              int32_t n_seqs, const float *h0, void *o, float *hT, void *stream) {
  Problem p;
  int32_t st = make_problem(B, T, H_qk, H_v, d_k, d_v, dtype, q, k, v, alpha, beta, cu_seqlens,
                            n_seqs, h0, o, hT, &p);
  if (st != GDN_SUCCESS) return st;
  if (!aligned16(alpha)) return GDN_ERROR_INVALID_VALUE;
  p.per_channel = 1;
  return status_of(launch_recurrent(p, static_cast<hipStream_t>(stream)));
}

size_t gdn_kda_chunk_fwd_workspace_bytes(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k,
                                         int32_t d_v, int32_t dtype, int32_t chunk, int32_t n_seqs) {
  if (!query_ok(B, T, H_qk, H_v, d_k, d_v, dtype, chunk, n_seqs)) return 0;
  Problem p = query_problem(B, T, H_qk, H_v, d_k, d_v, dtype, chunk, n_seqs);
  p.per_channel = 1;
  return workspace_layout(p, nullptr, nullptr);
}

int32_t gdn_kda_chunk_fwd(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k, int32_t d_v,
                          int32_t dtype, const void *q, const void *k, const void *v, const float *alpha,
                          const float *beta, const int32_t *cu_seqlens, int32_t n_seqs, const float *h0,
                          void *o, float *hT, int32_t chunk, void *workspace, size_t workspace_bytes,
                          void *stream) {
  Problem p;
  int32_t st = make_problem(B, T, H_qk, H_v, d_k, d_v, dtype, q, k, v, alpha, beta, cu_seqlens,
                            n_seqs, h0, o, hT, &p);
  if (st != GDN_SUCCESS) return st;
  if (!aligned16(alpha)) return GDN_ERROR_INVALID_VALUE;
  if (chunk != 16 && chunk != 32 && chunk != 64) return GDN_ERROR_NOT_SUPPORTED;
  p.chunk = chunk;
  p.per_channel = 1;
  const size_t need = workspace_layout(p, nullptr, nullptr);
  if (!workspace || workspace_bytes < need) return GDN_ERROR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return GDN_ERROR_WORKSPACE;
  Workspace ws;
  workspace_layout(p, workspace, &ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_chunk_offsets(p, ws, s);
  if (e == hipSuccess) e = launch_kda_chunk(p, ws, s);
  return status_of(e);
}

int32_t gdn_kda_decode_step(int32_t B, int32_t H_qk, int32_t H_v, int32_t d_k, int32_t d_v,
                            int32_t dtype, const void *q, const void *k, const void *v,
                            const float *alpha, const float *beta, float *state, void *o,
                            void *stream) {
  int32_t st = check_common(B, 1, H_qk, H_v, d_k, d_v, dtype, q, k, v, alpha, beta, o);
  if (st != GDN_SUCCESS) return st;
  if ((B > 0 && !state) || !aligned16(state) || !aligned16(alpha)) return GDN_ERROR_INVALID_VALUE;
  Problem p{};
  p.B = B;
  p.T = 1;
  p.H_qk = H_qk;
  p.H_v = H_v;
  p.d_k = d_k;
  p.d_v = d_v;
  p.dtype = dtype;
  p.q = q;
  p.k = k;
  p.v = v;
  p.alpha = alpha;
  p.beta = beta;
  p.o = o;
  p.n_seqs = B;
  p.per_channel = 1;
  return status_of(launch_decode(p, state, static_cast<hipStream_t>(stream)));
}

int32_t gdn_block_prologue(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k,
                           int32_t d_v, int32_t dtype, const void *q_raw, const void *k_raw,
                           const void *v_raw, const float *conv_q, const float *conv_k,
                           const float *conv_v, const float *conv_q_bias,
                           const float *conv_k_bias, const float *conv_v_bias,
                           const float *a_raw, const float *b_raw, const float *log_A,
                           const float *v_norm_weight, float eps, float q_scale,
                           const int32_t *cu_seqlens, int32_t n_seqs, void *q, void *k, void *v,
                           float *alpha, float *beta, void *stream) {
  int32_t st = check_shapes(B, T, H_qk, H_v, d_k, d_v, dtype);
  if (st != GDN_SUCCESS) return st;
  if (!(eps >= 0.0f) || !std::isfinite(eps) || !std::isfinite(q_scale)) return GDN_ERROR_INVALID_VALUE;
  const int64_t tokens = int64_t(B) * T;
  // at most one wave per (16 tokens, head) in a one-dimensional grid, and a
  // token's row of one tensor below 2^24 bytes (32-bit buffer offsets)
  if ((tokens + kPrologueMinTokens - 1) / kPrologueMinTokens > INT32_MAX / (2 * int64_t(H_qk) + H_v))
    return GDN_ERROR_NOT_SUPPORTED;
  const int64_t elem = dtype == GDN_BF16 ? 2 : 4;
  if (int64_t(H_qk) * d_k * elem >= (1 << 24) || int64_t(H_v) * d_v * elem >= (1 << 24))
    return GDN_ERROR_NOT_SUPPORTED;
  if (cu_seqlens) {
    if (B != 1 || n_seqs < 0 || (tokens > 0 && n_seqs < 1)) return GDN_ERROR_INVALID_VALUE;
  } else if (n_seqs != 0 && n_seqs != B) {
    return GDN_ERROR_INVALID_VALUE;
  }
  if (tokens > 0 && (!q_raw || !k_raw || !v_raw || !conv_q || !conv_k || !conv_v || !a_raw || !b_raw ||
                     !log_A || !q || !k || !v || !alpha || !beta))
    return GDN_ERROR_INVALID_VALUE;
  for (const void *t : {q_raw, k_raw, v_raw, static_cast<const void *>(q), static_cast<const void *>(k),
                        static_cast<const void *>(v)})
    if (!aligned16(t)) return GDN_ERROR_INVALID_VALUE;
  BlockProblem p{};
  p.B = B;
  p.T = T;
  p.H_qk = H_qk;
  p.H_v = H_v;
  p.d_k = d_k;
  p.d_v = d_v;
  p.dtype = dtype;
  p.raw[0] = q_raw;
  p.raw[1] = k_raw;
  p.raw[2] = v_raw;
  p.out[0] = q;
  p.out[1] = k;
  p.out[2] = v;
  p.conv[0] = conv_q;
  p.conv[1] = conv_k;
  p.conv[2] = conv_v;
  p.bias[0] = conv_q_bias;
  p.bias[1] = conv_k_bias;
  p.bias[2] = conv_v_bias;
  p.a_raw = a_raw;
  p.b_raw = b_raw;
  p.log_A = log_A;
  p.norm_w = v_norm_weight;
  p.alpha = alpha;
  p.beta = beta;
  p.cu_seqlens = cu_seqlens;
  p.n_seqs = cu_seqlens ? n_seqs : B;
  p.eps = eps;
  p.q_scale = q_scale;
  return status_of(launch_block_prologue(p, static_cast<hipStream_t>(stream)));
}

int32_t gdn_block_epilogue(int32_t B, int32_t T, int32_t H_v, int32_t d_v, int32_t dtype,
                           const void *o, const void *g, const float *o_norm_weight, float eps,
                           void *y, void *stream) {
  int32_t st = check_shapes(B, T, 1, H_v, 16, d_v, dtype);
  if (st != GDN_SUCCESS) return st;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return GDN_ERROR_INVALID_VALUE;
  if (int64_t(B) * T > 0 && (!o || !g || !y)) return GDN_ERROR_INVALID_VALUE;
  if (!aligned16(o) || !aligned16(g) || !aligned16(y)) return GDN_ERROR_INVALID_VALUE;
  BlockProblem p{};
  p.B = B;
  p.T = T;
  p.H_v = H_v;
  p.d_v = d_v;
  p.dtype = dtype;
  p.raw[0] = o;
  p.raw[1] = g;
  p.out[0] = y;
  p.norm_w = o_norm_weight;
  p.eps = eps;
  return status_of(launch_block_epilogue(p, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
