// Internal launchers of the libgdn kernels (host side).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"

namespace gdn {

struct Problem {
  int32_t B, T, H_qk, H_v, d_k, d_v, dtype;
  const void *q, *k, *v;
  const float *alpha, *beta;
  const int32_t *cu_seqlens;
  int32_t n_seqs;  // sequences (B for a uniform batch)
  const float *h0;
  void *o;
  float *hT;
  int32_t chunk;
  int32_t per_channel = 0;  // alpha holds one rate per key channel: [.., H_v, d_k]
  int64_t n_tokens() const { return int64_t(B) * T; }
};

// Chunk slots reserved for a problem: an upper bound on the number of chunks
// for any packed layout with the same totals.
int64_t chunk_slots(const Problem &p);

// One workspace entry per (chunk slot, value head) holds the intra-chunk
// factors of that chunk; its layout depends on the path (below).  Factors in
// MFMA fragment order are fragments of 64 lanes x 8 elements of the operand
// type.  A gate block holds fp32 gamma_t = 2^g_t for the 64 slots, then
// s_t = 2^(g_C - g_t), then g_t.  (g_t is the chunk-local cumulative log2
// gate; padded slots repeat the last token's gate, so gamma_63 = gamma_C and
// s = 1 there.)
constexpr int kFragElems = 64 * 8;

// The staged path: bf16 operands, d_k = 128, d_v a multiple of 32 (the factor
// kernel and the staged scan).  The scan forms P itself, and T's zeros are
// left out: the two all-zero fragments (rows 0-31, columns 32-63) entirely,
// and the zero halves of the two diagonal fragments 0 and 5 (t_entry_byte,
// tile_index.hpp).  An entry is 5,888 bytes: 5 KiB of T, then the gate
// block without its padding (gamma, s, g: 768 bytes; 23 x 256 bytes in all).
inline bool staged_path(const Problem &p) { return p.dtype == 1 && p.d_k == 128 && p.d_v % 32 == 0; }
constexpr int kStagedGateOffset = 5 * 1024;
constexpr int kStagedGateBytes = 3 * 64 * 4;
constexpr int64_t kStagedEntryBytes = kStagedGateOffset + kStagedGateBytes;
// Per-channel gate (kda_chunk.hip): 64 fragments (T, P, Khat, Qhat, Ktil^T)
// then Gamma_C, 128 fp32.
constexpr int kKdaFrags = 64;
template <typename T> constexpr int64_t kda_entry_bytes() {
  return int64_t(kKdaFrags) * kFragElems * sizeof(T) + 128 * 4;
}
// The chained path (launch_chain_fwd, bwd.hip): every scalar-gate chunked
// forward off the staged path (fp32 inputs, d_k < 128, or d_v not a multiple
// of 32), one-pass and segmented.  Its entry holds M = (I + A)^-1 and P in
// fp32 (C x C each, row-major) and a 256-float gate block: the head of a
// backward entry.
inline bool chain_path(const Problem &p) { return !p.per_channel && !staged_path(p); }
constexpr int64_t chain_entry_bytes(int C) { return (int64_t(2) * C * C + 256) * 4; }
inline int64_t entry_stride(const Problem &p) {
  if (p.per_channel) return p.dtype == 1 ? kda_entry_bytes<uint16_t>() : kda_entry_bytes<float>();
  if (staged_path(p)) return kStagedEntryBytes;
  return chain_entry_bytes(p.chunk);
}

struct Workspace {
  int32_t *chunk_off;  // [n_seqs + 1] chunk prefix sums (packed batches)
  int32_t *seq_order;  // [n_seqs] sequences, most chunks first (packed batches)
  void *entries;       // [chunk_slots, H_v] entries
};
size_t workspace_layout(const Problem &p, void *base, Workspace *ws);

hipError_t launch_chunk_offsets(const Problem &p, const Workspace &ws, hipStream_t st);
hipError_t launch_prep(const Problem &p, const Workspace &ws, hipStream_t st);
hipError_t launch_scan(const Problem &p, const Workspace &ws, hipStream_t st, float *mb = nullptr);
hipError_t launch_recurrent(const Problem &p, hipStream_t st);

// Backward pass of the chunked form (bwd.hip).
struct BwdProblem {
  Problem p;             // the forward problem (its o and hT are unused)
  Workspace ws;          // chunk offsets of a packed batch
  const void *d_o;       // dL/do, [tokens, H_v, d_v] in the input dtype
  const float *dhT;      // dL/dS_T or null
  float *entries;        // [chunk slots * H_v] per-chunk intermediates, bwd_entry_floats each
  float *dq_part, *dk_part;  // [tokens, H_v, d_k]: per value head (grouped heads only)
  float *dq, *dk, *dv, *dalpha, *dbeta, *dh0;
};
size_t bwd_entry_floats(int chunk, int d_k, int d_v);
hipError_t launch_chunk_bwd(const BwdProblem &b, hipStream_t st);
// The chained forward (chain_path problems): with factors, the per-chunk
// factors first; then one block per (unit, 16 or 32 columns) walking the
// chunks with the state in MFMA accumulators and writing o (and hT), or, with
// mb, the transition pass of the segment-parallel form (each unit's [B | M]
// into mb, [units, d_k, d_v + d_k]).
hipError_t launch_chain_fwd(const Problem &p, const Workspace &ws, hipStream_t st, float *mb = nullptr,
                            bool factors = true);
hipError_t launch_kda_chunk(const Problem &p, const Workspace &ws, hipStream_t st);
// Segment-parallel path (seqmap.hip, fold.hip).
hipError_t launch_segment_map(const Problem &p, int seg_tokens, int n_seg_bound, int32_t *seg_cu,
                              int32_t *seg_first, hipStream_t st);
hipError_t launch_fold(const float *mb, const float *h0, float *s_in, float *hT, const int32_t *seg_first,
                       int n_seqs, int n_segs, int H_v, int d_k, int d_v, hipStream_t st);

// The block prologue and epilogue (block.hip).  Prologue: raw = q_raw, k_raw,
// v_raw and out = q, k, v; epilogue: raw[0] = o, raw[1] = the output gate's
// projection, out[0] = y.
struct BlockProblem {
  int32_t B, T, H_qk, H_v, d_k, d_v, dtype;
  const void *raw[3];
  void *out[3];
  const float *conv[3], *bias[3];
  const float *a_raw, *b_raw, *log_A, *norm_w;
  float *alpha, *beta;
  const int32_t *cu_seqlens;
  int32_t n_seqs;
  float eps, q_scale;
};
constexpr int kPrologueMinTokens = 16;  // tokens per prologue wave, at least (a bound for the grid size)
hipError_t launch_block_prologue(const BlockProblem &p, hipStream_t st);
hipError_t launch_block_epilogue(const BlockProblem &p, hipStream_t st);
hipError_t launch_decode(const Problem &p, float *state, hipStream_t st);

SeqGeom make_geom(const Problem &p, const Workspace *ws);

// Host-side steps of the chunked forward shared by its entry points (api.hip).
int32_t make_problem(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k, int32_t d_v, int32_t dtype,
                     const void *q, const void *k, const void *v, const float *alpha, const float *beta,
                     const int32_t *cu_seqlens, int32_t n_seqs, const float *h0, void *o, float *hT,
                     Problem *p);
int32_t plan_segment_chunks(const Problem &p);
size_t chunk_workspace_bytes(const Problem &p, int32_t seg_chunks);
int32_t run_chunk_fwd(Problem p, int32_t seg_chunks, void *workspace, size_t workspace_bytes, hipStream_t s);

}  // namespace gdn
