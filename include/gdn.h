/*
 * libgdn -- the gated delta rule on AMD Instinct MI355X (gfx950).
 *
 * The operation (per unit = one sequence and one value head, state S of
 * d_k x d_v, S_0 = h0 or 0), once per token t:
 *
 *   S'  = alpha_t S_{t-1}                    decay
 *   vhat = S'^T k_t                          predict from the decayed state
 *   S_t = S' + beta_t k_t (v_t - vhat)^T     correct along the key
 *   o_t = S_t^T q_t                          read after the write
 *
 * Source: "Linear attention" (arsalanzafar.ai), section "How it works",
 * Eqs. (1)-(4); the same update, transposed, is "The gated delta rule" of
 * "How linear attention works: a small memory matrix and the gated delta rule"
 * (joelfernandes.org).  There is no score scale and no normaliser: callers
 * pre-scale and L2-normalise q and k themselves.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors are dense, row-major and contiguous; there are no stride arguments.
 *   q, k     [B, T, H_qk, d_k]   element type `dtype`
 *   v, o     [B, T, H_v,  d_v]   element type `dtype`
 *   alpha, beta [B, T, H_v]      float32 (one scalar per token and value head)
 *   h0, hT, state [N, H_v, d_k, d_v] float32, d_v fastest (the state is
 *                                stored as keys x values)
 * Value head j reads query/key head (j * H_qk) / H_v: H_v must be a multiple
 * of H_qk and each query/key head serves H_v / H_qk consecutive value heads.
 * Packed (variable-length) batches: pass `cu_seqlens` (device pointer, int32,
 * n_seqs + 1 non-decreasing offsets with cu_seqlens[0] = 0 and
 * cu_seqlens[n_seqs] = T) with B == 1; the state restarts at every boundary
 * and N = n_seqs.  Otherwise pass NULL and N = B.
 * Supported sizes: d_k, d_v in {16, 32, 64, 128}; dtype GDN_F32 or GDN_BF16.
 * The state and all accumulation are float32; o is written in `dtype`.
 *
 * Alignment: q, k, v, o, h0, hT, state and the block entry points' token-major
 * tensors (q_raw, k_raw, v_raw, g, y) start at 16-byte aligned addresses
 * (they are accessed 16 bytes per lane); other pointers need only the
 * alignment of their element type.  A misaligned tensor is rejected with
 * GDN_ERROR_INVALID_VALUE.
 *
 * Ownership: every buffer is allocated by the caller and lives on the current
 * HIP device (device pointers).  The library allocates nothing, frees nothing
 * and keeps no pointer after a call returns.  Calls are asynchronous on the
 * given stream (NULL = the default stream); results are ready when the caller
 * synchronises that stream.  o must not alias any input.
 *
 * Errors: arguments are checked before anything is launched.  On an error
 * nothing is launched and no output is touched; the status says why.  A
 * failed launch returns GDN_ERROR_LAUNCH.  Execution faults surface at the
 * caller's next synchronisation.  No call keeps global mutable state; calls
 * on different streams with disjoint buffers may run concurrently.
 * Results are bitwise reproducible run to run (no atomics).
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define GDN_SUCCESS 0
#define GDN_ERROR_INVALID_VALUE 1 /* a null pointer, a negative or inconsistent size */
#define GDN_ERROR_NOT_SUPPORTED 2 /* a size or dtype outside the supported set */
#define GDN_ERROR_WORKSPACE 3     /* workspace missing or smaller than required */
#define GDN_ERROR_LAUNCH 4        /* the HIP runtime rejected a kernel launch */

/* Element types of q, k, v and o. */
#define GDN_F32 0
#define GDN_BF16 1

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t gdn_version(void);

/* A static, human-readable description of a status code (never NULL). */
const char *gdn_status_string(int32_t status);

/*
 * gdn_recurrent_fwd -- the recurrence token by token.
 *
 * Evaluates Eqs. (1)-(4) of "Linear attention" ("How it works") one token at
 * a time with the state held in registers: the direct form whose cost
 * "How linear attention works" (section "Why it is called linear attention")
 * puts at O(d_v d_k) per token.
 *
 *   h0  nullable: initial state per (sequence, value head); NULL = zeros.
 *   hT  nullable: receives the final state.
 *   cu_seqlens, n_seqs: see "Packed batches" above (NULL and 0 otherwise).
 * T == 0 (or an empty packed sequence) is allowed: hT receives h0 (or zeros).
 */
int32_t gdn_recurrent_fwd(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k,
                          int32_t d_v, int32_t dtype, const void *q, const void *k, const void *v,
                          const float *alpha, const float *beta, const int32_t *cu_seqlens,
                          int32_t n_seqs, const float *h0, void *o, float *hT, void *stream);

/*
 * Bytes of device workspace gdn_chunk_fwd needs for these sizes (0 when the
 * arguments are unsupported).  The bound holds for every cu_seqlens with the
 * given T and n_seqs.  It includes the segment-parallel form's buffers when
 * gdn_chunk_fwd_plan_segments picks that form for these sizes.
 */
size_t gdn_chunk_fwd_workspace_bytes(int32_t B, int32_t T, int32_t H_qk, int32_t H_v,
                                     int32_t d_k, int32_t d_v, int32_t dtype, int32_t chunk,
                                     int32_t n_seqs);

/*
 * gdn_chunk_fwd -- the same result, computed chunk by chunk.
 *
 * Tokens are grouped into chunks of `chunk` tokens (16, 32 or 64; a
 * sequence's last chunk may be shorter and chunks never cross a sequence
 * boundary).  Inside a chunk one triangular solve turns the values into
 * pseudo-values and the rest is chunked linear attention; only the boundary
 * state passes from chunk to chunk ("Attention as Matrix Algebra: From
 * Softmax to the Delta Rule", section 8 "Training the delta rule in chunks";
 * "From KV Cache to a State Matrix: Linear Attention and DeltaNet", section
 * "Chunkwise training for DeltaNet"), with the decay gate of "Linear
 * attention", Eq. (1), carried as chunk-local cumulative log gates.
 *
 * Precision: bf16 inputs run the chunk products on the bf16 matrix cores
 * (operands such as the chunk's pseudo-values and the state rounded to bf16
 * where they enter a product, fp32 sums, the state kept in fp32), except in
 * the one-pass form with d_k < 128 or d_v = 16, which, like fp32 inputs,
 * keeps every product in fp32.
 *
 * Arguments as gdn_recurrent_fwd, plus:
 *   chunk       16, 32 or 64.
 *   workspace   device memory of at least gdn_chunk_fwd_workspace_bytes(...)
 *               bytes, 256-byte aligned; its contents on entry do not matter
 *               and are undefined on return.  Concurrent calls need separate
 *               workspaces.
 */
int32_t gdn_chunk_fwd(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k, int32_t d_v,
                      int32_t dtype, const void *q, const void *k, const void *v,
                      const float *alpha, const float *beta, const int32_t *cu_seqlens,
                      int32_t n_seqs, const float *h0, void *o, float *hT, int32_t chunk,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * Segment-parallel form of gdn_chunk_fwd (same result, up to rounding).
 *
 * The chunk updates of a sequence compose: the effect of a run of chunks on
 * the state is one affine map S_out = M S_in + B, because the delta rule is
 * linear in the state and the values ("From KV Cache to a State Matrix:
 * Linear Attention and DeltaNet", section "Chunkwise training for DeltaNet";
 * "Attention as Matrix Algebra", section 8).  Each sequence is cut into
 * segments of `seg_chunks` chunks (its last segment may be shorter); the
 * segments are scanned as independent units for their maps (B from a zero
 * state, M from the identity with the values set to zero), the maps are
 * folded in sequence order in fp32 (the state entering each segment, and the
 * final state), and the segments are scanned again from those states for the
 * outputs.  This spreads a problem with few (sequence, value head) units --
 * a long single sequence -- over the whole GPU, at about three times the
 * scan work.  gdn_chunk_fwd takes this form by itself when the one-pass scan
 * would keep fewer than half of the GPU's compute units busy.
 *
 * gdn_chunk_fwd_plan_segments: the segment length gdn_chunk_fwd uses for these
 *   sizes, in chunks (0 = one pass; -1 = unsupported arguments).
 * gdn_chunk_fwd_segmented_workspace_bytes: workspace bytes of
 *   gdn_chunk_fwd_segmented for the given seg_chunks (0 = unsupported).
 *   gdn_chunk_fwd_workspace_bytes is this value for the planned length.
 * gdn_chunk_fwd_segmented: arguments as gdn_chunk_fwd, plus
 *   seg_chunks  chunks per segment, >= 0 (0 = one pass, as gdn_chunk_fwd
 *               without segments).  GDN_ERROR_INVALID_VALUE when negative;
 *               GDN_ERROR_NOT_SUPPORTED when a segment would exceed 2^31 - 1
 *               tokens or the batch would need 2^30 segments or more.
 */
int32_t gdn_chunk_fwd_plan_segments(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k,
                                    int32_t d_v, int32_t dtype, int32_t chunk, int32_t n_seqs);
size_t gdn_chunk_fwd_segmented_workspace_bytes(int32_t B, int32_t T, int32_t H_qk, int32_t H_v,
                                               int32_t d_k, int32_t d_v, int32_t dtype, int32_t chunk,
                                               int32_t n_seqs, int32_t seg_chunks);
int32_t gdn_chunk_fwd_segmented(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k, int32_t d_v,
                                int32_t dtype, const void *q, const void *k, const void *v,
                                const float *alpha, const float *beta, const int32_t *cu_seqlens,
                                int32_t n_seqs, const float *h0, void *o, float *hT, int32_t chunk,
                                int32_t seg_chunks, void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_chunk_fwd_noalloc -- gdn_chunk_fwd for callers that cannot allocate
 * device memory around a call (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same arguments without the
 * workspace, the same result.
 *
 * The scratch lives in one static device array of 32 MiB (33,554,432 bytes)
 * per GPU, held until the process ends; the call allocates and frees
 * nothing.  A problem whose gdn_chunk_fwd_workspace_bytes(...) exceeds
 * 32 MiB is rejected with GDN_ERROR_WORKSPACE before anything is launched
 * (the prefill batch B=4, T=4096, H=16, d=128 needs about 24 MB).  All calls
 * on one GPU share that array: calls that overlap on one GPU (on different
 * streams, or from different threads) race on it and must be ordered by the
 * caller.  The first call on a device looks the array's address up on that
 * device (the current one).
 */
int32_t gdn_chunk_fwd_noalloc(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k, int32_t d_v,
                              int32_t dtype, const void *q, const void *k, const void *v,
                              const float *alpha, const float *beta, const int32_t *cu_seqlens,
                              int32_t n_seqs, const float *h0, void *o, float *hT, int32_t chunk,
                              void *stream);

/*
 * gdn_chunk_bwd -- gradients of the gated delta rule for training in chunks.
 *
 * The pages motivate chunked training ("From KV Cache to a State Matrix:
 * Linear Attention and DeltaNet", section "Chunkwise training for DeltaNet";
 * "Attention as Matrix Algebra", section 8) and print no gradients; these
 * are the reverse-mode derivatives of the forward of gdn_recurrent_fwd
 * ("Linear attention", Eqs. (1)-(4)) for the loss
 *   L = sum_t <d_o_t, o_t> + <dhT, S_T>   (per sequence and value head),
 * evaluated in the chunk form, in fp32: the chunk-start states and the
 * gradients reaching each chunk's end are carried chunk to chunk, and every
 * chunk's gradients then follow independently.  With bf16 inputs the
 * products whose other factor is an input (k, q or d_o, exact in bf16) take
 * their fp32 factor split as hi + lo in bf16 (about 16 significant bits) on
 * the bf16 matrix cores; every other product is fp32.  Deterministic (no atomics):
 * two calls on the same inputs give bitwise equal results.
 *
 * Inputs as gdn_chunk_fwd (q, k, v, alpha, beta, cu_seqlens, n_seqs, h0,
 * chunk, workspace), plus:
 *   d_o    dL/do, [B, T, H_v, d_v] in the input dtype (required when T > 0).
 *   dhT    dL/dS_T, [N, H_v, d_k, d_v] fp32, or NULL (zero).
 * Outputs, all fp32 and written in full:
 *   dq, dk     [B, T, H_qk, d_k]: summed over the value heads that read each
 *              query/key head (v head j reads qk head floor(j H_qk / H_v)).
 *   dv         [B, T, H_v, d_v].
 *   dalpha     [B, T, H_v]: dL/dalpha, computed as dL/d(ln alpha) / alpha, so
 *              alpha must be > 0 for a finite result.
 *   dbeta      [B, T, H_v].
 *   dh0        [N, H_v, d_k, d_v], or NULL (not written).
 * gdn_chunk_bwd_workspace_bytes gives the workspace bytes (0 = unsupported
 * arguments): per (chunk slot, value head) 3 C^2 + 256 + 2 d_k d_v + 2 C d_v
 * floats of intermediates (0.94 GiB for B=4, T=4096, H=16, d=128, C=64),
 * plus the per-value-head dq and dk when H_v > H_qk.  The caller owns the
 * workspace; it must be 256-byte aligned (else GDN_ERROR_WORKSPACE), and
 * nothing in it is needed after the call.
 * Errors as gdn_chunk_fwd; GDN_ERROR_INVALID_VALUE when an output is NULL
 * for a non-empty batch or a pointer is misaligned.
 */
size_t gdn_chunk_bwd_workspace_bytes(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k,
                                     int32_t d_v, int32_t dtype, int32_t chunk, int32_t n_seqs);
int32_t gdn_chunk_bwd(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k, int32_t d_v, int32_t dtype,
                      const void *q, const void *k, const void *v, const float *alpha, const float *beta,
                      const int32_t *cu_seqlens, int32_t n_seqs, const float *h0, const void *d_o,
                      const float *dhT, float *dq, float *dk, float *dv, float *dalpha, float *dbeta, float *dh0,
                      int32_t chunk, void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_decode_step -- one new token per sequence, state updated in place.
 *
 * The generation step of "Attention as Matrix Algebra" (section 9: about 6rd
 * operations and rd numbers of state per step and head) for the gated rule:
 * with S the stored state, a = S^T k, b = S^T q, vhat = alpha a,
 * u = beta (v - vhat), o = alpha b + (q^T k) u and S <- alpha S + k u^T.
 *
 *   q, k   [B, 1, H_qk, d_k];  v, o [B, 1, H_v, d_v];  alpha, beta [B, 1, H_v]
 *   state  [B, H_v, d_k, d_v] float32, read and overwritten in place.
 */
int32_t gdn_decode_step(int32_t B, int32_t H_qk, int32_t H_v, int32_t d_k, int32_t d_v,
                        int32_t dtype, const void *q, const void *k, const void *v,
                        const float *alpha, const float *beta, float *state, void *o,
                        void *stream);

/*
 * Per-channel gate (Kimi Delta Attention: "Attention as Matrix Algebra",
 * section 10, gives each feature channel its own forget rate).  The channels
 * are the key features, the rows of the keys x values state, so the decay of
 * step t is diag(alpha_t) with alpha_t in R^{d_k}; the rest of the update is
 * unchanged:
 *
 *   S' = diag(alpha_t) S_{t-1};  vhat = S'^T k_t;
 *   S_t = S' + beta_t k_t (v_t - vhat)^T;  o_t = S_t^T q_t
 *
 * gdn_kda_recurrent_fwd takes the arguments of gdn_recurrent_fwd, with
 *   alpha  [B, T, H_v, d_k] float32 (one rate per token, value head and key
 *          channel), 16-byte aligned.
 * gdn_kda_decode_step takes the arguments of gdn_decode_step, with
 *   alpha  [B, 1, H_v, d_k] float32, 16-byte aligned.
 * Errors, ownership and the state layout as for the scalar-gate entry points.
 * Equal rates across the channels give the scalar-gate results.
 */
int32_t gdn_kda_recurrent_fwd(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k,
                              int32_t d_v, int32_t dtype, const void *q, const void *k, const void *v,
                              const float *alpha, const float *beta, const int32_t *cu_seqlens,
                              int32_t n_seqs, const float *h0, void *o, float *hT, void *stream);

/*
 * gdn_kda_chunk_fwd -- the per-channel-gate forward computed chunk by chunk
 * (the same result as gdn_kda_recurrent_fwd, up to rounding).
 *
 * The chunk algebra of "Attention as Matrix Algebra" section 8 with the
 * scalar cumulative gate replaced by one per key channel: with
 * G_t = sum_{i<=t} log alpha_i inside the chunk (a vector over channels),
 *   A_ti = beta_t sum_c k_tc k_ic e^(G_tc - G_ic) (i < t),  T = (I + A)^-1 diag(beta),
 *   U = T (V - (e^G . K) S),  O = (e^G . Q) S + P U,  P_ti = sum_c q_tc k_ic e^(G_tc - G_ic) (i <= t),
 *   S <- diag(e^(G_C)) S + (e^(G_C - G) . K)^T U.
 * Every factor of the state side is e to a non-positive power.  The channel
 * sums of A and P are evaluated in fp32: as (e^G . K)(e^-G . K)^T and
 * (e^G . Q)(e^-G . K)^T on matrix cores when every cumulative log2 gate of
 * the chunk lies within [-60, 60] (no factor leaves [2^-60, 2^60]), else
 * pair by pair with the exact factor e^(G_tc - G_ic).
 *
 * Arguments as gdn_kda_recurrent_fwd (alpha [B, T, H_v, d_k] float32,
 * 16-byte aligned), plus chunk (16, 32 or 64) and a caller-provided
 * workspace of at least gdn_kda_chunk_fwd_workspace_bytes(...) bytes,
 * 256-byte aligned (contents on entry do not matter, undefined on return;
 * concurrent calls need separate workspaces).  Errors as gdn_chunk_fwd.
 */
size_t gdn_kda_chunk_fwd_workspace_bytes(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k,
                                         int32_t d_v, int32_t dtype, int32_t chunk, int32_t n_seqs);
int32_t gdn_kda_chunk_fwd(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k, int32_t d_v,
                          int32_t dtype, const void *q, const void *k, const void *v, const float *alpha,
                          const float *beta, const int32_t *cu_seqlens, int32_t n_seqs, const float *h0,
                          void *o, float *hT, int32_t chunk, void *workspace, size_t workspace_bytes,
                          void *stream);
int32_t gdn_kda_decode_step(int32_t B, int32_t H_qk, int32_t H_v, int32_t d_k, int32_t d_v,
                            int32_t dtype, const void *q, const void *k, const void *v,
                            const float *alpha, const float *beta, float *state, void *o,
                            void *stream);

/*
 * gdn_block_prologue -- the GDN block's steps between the projections and
 * the recurrence, fused ("Linear attention", section "A naive PyTorch
 * implementation"):
 *   x <- SiLU(bias + sum_j w[c][j] x[t - 3 + j])   per channel c of q, k and v
 *       (a causal depthwise convolution of width 4; tokens before the start
 *       of t's sequence count as zeros);
 *   q <- q_scale * q / max(|q|, 1e-12),  k <- k / max(|k|, 1e-12)   per head;
 *   v <- v / sqrt(mean(v^2) + eps) * v_norm_weight                 per head;
 *   alpha = exp(-exp(log_A[h]) * log(1 + exp(a_raw))),  beta = 1 / (1 + exp(-b_raw)).
 *
 *   q_raw, k_raw   [B, T, H_qk, d_k];  v_raw [B, T, H_v, d_v]   (dtype; the
 *                  projections of the block's input)
 *   conv_q, conv_k [H_qk * d_k, 4];  conv_v [H_v * d_v, 4]      float32 taps of
 *                  each channel, oldest token first (channel = head * d + i)
 *   conv_*_bias    [H * d] float32, or NULL for none
 *   a_raw, b_raw   [B, T, H_v] float32 gate projections;  log_A [H_v] float32
 *   v_norm_weight  [d_v] float32, or NULL for ones;  eps >= 0;  q_scale finite
 *                  (1 on the page; 1/sqrt(d_k) folds the attention scale in)
 *   cu_seqlens, n_seqs   as gdn_recurrent_fwd (a packed batch needs n_seqs >= 1
 *                  when T > 0); the convolution restarts at every sequence
 *   q, k, v        outputs shaped like q_raw, k_raw, v_raw (dtype);
 *   alpha, beta    outputs [B, T, H_v] float32 -- the inputs of gdn_chunk_fwd.
 * Outputs must not alias inputs.  Errors as gdn_recurrent_fwd, plus
 * GDN_ERROR_NOT_SUPPORTED when one token's row of q, k or v (H * d elements)
 * takes 2^24 bytes or more, or the batch needs more than 2^31 waves.
 */
int32_t gdn_block_prologue(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k,
                           int32_t d_v, int32_t dtype, const void *q_raw, const void *k_raw,
                           const void *v_raw, const float *conv_q, const float *conv_k,
                           const float *conv_v, const float *conv_q_bias,
                           const float *conv_k_bias, const float *conv_v_bias,
                           const float *a_raw, const float *b_raw, const float *log_A,
                           const float *v_norm_weight, float eps, float q_scale,
                           const int32_t *cu_seqlens, int32_t n_seqs, void *q, void *k, void *v,
                           float *alpha, float *beta, void *stream);

/*
 * gdn_block_epilogue -- the GDN block's steps after the recurrence, fused
 * ("Linear attention", section "A naive PyTorch implementation"): each
 * head's output RMS-normalised, times a weight, times SiLU of the output
 * gate's projection:
 *   y = o / sqrt(mean(o^2) + eps) * o_norm_weight * g / (1 + exp(-g)).
 *
 *   o, g, y        [B, T, H_v, d_v] (dtype); g is the output gate's projection
 *   o_norm_weight  [d_v] float32, or NULL for ones;  eps >= 0
 * y must not alias o or g.  Errors as gdn_recurrent_fwd.
 */
int32_t gdn_block_epilogue(int32_t B, int32_t T, int32_t H_v, int32_t d_v, int32_t dtype,
                           const void *o, const void *g, const float *o_norm_weight, float eps,
                           void *y, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
