// Segment-parallel chunked forward, the fold.
//
// A long sequence is cut into segments that the scan runs as independent
// units.  The delta rule is linear in the state and the values, so a
// segment's effect on the state is an affine map S_out = M S_in + B: chunk
// updates compose into one ("From KV Cache to a State Matrix", section
// "Chunkwise training for DeltaNet"; the prefix-product structure of
// "Attention as Matrix Algebra", section 8).  The transition-mode scan leaves
// B (the segment's final state from zero) and M (d_k x d_k) per (segment,
// value head).  This kernel walks each (sequence, value head)'s segments in
// order: the state entering segment j is written out for the output pass,
// then S <- M_j S + B_j; after the last segment S is the sequence's final
// state.
//
// One block per (sequence, value head, 16 state columns), one wave per 16
// state rows.  Each step is a d_k x d_k by d_k x 16 product on fp32 MFMA
// (v_mfma_f32_16x16x4f32), so the fold carries full fp32 precision.  The
// current state sits in LDS, transposed (16 columns x d_k rows, padded), so
// that a lane reads its four contraction values with one 16-byte read.
#include "launch.hpp"
#include "stage.hpp"

namespace gdn {

struct FoldArgs {
  const float *mb;            // [n_segs, H_v, d_k, d_v + d_k]: B, then M
  const float *h0;            // [n_seqs, H_v, d_k, d_v] or null (zeros)
  float *s_in;                // [n_segs, H_v, d_k, d_v]: the state entering each segment
  float *hT;                  // [n_seqs, H_v, d_k, d_v] or null
  const int32_t *seg_first;   // [n_seqs + 1]: segments of sequence s are seg_first[s] .. seg_first[s + 1] - 1
  int n_seqs, n_segs, H_v, d_k, d_v;  // n_segs: segment slots of mb and s_in
};

constexpr int kFoldRow = 128 + 4;  // floats per transposed row (one state column), padded

__global__ __launch_bounds__(512) void fold_kernel(FoldArgs a) {
  const int unit = blockIdx.x, ct = blockIdx.y;
  const int s = unit / a.H_v, h = unit % a.H_v;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r0 = lane & 15, g = lane >> 4;
  const int ld = a.d_v + a.d_k;
  const int nk4 = a.d_k >> 4;  // float4 groups of M per lane and step
  __shared__ __attribute__((aligned(16))) float st[2][16 * kFoldRow];

  // this lane's accumulator elements: rows 16 w + 4 g + i, column 16 ct + r0
  const int col = 16 * ct + r0;
  const int64_t unit_off = (int64_t(s) * a.H_v + h) * a.d_k * a.d_v;
  f32x4_t S;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    S[i] = a.h0 ? a.h0[unit_off + int64_t(16 * w + 4 * g + i) * a.d_v + col] : 0.0f;

  // (clamped: a malformed cu_seqlens can never index past the segment slots)
  const int j_end = min(max(a.seg_first[a.n_seqs], 0), a.n_segs);
  const int j0 = min(max(a.seg_first[s], 0), j_end);
  const int j1 = min(max(a.seg_first[s + 1], j0), j_end);
  // operands of step j: M row 16 w + r0, columns 16 m + 4 g .. + 3 (contraction
  // order: MFMA 4 m + i of a step takes index 16 m + 4 g + i in both
  // operands), and B at this lane's accumulator elements.  Three register
  // sets: the maps of the next two segments are in flight while one step runs
  // (the step's products are short next to a map's load latency).
  struct Ops {
    f32x4_t m[8], b;
  };
  auto load_step = [&](int j, Ops &r) {
    const float *base = a.mb + (int64_t(j) * a.H_v + h) * a.d_k * ld;
    const float *mrow = base + int64_t(16 * w + r0) * ld + a.d_v + 4 * g;
#pragma unroll
    for (int m = 0; m < 8; ++m)
      if (m < nk4) r.m[m] = *reinterpret_cast<const f32x4_t *>(mrow + 16 * m);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.b[i] = base[int64_t(16 * w + 4 * g + i) * ld + col];
  };
  int buf = 0;
  // S <- M_j S + B_j, after writing out the state entering segment j
  auto step = [&](int j, const Ops &r) {
    float *sin = a.s_in + (int64_t(j) * a.H_v + h) * a.d_k * a.d_v;
#pragma unroll
    for (int i = 0; i < 4; ++i) sin[int64_t(16 * w + 4 * g + i) * a.d_v + col] = S[i];
    *reinterpret_cast<f32x4_t *>(&st[buf][r0 * kFoldRow + 16 * w + 4 * g]) = S;
    __syncthreads();
    f32x4_t acc = r.b;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if (m < nk4) {
        const f32x4_t sv = *reinterpret_cast<const f32x4_t *>(&st[buf][r0 * kFoldRow + 16 * m + 4 * g]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(r.m[m][i], sv[i], acc, 0, 0, 0);
      }
    }
    S = acc;
    buf ^= 1;  // the next step writes the other buffer: no wave still reads it
  };
  Ops r0s, r1s, r2s;
  if (j0 < j1) load_step(j0, r0s);
  if (j0 + 1 < j1) load_step(j0 + 1, r1s);
  if (j0 + 2 < j1) load_step(j0 + 2, r2s);
  for (int j = j0; j < j1; j += 3) {
    step(j, r0s);
    if (j + 3 < j1) load_step(j + 3, r0s);
    if (j + 1 < j1) {
      step(j + 1, r1s);
      if (j + 4 < j1) load_step(j + 4, r1s);
    }
    if (j + 2 < j1) {
      step(j + 2, r2s);
      if (j + 5 < j1) load_step(j + 5, r2s);
    }
  }
  if (a.hT) {
#pragma unroll
    for (int i = 0; i < 4; ++i) a.hT[unit_off + int64_t(16 * w + 4 * g + i) * a.d_v + col] = S[i];
  }
}

hipError_t launch_fold(const float *mb, const float *h0, float *s_in, float *hT, const int32_t *seg_first,
                       int n_seqs, int n_segs, int H_v, int d_k, int d_v, hipStream_t st) {
  if (int64_t(n_seqs) * H_v == 0) return hipSuccess;
  FoldArgs a{mb, h0, s_in, hT, seg_first, n_seqs, n_segs, H_v, d_k, d_v};
  hipLaunchKernelGGL(fold_kernel, dim3(unsigned(n_seqs * H_v), unsigned(d_v / 16)), dim3(64 * (d_k / 16)), 0,
                     st, a);
  return hipGetLastError();
}

}  // namespace gdn
