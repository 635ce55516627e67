// Packed-batch chunk map: chunk_off[s] = number of chunks in sequences
// 0..s-1, computed on the device from cu_seqlens (no host synchronisation).
// Chunks never cross a sequence boundary and a sequence's last chunk may be
// shorter ("Attention as Matrix Algebra", section 8: chunks of C tokens with a
// shorter final chunk), so sequence s owns ceil(L_s / C) chunks.
#include "launch.hpp"

namespace gdn {

// Sequences ranked for scheduling: order[r] = the sequence with the r-th most
// chunks (ties by index).  The per-(sequence, head) scans take time in
// proportion to their chunk counts, so starting the longest first shortens
// the tail of a packed batch.  Ranked directly up to kMaxRanked sequences;
// beyond that the order is the identity.
constexpr int kMaxRanked = 1024;

// chunk_off[s] = number of chunks in sequences 0..s-1, and the scheduling
// order (packed batches).
__global__ __launch_bounds__(256) void chunk_offsets_kernel(SeqGeom geo, int32_t *off, int32_t *order) {
  __shared__ int32_t cnt_sh[kMaxRanked];
  __shared__ int32_t sh[256];
  __shared__ int32_t carry;
  const int tid = threadIdx.x;
  if (tid == 0) {
    off[0] = 0;
    carry = 0;
  }
  __syncthreads();
  for (int base = 0; base < geo.n_seqs; base += 256) {
    const int s = base + tid;
    int cnt = 0;
    if (s < geo.n_seqs) {
      int start, end;
      geo.seq_bounds(s, start, end);
      cnt = (end - start + geo.chunk - 1) / geo.chunk;
      if (s < kMaxRanked) cnt_sh[s] = cnt;
    }
    sh[tid] = cnt;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
      const int add = tid >= d ? sh[tid - d] : 0;
      __syncthreads();
      sh[tid] += add;
      __syncthreads();
    }
    if (s < geo.n_seqs) off[s + 1] = carry + sh[tid];
    __syncthreads();
    if (tid == 255) carry += sh[255];
    __syncthreads();
  }
  if (geo.n_seqs > kMaxRanked) {
    for (int s = tid; s < geo.n_seqs; s += 256) order[s] = s;
    return;
  }
  for (int s = tid; s < geo.n_seqs; s += 256) {
    const int c = cnt_sh[s];
    int rank = 0;
    for (int j = 0; j < geo.n_seqs; ++j) {
      const int cj = cnt_sh[j];
      rank += (cj > c) || (cj == c && j < s);
    }
    order[rank] = s;
  }
}

// Segment map of the segment-parallel path: every sequence is cut into
// segments of `seg_tokens` tokens (a multiple of the chunk size, so segment
// boundaries are chunk boundaries and the chunks are those of the whole
// sequence); its last segment may be shorter.  seg_first[s] = number of
// segments in sequences 0..s-1; seg_cu[i] = first token of segment i, and
// entries past the last segment hold the end of the last sequence (empty
// segments).  The segments then run as a packed batch.
__global__ __launch_bounds__(256) void segment_map_kernel(SeqGeom geo, int seg_tokens, int n_seg_bound,
                                                          int32_t *seg_cu, int32_t *seg_first) {
  __shared__ int32_t sh[256];
  __shared__ int32_t carry;
  const int tid = threadIdx.x;
  if (tid == 0) {
    seg_first[0] = 0;
    carry = 0;
  }
  __syncthreads();
  for (int base = 0; base < geo.n_seqs; base += 256) {
    const int s = base + tid;
    int cnt = 0, start = 0, end = 0;
    if (s < geo.n_seqs) {
      geo.seq_bounds(s, start, end);
      cnt = (end - start + seg_tokens - 1) / seg_tokens;
    }
    sh[tid] = cnt;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
      const int add = tid >= d ? sh[tid - d] : 0;
      __syncthreads();
      sh[tid] += add;
      __syncthreads();
    }
    if (s < geo.n_seqs) {
      const int first = carry + sh[tid] - cnt;
      seg_first[s + 1] = first + cnt;
      for (int j = 0; j < cnt && first + j < n_seg_bound; ++j) seg_cu[first + j] = start + j * seg_tokens;
    }
    __syncthreads();
    if (tid == 255) carry += sh[255];
    __syncthreads();
  }
  // the end of the last sequence closes the last segment and fills the rest
  int last_end = 0;
  if (geo.n_seqs > 0) {
    int start;
    geo.seq_bounds(geo.n_seqs - 1, start, last_end);
  }
  for (int i = min(carry, n_seg_bound) + tid; i <= n_seg_bound; i += 256) seg_cu[i] = last_end;
}

hipError_t launch_segment_map(const Problem &p, int seg_tokens, int n_seg_bound, int32_t *seg_cu,
                              int32_t *seg_first, hipStream_t st) {
  SeqGeom geo = make_geom(p, nullptr);
  hipLaunchKernelGGL(segment_map_kernel, dim3(1), dim3(256), 0, st, geo, seg_tokens, n_seg_bound, seg_cu,
                     seg_first);
  return hipGetLastError();
}

hipError_t launch_chunk_offsets(const Problem &p, const Workspace &ws, hipStream_t st) {
  if (!p.cu_seqlens) return hipSuccess;
  SeqGeom geo = make_geom(p, &ws);
  hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(256), 0, st, geo, ws.chunk_off, ws.seq_order);
  return hipGetLastError();
}

}  // namespace gdn
