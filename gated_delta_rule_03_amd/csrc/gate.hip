// Chunk geometry prepass and the cumulative log-gate kernel.
//
// The decay gate alpha_t of "Linear attention" (arsalanzafar.ai), Eq. (1),
// compounds inside a chunk: the state reaching token t from the chunk start
// has been scaled by prod_{i<=t} alpha_i.  The chunk kernels use that product
// in the log domain, g_t = sum_{i<=t} log2 alpha_i (chunk-local), so every
// factor they need is exp2 of a difference g_t - g_i <= 0 for i <= t (the
// prefix-product structure of "From KV Cache to a State Matrix", section
// "Chunkwise training for DeltaNet").
#include "launch.hpp"

namespace gdn {

// chunk_off[s] = number of chunks in sequences 0..s-1 (packed batches).
__global__ __launch_bounds__(256) void chunk_offsets_kernel(SeqGeom geo, int32_t *off) {
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
}

// One block per chunk slot; thread h owns value head h of the chunk.  All of
// the chunk's alpha loads are issued before the prefix sum, and consecutive
// threads touch consecutive heads of one token (coalesced).
__device__ __forceinline__ float clamped_log2(float a) {
  // log2 alpha, clamped below; alpha = 0 hits the floor, NaN and negative
  // gates propagate as NaN.
  if (a > 0.0f) return fmaxf(log2f(a), kLog2Floor);
  if (a == 0.0f) return kLog2Floor;
  return __builtin_nanf("");
}

__global__ __launch_bounds__(256) void gate_kernel(const float *__restrict__ alpha,
                                                   float *__restrict__ g, int H, SeqGeom geo) {
  int s, tok0, len;
  if (!geo.locate(blockIdx.x, s, tok0, len)) return;
  for (int h = threadIdx.x; h < H; h += blockDim.x) {
    float l[64];
#pragma unroll
    for (int t = 0; t < 64; ++t) l[t] = t < len ? alpha[int64_t(tok0 + t) * H + h] : 1.0f;
    float acc = 0.0f;
#pragma unroll
    for (int t = 0; t < 64; ++t) {
      acc += clamped_log2(l[t]);
      if (t < len) g[int64_t(tok0 + t) * H + h] = acc;
    }
  }
}

hipError_t launch_chunk_offsets(const Problem &p, const Workspace &ws, hipStream_t st) {
  if (!p.cu_seqlens) return hipSuccess;
  SeqGeom geo = make_geom(p, &ws);
  hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(256), 0, st, geo, ws.chunk_off);
  return hipGetLastError();
}

hipError_t launch_gate(const Problem &p, const Workspace &ws, hipStream_t st) {
  const int64_t slots = chunk_slots(p);
  if (slots == 0) return hipSuccess;
  SeqGeom geo = make_geom(p, &ws);
  hipLaunchKernelGGL(gate_kernel, dim3(unsigned(slots)), dim3(256), 0, st, p.alpha, ws.g, p.H_v,
                     geo);
  return hipGetLastError();
}

}  // namespace gdn
