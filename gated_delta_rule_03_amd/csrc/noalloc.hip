// gdn_chunk_fwd without a caller workspace: the scratch the chunked forward
// needs (chunk map, intra-chunk factors, and for the segment-parallel form
// the segment maps and entry states) lives in one file-scope device array of
// kScratchBytes per GPU, held by the library until the process ends.  For
// callers that cannot allocate device memory around a call (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation).
//
// The array's name is only a host-side stand-in: its device address is looked
// up once per device with hipGetSymbolAddress, with that device current, and
// that address is what the kernels receive.  Calls on one GPU share the
// array, so calls that overlap on one GPU (other streams, other threads) race
// on it; every byte the kernels read is written earlier in the same call, so
// nothing needs clearing between calls.
#include "../../include/gdn.h"

#include <mutex>

#include "launch.hpp"

namespace gdn {

constexpr size_t kScratchBytes = size_t(32) << 20;  // 32 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

static std::mutex scratch_mu;
static void *scratch_dev[kMaxDevices];  // device address of `scratch` on each GPU, once looked up

// The address of this GPU's copy of `scratch` (the current device's).
static hipError_t scratch_address(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return hipSuccess;
}

}  // namespace gdn

using namespace gdn;

extern "C" int32_t gdn_chunk_fwd_noalloc(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t d_k,
                                         int32_t d_v, int32_t dtype, const void *q, const void *k,
                                         const void *v, const float *alpha, const float *beta,
                                         const int32_t *cu_seqlens, int32_t n_seqs, const float *h0, void *o,
                                         float *hT, int32_t chunk, void *stream) {
  Problem p;
  int32_t st = make_problem(B, T, H_qk, H_v, d_k, d_v, dtype, q, k, v, alpha, beta, cu_seqlens, n_seqs, h0,
                            o, hT, &p);
  if (st != GDN_SUCCESS) return st;
  if (chunk != 16 && chunk != 32 && chunk != 64) return GDN_ERROR_NOT_SUPPORTED;
  p.chunk = chunk;
  const int32_t seg = plan_segment_chunks(p);
  if (chunk_workspace_bytes(p, seg) > kScratchBytes) return GDN_ERROR_WORKSPACE;
  void *ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return GDN_ERROR_LAUNCH;
  return run_chunk_fwd(p, seg, ws, kScratchBytes, static_cast<hipStream_t>(stream));
}
