// Inter-chunk state scan with the chunk output fused in.
//
// Only the boundary state passes from one chunk to the next ("From KV Cache
// to a State Matrix", section "Chunkwise training for DeltaNet"; "Attention
// as Matrix Algebra", section 5.1 and section 8).  For each chunk, from the
// state S at its start and the intra-chunk factors T, P, Ktilde^T:
//
//   Y = K S                      (d_k contraction)
//   U = T (V - diag(gamma) Y)    pseudo-values
//   O = diag(gamma) (Q S) + P U  the chunk's outputs
//   S <- gamma_C S + Ktilde^T U
//
// One wavefront owns 16 columns of the state (a d_k x 16 slice, fp32, in
// MFMA accumulator registers) for one (sequence, value head) and walks that
// sequence's chunks in order.  The delta-rule update acts on each value
// column separately ("Attention as Matrix Algebra", section 7.2: each write
// moves a column along the key only), so the column slices are independent.
// The accumulator layout of two stacked 16 x 16 tiles is the B-fragment
// layout, so Y, U and S feed the next product from registers.
//
// Launch: one 64-lane block per (unit, 16-column block).  Blocks of one unit
// are numbered so that they share blockIdx mod 8, i.e. they land on the same
// XCD and share its L2 for K, Q, T, P and Ktilde^T.
#include "launch.hpp"
#include "stage.hpp"

namespace gdn {

template <typename T>
struct ScanArgs {
  const T *q, *k, *v;
  const float *g;
  const T *entries;
  const float *h0;
  T *o;
  float *hT;
  int H_qk, H_v, d_k, d_v, group, n_units, n_colblk;
  SeqGeom geo;
};

template <typename T>
__global__ __launch_bounds__(64) void scan_kernel(ScanArgs<T> a) {
  const int lane = threadIdx.x;
  // XCD-aware decode: unit u's column blocks share bid % 8.
  const int per_group = 8 * a.n_colblk;
  const int bid = blockIdx.x;
  const int grp = bid / per_group, rem = bid - grp * per_group;
  const int cb = rem >> 3, u = grp * 8 + (rem & 7);
  if (u >= a.n_units) return;
  const int s = u / a.H_v, h = u - s * a.H_v, hq = h / a.group;
  const int col = 16 * cb + (lane & 15);  // this lane's state column
  const int nkt = a.d_k >> 4;             // 16-row tiles of the state

  // ---- state slice: S[rt] holds rows 16 rt + 4 (lane >> 4) + e, column col ----
  f32x4_t S[8];
  const int64_t st_base = (int64_t(s) * a.H_v + h) * a.d_k * a.d_v;
#pragma unroll
  for (int rt = 0; rt < 8; ++rt) {
    S[rt] = zero4();
    if (rt < nkt && a.h0) {
      for (int e = 0; e < 4; ++e) {
        const int m = 16 * rt + 4 * (lane >> 4) + e;
        S[rt][e] = a.h0[st_base + int64_t(m) * a.d_v + col];
      }
    }
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
    const T *entry = a.entries + (int64_t(c) * a.H_v + h) * kEntryElems;

    // gate of slot `lane` (padded slots repeat the last token's gate)
    const float gl = a.g[int64_t(tok0 + min(lane, len - 1)) * a.H_v + h];
    const float g_last = __shfl(gl, 63);
    const float gamma_C = exp2f(g_last);
    float gam[4][4];  // gamma of the rows this lane holds in a 64-row tile set
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) gam[rt][e] = exp2f(__shfl(gl, 16 * rt + 4 * (lane >> 4) + e));

    // state as B fragments (d_k contraction blocks of 32)
    Frag<T> Sf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) Sf[kk] = frag_from_acc<T>(S[2 * kk], S[2 * kk + 1]);
    const int nkb = (a.d_k + 31) >> 5;

    // ---- Y = K S,  OQ = Q S ----
    f32x4_t Y[4], OQ[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      Y[rt] = zero4();
      OQ[rt] = zero4();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (kk < nkb) {
          Frag<T> fk = load_row_frag(kb, qk_stride, 16 * rt + (lane & 15), len, 32 * kk, a.d_k, lane);
          Frag<T> fq = load_row_frag(qb, qk_stride, 16 * rt + (lane & 15), len, 32 * kk, a.d_k, lane);
          Y[rt] = mfma(fk, Sf[kk], Y[rt]);
          OQ[rt] = mfma(fq, Sf[kk], OQ[rt]);
        }
      }
    }

    // ---- X = V - gamma Y ----
    f32x4_t X[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * rt + 4 * (lane >> 4) + e;
        const float vv = t < len ? to_f32(vb[int64_t(t) * v_stride]) : 0.0f;
        X[rt][e] = vv - gam[rt][e] * Y[rt][e];
      }

    // ---- U = T X ----
    Frag<T> Xf[2];
    Xf[0] = frag_from_acc<T>(X[0], X[1]);
    Xf[1] = frag_from_acc<T>(X[2], X[3]);
    f32x4_t Uacc[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      Uacc[rt] = zero4();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        Uacc[rt] = mfma(load_frag(entry + (rt * 2 + kk) * kFragElems, lane), Xf[kk], Uacc[rt]);
    }
    Frag<T> Uf[2];
    Uf[0] = frag_from_acc<T>(Uacc[0], Uacc[1]);
    Uf[1] = frag_from_acc<T>(Uacc[2], Uacc[3]);

    // ---- O = gamma (Q S) + P U ----
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f32x4_t acc;
      for (int e = 0; e < 4; ++e) acc[e] = gam[rt][e] * OQ[rt][e];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        acc = mfma(load_frag(entry + (8 + rt * 2 + kk) * kFragElems, lane), Uf[kk], acc);
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * rt + 4 * (lane >> 4) + e;
        if (t < len) a.o[int64_t(tok0 + t) * v_stride + int64_t(h) * a.d_v + col] = from_f32<T>(acc[e]);
      }
    }

    // ---- S <- gamma_C S + Ktilde^T U ----
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) {
      if (rt < nkt) {
        f32x4_t acc;
        for (int e = 0; e < 4; ++e) acc[e] = gamma_C * S[rt][e];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          acc = mfma(load_frag(entry + (16 + rt * 2 + kk) * kFragElems, lane), Uf[kk], acc);
        S[rt] = acc;
      }
    }
  }

  if (a.hT) {
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) {
      if (rt < nkt) {
        for (int e = 0; e < 4; ++e) {
          const int m = 16 * rt + 4 * (lane >> 4) + e;
          a.hT[st_base + int64_t(m) * a.d_v + col] = S[rt][e];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Pipelined variant for bf16 with d_k = 128 and d_v a multiple of 32.
//
// Two waves per block own 32 state columns (16 each).  A chunk's operands --
// the k and q rows (swizzled row tiles), the 32 fragments T, P, Ktilde^T, the
// 64 x 32 block of v and the 64 gates -- are copied into an LDS stage with
// global_load_lds while the previous chunk is computed from the other stage,
// so the sequential chunk chain never waits on global memory.  Rows past a
// partial chunk repeat its last row (finite filler that meets exact zeros).
// ---------------------------------------------------------------------------
constexpr int kStageK = 0;                       // 64 x 128 bf16
constexpr int kStageQ = 16384;                   // 64 x 128 bf16
constexpr int kStageF = 32768;                   // 32 fragments x 1 KiB
constexpr int kStageV = 65536;                   // 64 x 32 bf16
constexpr int kStageG = 69632;                   // 64 fp32
constexpr int kStageBytes = 69888;

__device__ __forceinline__ int vtile_off(int row, int col) {
  // 64 rows x 32 bf16 (64 B per row); 16-byte chunks swizzled by row / 4 so
  // the four row groups of an accumulator tile read different banks.
  return row * 32 + 8 * ((col >> 3) ^ ((row >> 2) & 3)) + (col & 7);
}

__global__ __launch_bounds__(128) void scan_kernel_staged(ScanArgs<bf16_t> a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kStageBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int per_group = 8 * a.n_colblk;  // n_colblk = d_v / 32
  const int bid = blockIdx.x;
  const int grp = bid / per_group, rem = bid - grp * per_group;
  const int cb = rem >> 3, u = grp * 8 + (rem & 7);
  if (u >= a.n_units) return;
  const int s = u / a.H_v, h = u - s * a.H_v, hq = h / a.group;
  const int wcol = 16 * wave + (lane & 15);  // column inside the block's 32
  const int col = 32 * cb + wcol;            // state column

  f32x4_t S[8];
  const int64_t st_base = (int64_t(s) * a.H_v + h) * 128 * a.d_v;
#pragma unroll
  for (int rt = 0; rt < 8; ++rt) {
    S[rt] = zero4();
    if (a.h0)
      for (int e = 0; e < 4; ++e)
        S[rt][e] = a.h0[st_base + int64_t(16 * rt + 4 * (lane >> 4) + e) * a.d_v + col];
  }

  int start, end;
  a.geo.seq_bounds(s, start, end);
  const int C = a.geo.chunk;
  const int n_chunks = (end - start + C - 1) / C;
  const int c_first = a.geo.first_chunk(s);
  const int64_t qk_stride = int64_t(a.H_qk) * 128;
  const int64_t v_stride = int64_t(a.H_v) * a.d_v;

  auto stage = [&](int cc, int buf) {
    const int c = c_first + cc;
    const int tok0 = start + cc * C;
    const int len = min(C, end - tok0);
    char *base = smem + buf * kStageBytes;
    const bf16_t *entry = a.entries + (int64_t(c) * a.H_v + h) * kEntryElems;
    if (wave == 0) {
      stage_rowtile(reinterpret_cast<bf16_t *>(base + kStageK),
                    a.k + int64_t(tok0) * qk_stride + int64_t(hq) * 128, qk_stride, len, lane, 0,
                    16);
      for (int f = 0; f < 16; ++f)
        copy16_to_lds(entry + f * kFragElems + 8 * lane, base + kStageF + 1024 * f);
      copy4_to_lds(a.g + int64_t(tok0 + min(lane, len - 1)) * a.H_v + h, base + kStageG);
    } else {
      stage_rowtile(reinterpret_cast<bf16_t *>(base + kStageQ),
                    a.q + int64_t(tok0) * qk_stride + int64_t(hq) * 128, qk_stride, len, lane, 0,
                    16);
      for (int f = 16; f < 32; ++f)
        copy16_to_lds(entry + f * kFragElems + 8 * lane, base + kStageF + 1024 * f);
    }
    // v block: 4 pieces of 16 rows x 32 columns, two per wave
    for (int i = 2 * wave; i < 2 * wave + 2; ++i) {
      const int row = 16 * i + (lane >> 2);
      const int logical = (lane & 3) ^ ((row >> 2) & 3);
      const int r = row < len ? row : len - 1;
      copy16_to_lds(a.v + int64_t(tok0 + r) * v_stride + int64_t(h) * a.d_v + 32 * cb + 8 * logical,
                    base + kStageV + 1024 * i);
    }
  };

  const bool any = n_chunks > 0 && c_first < a.geo.n_slots;
  if (any) stage(0, 0);
  wait_vmem();
  __syncthreads();

  for (int cc = 0; cc < n_chunks; ++cc) {
    const int c = c_first + cc;
    if (c >= a.geo.n_slots) break;
    const int buf = cc & 1;
    if (cc + 1 < n_chunks && c + 1 < a.geo.n_slots) stage(cc + 1, buf ^ 1);

    const char *base = smem + buf * kStageBytes;
    const bf16_t *sK = reinterpret_cast<const bf16_t *>(base + kStageK);
    const bf16_t *sQ = reinterpret_cast<const bf16_t *>(base + kStageQ);
    const bf16_t *sF = reinterpret_cast<const bf16_t *>(base + kStageF);
    const bf16_t *sV = reinterpret_cast<const bf16_t *>(base + kStageV);
    const float *sG = reinterpret_cast<const float *>(base + kStageG);
    const int tok0 = start + cc * C;
    const int len = min(C, end - tok0);

    const float gamma_C = exp2f(sG[63]);
    float gam[4][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) gam[rt][e] = exp2f(sG[16 * rt + 4 * (lane >> 4) + e]);

    Frag<bf16_t> Sf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) Sf[kk] = frag_from_acc<bf16_t>(S[2 * kk], S[2 * kk + 1]);

    // Y = K S, OQ = Q S
    f32x4_t Y[4], OQ[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      Y[rt] = zero4();
      OQ[rt] = zero4();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        Y[rt] = mfma(rowtile_frag(sK, rt, kk, lane), Sf[kk], Y[rt]);
        OQ[rt] = mfma(rowtile_frag(sQ, rt, kk, lane), Sf[kk], OQ[rt]);
      }
    }
    // X = V - gamma Y
    f32x4_t X[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * rt + 4 * (lane >> 4) + e;
        X[rt][e] = to_f32(sV[vtile_off(t, wcol)]) - gam[rt][e] * Y[rt][e];
      }
    // U = T X
    Frag<bf16_t> Xf[2];
    Xf[0] = frag_from_acc<bf16_t>(X[0], X[1]);
    Xf[1] = frag_from_acc<bf16_t>(X[2], X[3]);
    f32x4_t Ua[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      Ua[rt] = zero4();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        Ua[rt] = mfma(load_frag(sF + (rt * 2 + kk) * kFragElems, lane), Xf[kk], Ua[rt]);
    }
    Frag<bf16_t> Uf[2];
    Uf[0] = frag_from_acc<bf16_t>(Ua[0], Ua[1]);
    Uf[1] = frag_from_acc<bf16_t>(Ua[2], Ua[3]);
    // O = gamma (Q S) + P U
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f32x4_t acc;
      for (int e = 0; e < 4; ++e) acc[e] = gam[rt][e] * OQ[rt][e];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        acc = mfma(load_frag(sF + (8 + rt * 2 + kk) * kFragElems, lane), Uf[kk], acc);
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * rt + 4 * (lane >> 4) + e;
        if (t < len)
          a.o[int64_t(tok0 + t) * v_stride + int64_t(h) * a.d_v + col] = from_f32<bf16_t>(acc[e]);
      }
    }
    // S <- gamma_C S + Ktilde^T U
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) {
      f32x4_t acc;
      for (int e = 0; e < 4; ++e) acc[e] = gamma_C * S[rt][e];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        acc = mfma(load_frag(sF + (16 + rt * 2 + kk) * kFragElems, lane), Uf[kk], acc);
      S[rt] = acc;
    }
    wait_vmem();
    __syncthreads();
  }

  if (a.hT) {
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
      for (int e = 0; e < 4; ++e)
        a.hT[st_base + int64_t(16 * rt + 4 * (lane >> 4) + e) * a.d_v + col] = S[rt][e];
  }
}

template <typename T>
static hipError_t launch_scan_t(const Problem &p, const Workspace &ws, hipStream_t st) {
  ScanArgs<T> a;
  a.q = static_cast<const T *>(p.q);
  a.k = static_cast<const T *>(p.k);
  a.v = static_cast<const T *>(p.v);
  a.g = ws.g;
  a.entries = static_cast<const T *>(ws.entries);
  a.h0 = p.h0;
  a.o = static_cast<T *>(p.o);
  a.hT = p.hT;
  a.H_qk = p.H_qk;
  a.H_v = p.H_v;
  a.d_k = p.d_k;
  a.d_v = p.d_v;
  a.group = p.H_v / p.H_qk;
  a.n_units = p.n_seqs * p.H_v;
  a.n_colblk = p.d_v / 16;
  a.geo = make_geom(p, &ws);
  const int64_t groups = (int64_t(a.n_units) + 7) / 8;
  const int64_t blocks = groups * 8 * a.n_colblk;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(scan_kernel<T>, dim3(unsigned(blocks)), dim3(64), 0, st, a);
  return hipGetLastError();
}

static hipError_t launch_scan_staged(const Problem &p, const Workspace &ws, hipStream_t st) {
  ScanArgs<bf16_t> a;
  a.q = static_cast<const bf16_t *>(p.q);
  a.k = static_cast<const bf16_t *>(p.k);
  a.v = static_cast<const bf16_t *>(p.v);
  a.g = ws.g;
  a.entries = static_cast<const bf16_t *>(ws.entries);
  a.h0 = p.h0;
  a.o = static_cast<bf16_t *>(p.o);
  a.hT = p.hT;
  a.H_qk = p.H_qk;
  a.H_v = p.H_v;
  a.d_k = p.d_k;
  a.d_v = p.d_v;
  a.group = p.H_v / p.H_qk;
  a.n_units = p.n_seqs * p.H_v;
  a.n_colblk = p.d_v / 32;
  a.geo = make_geom(p, &ws);
  const int64_t groups = (int64_t(a.n_units) + 7) / 8;
  const int64_t blocks = groups * 8 * a.n_colblk;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(scan_kernel_staged, dim3(unsigned(blocks)), dim3(128), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_scan(const Problem &p, const Workspace &ws, hipStream_t st) {
  if (p.dtype == 1 && p.d_k == 128 && p.d_v % 32 == 0) return launch_scan_staged(p, ws, st);
  return p.dtype == 1 ? launch_scan_t<bf16_t>(p, ws, st) : launch_scan_t<float>(p, ws, st);
}

}  // namespace gdn
