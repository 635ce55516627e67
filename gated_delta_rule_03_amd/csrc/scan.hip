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

hipError_t launch_scan(const Problem &p, const Workspace &ws, hipStream_t st) {
  return p.dtype == 1 ? launch_scan_t<bf16_t>(p, ws, st) : launch_scan_t<float>(p, ws, st);
}

}  // namespace gdn
