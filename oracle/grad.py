"""Float64 gradients of the gated delta rule's token loop (test infrastructure).

TEST INFRASTRUCTURE ONLY, like the rest of this package: the tests, the
smoke check and the benchmark's CPU baseline are the only callers.

The pages motivate training in chunks ("From KV Cache to a State Matrix",
section "Chunkwise training for DeltaNet"; "Attention as Matrix Algebra",
section 8) but print no gradients.  This module differentiates the token
loop of "Linear attention" (arsalanzafar.ai), section "How it works",
Eqs. (1)-(4), by reverse-mode accumulation, one token at a time in reverse:

  forward, per unit and token t:
    S'  = alpha_t S_{t-1}                 (1)
    e_t = v_t - S'^T k_t                  (2)  the prediction error
    S_t = S' + beta_t k_t e_t^T           (3)
    o_t = S_t^T q_t                       (4)

  given upstream gradients do_t = dL/do_t and dhT = dL/dS_T, with
  D = dL/dS_t carried backwards from D = dhT:
    (4)  D     += q_t do_t^T,        dq_t = S_t do_t
    (3)  dS'    = D,                 dbeta_t = k_t^T D e_t,
         dk_t   = beta_t D e_t,      de_t = beta_t D^T k_t
    (2)  dv_t   = de_t,              dS' -= k_t de_t^T,     dk_t -= S' de_t
    (1)  dalpha_t = <S_{t-1}, dS'>,  D = alpha_t dS'   (the gradient reaching S_{t-1})
  and dh0 = D after the first token.

A value head reads query/key head floor(j H_qk / H_v), so the gradients of q
and k sum over the value heads that share them; a packed batch restarts the
state at every sequence boundary, exactly as the forward oracle.

Pins (``tests/test_oracle_grad_pins.py``): central differences of the
float64 forward oracle (the check "Attention as Matrix Algebra", section 7.1,
applies to one step), closed forms at beta = 0 and for a single step, and
planted mistakes that each fail a pin.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import _as_f64, qk_head


def backward_units(q, k, v, alpha, beta, do, dhT=None, h0=None, mutant: int = 0):
    """Gradients of L = sum_t <do_t, o_t> + <dhT, S_T> for independent units.

    q, k: [U, T, d_k]; v, do: [U, T, d_v]; alpha, beta: [U, T];
    dhT, h0: [U, d_k, d_v] or None.  Returns (dq, dk, dv, dalpha, dbeta, dh0)
    in float64, shaped like the inputs (dh0 [U, d_k, d_v]).

    ``mutant`` > 0 plants one deliberate mistake (for the pin tests only).
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    alpha, beta = np.asarray(alpha, np.float64), np.asarray(beta, np.float64)
    U, T, dk_ = q.shape
    dv_ = v.shape[2]
    S = np.zeros((U, dk_, dv_)) if h0 is None else np.array(h0, dtype=np.float64)
    # forward, keeping every state: S_hist[:, t] = S_t (S_hist[:, 0] = S_0)
    S_hist = np.empty((U, T + 1, dk_, dv_))
    S_hist[:, 0] = S
    for t in range(T):
        Sd = alpha[:, t, None, None] * S
        e = v[:, t] - np.einsum("ukv,uk->uv", Sd, k[:, t])
        S = Sd + beta[:, t, None, None] * k[:, t, :, None] * e[:, None, :]
        S_hist[:, t + 1] = S

    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dalpha, dbeta = np.zeros_like(alpha), np.zeros_like(beta)
    D = np.zeros((U, dk_, dv_)) if dhT is None else np.array(dhT, dtype=np.float64)
    for t in range(T - 1, -1, -1):
        S_prev, S_t = S_hist[:, t], S_hist[:, t + 1]
        kt, qt, a, b = k[:, t], q[:, t], alpha[:, t], beta[:, t]
        Sd = a[:, None, None] * S_prev
        e = v[:, t] - np.einsum("ukv,uk->uv", Sd, kt)
        # (4) o_t = S_t^T q_t
        D = D + qt[:, :, None] * do[:, t, None, :]
        dq[:, t] = np.einsum("ukv,uv->uk", S_t, do[:, t])
        # (3) S_t = S' + beta_t k_t e_t^T
        De = np.einsum("ukv,uv->uk", D, e)
        dbeta[:, t] = np.einsum("uk,uk->u", kt, De)
        dk[:, t] = b[:, None] * De
        de = b[:, None] * np.einsum("ukv,uk->uv", D, kt)
        dSd = D.copy()
        # (2) e_t = v_t - S'^T k_t
        dv[:, t] = de
        if mutant != 2:
            dSd -= kt[:, :, None] * de[:, None, :]
        else:
            dSd += kt[:, :, None] * de[:, None, :]
        if mutant != 1:
            dk[:, t] -= np.einsum("ukv,uv->uk", Sd, de)
        # (1) S' = alpha_t S_{t-1}
        dalpha[:, t] = np.einsum("ukv,ukv->u", S_t if mutant == 3 else S_prev, dSd)
        D = dSd if mutant == 4 else a[:, None, None] * dSd
    return dq, dk, dv, dalpha, dbeta, D


def backward(q, k, v, alpha, beta, do, dhT=None, *, cu_seqlens=None, h0=None, mutant: int = 0):
    """Gradients for a batch laid out as the library receives it.

    q, k: [B, T, H_qk, d_k]; v, do: [B, T, H_v, d_v] (float values or bf16
    bits for q, k, v); alpha, beta: [B, T, H_v]; dhT, h0: [N, H_v, d_k, d_v]
    or None (N = B, or the number of packed sequences).  Returns (dq, dk, dv,
    dalpha, dbeta, dh0) in float64; dq and dk sum over the value heads that
    read each query/key head.
    """
    q, k, v = _as_f64(np.asarray(q)), _as_f64(np.asarray(k)), _as_f64(np.asarray(v))
    do = np.asarray(do, dtype=np.float64)
    alpha, beta = np.asarray(alpha, np.float64), np.asarray(beta, np.float64)
    B, T, H_qk, dk_ = q.shape
    H_v, dv_ = v.shape[2], v.shape[3]
    if cu_seqlens is None:
        seqs = [(b, 0, T) for b in range(B)]
    else:
        if B != 1:
            raise ValueError("oracle: a packed batch has B == 1")
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        seqs = [(0, int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)]
    heads = [qk_head(j, H_qk, H_v) for j in range(H_v)]
    dq, dk = np.zeros_like(q), np.zeros_like(k)
    dv, dalpha, dbeta = np.zeros_like(v), np.zeros_like(alpha), np.zeros_like(beta)
    dh0 = np.zeros((len(seqs), H_v, dk_, dv_))
    for i, (b, s, e) in enumerate(seqs):
        qs = np.stack([q[b, s:e, hq] for hq in heads])
        ks = np.stack([k[b, s:e, hq] for hq in heads])
        vs = np.transpose(v[b, s:e], (1, 0, 2))
        dos = np.transpose(do[b, s:e], (1, 0, 2))
        a_s, b_s = alpha[b, s:e].T, beta[b, s:e].T
        g = backward_units(qs, ks, vs, a_s, b_s, dos,
                           None if dhT is None else np.asarray(dhT[i], np.float64),
                           None if h0 is None else np.asarray(h0[i], np.float64), mutant=mutant)
        gq, gk, gv, ga, gb, gh = g
        for j, hq in enumerate(heads):
            dq[b, s:e, hq] += gq[j]
            dk[b, s:e, hq] += gk[j]
        dv[b, s:e] = np.transpose(gv, (1, 0, 2))
        dalpha[b, s:e] = ga.T
        dbeta[b, s:e] = gb.T
        dh0[i] = gh
    return dq, dk, dv, dalpha, dbeta, dh0
