"""Float64 oracle of the delta rule with one decay rate per key channel (test infrastructure).

TEST INFRASTRUCTURE ONLY, like the rest of this package: the tests, the
smoke check and the benchmark's CPU baseline are the only callers.

"Attention as Matrix Algebra: From Softmax to the Delta Rule"
(hananather.com), section 10 "Where this goes next", names Kimi Delta
Attention as the gated delta rule with its own forget rate for each feature
channel instead of one rate per head.  Reading taken (the figure that shows
the update is not in the text): the channels are the key features, i.e. the
rows of the keys x values state, so the scalar decay of "Linear attention"
(arsalanzafar.ai), section "How it works", Eqs. (1)-(4), becomes a diagonal
one.  Per unit (sequence, value head) and token t, with a_t in R^{d_k}:

    S'   = diag(a_t) S_{t-1}        decay each key row by its own rate
    vhat = S'^T k_t                 predict from the decayed state
    S_t  = S' + beta_t k_t (v_t - vhat)^T
    o_t  = S_t^T q_t                read after the write

With every entry of a_t equal to one scalar this is the scalar-gated rule;
``tests/test_oracle_kda_pins.py`` pins it to that oracle and to closed forms.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import _as_f64, qk_head


def _sequences(B: int, T: int, cu_seqlens):
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    if B != 1:
        raise ValueError("oracle: a packed batch has B == 1")
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return [(0, int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)]


def forward(q, k, v, alpha, beta, *, cu_seqlens=None, h0: Optional[np.ndarray] = None):
    """Token-by-token forward over a batch laid out as the library receives it.

    q, k: [B, T, H_qk, d_k]; v: [B, T, H_v, d_v] (float values or bf16 bits);
    alpha: [B, T, H_v, d_k] (one rate per key channel); beta: [B, T, H_v];
    h0: [N, H_v, d_k, d_v] or None.  Returns (o [B, T, H_v, d_v],
    hT [N, H_v, d_k, d_v]) in float64.
    """
    q, k, v = _as_f64(np.asarray(q)), _as_f64(np.asarray(k)), _as_f64(np.asarray(v))
    alpha = np.asarray(alpha, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    B, T, H_qk, dk = q.shape
    H_v, dv = v.shape[2], v.shape[3]
    heads = np.array([qk_head(j, H_qk, H_v) for j in range(H_v)])
    seqs = _sequences(B, T, cu_seqlens)
    o = np.zeros((B, T, H_v, dv))
    hT = np.zeros((len(seqs), H_v, dk, dv))
    for i, (b, s, e) in enumerate(seqs):
        S = np.zeros((H_v, dk, dv)) if h0 is None else np.array(h0[i], dtype=np.float64)
        for t in range(s, e):
            kt, qt = k[b, t, heads], q[b, t, heads]                # [H_v, d_k]
            Sd = alpha[b, t][:, :, None] * S                       # decay
            vhat = np.einsum("hkv,hk->hv", Sd, kt)                 # predict
            S = Sd + beta[b, t][:, None, None] * kt[:, :, None] * (v[b, t] - vhat)[:, None, :]  # correct
            o[b, t] = np.einsum("hkv,hk->hv", S, qt)               # read
        hT[i] = S
    return o, hT


def decode(state, q, k, v, alpha, beta):
    """One token per sequence from ``state`` [B, H_v, d_k, d_v]; alpha
    [B, 1, H_v, d_k].  Returns (o [B, 1, H_v, d_v], new state)."""
    return forward(q, k, v, alpha, beta, h0=state)
