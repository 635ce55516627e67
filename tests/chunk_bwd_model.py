"""Float64 model of the gradients of the gated chunk form -- test-side only.

Not the oracle (that is oracle/grad.py, the token loop differentiated).  It
writes out in NumPy the chunk-level backward pass that the HIP backward
kernels implement, so that a test can show it equals the oracle's gradients
before any kernel is trusted.  Shares no code with the HIP path.

Forward inside a chunk from state S (see chunk_model.py): g_t = sum_{i<=t}
ln alpha_i, gamma_t = e^{g_t}, Gamma_ti = e^{g_t - g_i} (i <= t),
s_t = e^{g_C - g_t}, gamma_C = e^{g_C}; A = strict_lower(diag(beta) (Gamma . K K^T)),
M = (I + A)^-1, T = M diag(beta), X = V - diag(gamma) K S, U = T X,
P = lower(Gamma . Q K^T), O = diag(gamma) Q S + P U,
S' = gamma_C S + (diag(s) K)^T U.

Backward, given dO and dS' (the gradient reaching the chunk's end state):
  dU   = P^T dO + diag(s) K dS'
  dX   = T^T dU,  dV = dX
  dS   = gamma_C dS' + Q^T diag(gamma) dO - K^T diag(gamma) dX     (to the previous chunk)
  dP   = lower(dO U^T)
  dQ   = diag(gamma) dO S^T + (dP . Gamma) K
  dY   = M^T dU (Y = diag(beta) X),  dbeta = rowsum(dY . X) + rowsum(dA . Gamma . KK^T)
  dA   = strict_lower(-M^T (dU Y^T) M^T)
  dK   = (dP . Gamma)^T Q - diag(gamma) dX S^T + diag(s) U dS'^T + (dG + dG^T) K,
         dG = dA . diag(beta) Gamma
  gates: dgamma_t = rowsum(dO . QS - dX . KS), dGamma = dA . diag(beta) KK^T + dP . QK^T,
         ds_t = rowsum(K dS' . U), dgamma_C = <S, dS'>;
         dg = gamma . dgamma + rowsum(Gamma . dGamma) - colsum(Gamma . dGamma) - s . ds,
         dg_C += gamma_C dgamma_C + sum(s . ds);  d ln alpha_i = sum_{t >= i} dg_t.
"""
import numpy as np


def chunked_backward(q, k, v, alpha, beta, do, C, dhT=None, h0=None):
    """One unit.  Returns (dq, dk, dv, dalpha, dbeta, dh0)."""
    T, dk_ = k.shape
    dv_ = v.shape[1]
    S = np.zeros((dk_, dv_)) if h0 is None else np.array(h0, dtype=np.float64)
    saved = []
    for c0 in range(0, T, C):
        sl = slice(c0, min(c0 + C, T))
        Q, K, V, b = q[sl], k[sl], v[sl], beta[sl]
        n = len(b)
        g = np.cumsum(np.log(alpha[sl]))
        gamma, s, gC = np.exp(g), np.exp(g[-1] - g), np.exp(g[-1])
        Gamma = np.tril(np.exp(g[:, None] - np.maximum(g[None, :], g[:, None])))
        KK, QK = K @ K.T, Q @ K.T
        A = np.tril(b[:, None] * Gamma * KK, -1)
        M = np.linalg.inv(np.eye(n) + A)
        Tm = M * b[None, :]
        KS, QS = K @ S, Q @ S
        X = V - gamma[:, None] * KS
        U = Tm @ X
        P = np.tril(QK * Gamma)
        saved.append((sl, S, b, g, gamma, s, gC, Gamma, KK, QK, M, Tm, KS, QS, X, U, P))
        S = gC * S + (s[:, None] * K).T @ U
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    da, db = np.zeros_like(alpha), np.zeros_like(beta)
    dS = np.zeros((dk_, dv_)) if dhT is None else np.array(dhT, dtype=np.float64)
    for (sl, S, b, g, gamma, s, gC, Gamma, KK, QK, M, Tm, KS, QS, X, U, P) in reversed(saved):
        Q, K, dO = q[sl], k[sl], do[sl]
        KdS = K @ dS
        dU = P.T @ dO + s[:, None] * KdS
        dX = Tm.T @ dU
        dS_prev = gC * dS + Q.T @ (gamma[:, None] * dO) - K.T @ (gamma[:, None] * dX)
        dP = np.tril(dO @ U.T)
        dQ = gamma[:, None] * (dO @ S.T) + (dP * Gamma) @ K
        dY = M.T @ dU
        dA = np.tril(-M.T @ (dU @ (b[:, None] * X).T) @ M.T, -1)
        dbeta = np.sum(dY * X, axis=1) + np.sum(dA * Gamma * KK, axis=1)
        dG = dA * b[:, None] * Gamma
        dK = (dP * Gamma).T @ Q - gamma[:, None] * (dX @ S.T) + s[:, None] * (U @ dS.T) + (dG + dG.T) @ K
        dgamma = np.sum(dO * QS, axis=1) - np.sum(dX * KS, axis=1)
        dGamma = dA * b[:, None] * KK + dP * QK
        ds = np.sum(KdS * U, axis=1)
        GdG = Gamma * dGamma
        dg = gamma * dgamma + GdG.sum(axis=1) - GdG.sum(axis=0) - s * ds
        dg[-1] += gC * np.sum(S * dS) + np.sum(s * ds)
        da[sl] = np.cumsum(dg[::-1])[::-1] / alpha[sl]
        dq[sl], dk[sl], dv[sl], db[sl] = dQ, dK, dX, dbeta
        dS = dS_prev
    return dq, dk, dv, da, db, dS
