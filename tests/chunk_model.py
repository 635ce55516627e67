"""Float64 model of the gated chunkwise (WY / UT) form -- test-side only.

Not the oracle.  It writes out, in NumPy, the chunk equations that the HIP
chunk kernels implement, so that a test can show they equal the token-by-token
oracle before any kernel is trusted.  It shares no code with the HIP path.

Derivation (the pages give only the ungated form: "Attention as Matrix
Algebra", section 8, and "From KV Cache to a State Matrix", section "Chunkwise
training for DeltaNet"; the gate is "Linear attention", Eq. (1)).  Inside a
chunk that starts from state S, let g_t = sum_{i<=t} ln alpha_i (chunk-local),
gamma_t = e^{g_t} and Gamma_ti = e^{g_t - g_i} (i <= t).  With the
pseudo-value u_t = beta_t (v_t - alpha_t S_{t-1}^T k_t) the state is
S_t = alpha_t S_{t-1} + k_t u_t^T, so

    S_t = gamma_t S + sum_{i<=t} Gamma_ti k_i u_i^T
    (I + A) U = diag(beta) (V - diag(gamma) K S),  A_ti = beta_t Gamma_ti k_t^T k_i (i < t)
    U = T (V - diag(gamma) K S),                    T = (I + A)^{-1} diag(beta)
    O = diag(gamma) Q S + (Q K^T . Gamma . L_C) U
    S <- gamma_C S + Ktilde^T U,                    Ktilde_i = e^{g_C - g_i} k_i

With alpha = 1 these reduce to the page's (I + L) U = diag(beta)(V - KS),
O = QS + (QK^T . L_C) U, S <- S + K^T U.
"""
import numpy as np
from scipy.linalg import solve_triangular

LOG_FLOOR = -690.0  # ln alpha is clamped here so that alpha = 0 stays finite in logs


def chunked(q, k, v, alpha, beta, C, h0=None):
    """One unit: q, k [T, d_k], v [T, d_v], alpha, beta [T]; returns (o, S_T)."""
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if h0 is None else np.array(h0, dtype=np.float64)
    o = np.empty((T, dv))
    for c0 in range(0, T, C):
        sl = slice(c0, min(c0 + C, T))
        Q, K, V = q[sl], k[sl], v[sl]
        b = beta[sl]
        n = len(b)
        with np.errstate(divide="ignore"):
            g = np.cumsum(np.maximum(np.log(np.maximum(alpha[sl], 0.0)), LOG_FLOOR))
        gamma = np.exp(g)
        Gamma = np.tril(np.exp(g[:, None] - np.maximum(g[None, :], g[:, None])))
        A = np.tril(b[:, None] * Gamma * (K @ K.T), -1)
        Tm = solve_triangular(np.eye(n) + A, np.diag(b), lower=True)
        U = Tm @ (V - gamma[:, None] * (K @ S))
        o[sl] = gamma[:, None] * (Q @ S) + (np.tril(Q @ K.T) * Gamma) @ U
        Kt = np.exp(g[-1] - g)[:, None] * K
        S = gamma[-1] * S + Kt.T @ U
    return o, S


def wy_transition(k, alpha, beta):
    """gamma_C I - Ktilde^T W with W = T diag(gamma) K: the chunk's state map."""
    n, dk = k.shape
    g = np.cumsum(np.log(alpha))
    gamma = np.exp(g)
    Gamma = np.tril(np.exp(g[:, None] - g[None, :]))
    A = np.tril(beta[:, None] * Gamma * (k @ k.T), -1)
    Tm = solve_triangular(np.eye(n) + A, np.diag(beta), lower=True)
    W = Tm @ (gamma[:, None] * k)
    Kt = np.exp(g[-1] - g)[:, None] * k
    return gamma[-1] * np.eye(dk) - Kt.T @ W
