"""Pins of the float64 gradient oracle (oracle/grad.py).

None of these retypes the backward recurrence.  Each compares it with an
independent fact:
  * central differences of the float64 forward oracle (gdn_oracle.c), input
    by input, on a packed batch with grouped heads and an initial state --
    the finite-difference check "Attention as Matrix Algebra", section 7.1
    ("One step of online regression") runs on one step;
  * closed forms: beta = 0 leaves only the decay of h0, so o_t =
    (prod_{i<=t} alpha_i) h0^T q_t and every gradient is a sum of products;
    one step from h0 differentiates by hand;
  * planted mistakes in the backward pass, each caught by a pin.
"""
import numpy as np
import pytest

import oracle
from oracle import grad

EPS = 1e-6


def loss(w, do, dhT):
    o, hT = oracle.forward(w["q"], w["k"], w["v"], w["alpha"], w["beta"], cu_seqlens=w.get("cu"),
                           h0=w.get("h0"))
    return float(np.sum(o * do) + np.sum(hT * dhT))


def batch(rng, packed=True):
    """2 packed sequences (5 and 7 tokens) or B=2 x 6 tokens; 1 query/key head
    shared by 2 value heads; d_k = 3, d_v = 2; unit-length keys."""
    if packed:
        B, T, cu, N = 1, 12, np.array([0, 5, 12], dtype=np.int32), 2
    else:
        B, T, cu, N = 2, 6, None, 2
    H_qk, H_v, dk, dv = 1, 2, 3, 2
    k = rng.standard_normal((B, T, H_qk, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    w = {"q": rng.standard_normal((B, T, H_qk, dk)) * 0.7, "k": k,
         "v": rng.standard_normal((B, T, H_v, dv)),
         "alpha": rng.uniform(0.5, 1.0, (B, T, H_v)), "beta": rng.uniform(0.1, 1.0, (B, T, H_v)),
         "h0": rng.standard_normal((N, H_v, dk, dv)) * 0.5}
    if cu is not None:
        w["cu"] = cu
    do = rng.standard_normal((B, T, H_v, dv))
    dhT = rng.standard_normal((N, H_v, dk, dv))
    return w, do, dhT


def grads(w, do, dhT, mutant=0):
    g = grad.backward(w["q"], w["k"], w["v"], w["alpha"], w["beta"], do, dhT, cu_seqlens=w.get("cu"),
                      h0=w.get("h0"), mutant=mutant)
    return dict(zip(("q", "k", "v", "alpha", "beta", "h0"), g))


def central_difference_error(w, do, dhT, g):
    """Largest |analytic - numeric| over every element of every input,
    relative to max(1, |numeric|)."""
    worst = 0.0
    for name in ("q", "k", "v", "alpha", "beta", "h0"):
        x = w[name]
        for idx in np.ndindex(x.shape):
            orig = x[idx]
            x[idx] = orig + EPS
            lp = loss(w, do, dhT)
            x[idx] = orig - EPS
            lm = loss(w, do, dhT)
            x[idx] = orig
            num = (lp - lm) / (2 * EPS)
            worst = max(worst, abs(g[name][idx] - num) / max(1.0, abs(num)))
    return worst


@pytest.mark.parametrize("packed", [True, False])
def test_gradients_match_central_differences(packed):
    rng = np.random.default_rng(70 + packed)
    w, do, dhT = batch(rng, packed)
    err = central_difference_error(w, do, dhT, grads(w, do, dhT))
    assert err < 1e-7, err


def test_beta_zero_closed_form():
    """beta = 0: S_t = (prod_{i<=t} alpha_i) h0, so with P_t = prod_{i<=t} alpha_i
    dq_t = P_t h0 do_t, dv = dk = 0, dh0 = sum_t P_t q_t do_t^T + P_T dhT,
    dalpha_t = sum_{s>=t} (P_s / alpha_t) (q_s^T h0 do_s) + (P_T / alpha_t) <h0, dhT>,
    dbeta_t = k_t^T D_t e_t with D_t = sum_{s>=t} (P_s/P_t) q_s do_s^T + (P_T/P_t) dhT
    and e_t = v_t - P_t h0^T k_t."""
    rng = np.random.default_rng(72)
    T, dk, dv = 7, 4, 3
    q, k, v = (rng.standard_normal((1, T, dk)), rng.standard_normal((1, T, dk)), rng.standard_normal((1, T, dv)))
    a = rng.uniform(0.4, 1.0, (1, T))
    b = np.zeros((1, T))
    h0 = rng.standard_normal((1, dk, dv))
    do, dhT = rng.standard_normal((1, T, dv)), rng.standard_normal((1, dk, dv))
    gq, gk, gv, ga, gb, gh = grad.backward_units(q, k, v, a, b, do, dhT, h0)
    P = np.cumprod(a[0])
    H = h0[0]
    assert np.allclose(gq[0], (P[:, None] * (H @ do[0].T).T), atol=1e-13)
    assert np.all(gv == 0) and np.all(gk == 0)
    want_h0 = sum(P[t] * np.outer(q[0, t], do[0, t]) for t in range(T)) + P[-1] * dhT[0]
    assert np.allclose(gh[0], want_h0, atol=1e-13)
    qhd = np.array([q[0, s] @ H @ do[0, s] for s in range(T)])
    want_a = [(sum(P[s] * qhd[s] for s in range(t, T)) + P[-1] * np.sum(H * dhT[0])) / a[0, t] for t in range(T)]
    assert np.allclose(ga[0], want_a, atol=1e-12)
    for t in range(T):
        D = sum(P[s] / P[t] * np.outer(q[0, s], do[0, s]) for s in range(t, T)) + P[-1] / P[t] * dhT[0]
        e = v[0, t] - P[t] * (H.T @ k[0, t])
        assert abs(gb[0, t] - k[0, t] @ D @ e) < 1e-12


def test_single_step_closed_form():
    """One token from h0: S_1 = a h0 + b k (v - a h0^T k)^T, o = S_1^T q, and
    L = <do, o> (no dhT): dq = S_1 do, dv = b (q^T k) do,
    dk = b (q^T k)... by hand: L = a q^T h0 do + b (q^T k)(v - a h0^T k)^T do, so
    dk = b q ((v - a h0^T k)^T do) - a b (q^T k) h0 do,
    dbeta = (q^T k)(v - a h0^T k)^T do, dalpha = q^T h0 do - b (q^T k) k^T h0 do,
    dh0 = a q do^T - a b (q^T k) k do^T."""
    rng = np.random.default_rng(73)
    dk, dv = 5, 4
    q, k, v = rng.standard_normal(dk), rng.standard_normal(dk), rng.standard_normal(dv)
    a, b = 0.8, 0.6
    h0, do = rng.standard_normal((dk, dv)), rng.standard_normal(dv)
    gq, gk, gv, ga, gb, gh = grad.backward_units(q[None, None], k[None, None], v[None, None], np.array([[a]]),
                                                 np.array([[b]]), do[None, None], None, h0[None])
    S1 = a * h0 + b * np.outer(k, v - a * h0.T @ k)
    qk = q @ k
    err = v - a * h0.T @ k
    assert np.allclose(gq[0, 0], S1 @ do, atol=1e-14)
    assert np.allclose(gv[0, 0], b * qk * do, atol=1e-14)
    assert np.allclose(gk[0, 0], b * q * (err @ do) - a * b * qk * (h0 @ do), atol=1e-14)
    assert abs(gb[0, 0] - qk * (err @ do)) < 1e-14
    assert abs(ga[0, 0] - (q @ h0 @ do - b * qk * (k @ h0 @ do))) < 1e-14
    assert np.allclose(gh[0], a * np.outer(q, do) - a * b * qk * np.outer(k, do), atol=1e-14)


@pytest.mark.parametrize("mutant", [1, 2, 3, 4])
def test_pins_catch_planted_mistakes(mutant):
    """Dropping the -S' de term of dk, flipping the sign of the -k de^T term,
    taking dalpha from S_t instead of S_{t-1}, or passing dS' to S_{t-1}
    without alpha: each fails the central-difference pin."""
    rng = np.random.default_rng(74)
    w, do, dhT = batch(rng, True)
    assert central_difference_error(w, do, dhT, grads(w, do, dhT, mutant=mutant)) > 1e-3
