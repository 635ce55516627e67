"""Pins of the per-channel-decay oracle (oracle/kda.py) against independent facts.

None of these retypes its update: each compares it with the scalar-gate
oracle (itself pinned to the pages' worked examples), with a closed form, or
with an invariant of the update ("Attention as Matrix Algebra", section 10,
names the per-channel rate; "Linear attention", Eqs. (1)-(4), the rest).
"""
import numpy as np

import oracle
from oracle import kda

TOL = 1e-12


def rng(seed):
    return np.random.default_rng(seed)


def inputs(seed, B=2, T=9, H_qk=1, H_v=2, dk=4, dv=3):
    r = rng(seed)
    q = r.standard_normal((B, T, H_qk, dk))
    k = r.standard_normal((B, T, H_qk, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, T, H_v, dv))
    beta = r.uniform(0.1, 0.9, (B, T, H_v))
    return q, k, v, beta


def test_equal_rates_reduce_to_the_scalar_gate_oracle():
    """Every channel at the same rate: the scalar-gated rule, including grouped
    heads, a packed batch and an initial state."""
    q, k, v, beta = inputs(1, B=1, T=23, H_qk=2, H_v=4)
    a = rng(2).uniform(0.5, 1.0, (1, 23, 4))
    cu = np.array([0, 5, 5, 17, 23])
    h0 = rng(3).standard_normal((4, 4, 4, 3))
    a_vec = np.repeat(a[..., None], 4, axis=-1)
    o1, h1 = kda.forward(q, k, v, a_vec, beta, cu_seqlens=cu, h0=h0)
    o2, h2 = oracle.forward(q, k, v, a, beta, cu_seqlens=cu, h0=h0)
    assert np.max(np.abs(o1 - o2)) <= TOL and np.max(np.abs(h1 - h2)) <= TOL


def test_beta_zero_scales_each_key_row_by_its_rates():
    """With beta = 0 nothing is written: S_t = diag(prod of a) S_0, so row j of
    the state is S_0's row j times the product of channel j's rates."""
    q, k, v, beta = inputs(4, dk=4, dv=4)
    a = rng(5).uniform(0.2, 1.0, (2, 9, 2, 4))
    h0 = rng(6).standard_normal((2, 2, 4, 4))
    o, hT = kda.forward(q, k, v, a, np.zeros_like(beta), h0=h0)
    cum = np.cumprod(a, axis=1)  # [B, T, H_v, d_k]
    want_hT = cum[:, -1][..., None] * h0
    assert np.max(np.abs(hT - want_hT)) <= TOL
    for t in range(9):
        St = cum[:, t][..., None] * h0  # [B, H_v, d_k, d_v]
        want_o = np.einsum("bhkv,bhk->bhv", St, q[:, t, [0, 0]])
        assert np.max(np.abs(o[:, t] - want_o)) <= TOL


def test_first_token_from_zero_state():
    """From S_0 = 0 the decay has nothing to act on: S_1 = beta k v^T and
    o_1 = beta (q . k) v, whatever the rates."""
    q, k, v, beta = inputs(7, T=1)
    a = rng(8).uniform(0.0, 1.0, (2, 1, 2, 4))
    o, hT = kda.forward(q, k, v, a, beta)
    for b in range(2):
        for j in range(2):
            kk, qq = k[b, 0, 0], q[b, 0, 0]
            assert np.max(np.abs(hT[b, j] - beta[b, 0, j] * np.outer(kk, v[b, 0, j]))) <= TOL
            assert np.max(np.abs(o[b, 0, j] - beta[b, 0, j] * (qq @ kk) * v[b, 0, j])) <= TOL


def test_a_zero_rate_forgets_that_key_row():
    """A rate of 0 on channel j at token t erases row j of the state before
    the token's write.  At t = 0 that state is h0, so row j of h0 has no
    effect on anything; with the rate at 1 instead, it does."""
    q, k, v, beta = inputs(9, B=1, T=8)
    a = rng(10).uniform(0.5, 1.0, (1, 8, 2, 4))
    h0 = rng(11).standard_normal((1, 2, 4, 3))
    h0b = h0.copy()
    h0b[:, :, 2, :] += 5.0
    a[0, 0, :, 2] = 0.0
    o1, h1 = kda.forward(q, k, v, a, beta, h0=h0)
    o2, h2 = kda.forward(q, k, v, a, beta, h0=h0b)
    assert np.max(np.abs(o1 - o2)) <= TOL and np.max(np.abs(h1 - h2)) <= TOL
    a[0, 0, :, 2] = 1.0
    o3, _ = kda.forward(q, k, v, a, beta, h0=h0)
    o4, _ = kda.forward(q, k, v, a, beta, h0=h0b)
    assert np.max(np.abs(o3 - o4)) > 1e-3


def test_decode_is_the_one_token_forward():
    q, k, v, beta = inputs(12, T=1)
    a = rng(13).uniform(0.5, 1.0, (2, 1, 2, 4))
    state = rng(14).standard_normal((2, 2, 4, 3))
    o1, s1 = kda.decode(state, q, k, v, a, beta)
    o2, s2 = kda.forward(q, k, v, a, beta, h0=state)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
