"""The gated chunk equations the HIP chunk path implements equal the oracle.

Mirrors the checks of "Attention as Matrix Algebra", section 8 (chunks of
C = 1, 5, 16, 64 equal the recurrence; the WY product of 6 transitions), with
the decay gate added, partial last chunks, alpha = 0 tokens and a nonzero
initial state.
"""
import numpy as np
import pytest

import oracle
from chunk_model import chunked, wy_transition


def data(T=64, dk=16, dv=12, seed=0):
    rng = np.random.default_rng(seed)
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    q = unit(rng.standard_normal((T, dk)))
    k = unit(rng.standard_normal((T, dk)))
    v = rng.standard_normal((T, dv))
    a = 1.0 / (1.0 + np.exp(-(2.0 + 0.5 * rng.standard_normal(T))))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    return q, k, v, a, b


@pytest.mark.parametrize("C", [1, 5, 7, 16, 64])
def test_chunks_equal_the_recurrence(C):
    q, k, v, a, b = data(seed=C)
    h0 = np.random.default_rng(99).standard_normal((16, 12))
    for init in (None, h0):
        o_ref, S_ref = oracle.forward_units(q[None], k[None], v[None], a[None], b[None],
                                            None if init is None else init[None])
        o, S = chunked(q, k, v, a, b, C, h0=init)
        assert np.max(np.abs(o - o_ref[0])) < 1e-12
        assert np.max(np.abs(S - S_ref[0])) < 1e-12


def test_alpha_zero_inside_a_chunk():
    q, k, v, a, b = data(T=70, seed=3)
    a[5] = 0.0
    a[40] = 0.0
    o_ref, S_ref = oracle.forward_units(q[None], k[None], v[None], a[None], b[None])
    o, S = chunked(q, k, v, a, b, 16)
    assert np.max(np.abs(o - o_ref[0])) < 1e-12
    assert np.max(np.abs(S - S_ref[0])) < 1e-12


def test_gated_wy_product_of_six_transitions():
    q, k, v, a, b = data(T=6, dk=8, dv=8, seed=4)
    P = np.eye(8)
    for t in range(6):
        P = a[t] * (np.eye(8) - b[t] * np.outer(k[t], k[t])) @ P
    assert np.max(np.abs(wy_transition(k, a, b) - P)) < 1e-14
