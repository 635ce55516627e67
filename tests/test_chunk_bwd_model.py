"""The chunk-level backward pass that the HIP backward kernels implement
equals the oracle's token-level gradients (oracle/grad.py), for chunks of
1, 5, 16 and 64 tokens, partial last chunks, an initial state and an
upstream gradient of the final state."""
import numpy as np
import pytest

from chunk_bwd_model import chunked_backward
from oracle import grad


@pytest.mark.parametrize("C", [1, 5, 16, 64])
def test_chunked_backward_equals_token_gradients(C):
    rng = np.random.default_rng(80 + C)
    T, dk, dv = 70, 16, 12
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    q, k = unit(rng.standard_normal((T, dk))) * 0.5, unit(rng.standard_normal((T, dk)))
    v = rng.standard_normal((T, dv))
    a = 1.0 / (1.0 + np.exp(-(2.0 + 0.5 * rng.standard_normal(T))))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    h0, dhT = rng.standard_normal((dk, dv)), rng.standard_normal((dk, dv))
    do = rng.standard_normal((T, dv))
    got = chunked_backward(q, k, v, a, b, do, C, dhT=dhT, h0=h0)
    want = grad.backward_units(q[None], k[None], v[None], a[None], b[None], do[None], dhT[None], h0[None])
    for name, x, y in zip(("dq", "dk", "dv", "dalpha", "dbeta", "dh0"), got, want):
        err = np.max(np.abs(x - y[0])) / max(1.0, np.max(np.abs(y[0])))
        assert err < 1e-10, (name, err)
