"""The seeded input generators: shapes, determinism, rounding and distributions."""
import math

import numpy as np

import gdn_inputs as gi


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.4e38, np.inf],
                 dtype=np.float32)
    b = gi.f32_to_bf16_bits(x)
    back = gi.bf16_bits_to_f32(b)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins.
    assert back[0] == 1.0 and back[1] == 1.0
    assert back[2] == np.float32(1.0 + 4 * 2 ** -8)
    assert back[3] == 1.0
    assert back[4] == -2.5
    assert np.isinf(back[5]) and np.isinf(back[6])
    assert np.isnan(gi.bf16_bits_to_f32(gi.f32_to_bf16_bits(np.array([np.nan], np.float32))))[0]


def test_tiny_config():
    w = gi.generate(gi.config(1))
    assert w.q.dtype == np.float32 and w.q.shape == (1, 64, 1, 16)
    assert w.alpha.shape == (1, 64, 1) and w.alpha.dtype == np.float32
    n = np.linalg.norm(w.q, axis=-1)
    assert np.allclose(n, 1.0, atol=1e-6)
    assert np.all((w.alpha > 0) & (w.alpha < 1)) and np.all((w.beta > 0) & (w.beta < 1))
    w2 = gi.generate(gi.config(1))
    assert np.array_equal(w.q, w2.q) and np.array_equal(w.alpha, w2.alpha)


def test_prefill_shaped_small():
    spec = gi.config(2, B=2, T=100, H_qk=3, H_v=3)
    w = gi.generate(spec)
    assert w.q.dtype == np.uint16 and w.q.shape == (2, 100, 3, 128)
    qn = np.linalg.norm(w.values("q"), axis=-1)
    assert np.allclose(qn, 1 / math.sqrt(128), rtol=1e-2)
    kn = np.linalg.norm(w.values("k"), axis=-1)
    assert np.allclose(kn, 1.0, rtol=1e-2)
    la = np.log(w.alpha.astype(np.float64))
    assert np.all(la < 0)
    # A_h = exp(U(-4, 0)) per head: log alpha / softplus(z) is constant per head;
    # at least check the gate stays in (0, 1).
    assert np.all((w.alpha > 0) & (w.alpha < 1))


def test_packed_lengths_and_offsets():
    spec = gi.config(5)
    L = gi.packed_lengths(spec)
    assert len(L) == 32 and min(L) >= 128 and max(L) <= 16384
    small = gi.config(5, lengths=(3, 70, 1, 64), H_qk=2, H_v=4, d_k=16, d_v=8)
    w = gi.generate(small)
    assert list(w.cu_seqlens) == [0, 3, 73, 74, 138]
    assert w.q.shape == (1, 138, 2, 16) and w.v.shape == (1, 138, 4, 8)


def test_long_memory_gate_scaling():
    a = gi.generate(gi.config(2, B=1, T=64, H_qk=2, H_v=2))
    b = gi.generate(gi.config(2, B=1, T=64, H_qk=2, H_v=2, log_alpha_scale=1 / 64))
    la, lb = np.log(a.alpha.astype(np.float64)), np.log(b.alpha.astype(np.float64))
    assert np.allclose(lb, la / 64, rtol=1e-3, atol=1e-6)  # alpha is stored in float32
