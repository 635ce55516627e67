"""Pins of the block oracle (oracle/block.py) against independent facts.

None of these retypes the oracle's formulas: each compares it with a library
routine (PyTorch CPU operators, numpy.convolve), a closed form, or an
invariant of the operation ("Linear attention", section "A naive PyTorch
implementation", describes the steps).  Tolerance 1e-12 unless stated.
"""
import numpy as np
import pytest
import torch

from oracle import block

TOL = 1e-12


def close(a, b, tol=TOL):
    d = np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))
    return d.size == 0 or float(np.max(d)) <= tol


def rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# Causal depthwise convolution
# ---------------------------------------------------------------------------

def test_conv_one_hot_taps_are_token_shifts():
    x = rng(1).standard_normal((2, 9, 5))
    for j, shift in ((3, 0), (2, 1), (1, 2), (0, 3)):
        w = np.zeros((5, 4))
        w[:, j] = 1.0
        y = block.causal_conv(x, w)
        want = np.zeros_like(x)
        want[:, shift:] = x[:, :9 - shift]
        assert close(y, want), (j, shift)


def test_conv_matches_numpy_convolve_per_channel():
    r = rng(2)
    x = r.standard_normal((1, 23, 6))
    w = r.standard_normal((6, 4))
    bias = r.standard_normal(6)
    y = block.causal_conv(x, w, bias)
    for c in range(6):
        # tap j reads token t - 3 + j: the causal filter h[s] = w[3 - s]
        want = np.convolve(x[0, :, c], w[c, ::-1])[:23] + bias[c]
        assert close(y[0, :, c], want)


def test_conv_silu_matches_torch_left_padded_depthwise_conv():
    r = rng(3)
    B, T, C = 2, 17, 8
    x = r.standard_normal((B, T, C))
    w = r.standard_normal((C, 4))
    bias = r.standard_normal(C)
    xt = torch.nn.functional.pad(torch.from_numpy(x), (0, 0, 3, 0))  # three zero tokens in front
    yt = torch.nn.functional.conv1d(xt.transpose(1, 2), torch.from_numpy(w)[:, None, :],
                                    torch.from_numpy(bias), groups=C)
    want = torch.nn.functional.silu(yt).transpose(1, 2).numpy()
    assert close(block.causal_conv_silu(x, w, bias), want)


def test_conv_is_causal_and_local():
    r = rng(4)
    x = r.standard_normal((1, 20, 3))
    w = r.standard_normal((3, 4))
    y0 = block.causal_conv(x, w)
    x2 = x.copy()
    x2[0, 10] += 1.0
    changed = np.any(block.causal_conv(x2, w) != y0, axis=(0, 2))
    assert list(np.nonzero(changed)[0]) == [10, 11, 12, 13]


def test_conv_packed_batch_pads_each_sequence():
    r = rng(5)
    lengths = [5, 1, 0, 9, 2]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    x = r.standard_normal((1, int(cu[-1]), 4))
    w = r.standard_normal((4, 4))
    bias = r.standard_normal(4)
    y = block.causal_conv(x, w, bias, cu_seqlens=cu)
    for i, L in enumerate(lengths):
        s = int(cu[i])
        alone = block.causal_conv(x[:, s:s + L], w, bias)
        assert close(y[:, s:s + L], alone)


# ---------------------------------------------------------------------------
# Pointwise maps and normalisations
# ---------------------------------------------------------------------------

def test_silu_and_softplus_against_torch_and_odd_parts():
    x = np.linspace(-30.0, 30.0, 121)
    assert close(block.silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy())
    assert close(block.silu(x) - block.silu(-x), x)  # x s(x) + x s(-x) = x
    assert block.silu(0.0) == 0.0
    sp = block.softplus(x)
    assert close(sp, torch.nn.functional.softplus(torch.from_numpy(x), threshold=1e9).numpy(), 1e-12)
    assert close(sp - block.softplus(-x), x)  # log(1 + e^x) - log(1 + e^-x) = x
    assert abs(block.softplus(0.0) - np.log(2.0)) <= TOL
    assert close(block.sigmoid(x) + block.sigmoid(-x), np.ones_like(x))


def test_unit_rows_against_torch_normalize():
    x = rng(6).standard_normal((3, 4, 16))
    u = block.unit_rows(x)
    assert close(np.linalg.norm(u, axis=-1), np.ones((3, 4)))
    assert close(u, torch.nn.functional.normalize(torch.from_numpy(x), dim=-1).numpy())
    assert close(block.unit_rows(7.5 * x), u)
    assert np.all(block.unit_rows(np.zeros((2, 8))) == 0.0)  # the 1e-12 floor keeps zero rows zero


def test_rms_norm_against_torch_and_invariants():
    r = rng(7)
    x = r.standard_normal((5, 32)) * 3.0
    w = r.standard_normal(32)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (32,), torch.from_numpy(w), eps=1e-6).numpy()
    assert close(block.rms_norm(x, w, 1e-6), want)
    y = block.rms_norm(x, None, 0.0)
    assert close(np.mean(y * y, axis=-1), np.ones(5))  # unit root mean square without eps
    assert close(block.rms_norm(4.0 * x, None, 0.0), y)  # scale invariant without eps


def test_gates_closed_forms():
    # a = 0: softplus(0) = ln 2, so alpha = exp(-A ln 2) = 2^-A
    log_A = np.log(np.array([1.0, 2.0, 0.5, 16.0]))
    alpha, beta = block.gates(np.zeros((3, 4)), np.zeros((3, 4)), log_A)
    assert close(alpha, np.broadcast_to(2.0 ** -np.exp(log_A), (3, 4)))
    assert close(beta, np.full((3, 4), 0.5))
    # a -> -inf: no forgetting; a -> +inf: alpha -> 0; alpha falls as a rises
    alpha, _ = block.gates(np.array([-800.0, 800.0]), np.zeros(2), np.zeros(2))
    assert alpha[0] == 1.0 and alpha[1] == 0.0
    a = np.linspace(-10, 10, 41)
    alpha, _ = block.gates(a, a, np.zeros(41))
    assert np.all(np.diff(alpha) < 0) and np.all((alpha > 0) & (alpha < 1))


def test_epilogue_against_torch_composition():
    r = rng(8)
    o = r.standard_normal((2, 3, 4, 16))
    g = r.standard_normal((2, 3, 4, 16)) * 2.0
    w = r.standard_normal(16)
    ot = torch.from_numpy(o)
    want = (torch.nn.functional.rms_norm(ot, (16,), torch.from_numpy(w), eps=1e-6)
            * torch.nn.functional.silu(torch.from_numpy(g))).numpy()
    assert close(block.epilogue(o, g, w), want)
    assert np.all(block.epilogue(o, np.zeros_like(g), w) == 0.0)


def test_prologue_against_torch_composition():
    """The prologue against the same steps composed from PyTorch CPU operators
    (conv1d on left-padded tokens, SiLU, normalize, rms_norm, softplus,
    sigmoid)."""
    r = rng(9)
    B, T, H, d = 2, 11, 2, 8
    q, k, v = (r.standard_normal((B, T, H, d)) for _ in range(3))
    cq, ck, cv = (r.standard_normal((H * d, 4)) for _ in range(3))
    bq, bk, bv = (r.standard_normal(H * d) for _ in range(3))
    a_raw, b_raw = r.standard_normal((B, T, H)), r.standard_normal((B, T, H))
    log_A = np.log(r.uniform(0.5, 16.0, H))
    nw = r.standard_normal(d)

    def tconv(x, w, b):
        xt = torch.nn.functional.pad(torch.from_numpy(x.reshape(B, T, H * d)), (0, 0, 3, 0))
        y = torch.nn.functional.conv1d(xt.transpose(1, 2), torch.from_numpy(w)[:, None, :], torch.from_numpy(b),
                                       groups=H * d)
        return torch.nn.functional.silu(y).transpose(1, 2).reshape(B, T, H, d)

    tq = torch.nn.functional.normalize(tconv(q, cq, bq), dim=-1) * 0.25
    tk = torch.nn.functional.normalize(tconv(k, ck, bk), dim=-1)
    tv = torch.nn.functional.rms_norm(tconv(v, cv, bv), (d,), torch.from_numpy(nw), eps=1e-6)
    ta = torch.exp(-torch.exp(torch.from_numpy(log_A)) * torch.nn.functional.softplus(torch.from_numpy(a_raw),
                                                                                       threshold=1e9))
    tb = torch.sigmoid(torch.from_numpy(b_raw))
    got = block.prologue(q, k, v, cq, ck, cv, a_raw, b_raw, log_A, conv_q_bias=bq, conv_k_bias=bk,
                         conv_v_bias=bv, norm_weight=nw, q_scale=0.25)
    for g_, t_ in zip(got, (tq, tk, tv, ta, tb)):
        assert close(g_, t_.numpy())
