"""Pins of the float64 oracle against what the pages and the mathematics fix.

None of these retypes the oracle's own formula.  Each compares the oracle with
an independent fact: numbers a page prints for a worked example (fixtures in
tests/golden/, each with its citation), a closed form, a library routine, an
invariant, or brute force.  Tolerance 1e-12 (the float64 convention of
"Attention as Matrix Algebra", section 1, the ``check`` helper) unless stated.
"""
import numpy as np
import pytest
from scipy.linalg import solve_triangular

import oracle
from conftest import golden

TOL = 1e-12


def run(q, k, v, alpha, beta, h0=None, delta=True, lib=None):
    """One unit through the oracle; returns (o [T, d_v], S_T [d_k, d_v])."""
    o, hT = oracle.forward_units(np.asarray(q)[None], np.asarray(k)[None], np.asarray(v)[None],
                                 np.asarray(alpha)[None], np.asarray(beta)[None],
                                 None if h0 is None else np.asarray(h0)[None], delta=delta,
                                 lib=lib)
    return o[0], hT[0]


def unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def close(a, b, tol=TOL):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) <= tol


# ---------------------------------------------------------------------------
# Worked examples printed on the pages
# ---------------------------------------------------------------------------

def check_walkthrough(lib=None):
    g = golden("walkthrough_2x3.json")
    q, k, v = (np.array(g[x]) for x in ("q", "k", "v"))
    a, b, e = np.array(g["alpha"]), np.array(g["beta"]), g["expect"]
    ok = []
    o2, S2 = run(q[:2], k[:2], v[:2], a[:2], b[:2], lib=lib)
    ok.append(close(S2, e["S_2"]))
    ok.append(close(o2[1], e["o_2"]))
    o3, S3 = run(q, k, v, a, b, lib=lib)
    ok.append(close(S3, e["S_3"]))
    ok.append(close(o3[2], e["o_3"]))
    ok.append(close(S3.T @ np.array([1.0, 0.0]), e["read_k1_after_3"]))
    ok.append(close(S3.T @ np.array([0.0, 1.0]), e["read_k2_after_3"]))
    # The decayed prediction and the error of token 3 follow from the write:
    # S_3 - alpha_3 S_2 = beta_3 k_3 (v_3 - vhat)^T.
    write = S3 - a[2] * S2
    err = write[0] / b[2]
    ok.append(close(err, e["error_3"]))
    ok.append(close(v[2] - err, e["decayed_prediction_3"]))
    # The "runnable check": one step from the page's S_old (transposed).
    S_old = S2
    o1, S1 = run(q[2:], k[2:], v[2:], a[2:], b[2:], h0=S_old, lib=lib)
    ok.append(close(S1, e["S_3"]))
    ok.append(close(o1[0], e["o_3"]))
    return all(ok)


def test_walkthrough_2_keys_3_values():
    assert check_walkthrough()


def check_figure6(lib=None):
    g = golden("delta_rule_figure6.json")
    keys, values, e = np.array(g["keys"]), np.array(g["values"]), g["expect"]
    ones = np.ones(3)
    _, S_add = run(keys, keys, values, ones, ones, delta=False, lib=lib)
    _, S3 = run(keys, keys, values, ones, ones, lib=lib)
    _, S2 = run(keys[:2], keys[:2], values[:2], ones[:2], ones[:2], lib=lib)
    u3 = (S3 - S2)[0]  # k_3 = e_1, so the write k_3 u_3^T is the first row
    return close(S_add, e["additive_S_3"]) and close(S3, e["delta_S_3"]) \
        and close(u3, e["pseudo_value_u_3"])


def test_delta_rule_figure6():
    assert check_figure6()


def test_additive_figure5():
    g = golden("additive_figure5.json")
    keys, values, e = np.array(g["keys"]), np.array(g["values"]), g["expect"]
    ones = np.ones(3)
    _, S2 = run(keys[:2], keys[:2], values[:2], ones[:2], ones[:2], delta=False)
    _, S3 = run(keys, keys, values, ones, ones, delta=False)
    assert close(S2, e["S_2"])
    assert close(S3, e["S_3"])
    reads = keys @ S3 / (keys ** 2).sum(axis=1, keepdims=True)
    assert close(reads - values, e["crosstalk_after_3"])


def test_kaczmarz_sweeps_converge():
    g = golden("kaczmarz.json")
    rng = np.random.default_rng(44)
    d, n, sweeps = g["dim"], g["pairs"], g["sweeps"]
    K, V = unit_rows(rng.standard_normal((n, d))), unit_rows(rng.standard_normal((n, d)))
    Ks, Vs = np.tile(K, (sweeps, 1)), np.tile(V, (sweeps, 1))
    ones = np.ones(n * sweeps)
    _, S = run(Ks, Ks, Vs, ones, ones)
    assert np.max(np.abs(K @ S - V)) < g["tolerance"]


def test_recall_table1_statistics():
    """Delta rule read errors of Table 1 (beta = 1), to +-0.03."""
    g = golden("recall_table1.json")
    r, reps, tol = g["r"], g["repetitions"], g["tolerance"]
    rng = np.random.default_rng(2024)
    for col, n in enumerate(g["n"]):
        K = unit_rows(rng.standard_normal((reps, n, r)))
        V = unit_rows(rng.standard_normal((reps, n, r)))
        ones = np.ones((reps, n))
        _, S = oracle.forward_units(K, K, V, ones, ones)
        _, S_add = oracle.forward_units(K, K, V, ones, ones, delta=False)
        err = ((np.einsum("unk,ukv->unv", K, S) - V) ** 2).sum(axis=2)       # [reps, n]
        err_add = ((np.einsum("unk,ukv->unv", K, S_add) - V) ** 2).sum(axis=2)
        assert abs(np.sqrt(err.mean(axis=1).mean()) - g["delta_all_pairs"][col]) < tol
        assert abs(np.sqrt(err[:, -8:].mean(axis=1).mean()) - g["delta_8_newest"][col]) < tol
        assert abs(np.sqrt(err_add.mean(axis=1).mean()) - g["additive"][col]) < tol


# ---------------------------------------------------------------------------
# Closed forms and library routines
# ---------------------------------------------------------------------------

def random_unit(T=48, dk=8, dv=5, seed=0, unit=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    if unit:
        q, k = unit_rows(q), unit_rows(k)
    v = rng.standard_normal((T, dv))
    alpha = rng.uniform(0.5, 1.0, T)
    beta = rng.uniform(0.0, 1.0, T)
    return q, k, v, alpha, beta


def check_additive_brute_force(lib=None):
    """alpha = beta = 1, no delta term: o_t = sum_{j<=t} (q_t^T k_j) v_j = tril(QK^T) V."""
    q, k, v, _, _ = random_unit(T=64, dk=16, dv=12, seed=1, unit=False)
    ones = np.ones(64)
    o, S = run(q, k, v, ones, ones, delta=False, lib=lib)
    return close(o, np.tril(q @ k.T) @ v, 1e-11) and close(S, k.T @ v, 1e-11)


def test_additive_equals_unnormalised_causal_attention():
    assert check_additive_brute_force()


def test_decayed_additive_closed_form():
    """No delta term, general alpha and beta:
    o_t = sum_{j<=t} (prod_{j<i<=t} alpha_i) beta_j (q_t^T k_j) v_j."""
    q, k, v, a, b = random_unit(T=40, dk=6, dv=7, seed=2)
    o, _ = run(q, k, v, a, b, delta=False)
    want = np.zeros_like(o)
    for t in range(40):
        for j in range(t + 1):
            decay = np.prod(a[j + 1:t + 1])
            want[t] += decay * b[j] * (q[t] @ k[j]) * v[j]
    assert close(o, want)


def check_whole_sequence_solve(lib=None):
    """S_0 = 0, the whole sequence as one block (the C = n case of the chunked
    delta rule of "Attention as Matrix Algebra", section 8, with the decay of
    "Linear attention", Eq. (1)):  (I + A) U = diag(beta) V with
    A_ti = beta_t Gamma_ti k_t^T k_i (i < t), Gamma_ti = prod_{i<s<=t} alpha_s,
    and O = (QK^T . Gamma . L) U -- solved by SciPy's triangular solver."""
    q, k, v, a, b = random_unit(T=96, dk=8, dv=6, seed=3)
    T = len(a)
    logc = np.cumsum(np.log(a))
    Gamma = np.tril(np.exp(logc[:, None] - logc[None, :]))
    A = np.tril(b[:, None] * Gamma * (k @ k.T), -1)
    U = solve_triangular(np.eye(T) + A, b[:, None] * v, lower=True)
    O = (np.tril(q @ k.T) * Gamma) @ U
    o, _ = run(q, k, v, a, b, lib=lib)
    return close(o, O, 1e-11)


def test_whole_sequence_triangular_solve():
    assert check_whole_sequence_solve()


def test_transition_product_is_householder_product():
    """With v = 0 the map S_0 -> S_T is the product of the transitions
    alpha_t (I - beta_t k_t k_t^T) ("How linear attention works", factored form;
    "Attention as Matrix Algebra", section 8, WY product check)."""
    q, k, v, a, b = random_unit(T=6, dk=8, dv=8, seed=4)
    _, S = run(q, k, np.zeros_like(v), a, b, h0=np.eye(8))
    P = np.eye(8)
    for t in range(6):
        P = a[t] * (np.eye(8) - b[t] * np.outer(k[t], k[t])) @ P
    assert close(S, P)


def test_factored_form_stepwise():
    """S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T with
    non-unit keys ("How linear attention works", section "The gated delta rule",
    the expanded form; "Attention as Matrix Algebra", section 7, Householder form)."""
    q, k, v, a, b = random_unit(T=20, dk=5, dv=3, seed=5, unit=False)
    S0 = np.random.default_rng(6).standard_normal((5, 3))
    S = S0.copy()
    for t in range(20):
        S = a[t] * (np.eye(5) - b[t] * np.outer(k[t], k[t])) @ S + b[t] * np.outer(k[t], v[t])
    _, ST = run(q, k, v, a, b, h0=S0)
    assert close(ST, S, 1e-11)


def test_gradient_step_central_difference():
    """One step is a gradient step of size beta on 1/2 |S'^T k - v|^2 at the
    decayed state S' ("Attention as Matrix Algebra", section 7.1; "From KV Cache
    to a State Matrix", section "L2 loss and the delta rule").  The gradient is
    taken by central differences, not by formula."""
    rng = np.random.default_rng(7)
    dk, dv = 4, 3
    S_prev = rng.standard_normal((dk, dv))
    k = rng.standard_normal(dk)
    v = rng.standard_normal(dv)
    q = rng.standard_normal(dk)
    a, b = 0.8, 0.6
    Sp = a * S_prev

    def loss(M):
        r = M.T @ k - v
        return 0.5 * float(r @ r)

    h = 1e-6
    grad = np.zeros_like(Sp)
    for i in range(dk):
        for j in range(dv):
            E = np.zeros_like(Sp)
            E[i, j] = h
            grad[i, j] = (loss(Sp + E) - loss(Sp - E)) / (2 * h)
    _, S1 = run(q[None], k[None], v[None], [a], [b], h0=S_prev)
    assert close(S1, Sp - b * grad, 1e-8)


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------

def test_orthonormal_keys_read_back_exactly():
    rng = np.random.default_rng(8)
    dk, dv = 16, 9
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm.T  # d_k orthonormal rows
    v = rng.standard_normal((dk, dv))
    ones = np.ones(dk)
    _, S = run(keys, keys, v, ones, ones)
    assert close(keys @ S, v)


def test_beta_zero_leaves_only_the_decay():
    rng = np.random.default_rng(9)
    q, k, v, a, _ = random_unit(T=30, dk=6, dv=4, seed=10)
    S0 = rng.standard_normal((6, 4))
    zeros = np.zeros(30)
    _, S = run(q, k, v, np.ones(30), zeros, h0=S0)
    assert np.array_equal(S, S0)
    _, S = run(q, k, v, a, zeros, h0=S0)
    assert close(S, np.prod(a) * S0)


def test_read_back_mixes_old_read_and_new_value():
    """S_t^T k_t = vhat + beta ||k||^2 (v - vhat), vhat = alpha S_{t-1}^T k
    ("Linear attention", the unit-length remark; "How linear attention works",
    section "Correct the association at this key")."""
    q, k, v, a, b = random_unit(T=12, dk=7, dv=5, seed=11, unit=False)
    S = np.random.default_rng(12).standard_normal((7, 5))
    for t in range(12):
        _, S_new = run(q[t:t + 1], k[t:t + 1], v[t:t + 1], a[t:t + 1], b[t:t + 1], h0=S)
        vhat = a[t] * S.T @ k[t]
        want = vhat + b[t] * (k[t] @ k[t]) * (v[t] - vhat)
        assert close(S_new.T @ k[t], want, 1e-11)
        S = S_new


def test_orthogonal_directions_only_decay():
    q, k, v, a, b = random_unit(T=8, dk=6, dv=4, seed=13)
    rng = np.random.default_rng(14)
    S = rng.standard_normal((6, 4))
    for t in range(8):
        x = rng.standard_normal(6)
        x -= (x @ k[t]) * k[t]  # unit k: project out the key direction
        _, S_new = run(q[t:t + 1], k[t:t + 1], v[t:t + 1], a[t:t + 1], b[t:t + 1], h0=S)
        assert close(S_new.T @ x, a[t] * S.T @ x)
        S = S_new


def test_transition_does_not_amplify():
    """Spectral norm bound for unit keys and beta in [0, 2]:
    ||S_t||_2 <= alpha_t ||S_{t-1}||_2 + |beta_t| ||v_t|| ("Attention as Matrix
    Algebra", section 7.2)."""
    rng = np.random.default_rng(15)
    S = rng.standard_normal((8, 8))
    for t in range(50):
        k = unit_rows(rng.standard_normal((1, 8)))
        v = rng.standard_normal((1, 8))
        a, b = rng.uniform(0.2, 1.0), rng.uniform(0.0, 2.0)
        _, S_new = run(k, k, v, [a], [b], h0=S)
        assert np.linalg.norm(S_new, 2) <= a * np.linalg.norm(S, 2) + b * np.linalg.norm(v) + 1e-12
        S = S_new


def test_split_invariance_and_state_carry():
    """Carrying the state across calls ("How linear attention works", the state
    is carried across tokens and processing batches) gives identical results."""
    q, k, v, a, b = random_unit(T=50, dk=6, dv=5, seed=16)
    o, S = run(q, k, v, a, b)
    o1, S1 = run(q[:23], k[:23], v[:23], a[:23], b[:23])
    o2, S2 = run(q[23:], k[23:], v[23:], a[23:], b[23:], h0=S1)
    assert np.array_equal(np.concatenate([o1, o2]), o)
    assert np.array_equal(S2, S)


def test_units_are_independent():
    rng = np.random.default_rng(17)
    U, T, dk, dv = 5, 20, 6, 4
    q = unit_rows(rng.standard_normal((U, T, dk)))
    k = unit_rows(rng.standard_normal((U, T, dk)))
    v = rng.standard_normal((U, T, dv))
    a = rng.uniform(0.5, 1, (U, T))
    b = rng.uniform(0, 1, (U, T))
    o, S = oracle.forward_units(q, k, v, a, b)
    perm = np.array([3, 0, 4, 1, 2])
    o2, S2 = oracle.forward_units(q[perm], k[perm], v[perm], a[perm], b[perm])
    assert np.array_equal(o2, o[perm]) and np.array_equal(S2, S[perm])
    for u in range(U):
        ou, Su = run(q[u], k[u], v[u], a[u], b[u])
        assert np.array_equal(ou, o[u]) and np.array_equal(Su, S[u])


def test_alpha_zero_clears_the_state():
    """alpha = 0 (the limiting case of the forget gate) erases everything before."""
    q, k, v, a, b = random_unit(T=20, dk=6, dv=4, seed=18)
    a[9] = 0.0
    o, S = run(q, k, v, a, b, h0=np.ones((6, 4)))
    o2, S2 = run(q[9:], k[9:], v[9:], a[9:], b[9:])
    assert close(o[9:], o2) and close(S, S2)


# ---------------------------------------------------------------------------
# Layout helpers of the oracle (grouped heads, packed batches, decode)
# ---------------------------------------------------------------------------

def test_batch_layout_grouped_heads_and_packing():
    rng = np.random.default_rng(19)
    lens = [5, 17, 1, 9]
    N, H_qk, H_v, dk, dv = sum(lens), 2, 4, 6, 3
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = rng.standard_normal((1, N, H_qk, dk)).astype(np.float32)
    k = rng.standard_normal((1, N, H_qk, dk)).astype(np.float32)
    v = rng.standard_normal((1, N, H_v, dv)).astype(np.float32)
    a = rng.uniform(0.5, 1, (1, N, H_v)).astype(np.float32)
    b = rng.uniform(0, 1, (1, N, H_v)).astype(np.float32)
    h0 = rng.standard_normal((len(lens), H_v, dk, dv)).astype(np.float32)
    o, hT = oracle.forward(q, k, v, a, b, cu_seqlens=cu, h0=h0)
    for i in range(len(lens)):
        s, e = cu[i], cu[i + 1]
        for j in range(H_v):
            hq = j // (H_v // H_qk)
            ou, Su = run(q[0, s:e, hq], k[0, s:e, hq], v[0, s:e, j], a[0, s:e, j], b[0, s:e, j],
                         h0=h0[i, j])
            assert np.array_equal(o[0, s:e, j], ou)
            assert np.array_equal(hT[i, j], Su)
    sub = oracle.forward(q, k, v, a, b, cu_seqlens=cu, h0=h0, units=[(1, 3), (3, 0)])
    assert np.array_equal(sub[(1, 3)][0], o[0, cu[1]:cu[2], 3])
    assert np.array_equal(sub[(3, 0)][1], hT[3, 0])


# ---------------------------------------------------------------------------
# Planted mistakes: each mutant of the oracle must fail at least one pin.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mutant", [1, 2, 3, 4, 5])
def test_pins_catch_planted_mistakes(mutant):
    lib = oracle.load_mutant(mutant)
    assert lib.gdn_oracle_mutant() == mutant
    results = [check_walkthrough(lib), check_figure6(lib), check_additive_brute_force(lib),
               check_whole_sequence_solve(lib)]
    assert not all(results), f"mutant {mutant} passed every pin"


# ---------------------------------------------------------------------------
# The bf16 widening the oracle applies to uint16 bit patterns
# ---------------------------------------------------------------------------

def test_bf16_widening_exact_values():
    """bf16 is the top half of an IEEE binary32: sign, 8 exponent bits, 7
    mantissa bits.  Bit patterns with known values: 1, -2.5, the smallest
    subnormal 2^-133, the largest finite value (2 - 2^-7) 2^127, infinities
    and a NaN."""
    bits = np.array([0x3F80, 0xC020, 0x0001, 0x8001, 0x7F7F, 0x7F80, 0xFF80, 0x0000, 0x8000,
                     0x3E80, 0x4049], dtype=np.uint16)
    want = np.array([1.0, -2.5, 2.0 ** -133, -(2.0 ** -133), (2.0 - 2.0 ** -7) * 2.0 ** 127,
                     np.inf, -np.inf, 0.0, -0.0, 0.25, 3.140625])
    got = oracle._as_f64(bits)
    assert got.dtype == np.float64
    assert np.array_equal(got, want)
    assert np.signbit(got[8]) and not np.signbit(got[7])
    assert np.isnan(oracle._as_f64(np.array([0x7FC0], dtype=np.uint16)))[0]


def test_bf16_widening_matches_torch_on_every_pattern():
    """Every one of the 65,536 patterns widens as torch's bfloat16 -> float64."""
    import torch
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle._as_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_forward_on_bf16_bits_equals_forward_on_their_values():
    """A batch handed over as bf16 bit patterns gives the result of the same
    batch handed over as the float64 values torch assigns those patterns."""
    import torch
    rng = np.random.default_rng(11)
    B, T, H_qk, H_v, dk, dv = 2, 9, 1, 2, 8, 4
    def bf16(shape, scale=1.0):
        x = torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32))
        return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    q, k, v = bf16((B, T, H_qk, dk), 0.3), bf16((B, T, H_qk, dk), 0.3), bf16((B, T, H_v, dv))
    alpha = rng.uniform(0.5, 1.0, (B, T, H_v))
    beta = rng.uniform(0.0, 1.0, (B, T, H_v))
    def widen(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    o_bits, h_bits = oracle.forward(q, k, v, alpha, beta)
    o_vals, h_vals = oracle.forward(widen(q), widen(k), widen(v), alpha, beta)
    assert np.array_equal(o_bits, o_vals) and np.array_equal(h_bits, h_vals)
    # and the bits are not read as integers: the result differs from that reading
    o_int, _ = oracle.forward(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                              alpha, beta)
    assert not np.allclose(o_int, o_bits)
