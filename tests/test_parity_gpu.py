"""GPU parity: every entry point of libgdn, through the C ABI, against the oracle.

Small cases span several 64-token chunks and a ragged tail and finish in
seconds on the oracle; the full-size cases use the five target workloads in
the launch configuration the benchmark times.  Bars (max per-unit relative
error): 1e-4 for float32 inputs, 2e-2 for bf16 inputs with a float32 state.
"""
import numpy as np
import pytest

import gdn_inputs as gi
import oracle
from gpu_util import ELEM_TOL, TOL, dev_tensor, host_f64, local_errors, log, to_device, unit_rel_errors

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import torch
    import gated_delta_rule_03_amd as g
    assert torch.cuda.is_available()
    g.load()
    return g


def run_path(gdn, path, w, h0=None, chunk=None):
    import torch
    d = to_device(w)
    h0_t = None if h0 is None else dev_tensor(h0)
    if path == "chunk":
        o, hT = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                              chunk=chunk or w.spec.chunk, cu_seqlens=d["cu_seqlens"], h0=h0_t)
    else:
        o, hT = gdn.recurrent_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                  cu_seqlens=d["cu_seqlens"], h0=h0_t)
    torch.cuda.synchronize()
    return host_f64(o), host_f64(hT)


def check(gdn, path, w, h0=None, chunk=None, tol=None, units=None):
    log(f"[{path}] {w.spec.name} dtype={w.spec.dtype} B={w.B} T={w.T} H_qk={w.spec.H_qk} "
        f"H_v={w.spec.H_v} d_k={w.spec.d_k} d_v={w.spec.d_v} chunk={chunk or w.spec.chunk} "
        f"packed={w.cu_seqlens is not None} h0={h0 is not None}")
    o, hT = run_path(gdn, path, w, h0=h0, chunk=chunk)
    o_ref, hT_ref = oracle.forward(w.q, w.k, w.v, w.alpha, w.beta, cu_seqlens=w.cu_seqlens,
                                   h0=h0)
    eo, eh, unit = unit_rel_errors(o, hT, o_ref, hT_ref, w.seq_slices(), w.spec.H_v)
    ew, ee = local_errors(o, o_ref, w.seq_slices(), w.spec.H_v)
    bar = tol or TOL[w.spec.dtype]
    log(f"    max rel err o={eo:.3e} hT={eh:.3e} (worst unit {unit}) bar={bar}; "
        f"64-token windows o={ew:.3e}; elementwise o={ee:.3e} bar={ELEM_TOL[w.spec.dtype]}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(hT))
    assert eo <= bar and eh <= bar
    assert ew <= bar and ee <= ELEM_TOL[w.spec.dtype]
    return o, hT


def small(dtype, B, T, H_qk, H_v, d_k, d_v, chunk, seed, lengths=None):
    gates = "tiny" if dtype == "f32" else "prefill"
    return gi.generate(gi.Spec(f"small-{dtype}", B=B, T=T, H_qk=H_qk, H_v=H_v, d_k=d_k, d_v=d_v,
                               dtype=dtype, chunk=chunk, gates=gates, q_scale=dtype == "bf16",
                               lengths=lengths, seed=seed))


SMALL = [
    # dtype, B, T, H_qk, H_v, d_k, d_v, chunk
    ("f32", 2, 200, 2, 2, 64, 32, 64),
    ("f32", 1, 100, 1, 2, 32, 64, 32),
    ("f32", 1, 130, 1, 1, 128, 128, 64),
    ("f32", 2, 77, 1, 1, 16, 16, 16),
    ("bf16", 2, 300, 4, 4, 128, 128, 64),
    ("bf16", 1, 129, 2, 4, 64, 128, 64),
    ("bf16", 1, 190, 2, 2, 128, 64, 32),
]


def test_tiny_config_recurrent_and_chunked_agree(gdn):
    """Config 1: both paths match the oracle to 1e-4 and each other to 1e-4."""
    w = gi.generate(gi.config(1))
    o_c, h_c = check(gdn, "chunk", w)
    o_r, h_r = check(gdn, "recurrent", w)
    scale = max(np.max(np.abs(o_r)), 1e-30)
    assert np.max(np.abs(o_c - o_r)) / scale <= 1e-4
    assert np.max(np.abs(h_c - h_r)) / max(np.max(np.abs(h_r)), 1e-30) <= 1e-4


@pytest.mark.parametrize("case", SMALL, ids=[f"{c[0]}-B{c[1]}T{c[2]}H{c[3]}_{c[4]}d{c[5]}_{c[6]}C{c[7]}"
                                              for c in SMALL])
@pytest.mark.parametrize("path", ["chunk", "recurrent"])
def test_small_uniform(gdn, case, path):
    dtype, B, T, H_qk, H_v, d_k, d_v, chunk = case
    w = small(dtype, B, T, H_qk, H_v, d_k, d_v, chunk, seed=100 + SMALL.index(case))
    h0 = gi.random_state((B, H_v, d_k, d_v), seed=7, scale=0.3)
    check(gdn, path, w, chunk=chunk)
    check(gdn, path, w, h0=h0, chunk=chunk)


# Off the staged path (fp32 inputs, d_k < 128, d_v = 16) the chunked forward
# runs the chained kernels.  Below 256 blocks of 32 value columns they use
# 16-column blocks (every small case above); these have enough units for
# 32-column blocks, with grouped heads, packed sequences and every chunk size.
CHAINED_WIDE = [
    # dtype, B, T, H_qk, H_v, d_k, d_v, chunk
    ("f32", 4, 70, 16, 16, 128, 128, 64),
    ("bf16", 2, 100, 64, 128, 64, 64, 32),
    ("f32", 8, 40, 32, 32, 32, 32, 16),
]


@pytest.mark.parametrize("case", CHAINED_WIDE, ids=[f"{c[0]}-B{c[1]}T{c[2]}H{c[3]}_{c[4]}d{c[5]}_{c[6]}C{c[7]}"
                                                    for c in CHAINED_WIDE])
def test_chained_wide_blocks(gdn, case):
    dtype, B, T, H_qk, H_v, d_k, d_v, chunk = case
    assert B * H_v * (d_v // 32) >= 256
    w = small(dtype, B, T, H_qk, H_v, d_k, d_v, chunk, seed=150 + CHAINED_WIDE.index(case))
    check(gdn, "chunk", w, chunk=chunk)
    check(gdn, "chunk", w, h0=gi.random_state((B, H_v, d_k, d_v), seed=13, scale=0.3), chunk=chunk)


def test_chained_wide_blocks_packed(gdn):
    lengths = (0, 1, 63, 64, 65, 130, 7, 200) * 4
    w = small("f32", 1, 0, 8, 32, 64, 64, 64, seed=160, lengths=lengths)
    assert len(lengths) * 32 * 2 >= 256
    check(gdn, "chunk", w)
    check(gdn, "chunk", w, h0=gi.random_state((len(lengths), 32, 64, 64), seed=14, scale=0.3))


# bf16 with d_k = 128 and d_v a multiple of 32 runs the staged kernels: value
# widths of one and two 32-column blocks, unit counts that are not a
# multiple of the eight-unit block groups, a single partial chunk, one token,
# and the small chunk sizes.
STAGED = [
    # B, T, H_qk, H_v, d_v, chunk
    (3, 150, 3, 3, 32, 64),
    (1, 333, 1, 3, 64, 64),
    (3, 50, 1, 1, 128, 64),
    (2, 1, 2, 2, 128, 64),
    (1, 200, 1, 2, 64, 16),
    (1, 97, 2, 2, 128, 32),
]


@pytest.mark.parametrize("case", STAGED, ids=[f"B{c[0]}T{c[1]}H{c[2]}_{c[3]}dv{c[4]}C{c[5]}" for c in STAGED])
def test_staged_shapes(gdn, case):
    B, T, H_qk, H_v, d_v, chunk = case
    w = small("bf16", B, T, H_qk, H_v, 128, d_v, chunk, seed=200 + STAGED.index(case))
    check(gdn, "chunk", w, chunk=chunk)
    check(gdn, "chunk", w, h0=gi.random_state((B, H_v, 128, d_v), seed=11, scale=0.3), chunk=chunk)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("path,chunk", [("chunk", 64), ("chunk", 32), ("recurrent", None)])
def test_small_packed_grouped_heads(gdn, dtype, path, chunk):
    lengths = (1, 64, 65, 0, 130, 17, 128)
    w = small(dtype, 1, 0, 2, 4, 128, 128, chunk or 64, seed=31, lengths=lengths)
    h0 = gi.random_state((len(lengths), 4, 128, 128), seed=8, scale=0.3)
    check(gdn, path, w, chunk=chunk)
    check(gdn, path, w, h0=h0, chunk=chunk)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_many_packed_sequences(gdn, dtype):
    """1,100 ragged sequences of 0-40 tokens: more than the 1,024 the device
    ranks by length (beyond that the scan walks them in index order)."""
    rng = np.random.default_rng(77)
    lengths = tuple(int(x) for x in rng.integers(0, 41, size=1100))
    w = small(dtype, 1, 0, 1, 2, 128, 64 if dtype == "bf16" else 32, 64, seed=78, lengths=lengths)
    check(gdn, "chunk", w)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_small_decode(gdn, dtype):
    import torch
    w = small(dtype, 5, 1, 2, 4, 128, 64, 64, seed=41)
    state = gi.random_state((5, 4, 128, 64), seed=9, scale=0.5)
    log(f"[decode] small dtype={dtype}")
    d = to_device(w)
    st = dev_tensor(state)
    o = gdn.decode_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], st)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.decode(state, w.q, w.k, w.v, w.alpha, w.beta)
    eo, eh, _ = unit_rel_errors(host_f64(o), host_f64(st), o_ref, s_ref, w.seq_slices(), 4)
    log(f"    max rel err o={eo:.3e} state={eh:.3e}")
    assert eo <= TOL[dtype] and eh <= TOL[dtype]


def test_empty_sequences_return_initial_state(gdn):
    import torch
    w = small("f32", 2, 0, 1, 2, 32, 32, 64, seed=3)
    h0 = gi.random_state((2, 2, 32, 32), seed=4)
    for path in ("chunk", "recurrent"):
        log(f"[{path}] T = 0")
        _, hT = run_path(gdn, path, w, h0=h0)
        assert np.array_equal(hT, h0.astype(np.float64))


def test_beta_zero_keeps_state_bitwise(gdn):
    """beta = 0 and alpha = 1: no write and no decay, so the state is unchanged."""
    w = small("bf16", 1, 200, 2, 2, 128, 128, 64, seed=5)
    w.beta[:] = 0.0
    w.alpha[:] = 1.0
    h0 = gi.random_state((1, 2, 128, 128), seed=6)
    for path in ("chunk", "recurrent"):
        log(f"[{path}] beta = 0")
        _, hT = run_path(gdn, path, w, h0=h0)
        assert np.array_equal(hT, h0.astype(np.float64))


def test_alpha_zero_tokens(gdn):
    w = small("f32", 1, 150, 1, 1, 64, 64, 64, seed=12)
    w.alpha[0, [0, 40, 64, 99], 0] = 0.0
    for path in ("chunk", "recurrent"):
        check(gdn, path, w, h0=gi.random_state((1, 1, 64, 64), seed=2))


def test_bitwise_deterministic_and_split_invariant(gdn):
    import torch
    w = small("bf16", 2, 256, 2, 2, 128, 128, 64, seed=21)
    d = to_device(w)
    log("[chunk] determinism and split invariance")
    o1, h1 = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"])
    o2, h2 = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    cut = 128  # a chunk boundary: both halves run the same per-chunk arithmetic
    sl = lambda t, a, b: t[:, a:b].contiguous()
    oa, ha = gdn.chunk_fwd(*(sl(d[n], 0, cut) for n in ("q", "k", "v", "alpha", "beta")))
    ob, hb = gdn.chunk_fwd(*(sl(d[n], cut, 256) for n in ("q", "k", "v", "alpha", "beta")), h0=ha)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([oa, ob], dim=1), o1)
    assert torch.equal(hb, h1)


# ---------------------------------------------------------------------------
# Full-size workloads
# ---------------------------------------------------------------------------

def test_config2_prefill_full(gdn):
    w = gi.generate(gi.config(2))
    check(gdn, "chunk", w)


def test_config4_long_context_full(gdn):
    w = gi.generate(gi.config(4))
    check(gdn, "chunk", w)


def test_config5_packed_grouped_full(gdn):
    w = gi.generate(gi.config(5))
    log(f"    packed tokens = {w.n_tokens}, sequences = {w.n_seqs}")
    check(gdn, "chunk", w)


def test_config3_decode_full(gdn):
    """Config 3: state from the oracle's 512-token forward, then one token."""
    import torch
    spec = gi.config(3)
    warm = gi.generate(gi.decode_warmup_spec(spec))
    log("[decode] config 3: oracle warm-up over 512 tokens for 8192 units")
    _, S0 = oracle.forward(warm.q, warm.k, warm.v, warm.alpha, warm.beta, return_o=False)
    state = S0.astype(np.float32)
    w = gi.generate(spec)
    d = to_device(w)
    st = dev_tensor(state)
    o = gdn.decode_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], st)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.decode(state, w.q, w.k, w.v, w.alpha, w.beta)
    eo, eh, unit = unit_rel_errors(host_f64(o), host_f64(st), o_ref, s_ref, w.seq_slices(), 32)
    _, ee = local_errors(host_f64(o), o_ref, w.seq_slices(), 32)
    log(f"    max rel err o={eo:.3e} state={eh:.3e} (worst unit {unit}); elementwise o={ee:.3e}")
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"] and ee <= ELEM_TOL["bf16"]
