"""GPU parity of the segment-parallel chunked forward (gdn_chunk_fwd_segmented,
and gdn_chunk_fwd where it picks segments by itself) against the oracle.

The segmented form computes the same function as the one-pass chunked
forward: each sequence is cut into segments whose affine state maps are
folded in order, then every segment's outputs are computed from its true
incoming state.  Cases: several segment lengths (one chunk, a length that
leaves a short last segment, longer than the sequence), fp32 and bf16, the
staged and the chained kernels, packed batches with empty and short
sequences and grouped heads, h0, and the long-context workload at full size
(as given, and at the two-head share of one GPU of an eight-way head split).
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


def run_seg(gdn, w, seg_chunks, h0=None, chunk=None):
    import torch
    d = to_device(w)
    h0_t = None if h0 is None else dev_tensor(h0)
    o, hT = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], chunk=chunk or w.spec.chunk,
                          cu_seqlens=d["cu_seqlens"], h0=h0_t, seg_chunks=seg_chunks)
    torch.cuda.synchronize()
    return host_f64(o), host_f64(hT)


def check_seg(gdn, w, seg_chunks, h0=None, chunk=None, ref=None):
    log(f"[segmented seg_chunks={seg_chunks}] {w.spec.name} dtype={w.spec.dtype} B={w.B} T={w.T} "
        f"H_qk={w.spec.H_qk} H_v={w.spec.H_v} d_k={w.spec.d_k} d_v={w.spec.d_v} "
        f"chunk={chunk or w.spec.chunk} packed={w.cu_seqlens is not None} h0={h0 is not None}")
    o, hT = run_seg(gdn, w, seg_chunks, h0=h0, chunk=chunk)
    if ref is None:
        ref = oracle.forward(w.q, w.k, w.v, w.alpha, w.beta, cu_seqlens=w.cu_seqlens, h0=h0)
    o_ref, hT_ref = ref
    eo, eh, unit = unit_rel_errors(o, hT, o_ref, hT_ref, w.seq_slices(), w.spec.H_v)
    ew, ee = local_errors(o, o_ref, w.seq_slices(), w.spec.H_v)
    bar = TOL[w.spec.dtype]
    log(f"    max rel err o={eo:.3e} hT={eh:.3e} (worst unit {unit}) bar={bar}; "
        f"64-token windows o={ew:.3e}; elementwise o={ee:.3e}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(hT))
    assert eo <= bar and eh <= bar and ew <= bar and ee <= ELEM_TOL[w.spec.dtype]
    return o, hT


def small(dtype, B, T, H_qk, H_v, d_k, d_v, chunk, seed, lengths=None, log_alpha_scale=1.0):
    gates = "tiny" if dtype == "f32" else "prefill"
    return gi.generate(gi.Spec(f"seg-{dtype}", B=B, T=T, H_qk=H_qk, H_v=H_v, d_k=d_k, d_v=d_v,
                               dtype=dtype, chunk=chunk, gates=gates, q_scale=dtype == "bf16",
                               lengths=lengths, log_alpha_scale=log_alpha_scale, seed=seed))


# bf16 with d_k = 128 (staged kernels) and the chained kernels (fp32; bf16
# with d_k < 128 or d_v = 16), including d_k not a multiple of 32 (16-column
# transition blocks)
UNIFORM = [
    # dtype, B, T, H_qk, H_v, d_k, d_v, chunk, segment lengths (chunks)
    ("bf16", 2, 1000, 2, 2, 128, 128, 64, (1, 3, 4, 40)),
    ("bf16", 1, 700, 1, 2, 128, 64, 32, (2, 5)),
    ("f32", 1, 300, 1, 1, 32, 64, 32, (1, 2, 7)),
    ("f32", 2, 150, 2, 2, 16, 16, 16, (3,)),
    ("bf16", 1, 900, 2, 2, 64, 64, 64, (2, 5)),
    ("bf16", 2, 400, 1, 2, 32, 16, 32, (1, 4)),
]


@pytest.mark.parametrize("case", UNIFORM, ids=[f"{c[0]}-B{c[1]}T{c[2]}H{c[3]}_{c[4]}d{c[5]}_{c[6]}C{c[7]}"
                                                for c in UNIFORM])
def test_segmented_uniform(gdn, case):
    dtype, B, T, H_qk, H_v, d_k, d_v, chunk, segs = case
    w = small(dtype, B, T, H_qk, H_v, d_k, d_v, chunk, seed=300 + UNIFORM.index(case), log_alpha_scale=0.25)
    h0 = gi.random_state((B, H_v, d_k, d_v), seed=13, scale=0.3)
    ref0 = oracle.forward(w.q, w.k, w.v, w.alpha, w.beta)
    ref1 = oracle.forward(w.q, w.k, w.v, w.alpha, w.beta, h0=h0)
    for sc in segs:
        check_seg(gdn, w, sc, chunk=chunk, ref=ref0)
        check_seg(gdn, w, sc, h0=h0, chunk=chunk, ref=ref1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_segmented_packed_grouped_heads(gdn, dtype):
    """Empty, one-token and chunk-boundary sequences; segments restart at
    every sequence; grouped heads (two value heads per query/key head)."""
    lengths = (0, 1, 200, 513, 64, 130, 0, 65)
    w = small(dtype, 1, 0, 2, 4, 128, 128, 64, seed=41, lengths=lengths)
    h0 = gi.random_state((len(lengths), 4, 128, 128), seed=14, scale=0.3)
    ref = oracle.forward(w.q, w.k, w.v, w.alpha, w.beta, cu_seqlens=w.cu_seqlens, h0=h0)
    for sc in (1, 2, 3):
        check_seg(gdn, w, sc, h0=h0, ref=ref)


def test_segmented_equals_one_pass_closely(gdn):
    """Same arithmetic per chunk, a different state path: the two forms agree
    to well inside the bf16 bar."""
    import torch
    w = small("bf16", 1, 2048, 2, 2, 128, 128, 64, seed=51, log_alpha_scale=0.1)
    o1, h1 = run_seg(gdn, w, 0)
    o2, h2 = run_seg(gdn, w, 4)
    so = max(np.max(np.abs(o1)), 1e-30)
    sh = max(np.max(np.abs(h1)), 1e-30)
    log(f"[segmented vs one pass] o {np.max(np.abs(o1 - o2)) / so:.3e} hT {np.max(np.abs(h1 - h2)) / sh:.3e}")
    assert np.max(np.abs(o1 - o2)) / so <= 1e-2 and np.max(np.abs(h1 - h2)) / sh <= 1e-2


def test_plan_picks_segments_for_few_long_units(gdn):
    """gdn_chunk_fwd segments a few long units by itself and not a full batch."""
    bf = gdn.GDN_BF16
    assert gdn.chunk_fwd_plan_segments(4, 4096, 16, 16, 128, 128, bf, 64, 0) == 0
    assert gdn.chunk_fwd_plan_segments(1, 65536, 16, 16, 128, 128, bf, 64, 0) > 0
    assert gdn.chunk_fwd_plan_segments(1, 65536, 2, 2, 128, 128, bf, 64, 0) > 0
    w = small("bf16", 1, 8192, 1, 1, 128, 128, 64, seed=61, log_alpha_scale=0.1)
    plan = gdn.chunk_fwd_plan_segments(1, 8192, 1, 1, 128, 128, bf, 64, 0)
    log(f"[plan] B=1 T=8192 H=1: {plan} chunks per segment")
    assert plan > 0
    check_seg(gdn, w, None)


def test_config4_long_context_other_forms_full(gdn):
    """The long-context workload (B=1, H=16, T=65536), which gdn_chunk_fwd
    cuts into 128-chunk segments, through the one-pass scan and through
    64-chunk segments."""
    w = gi.generate(gi.config(4))
    ref = oracle.forward(w.q, w.k, w.v, w.alpha, w.beta)
    check_seg(gdn, w, 0, ref=ref)
    check_seg(gdn, w, 64, ref=ref)


def test_config4_two_heads_auto(gdn):
    """The long-context workload at one GPU's share of an eight-way head split
    (2 heads): gdn_chunk_fwd picks the segmented form."""
    w = gi.generate(gi.config(4, H_qk=2, H_v=2, name="long-2heads"))
    plan = gdn.chunk_fwd_plan_segments(1, 65536, 2, 2, 128, 128, gdn.GDN_BF16, 64, 0)
    log(f"[plan] long context, 2 heads: {plan} chunks per segment")
    assert plan > 0
    check_seg(gdn, w, None)


def test_long_context_chained_f32_two_heads_auto(gdn):
    """fp32 inputs run the chained kernels; at the two-head share of the
    long-context workload gdn_chunk_fwd cuts them into segments too."""
    w = gi.generate(gi.config(4, H_qk=2, H_v=2, dtype="f32", name="long-2heads-f32"))
    plan = gdn.chunk_fwd_plan_segments(1, 65536, 2, 2, 128, 128, gdn.GDN_F32, 64, 0)
    log(f"[plan] long context, fp32, 2 heads: {plan} chunks per segment")
    assert 0 < plan < 1024
    check_seg(gdn, w, None)
