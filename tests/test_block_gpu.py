"""GPU parity of the GDN block's prologue and epilogue kernels (through the C
ABI) against the float64 block oracle, and of a whole block -- prologue,
chunked recurrence, epilogue -- against the oracle composed the same way.

Metric as the other parity tests: per (sequence, head) slice, max |X - X_ref|
over max |X_ref|; bars 1e-4 (float32) and 2e-2 (bf16).
"""
import numpy as np
import pytest

import gdn_inputs as gi
import oracle
from oracle import block as ob
from gpu_util import TOL, dev_tensor, host_f64, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import torch
    import gated_delta_rule_03_amd as g
    assert torch.cuda.is_available()
    g.load()
    return g


def slices(x):
    if x["cu_seqlens"] is None:
        return [(b, 0, x["T"]) for b in range(x["B"])]
    cu = x["cu_seqlens"]
    return [(0, int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)]


def rel_err(got, ref, sl):
    """Max over (sequence, head) slices of max |got - ref| / max |ref|."""
    worst = 0.0
    for b, s, e in sl:
        if e == s:
            continue
        for h in range(ref.shape[2]):
            r = ref[b, s:e, h]
            den = max(float(np.max(np.abs(r))), 1e-30)
            worst = max(worst, float(np.max(np.abs(got[b, s:e, h] - r))) / den)
    return worst


def run_prologue(gdn, x, q_scale):
    d = {n: dev_tensor(x[n]) for n in ("q_raw", "k_raw", "v_raw", "conv_q", "conv_k", "conv_v", "conv_q_bias",
                                       "conv_k_bias", "conv_v_bias", "a_raw", "b_raw", "log_A", "v_norm")}
    cu = None if x["cu_seqlens"] is None else dev_tensor(x["cu_seqlens"])
    return gdn.block_prologue(d["q_raw"], d["k_raw"], d["v_raw"], d["conv_q"], d["conv_k"], d["conv_v"],
                              d["a_raw"], d["b_raw"], d["log_A"], conv_q_bias=d["conv_q_bias"],
                              conv_k_bias=d["conv_k_bias"], conv_v_bias=d["conv_v_bias"],
                              v_norm_weight=d["v_norm"], eps=1e-6, q_scale=q_scale, cu_seqlens=cu), cu


def oracle_prologue(x, q_scale):
    return ob.prologue(x["q_raw"], x["k_raw"], x["v_raw"], x["conv_q"], x["conv_k"], x["conv_v"], x["a_raw"],
                       x["b_raw"], x["log_A"], conv_q_bias=x["conv_q_bias"], conv_k_bias=x["conv_k_bias"],
                       conv_v_bias=x["conv_v_bias"], norm_weight=x["v_norm"], eps=1e-6, q_scale=q_scale,
                       cu_seqlens=x["cu_seqlens"])


PROLOGUE = [
    # dtype, B, T, H_qk, H_v, d_k, d_v, lengths
    ("f32", 2, 150, 2, 4, 128, 128, None),
    ("f32", 1, 0, 1, 2, 64, 32, (1, 2, 3, 0, 70, 5)),
    ("f32", 3, 37, 1, 1, 16, 16, None),
    ("bf16", 2, 150, 2, 4, 128, 128, None),
    ("bf16", 1, 0, 2, 2, 128, 64, (130, 1, 0, 64, 65, 3)),
]


@pytest.mark.parametrize("case", PROLOGUE, ids=[f"{c[0]}-B{c[1]}T{c[2]}H{c[3]}_{c[4]}d{c[5]}_{c[6]}"
                                                + ("-packed" if c[7] else "") for c in PROLOGUE])
def test_block_prologue(gdn, case):
    import torch
    dtype, B, T, H_qk, H_v, d_k, d_v, lengths = case
    x = gi.block_inputs(B, T, H_qk, H_v, d_k, d_v, dtype, seed=300 + PROLOGUE.index(case), lengths=lengths)
    log(f"[prologue] {case}")
    (q, k, v, alpha, beta), _ = run_prologue(gdn, x, 0.125)
    torch.cuda.synchronize()
    ref = oracle_prologue(x, 0.125)
    sl = slices(x)
    errs = [rel_err(host_f64(t), r, sl) for t, r in zip((q, k, v), ref[:3])]
    errs += [rel_err(host_f64(t)[..., None], r[..., None], sl) for t, r in zip((alpha, beta), ref[3:])]
    log(f"    max rel err q={errs[0]:.3e} k={errs[1]:.3e} v={errs[2]:.3e} alpha={errs[3]:.3e} beta={errs[4]:.3e}")
    # alpha and beta are float32 for either dtype
    assert max(errs[:3]) <= TOL[dtype] and max(errs[3:]) <= TOL["f32"]


@pytest.mark.parametrize("dtype,d_v", [("f32", 128), ("f32", 16), ("bf16", 128), ("bf16", 64)])
def test_block_epilogue(gdn, dtype, d_v):
    import torch
    x = gi.block_inputs(2, 77, 1, 3, 64, d_v, dtype, seed=320 + d_v)
    log(f"[epilogue] {dtype} d_v={d_v}")
    o, g = dev_tensor(x["v_raw"]), dev_tensor(x["g_raw"])
    y = gdn.block_epilogue(o, g, o_norm_weight=dev_tensor(x["o_norm"]), eps=1e-6)
    torch.cuda.synchronize()
    ref = ob.epilogue(x["v_raw"], x["g_raw"], x["o_norm"], 1e-6)
    err = rel_err(host_f64(y), ref, slices(x))
    log(f"    max rel err y={err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype,lengths", [("f32", None), ("bf16", None), ("bf16", (200, 1, 0, 96, 65))])
def test_whole_block(gdn, dtype, lengths):
    """Prologue -> chunked recurrence -> epilogue, against the float64 oracle of
    the same composition (the block's output before its final projection)."""
    import torch
    x = gi.block_inputs(2, 160, 2, 4, 128, 128, dtype, seed=340, lengths=lengths)
    log(f"[block] {dtype} packed={lengths is not None}")
    q_scale = 1.0 / np.sqrt(128.0)
    (q, k, v, alpha, beta), cu = run_prologue(gdn, x, q_scale)
    o, _ = gdn.chunk_fwd(q, k, v, alpha, beta, chunk=64, cu_seqlens=cu)
    y = gdn.block_epilogue(o, dev_tensor(x["g_raw"]), o_norm_weight=dev_tensor(x["o_norm"]), eps=1e-6)
    torch.cuda.synchronize()
    rq, rk, rv, ra, rb = oracle_prologue(x, q_scale)
    ro, _ = oracle.forward(rq, rk, rv, ra, rb, cu_seqlens=x["cu_seqlens"])
    ref = ob.epilogue(ro, x["g_raw"], x["o_norm"], 1e-6)
    err = rel_err(host_f64(y), ref, slices(x))
    log(f"    max rel err y={err:.3e}")
    assert np.all(np.isfinite(host_f64(y))) and err <= TOL[dtype]


def test_block_full_prefill_shape(gdn):
    """Prologue and epilogue at the bench's shape (B=4, T=4096, H=16, d=128,
    bf16), in the launch configuration the bench times, against the float64
    oracle on every output."""
    x = gi.block_inputs(4, 4096, 16, 16, 128, 128, "bf16", seed=360)
    log("[block full] B=4 T=4096 H=16 d=128 bf16")
    (q, k, v, alpha, beta), _ = run_prologue(gdn, x, 128 ** -0.5)
    y = gdn.block_epilogue(dev_tensor(x["v_raw"]), dev_tensor(x["g_raw"]), o_norm_weight=dev_tensor(x["o_norm"]),
                           eps=1e-6)
    import torch
    torch.cuda.synchronize()
    ref = oracle_prologue(x, 128 ** -0.5)
    sl = slices(x)
    errs = [rel_err(host_f64(t), r, sl) for t, r in zip((q, k, v), ref[:3])]
    errs += [rel_err(host_f64(t)[..., None], r[..., None], sl) for t, r in zip((alpha, beta), ref[3:])]
    ey = rel_err(host_f64(y), ob.epilogue(x["v_raw"], x["g_raw"], x["o_norm"], 1e-6), sl)
    log(f"    max rel err q={errs[0]:.3e} k={errs[1]:.3e} v={errs[2]:.3e} alpha={errs[3]:.3e} "
        f"beta={errs[4]:.3e} y={ey:.3e}")
    assert max(errs[:3] + [ey]) <= TOL["bf16"] and max(errs[3:]) <= TOL["f32"]


def test_block_prologue_many_short_sequences(gdn):
    """A packed batch of 700 sequences of 0 to 40 tokens: many sequence starts
    inside each 64-token run, empty sequences and sequences shorter than the
    convolution."""
    rng = np.random.default_rng(370)
    lengths = tuple(int(v) for v in rng.integers(0, 41, 700))
    x = gi.block_inputs(1, 0, 2, 4, 64, 128, "f32", seed=371, lengths=lengths)
    log(f"[prologue packed] {len(lengths)} sequences, {sum(lengths)} tokens")
    (q, k, v, alpha, beta), _ = run_prologue(gdn, x, 1.0)
    import torch
    torch.cuda.synchronize()
    ref = oracle_prologue(x, 1.0)
    sl = slices(x)
    errs = [rel_err(host_f64(t), r, sl) for t, r in zip((q, k, v), ref[:3])]
    log(f"    max rel err q={errs[0]:.3e} k={errs[1]:.3e} v={errs[2]:.3e}")
    assert max(errs) <= TOL["f32"]


def test_whole_block_unequal_head_dims(gdn):
    """Prologue (two launches: q/k at d_k = 64, v at d_v = 128) -> chunked
    recurrence on the chained path -> epilogue, packed, float32, against the
    float64 oracle of the same composition."""
    import torch
    x = gi.block_inputs(1, 0, 2, 4, 64, 128, "f32", seed=380, lengths=(90, 1, 0, 130))
    log("[block] f32 d_k=64 d_v=128 packed")
    (q, k, v, alpha, beta), cu = run_prologue(gdn, x, 0.125)
    o, _ = gdn.chunk_fwd(q, k, v, alpha, beta, chunk=32, cu_seqlens=cu)
    y = gdn.block_epilogue(o, dev_tensor(x["g_raw"]), o_norm_weight=dev_tensor(x["o_norm"]), eps=1e-6)
    torch.cuda.synchronize()
    rq, rk, rv, ra, rb = oracle_prologue(x, 0.125)
    ro, _ = oracle.forward(rq, rk, rv, ra, rb, cu_seqlens=x["cu_seqlens"])
    ref = ob.epilogue(ro, x["g_raw"], x["o_norm"], 1e-6)
    err = rel_err(host_f64(y), ref, slices(x))
    log(f"    max rel err y={err:.3e}")
    assert np.all(np.isfinite(host_f64(y))) and err <= TOL["f32"]
