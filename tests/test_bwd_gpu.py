"""GPU parity of the backward pass (gdn_chunk_bwd) against the float64
gradient oracle (oracle/grad.py), through the C ABI.

The loss is L = sum_t <d_o_t, o_t> + <dhT, S_T> per sequence and value head;
every gradient (q, k, v, alpha, beta, h0) is compared per unit slice,
max |g - g_ref| / max |g_ref|.  The kernels compute in fp32 from the exact
input values (bf16 widens exactly), so both dtypes are held to the fp32 bar
of 1e-4.  Cases: uniform and packed batches (empty and one-token sequences,
ragged last chunks), grouped heads, h0 and dhT, chunks of 16, 32 and 64, the
sizes d_k, d_v in {16, ..., 128}, bf16 inputs, and run-to-run bitwise
equality; and the prefill shape at full size (B=4, T=4096, H=16, d=128,
bf16, chunk 64: the launch the benchmark times), checked on sampled units.
"""
import numpy as np
import pytest

import gdn_inputs as gi
from oracle import grad as ograd
from gpu_util import dev_tensor, host_f64, log

pytestmark = pytest.mark.gpu

BAR = 1e-4


@pytest.fixture(scope="module")
def gdn():
    import torch
    import gated_delta_rule_03_amd as g
    assert torch.cuda.is_available()
    g.load()
    return g


def rel(got, ref, unit_axes):
    """Max over unit slices (all axes but `unit_axes` reduced) of max|d| / max|ref|."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    d = np.abs(got - ref)
    red = tuple(a for a in range(ref.ndim) if a not in unit_axes)
    num = d.max(axis=red) if red else d
    den = np.maximum(np.abs(ref).max(axis=red) if red else np.abs(ref), 1e-30)
    return float(np.max(num / den)) if num.size else 0.0


# dtype, B, T, H_qk, H_v, d_k, d_v, chunk, lengths, h0, dhT
CASES = [
    ("f32", 2, 37, 1, 2, 32, 16, 16, None, True, True),
    ("f32", 1, 64, 2, 2, 16, 32, 64, None, False, False),
    ("f32", 1, 0, 1, 2, 64, 64, 32, (20, 0, 1, 45, 64), True, True),
    ("f32", 2, 100, 2, 4, 128, 128, 64, None, True, False),
    ("bf16", 2, 70, 2, 2, 128, 64, 64, None, False, True),
    ("bf16", 1, 0, 2, 4, 64, 128, 16, (33, 3, 0, 80), True, True),
    # bf16 in chunks of 32, a 16-column value block and d_k = 16: the split
    # (hi + lo) operand layouts at their other sizes
    ("bf16", 2, 90, 1, 2, 16, 16, 32, None, True, True),
    ("bf16", 1, 75, 2, 2, 32, 64, 32, None, False, True),
]


def run_case(gdn, case, seed):
    import torch
    dtype, B, T, H_qk, H_v, d_k, d_v, chunk, lengths, use_h0, use_dhT = case
    w = gi.generate(gi.Spec("bwd", B=B, T=T, H_qk=H_qk, H_v=H_v, d_k=d_k, d_v=d_v, dtype=dtype, chunk=chunk,
                            lengths=lengths, seed=seed))
    B, T = w.q.shape[0], w.q.shape[1]
    cu = w.cu_seqlens
    N = B if cu is None else len(cu) - 1
    h0 = gi.random_state((N, H_v, d_k, d_v), seed=seed + 1, scale=0.3) if use_h0 else None
    dhT = gi.random_state((N, H_v, d_k, d_v), seed=seed + 2, scale=0.5) if use_dhT else None
    do32 = gi.random_state((B, T, H_v, d_v), seed=seed + 3)
    do_dev = gi.f32_to_bf16_bits(do32) if dtype == "bf16" else do32
    do_ref = gi.bf16_bits_to_f32(do_dev) if dtype == "bf16" else do32
    log(f"[bwd] {dtype} B={B} T={T} H_qk={H_qk} H_v={H_v} d_k={d_k} d_v={d_v} chunk={chunk} "
        f"packed={cu is not None} h0={use_h0} dhT={use_dhT}")
    got = gdn.chunk_bwd(dev_tensor(w.q), dev_tensor(w.k), dev_tensor(w.v), dev_tensor(w.alpha),
                        dev_tensor(w.beta), dev_tensor(do_dev), chunk=chunk,
                        cu_seqlens=None if cu is None else dev_tensor(cu),
                        h0=None if h0 is None else dev_tensor(h0), dhT=None if dhT is None else dev_tensor(dhT))
    torch.cuda.synchronize()
    ref = ograd.backward(w.q, w.k, w.v, w.alpha, w.beta, do_ref, dhT, cu_seqlens=cu, h0=h0)
    return [host_f64(g) for g in got], ref, cu


def check(got, ref, cu):
    names = ("dq", "dk", "dv", "dalpha", "dbeta", "dh0")
    errs = {}
    if cu is None:
        # unit slices: (sequence, head) of the token-major tensors
        axes = {"dq": (0, 2), "dk": (0, 2), "dv": (0, 2), "dalpha": (0, 2), "dbeta": (0, 2), "dh0": (0, 1)}
        for n, g, r in zip(names, got, ref):
            errs[n] = rel(g, r, axes[n])
    else:
        for n, g, r in zip(names[:5], got[:5], ref[:5]):
            worst = 0.0
            for i in range(len(cu) - 1):
                s, e = int(cu[i]), int(cu[i + 1])
                if e > s:
                    worst = max(worst, rel(g[:, s:e], r[:, s:e], (2,)))
            errs[n] = worst
        errs["dh0"] = rel(got[5], ref[5], (0, 1))
    log("    " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= BAR}
    assert not bad, f"gradients off the oracle: {bad}"


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-B{c[1]}T{c[2]}H{c[3]}_{c[4]}d{c[5]}_{c[6]}C{c[7]}"
                                             + ("-packed" if c[8] else "") for c in CASES])
def test_chunk_bwd_matches_gradient_oracle(gdn, case):
    got, ref, cu = run_case(gdn, case, 700 + CASES.index(case))
    check(got, ref, cu)


def test_chunk_bwd_chunk_sizes_agree_and_repeat_bitwise(gdn):
    """Chunks of 16, 32 and 64 give the oracle's gradients; a second call is bitwise equal."""
    import torch
    base = ("f32", 1, 90, 1, 2, 64, 32, 16, None, True, True)
    outs = []
    for chunk in (16, 32, 64):
        case = base[:7] + (chunk,) + base[8:]
        got, ref, cu = run_case(gdn, case, 760)
        check(got, ref, cu)
        outs.append(got)
    again, _, _ = run_case(gdn, base[:7] + (64,) + base[8:], 760)
    for a, b in zip(outs[2], again):
        assert np.array_equal(a, b)
    torch.cuda.synchronize()


def test_chunk_bwd_prefill_shape_sampled_units(gdn):
    """The prefill workload at full size through one call; three units (first,
    last and one between, all 64 chunks of each) against the gradient oracle.
    Units are independent (one value head per query/key head here), so the
    oracle runs on those units alone."""
    import torch
    spec = gi.config(2)
    w = gi.generate(spec)
    B, T, H = w.q.shape[0], w.q.shape[1], w.q.shape[2]
    do32 = gi.random_state((B, T, H, spec.d_v), seed=spec.seed + 11)
    do_bits = gi.f32_to_bf16_bits(do32)
    log(f"[bwd] prefill shape B={B} T={T} H={H} d={spec.d_k} bf16 chunk 64")
    got = gdn.chunk_bwd(dev_tensor(w.q), dev_tensor(w.k), dev_tensor(w.v), dev_tensor(w.alpha),
                        dev_tensor(w.beta), dev_tensor(do_bits), chunk=64)
    torch.cuda.synchronize()
    got = [host_f64(g) for g in got]
    do_ref = gi.bf16_bits_to_f32(do_bits)
    for b, h in ((0, 0), (2, 7), (B - 1, H - 1)):
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        ref = ograd.backward(w.q[sl], w.k[sl], w.v[sl], w.alpha[sl], w.beta[sl], do_ref[sl], None)
        mine = [g[sl] for g in got[:5]] + [got[5][b:b + 1, h:h + 1]]
        log(f"    unit (b={b}, h={h})")
        check(mine, ref, None)
