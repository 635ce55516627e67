"""Non-finite inputs: a NaN or an Inf planted in one unit's input reaches that
unit's outputs (or state), every other unit's results stay bitwise equal to a
clean run, and every call returns (no kernel has a data-dependent loop).

Units are independent (one value head per query/key head here, so nothing is
summed across heads), which is what makes the bitwise comparison exact.  The
chunked form multiplies whole chunks through its triangular matrices, and on
MFMA 0 x NaN is NaN, so inside the planted unit a NaN may also reach tokens
of its chunk that come before it; the token loop does not do that.  The test
therefore asks only that the planted unit is affected, not where.
"""
import numpy as np
import pytest

import gdn_inputs as gi
from gpu_util import dev_tensor, host_f64, log

pytestmark = pytest.mark.gpu

B, T, H, D, CHUNK = 2, 100, 2, 128, 64
UNIT = (1, 1)       # (sequence, head) that gets the non-finite value
TOK, COL = 40, 5


@pytest.fixture(scope="module")
def gdn():
    import torch
    import gated_delta_rule_03_amd as g
    assert torch.cuda.is_available()
    g.load()
    return g


def inputs(dtype, seed):
    w = gi.generate(gi.Spec(f"nan-{dtype}", B=B, T=T, H_qk=H, H_v=H, d_k=D, d_v=D, dtype=dtype, chunk=CHUNK,
                            gates="prefill", q_scale=True, seed=seed))
    return w


def plant(x, value, dtype, index):
    y = np.array(x, copy=True)
    y[index] = gi.f32_to_bf16_bits(np.array([value], np.float32))[0] if dtype == "bf16" else value
    return y


def split_units(a, unit_axes=(0, 2)):
    """The planted unit's slice and a mask of everything else."""
    b, h = UNIT
    idx = [slice(None)] * a.ndim
    idx[unit_axes[0]] = b
    idx[unit_axes[1]] = h
    mask = np.ones(a.shape, bool)
    mask[tuple(idx)] = False
    return a[tuple(idx)], mask


def check(name, clean, dirty, unit_axes):
    """clean, dirty: lists of host arrays (same order); unit_axes per array."""
    affected = False
    for c, d, ax in zip(clean, dirty, unit_axes):
        part, mask = split_units(d, ax)
        assert np.array_equal(c[mask], d[mask]), f"{name}: another unit changed"
        affected |= not np.isfinite(part).all()
    log(f"[nan] {name}: other units bitwise unchanged, planted unit non-finite={affected}")
    assert affected, f"{name}: the planted value did not reach its unit"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("value", [float("nan"), float("inf")])
def test_forward_paths(gdn, dtype, value):
    import torch
    w = inputs(dtype, 940 + (dtype == "f32"))
    v_bad = plant(w.v, value, dtype, (UNIT[0], TOK, UNIT[1], COL))
    rates = gi.channel_rates(B, T, H, D, 944)
    for fn in ("chunk_fwd", "recurrent_fwd", "kda_chunk_fwd"):
        outs = []
        for v in (w.v, v_bad):
            alpha = rates if fn == "kda_chunk_fwd" else w.alpha
            args = [dev_tensor(x) for x in (w.q, w.k, v, alpha, w.beta)]
            if fn == "recurrent_fwd":
                o, hT = gdn.recurrent_fwd(*args)
            elif fn == "kda_chunk_fwd":
                o, hT = gdn.kda_chunk_fwd(*args, chunk=CHUNK)
            else:
                o, hT = gdn.chunk_fwd(*args, chunk=CHUNK)
            torch.cuda.synchronize()
            outs.append([host_f64(o), host_f64(hT)])
        check(f"{fn} {dtype} v={value}", outs[0], outs[1], [(0, 2), (0, 1)])


@pytest.mark.parametrize("value", [float("nan"), float("inf")])
def test_decode(gdn, value):
    import torch
    w = gi.generate(gi.Spec("nan-decode", B=B, T=1, H_qk=H, H_v=H, d_k=D, d_v=D, dtype="bf16", chunk=CHUNK,
                            gates="prefill", q_scale=True, seed=946))
    state0 = gi.random_state((B, H, D, D), seed=947, scale=0.3)
    bad = np.array(state0, copy=True)
    bad[UNIT[0], UNIT[1], 3, COL] = value
    outs = []
    for st in (state0, bad):
        s = dev_tensor(st)
        o = gdn.decode_step(*[dev_tensor(x) for x in (w.q, w.k, w.v, w.alpha, w.beta)], s)
        torch.cuda.synchronize()
        outs.append([host_f64(o), host_f64(s)])
    check(f"decode state={value}", outs[0], outs[1], [(0, 2), (0, 1)])


@pytest.mark.parametrize("value", [float("nan"), float("inf")])
def test_backward(gdn, value):
    import torch
    w = inputs("bf16", 948)
    do32 = gi.random_state((B, T, H, D), seed=949)
    do = gi.f32_to_bf16_bits(do32)
    do_bad = plant(do, value, "bf16", (UNIT[0], TOK, UNIT[1], COL))
    outs = []
    for d_o in (do, do_bad):
        g = gdn.chunk_bwd(*[dev_tensor(x) for x in (w.q, w.k, w.v, w.alpha, w.beta)], dev_tensor(d_o), chunk=CHUNK)
        torch.cuda.synchronize()
        outs.append([host_f64(x) for x in g])
    check(f"chunk_bwd d_o={value}", outs[0], outs[1], [(0, 2)] * 5 + [(0, 1)])
