"""GPU parity of the per-channel-gate entry points (gdn_kda_recurrent_fwd,
gdn_kda_decode_step) against the float64 oracle ``oracle/kda.py``, through the
C ABI.  Metric as the other parity tests: per (sequence, head) and tensor,
max |X - X_ref| / max |X_ref|; bars 1e-4 (float32 inputs) and 2e-2 (bf16)."""
import numpy as np
import pytest

import gdn_inputs as gi
from oracle import kda
from gpu_util import TOL, dev_tensor, host_f64, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import torch
    import gated_delta_rule_03_amd as g
    assert torch.cuda.is_available()
    g.load()
    return g


def rel_err(got, ref):
    """Max over the leading (unit) slices of max |got - ref| / max |ref|."""
    g = got.reshape(-1, *got.shape[-2:]) if got.ndim > 3 else got
    r = ref.reshape(-1, *ref.shape[-2:]) if ref.ndim > 3 else ref
    worst = 0.0
    for a, b in zip(g, r):
        den = max(float(np.max(np.abs(b))), 1e-30)
        worst = max(worst, float(np.max(np.abs(a - b))) / den)
    return worst


CASES = [
    # dtype, B, T, H_qk, H_v, d_k, d_v, lengths
    ("f32", 2, 40, 1, 2, 16, 16, None),
    ("f32", 1, 0, 2, 4, 64, 128, (17, 0, 1, 30)),
    ("f32", 2, 33, 2, 2, 128, 64, None),
    ("bf16", 2, 64, 2, 4, 128, 128, None),
    ("bf16", 1, 0, 1, 4, 64, 32, (40, 3, 0, 77)),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-B{c[1]}T{c[2]}H{c[3]}_{c[4]}d{c[5]}_{c[6]}"
                                             + ("-packed" if c[7] else "") for c in CASES])
def test_kda_recurrent(gdn, case):
    import torch
    dtype, B, T, H_qk, H_v, d_k, d_v, lengths = case
    seed = 400 + CASES.index(case)
    w = gi.generate(gi.Spec("kda", B=B, T=T, H_qk=H_qk, H_v=H_v, d_k=d_k, d_v=d_v, dtype=dtype, chunk=64,
                            lengths=lengths, seed=seed))
    B, T = w.q.shape[0], w.q.shape[1]
    a = gi.channel_rates(B, T, H_v, d_k, seed + 50)
    cu = w.cu_seqlens
    N = B if cu is None else len(cu) - 1
    h0 = gi.random_state((N, H_v, d_k, d_v), seed=seed + 60, scale=0.3)
    log(f"[kda recurrent] {case}")
    o, hT = gdn.kda_recurrent_fwd(dev_tensor(w.q), dev_tensor(w.k), dev_tensor(w.v), dev_tensor(a),
                                  dev_tensor(w.beta), cu_seqlens=None if cu is None else dev_tensor(cu),
                                  h0=dev_tensor(h0))
    torch.cuda.synchronize()
    ro, rh = kda.forward(w.q, w.k, w.v, a, w.beta, cu_seqlens=cu, h0=h0)
    eo = max(rel_err(host_f64(o)[b, s:e].transpose(1, 0, 2), ro[b, s:e].transpose(1, 0, 2))
             for b, s, e in ([(b, 0, T) for b in range(B)] if cu is None else
                             [(0, int(cu[i]), int(cu[i + 1])) for i in range(N) if cu[i + 1] > cu[i]]))
    eh = rel_err(host_f64(hT), rh)
    log(f"    max rel err o={eo:.3e} hT={eh:.3e}")
    assert eo <= TOL[dtype] and eh <= TOL[dtype]


def test_kda_equal_rates_match_scalar_gate(gdn):
    """Every channel at one rate: the per-channel path gives the scalar-gate
    kernel's results (to rounding)."""
    import torch
    w = gi.generate(gi.Spec("kda-eq", B=2, T=50, H_qk=2, H_v=2, d_k=64, d_v=64, dtype="f32", chunk=64, seed=420))
    a = np.repeat(w.alpha[..., None], 64, axis=-1).astype(np.float32)
    args = [dev_tensor(x) for x in (w.q, w.k, w.v)]
    o1, h1 = gdn.kda_recurrent_fwd(*args, dev_tensor(a), dev_tensor(w.beta))
    o2, h2 = gdn.recurrent_fwd(*args, dev_tensor(w.alpha), dev_tensor(w.beta))
    torch.cuda.synchronize()
    e = max(rel_err(host_f64(o1), host_f64(o2)), rel_err(host_f64(h1), host_f64(h2)))
    log(f"[kda equal rates] max rel diff vs scalar gate {e:.3e}")
    assert e <= 1e-5


@pytest.mark.parametrize("dtype,B,H_qk,H_v,d", [("f32", 3, 1, 2, 32), ("f32", 5, 2, 8, 64),
                                               ("bf16", 256, 32, 32, 128)])
def test_kda_decode(gdn, dtype, B, H_qk, H_v, d):
    """One decode step from a random state; the bf16 case is the decode bench
    shape (B=256, H=32, d=128), every unit checked."""
    import torch
    w = gi.generate(gi.Spec("kda-dec", B=B, T=1, H_qk=H_qk, H_v=H_v, d_k=d, d_v=d, dtype=dtype, chunk=64,
                            seed=430 + B))
    a = gi.channel_rates(B, 1, H_v, d, 431 + B)
    state = gi.random_state((B, H_v, d, d), seed=432 + B, scale=0.3)
    log(f"[kda decode] {dtype} B={B} H={H_v} d={d}")
    st = dev_tensor(state)
    o = gdn.kda_decode_step(dev_tensor(w.q), dev_tensor(w.k), dev_tensor(w.v), dev_tensor(a), dev_tensor(w.beta), st)
    torch.cuda.synchronize()
    ro, rs = kda.decode(state, w.q, w.k, w.v, a, w.beta)
    eo = rel_err(host_f64(o)[:, 0], ro[:, 0])
    es = rel_err(host_f64(st), rs)
    log(f"    max rel err o={eo:.3e} state={es:.3e}")
    assert eo <= TOL[dtype] and es <= TOL["f32"]


# ---------------------------------------------------------------------------
# The chunked form (gdn_kda_chunk_fwd)
# ---------------------------------------------------------------------------

CHUNK_CASES = [
    # dtype, B, T, H_qk, H_v, d_k, d_v, chunk, lengths
    ("f32", 2, 150, 1, 2, 16, 16, 16, None),
    ("f32", 1, 200, 2, 2, 64, 32, 32, None),
    ("f32", 2, 130, 1, 1, 128, 64, 64, None),
    ("f32", 1, 0, 2, 4, 64, 128, 64, (17, 0, 1, 130, 64)),
    ("bf16", 2, 300, 2, 4, 128, 128, 64, None),
    ("bf16", 1, 0, 1, 4, 64, 32, 64, (40, 3, 0, 77, 200)),
    ("bf16", 1, 190, 2, 2, 128, 64, 32, None),
]


def kda_unit_errors(o, hT, ro, rh, slices):
    eo = max([rel_err(o[b, s:e].transpose(1, 0, 2), ro[b, s:e].transpose(1, 0, 2))
              for b, s, e in slices if e > s] or [0.0])
    return eo, rel_err(hT, rh)


@pytest.mark.parametrize("case", CHUNK_CASES, ids=[f"{c[0]}-B{c[1]}T{c[2]}H{c[3]}_{c[4]}d{c[5]}_{c[6]}C{c[7]}"
                                                   + ("-packed" if c[8] else "") for c in CHUNK_CASES])
def test_kda_chunk(gdn, case):
    import torch
    dtype, B, T, H_qk, H_v, d_k, d_v, chunk, lengths = case
    seed = 500 + CHUNK_CASES.index(case)
    w = gi.generate(gi.Spec("kda-chunk", B=B, T=T, H_qk=H_qk, H_v=H_v, d_k=d_k, d_v=d_v, dtype=dtype,
                            chunk=chunk, lengths=lengths, seed=seed))
    B, T = w.q.shape[0], w.q.shape[1]
    a = gi.channel_rates(B, T, H_v, d_k, seed + 50)
    cu = w.cu_seqlens
    N = B if cu is None else len(cu) - 1
    slices = w.seq_slices()
    args = [dev_tensor(x) for x in (w.q, w.k, w.v)] + [dev_tensor(a), dev_tensor(w.beta)]
    cu_t = None if cu is None else dev_tensor(cu)
    for h0 in (None, gi.random_state((N, H_v, d_k, d_v), seed=seed + 60, scale=0.3)):
        log(f"[kda chunk] {case} h0={h0 is not None}")
        o, hT = gdn.kda_chunk_fwd(*args, chunk=chunk, cu_seqlens=cu_t, h0=None if h0 is None else dev_tensor(h0))
        torch.cuda.synchronize()
        ro, rh = kda.forward(w.q, w.k, w.v, a, w.beta, cu_seqlens=cu, h0=h0)
        eo, eh = kda_unit_errors(host_f64(o), host_f64(hT), ro, rh, slices)
        log(f"    max rel err o={eo:.3e} hT={eh:.3e}")
        assert np.all(np.isfinite(host_f64(o))) and eo <= TOL[dtype] and eh <= TOL[dtype]


def test_kda_chunk_equal_rates_match_scalar_chunk(gdn):
    """Every channel at one rate: the per-channel chunked form gives the
    scalar-gate chunked forward's results (to rounding)."""
    import torch
    w = gi.generate(gi.Spec("kda-eq-chunk", B=2, T=300, H_qk=2, H_v=2, d_k=64, d_v=64, dtype="f32", chunk=64,
                            gates="tiny", seed=520))
    a = np.repeat(w.alpha[..., None], 64, axis=-1).astype(np.float32)
    args = [dev_tensor(x) for x in (w.q, w.k, w.v)]
    o1, h1 = gdn.kda_chunk_fwd(*args, dev_tensor(a), dev_tensor(w.beta))
    o2, h2 = gdn.chunk_fwd(*args, dev_tensor(w.alpha), dev_tensor(w.beta))
    torch.cuda.synchronize()
    e = max(rel_err(host_f64(o1), host_f64(o2)), rel_err(host_f64(h1), host_f64(h2)))
    log(f"[kda chunk equal rates] max rel diff vs scalar chunked forward {e:.3e}")
    assert e <= 1e-5


def test_kda_chunk_prefill_shape(gdn):
    """The prefill shape (B=4, T=4096, H=16, d=128, bf16, chunk 64) with one
    rate per key channel, every unit checked against the float64 oracle."""
    import torch
    w = gi.generate(gi.config(2, name="kda-prefill"))
    a = gi.channel_rates(4, 4096, 16, 128, 540)
    log("[kda chunk] prefill shape B=4 T=4096 H=16 d=128 bf16")
    o, hT = gdn.kda_chunk_fwd(*[dev_tensor(x) for x in (w.q, w.k, w.v)], dev_tensor(a), dev_tensor(w.beta))
    torch.cuda.synchronize()
    ro, rh = kda.forward(w.q, w.k, w.v, a, w.beta)
    eo, eh = kda_unit_errors(host_f64(o), host_f64(hT), ro, rh, w.seq_slices())
    log(f"    max rel err o={eo:.3e} hT={eh:.3e}")
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_kda_chunk_strong_decay_and_zero_rates(gdn, dtype):
    """Chunks whose per-channel cumulative decay leaves [2^-60, 2^60] (rates
    down to 0, some exactly 0) take the exact per-pair path of the chunked
    form; the others the factored one.  Both against the float64 oracle."""
    import torch
    B, T, H_qk, H_v, d_k, d_v = 1, 260, 1, 2, 64, 32
    w = gi.generate(gi.Spec("kda-decay", B=B, T=T, H_qk=H_qk, H_v=H_v, d_k=d_k, d_v=d_v, dtype=dtype,
                            chunk=64, seed=560))
    a = gi.channel_rates(B, T, H_v, d_k, 561)           # head 0: rates in [0.8, 1)
    a[:, :, 1] = gi.channel_rates(B, T, 1, d_k, 562, lo=0.0)[:, :, 0]  # head 1: rates in [0, 1)
    a[:, 100:103, 1, :5] = 0.0                           # some rates exactly 0
    a[:, 200, 0, 7] = 0.0                                # one zero in an otherwise slow-decay head
    args = [dev_tensor(x) for x in (w.q, w.k, w.v)] + [dev_tensor(a), dev_tensor(w.beta)]
    log(f"[kda chunk strong decay] {dtype}")
    o, hT = gdn.kda_chunk_fwd(*args, chunk=64)
    torch.cuda.synchronize()
    ro, rh = kda.forward(w.q, w.k, w.v, a, w.beta)
    eo, eh = kda_unit_errors(host_f64(o), host_f64(hT), ro, rh, w.seq_slices())
    log(f"    max rel err o={eo:.3e} hT={eh:.3e}")
    assert np.all(np.isfinite(host_f64(o))) and eo <= TOL[dtype] and eh <= TOL[dtype]
