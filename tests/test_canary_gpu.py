"""Guard bands: every output buffer (o, the final state, the workspace, the
decode state) sits inside a larger allocation whose bytes before and after
hold a sentinel pattern; after each call the bands must be bitwise
untouched.  Cases: the staged and chained chunk kernels on uniform batches
with a partial last chunk, a packed batch with empty and one-token sequences
and grouped heads, the segment-parallel form, the per-channel-gate chunked
and token-by-token forwards, the decode step, and the backward pass (every
gradient and its workspace, with h0 and dhT)."""
import numpy as np
import pytest

import gdn_inputs as gi
from gpu_util import dev_tensor, log

pytestmark = pytest.mark.gpu

BAND = 4096          # bytes on either side (a multiple of 256, so the guarded tensor stays aligned)
SENTINEL = 0xA5


@pytest.fixture(scope="module")
def gdn():
    import torch
    import gated_delta_rule_03_amd as g
    assert torch.cuda.is_available()
    g.load()
    return g


class Guarded:
    """A tensor of `shape` and `dtype` between two sentinel bands of one allocation."""

    def __init__(self, shape, dtype):
        import torch
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.n = n
        self.buf = torch.full((BAND + n + BAND,), SENTINEL, dtype=torch.uint8, device="cuda")
        self.t = self.buf[BAND:BAND + n].view(dtype).view(shape) if n else \
            torch.empty(shape, dtype=dtype, device="cuda")

    def intact(self):
        b = self.buf
        return bool((b[:BAND] == SENTINEL).all()) and bool((b[BAND + self.n:] == SENTINEL).all())


def guarded_ws(nbytes):
    import torch
    g = Guarded((nbytes,), torch.uint8)
    return g


def run_case(gdn, name, w, fn, per_channel=False, **kw):
    import torch
    B, T = w.q.shape[0], w.q.shape[1]
    H_v, d_k, d_v = w.spec.H_v, w.spec.d_k, w.spec.d_v
    dt = torch.bfloat16 if w.spec.dtype == "bf16" else torch.float32
    cu = None if w.cu_seqlens is None else dev_tensor(w.cu_seqlens)
    N = B if cu is None else cu.numel() - 1
    o, hT = Guarded((B, T, H_v, d_v), dt), Guarded((N, H_v, d_k, d_v), torch.float32)
    alpha = gi.channel_rates(B, T, H_v, d_k, 9) if per_channel else w.alpha
    args = [dev_tensor(x) for x in (w.q, w.k, w.v)] + [dev_tensor(alpha), dev_tensor(w.beta)]
    n_seqs = 0 if cu is None else N
    code = gdn.GDN_BF16 if w.spec.dtype == "bf16" else gdn.GDN_F32
    dims = (B, T, w.spec.H_qk, H_v, d_k, d_v, code, w.spec.chunk, n_seqs)
    ws = None
    if fn == "chunk_fwd":
        seg = kw.get("seg_chunks")
        nb = (gdn.chunk_fwd_workspace_bytes(*dims) if seg is None
              else gdn.chunk_fwd_segmented_workspace_bytes(*dims, seg))
        ws = guarded_ws(nb)
        gdn.chunk_fwd(*args, chunk=w.spec.chunk, cu_seqlens=cu, o=o.t, hT=hT.t, workspace=ws.t, seg_chunks=seg)
    elif fn == "kda_chunk_fwd":
        ws = guarded_ws(gdn.kda_chunk_fwd_workspace_bytes(*dims))
        gdn.kda_chunk_fwd(*args, chunk=w.spec.chunk, cu_seqlens=cu, o=o.t, hT=hT.t, workspace=ws.t)
    elif fn == "recurrent_fwd":
        gdn.recurrent_fwd(*args, cu_seqlens=cu, o=o.t, hT=hT.t)
    elif fn == "kda_recurrent_fwd":
        gdn.kda_recurrent_fwd(*args, cu_seqlens=cu, o=o.t, hT=hT.t)
    torch.cuda.synchronize()
    ok = o.intact() and hT.intact() and (ws is None or ws.intact())
    log(f"[canary] {name} {fn} {kw}: bands {'intact' if ok else 'OVERWRITTEN'}")
    assert ok
    assert torch.isfinite(o.t.float()).all()


def small(dtype, B, T, H_qk, H_v, d_k, d_v, chunk, seed, lengths=None):
    return gi.generate(gi.Spec(f"canary-{dtype}", B=B, T=T, H_qk=H_qk, H_v=H_v, d_k=d_k, d_v=d_v, dtype=dtype,
                               chunk=chunk, gates="tiny" if dtype == "f32" else "prefill",
                               q_scale=dtype == "bf16", lengths=lengths, seed=seed))


CASES = [
    ("staged uniform, partial chunk", ("bf16", 2, 300, 2, 2, 128, 128, 64, 701, None)),
    ("staged 16-column blocks", ("bf16", 1, 100, 1, 1, 128, 64, 64, 702, None)),
    ("staged packed, grouped heads", ("bf16", 1, 0, 2, 4, 128, 128, 64, 703, (1, 64, 65, 0, 130))),
    ("chained fp32, chunk 32", ("f32", 2, 77, 1, 2, 32, 64, 32, 704, None)),
    ("chained bf16 packed", ("bf16", 1, 0, 1, 2, 64, 32, 16, 705, (0, 17, 3, 40))),
]


@pytest.mark.parametrize("name,case", CASES, ids=[c[0] for c in CASES])
def test_bands_untouched(gdn, name, case):
    dtype, B, T, H_qk, H_v, d_k, d_v, chunk, seed, lengths = case
    w = small(dtype, B, T, H_qk, H_v, d_k, d_v, chunk, seed, lengths)
    run_case(gdn, name, w, "chunk_fwd")
    run_case(gdn, name, w, "chunk_fwd", seg_chunks=1)
    run_case(gdn, name, w, "recurrent_fwd")
    run_case(gdn, name, w, "kda_chunk_fwd", per_channel=True)
    run_case(gdn, name, w, "kda_recurrent_fwd", per_channel=True)


@pytest.mark.parametrize("per_channel", [False, True])
def test_decode_bands_untouched(gdn, per_channel):
    import torch
    w = small("bf16", 5, 1, 2, 4, 128, 64, 64, 706)
    st = Guarded((5, 4, 128, 64), torch.float32)
    st.t.copy_(torch.from_numpy(gi.random_state((5, 4, 128, 64), seed=707, scale=0.3)).cuda())
    o = Guarded((5, 1, 4, 64), torch.bfloat16)
    args = [dev_tensor(x) for x in (w.q, w.k, w.v)]
    if per_channel:
        gdn.kda_decode_step(*args, dev_tensor(gi.channel_rates(5, 1, 4, 128, 708)), dev_tensor(w.beta), st.t, o=o.t)
    else:
        gdn.decode_step(*args, dev_tensor(w.alpha), dev_tensor(w.beta), st.t, o=o.t)
    torch.cuda.synchronize()
    log(f"[canary] decode per_channel={per_channel}: bands {'intact' if st.intact() and o.intact() else 'OVERWRITTEN'}")
    assert st.intact() and o.intact()


@pytest.mark.parametrize("name,case", CASES, ids=[c[0] for c in CASES])
def test_backward_bands_untouched(gdn, name, case):
    import torch
    dtype, B, T, H_qk, H_v, d_k, d_v, chunk, seed, lengths = case
    w = small(dtype, B, T, H_qk, H_v, d_k, d_v, chunk, seed, lengths)
    B, T = w.q.shape[0], w.q.shape[1]
    cu = None if w.cu_seqlens is None else dev_tensor(w.cu_seqlens)
    N = B if cu is None else cu.numel() - 1
    n_seqs = 0 if cu is None else N
    f32 = torch.float32
    outs = [Guarded((B, T, H_qk, d_k), f32), Guarded((B, T, H_qk, d_k), f32), Guarded((B, T, H_v, d_v), f32),
            Guarded((B, T, H_v), f32), Guarded((B, T, H_v), f32), Guarded((N, H_v, d_k, d_v), f32)]
    code = gdn.GDN_BF16 if dtype == "bf16" else gdn.GDN_F32
    ws = guarded_ws(gdn.chunk_bwd_workspace_bytes(B, T, H_qk, H_v, d_k, d_v, code, chunk, n_seqs))
    do32 = gi.random_state((B, T, H_v, d_v), seed=seed + 1)
    d_o = dev_tensor(gi.f32_to_bf16_bits(do32) if dtype == "bf16" else do32)
    h0 = dev_tensor(gi.random_state((N, H_v, d_k, d_v), seed=seed + 2, scale=0.3))
    dhT = dev_tensor(gi.random_state((N, H_v, d_k, d_v), seed=seed + 3, scale=0.5))
    args = [dev_tensor(x) for x in (w.q, w.k, w.v, w.alpha, w.beta)]
    gdn.chunk_bwd(*args, d_o, chunk=chunk, cu_seqlens=cu, h0=h0, dhT=dhT, out=[g.t for g in outs],
                  workspace=ws.t)
    torch.cuda.synchronize()
    ok = all(g.intact() for g in outs) and ws.intact()
    log(f"[canary] {name} chunk_bwd: bands {'intact' if ok else 'OVERWRITTEN'}")
    assert ok
    assert all(bool(torch.isfinite(g.t).all()) for g in outs)
