"""gdn_chunk_fwd_noalloc (the library's static per-GPU scratch instead of a
caller workspace) against gdn_chunk_fwd with a workspace, through the C ABI:
two calls in a row, the second smaller, each bitwise equal to the workspace
entry point and within its dtype's bar of the float64 oracle; a problem whose
scratch would exceed the 32 MiB array is rejected before any launch."""
import ctypes

import numpy as np
import pytest

import gdn_inputs as gi
import oracle
from gpu_util import TOL, dev_tensor, host_f64, log, unit_rel_errors

pytestmark = pytest.mark.gpu


def test_noalloc_matches_workspace_entry_point():
    import torch
    import gated_delta_rule_03_amd as gdn
    lib = gdn.load()
    vp = ctypes.c_void_p
    stream = vp(torch.cuda.current_stream().cuda_stream)
    # calls in a row: a uniform batch, then a smaller packed batch with grouped
    # heads (both on the bf16 staged kernels), then fp32 inputs with d_k = 64
    # in chunks of 32 (the chained kernels), smaller again
    cases = [
        gi.Spec("noalloc-a", B=2, T=1000, H_qk=4, H_v=4, d_k=128, d_v=128, dtype="bf16", chunk=64, seed=601),
        gi.Spec("noalloc-b", B=1, T=0, H_qk=1, H_v=2, d_k=128, d_v=64, dtype="bf16", chunk=64,
                lengths=(100, 0, 37, 129), seed=602),
        gi.Spec("noalloc-c", B=2, T=150, H_qk=1, H_v=2, d_k=64, d_v=64, dtype="f32", chunk=32, gates="tiny",
                q_scale=False, seed=603),
    ]
    for spec in cases:
        w = gi.generate(spec)
        B, T = w.q.shape[0], w.q.shape[1]
        q, k, v, a, b = (dev_tensor(x) for x in (w.q, w.k, w.v, w.alpha, w.beta))
        cu = None if w.cu_seqlens is None else dev_tensor(w.cu_seqlens)
        n_seqs = 0 if cu is None else cu.numel() - 1
        N = B if cu is None else n_seqs
        code = gdn.GDN_BF16 if spec.dtype == "bf16" else gdn.GDN_F32
        o_ws, h_ws = gdn.chunk_fwd(q, k, v, a, b, cu_seqlens=cu, chunk=spec.chunk)
        o_na = torch.empty_like(o_ws)
        h_na = torch.empty_like(h_ws)
        st = lib.gdn_chunk_fwd_noalloc(B, T, spec.H_qk, spec.H_v, spec.d_k, spec.d_v, code,
                                       vp(q.data_ptr()), vp(k.data_ptr()), vp(v.data_ptr()), vp(a.data_ptr()),
                                       vp(b.data_ptr()), None if cu is None else vp(cu.data_ptr()), n_seqs, None,
                                       vp(o_na.data_ptr()), vp(h_na.data_ptr()), spec.chunk, stream)
        torch.cuda.synchronize()
        assert st == 0, gdn.status_string(st)
        assert torch.equal(o_na, o_ws) and torch.equal(h_na, h_ws)
        o_ref, h_ref = oracle.forward(w.q, w.k, w.v, w.alpha, w.beta, cu_seqlens=w.cu_seqlens)
        eo, eh, _ = unit_rel_errors(host_f64(o_na), host_f64(h_na), o_ref, h_ref, w.seq_slices(), spec.H_v)
        log(f"[noalloc] {spec.name}: bitwise equal to the workspace entry point; "
            f"max rel err o={eo:.3e} hT={eh:.3e} (N={N})")
        assert eo <= TOL[spec.dtype] and eh <= TOL[spec.dtype]


def test_noalloc_rejects_problems_beyond_its_scratch():
    import torch
    import gated_delta_rule_03_amd as gdn
    lib = gdn.load()
    vp = ctypes.c_void_p
    B, T, H, D = 8, 4096, 16, 128   # needs about 48 MB of scratch
    assert gdn.chunk_fwd_workspace_bytes(B, T, H, H, D, D, gdn.GDN_BF16, 64, 0) > (32 << 20)
    x = torch.zeros((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((B, T, H), dtype=torch.float32, device="cuda")
    o = torch.empty_like(x)
    st = lib.gdn_chunk_fwd_noalloc(B, T, H, H, D, D, gdn.GDN_BF16, vp(x.data_ptr()), vp(x.data_ptr()),
                                   vp(x.data_ptr()), vp(g.data_ptr()), vp(g.data_ptr()), None, 0, None,
                                   vp(o.data_ptr()), None, 64, vp(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    log(f"[noalloc] B={B} T={T} H={H}: status {st} ({gdn.status_string(st)})")
    assert st == gdn_status_workspace()


def gdn_status_workspace():
    return 3  # GDN_ERROR_WORKSPACE
