"""Helpers for the GPU parity tests: device copies of workloads and error metrics.

Error metric (per output tensor X in {o, final state} and per unit slice s,
a unit being one (sequence, value head)):
    rel_s = max_s |X - X_ref| / max_s |X_ref|
and a test reports max_s rel_s.  Bars: 1e-4 for float32 inputs, 2e-2 for
bf16 inputs with a float32 state.
"""
import sys

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_tensor(a, device="cuda"):
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(
            torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host_f64(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def to_device(w, device="cuda"):
    d = {name: dev_tensor(getattr(w, name), device) for name in ("q", "k", "v", "alpha", "beta")}
    d["cu_seqlens"] = None if w.cu_seqlens is None else dev_tensor(w.cu_seqlens, device)
    return d


def unit_rel_errors(o, hT, o_ref, hT_ref, seq_slices, H_v):
    """Per-unit relative errors.  Returns (max over units for o, max for hT, worst unit)."""
    worst_o, worst_h, worst_unit = 0.0, 0.0, None
    for i, (b, s, e) in enumerate(seq_slices):
        for j in range(H_v):
            if e > s:
                ref = o_ref[b, s:e, j]
                den = max(np.max(np.abs(ref)), 1e-30)
                r = float(np.max(np.abs(o[b, s:e, j] - ref)) / den)
                if r > worst_o:
                    worst_o, worst_unit = r, (i, j)
            if hT is not None:
                ref = hT_ref[i, j]
                den = max(np.max(np.abs(ref)), 1e-30)
                r = float(np.max(np.abs(hT[i, j] - ref)) / den)
                if r > worst_h:
                    worst_h = r
    return worst_o, worst_h, worst_unit
