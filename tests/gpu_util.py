"""Helpers for the GPU parity tests: device copies of workloads and error metrics.

Error metric (per output tensor X in {o, final state} and per unit slice s,
a unit being one (sequence, value head)):
    rel_s = max_s |X - X_ref| / max_s |X_ref|
and a test reports max_s rel_s.  Bars: 1e-4 for float32 inputs, 2e-2 for
bf16 inputs with a float32 state.

Two localised forms of the same comparison guard against an error in small
outputs that a unit's largest value would hide (an early token of a long
sequence, say):
  * windowed: the same ratio over every 64-token window of a unit's outputs,
    max_w |o - o_ref| / max_w |o_ref|, held to the same bars;
  * elementwise: |o - o_ref| / (|o_ref| + 1e-3 max_s |o_ref|) per element,
    reported, and held to ELEM_TOL.  For float32 inputs that is a real bar
    (errors ~1e-6 of the unit's scale).  With bf16 operands an output carries
    an absolute error of order 2^-9 of the terms that sum into it, which is
    about twice the 1e-3 floor, so near-zero elements score O(1) however
    correct the kernel is; the bf16 bar only catches gross failures, and the
    windowed metric is the local check.
"""
import sys

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}
ELEM_TOL = {"f32": 1e-2, "bf16": 16.0}
WINDOW = 64


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


def local_errors(o, o_ref, seq_slices, H_v, window=WINDOW):
    """Worst windowed relative error and worst elementwise error of o over all
    units (see the module docstring).  Returns (windowed, elementwise)."""
    worst_w, worst_e = 0.0, 0.0
    for (b, s, e) in seq_slices:
        if e <= s:
            continue
        ref = o_ref[b, s:e]          # [L, H_v, d_v]
        d = np.abs(o[b, s:e] - ref)
        a = np.abs(ref)
        unit_max = np.maximum(a.max(axis=(0, 2)), 1e-30)   # [H_v]
        worst_e = max(worst_e, float(np.max(d / (a + 1e-3 * unit_max[None, :, None]))))
        L = e - s
        nw = (L + window - 1) // window
        pad = nw * window - L
        if pad:
            d = np.concatenate([d, np.zeros((pad,) + d.shape[1:])])
            a = np.concatenate([a, np.zeros((pad,) + a.shape[1:])])
        dw = d.reshape(nw, window, H_v, -1).max(axis=(1, 3))
        aw = a.reshape(nw, window, H_v, -1).max(axis=(1, 3))
        nz = aw > 0
        if np.any(~nz & (dw > 0)):
            return float("inf"), float("inf")
        if np.any(nz):
            worst_w = max(worst_w, float(np.max(dw[nz] / aw[nz])))
    return worst_w, worst_e
