"""Python binding of libgdn (the gated delta rule on MI355X).

Thin ctypes marshalling over the C ABI declared in ``include/gdn.h``: it checks
tensor devices, dtypes, shapes and contiguity, passes raw device pointers and
the current HIP stream, and raises ``GDNError`` on a non-zero status.  Every
step of the computation runs in the HIP kernels of ``libgdn.so``; there is no
other implementation here and no fallback.  PyTorch only provides device
memory and streams.

Names follow the C ABI: ``recurrent_fwd``, ``chunk_fwd`` (with
``chunk_fwd_workspace_bytes``; ``seg_chunks`` selects the segment-parallel
form of ``gdn_chunk_fwd_segmented``, with ``chunk_fwd_plan_segments`` and
``chunk_fwd_segmented_workspace_bytes``), ``decode_step``, the GDN block's
``block_prologue`` and ``block_epilogue``, the per-channel-gate
``kda_recurrent_fwd``, ``kda_chunk_fwd`` and ``kda_decode_step``, and the
backward pass ``chunk_bwd`` (with ``chunk_bwd_workspace_bytes``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

__all__ = [
    "GDNError", "lib_path", "load", "version", "status_string", "recurrent_fwd",
    "chunk_fwd", "chunk_fwd_workspace_bytes", "chunk_fwd_plan_segments",
    "chunk_fwd_segmented_workspace_bytes", "chunk_fwd_noalloc", "decode_step", "block_prologue", "block_epilogue",
    "kda_recurrent_fwd", "kda_chunk_fwd", "kda_chunk_fwd_workspace_bytes", "kda_decode_step",
    "chunk_bwd", "chunk_bwd_workspace_bytes", "GDN_F32", "GDN_BF16",
]

GDN_SUCCESS = 0
GDN_F32 = 0
GDN_BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgdn.so")
_lib: Optional[ctypes.CDLL] = None

EXPORTS = ["gdn_version", "gdn_status_string", "gdn_recurrent_fwd",
           "gdn_chunk_fwd_workspace_bytes", "gdn_chunk_fwd", "gdn_chunk_fwd_plan_segments",
           "gdn_chunk_fwd_segmented_workspace_bytes", "gdn_chunk_fwd_segmented", "gdn_chunk_fwd_noalloc",
           "gdn_decode_step",
           "gdn_block_prologue", "gdn_block_epilogue", "gdn_kda_recurrent_fwd",
           "gdn_kda_chunk_fwd_workspace_bytes", "gdn_kda_chunk_fwd", "gdn_kda_decode_step",
           "gdn_chunk_bwd_workspace_bytes", "gdn_chunk_bwd"]


class GDNError(RuntimeError):
    """A libgdn call returned a non-zero status."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def lib_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libgdn.so from the package directory.  Raises if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"libgdn.so not found at {_LIB_PATH}: build it with "
            "`python -m gated_delta_rule_03_amd.build` (there is no fallback implementation)")
    lib = ctypes.CDLL(_LIB_PATH)
    i32, vp, fp = ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p
    lib.gdn_version.argtypes = []
    lib.gdn_version.restype = i32
    lib.gdn_status_string.argtypes = [i32]
    lib.gdn_status_string.restype = ctypes.c_char_p
    fwd = [i32] * 7 + [vp, vp, vp, fp, fp, vp, i32, fp, vp, fp]
    lib.gdn_recurrent_fwd.argtypes = fwd + [vp]
    lib.gdn_recurrent_fwd.restype = i32
    lib.gdn_chunk_fwd_workspace_bytes.argtypes = [i32] * 9
    lib.gdn_chunk_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_chunk_fwd.argtypes = fwd + [i32, vp, ctypes.c_size_t, vp]
    lib.gdn_chunk_fwd.restype = i32
    lib.gdn_chunk_fwd_plan_segments.argtypes = [i32] * 9
    lib.gdn_chunk_fwd_plan_segments.restype = i32
    lib.gdn_chunk_fwd_segmented_workspace_bytes.argtypes = [i32] * 10
    lib.gdn_chunk_fwd_segmented_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_chunk_fwd_segmented.argtypes = fwd + [i32, i32, vp, ctypes.c_size_t, vp]
    lib.gdn_chunk_fwd_segmented.restype = i32
    lib.gdn_chunk_fwd_noalloc.argtypes = fwd + [i32, vp]
    lib.gdn_chunk_fwd_noalloc.restype = i32
    lib.gdn_decode_step.argtypes = [i32] * 6 + [vp, vp, vp, fp, fp, fp, vp, vp]
    lib.gdn_kda_recurrent_fwd.argtypes = fwd + [vp]
    lib.gdn_kda_recurrent_fwd.restype = i32
    lib.gdn_kda_chunk_fwd_workspace_bytes.argtypes = [i32] * 9
    lib.gdn_kda_chunk_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_kda_chunk_fwd.argtypes = fwd + [i32, vp, ctypes.c_size_t, vp]
    lib.gdn_kda_chunk_fwd.restype = i32
    lib.gdn_kda_decode_step.argtypes = [i32] * 6 + [vp, vp, vp, fp, fp, fp, vp, vp]
    lib.gdn_kda_decode_step.restype = i32
    lib.gdn_decode_step.restype = i32
    f32 = ctypes.c_float
    lib.gdn_block_prologue.argtypes = ([i32] * 7 + [vp] * 3 + [fp] * 10 + [f32, f32, vp, i32]
                                       + [vp] * 3 + [fp, fp, vp])
    lib.gdn_block_prologue.restype = i32
    lib.gdn_block_epilogue.argtypes = [i32] * 5 + [vp, vp, fp, f32, vp, vp]
    lib.gdn_block_epilogue.restype = i32
    lib.gdn_chunk_bwd_workspace_bytes.argtypes = [i32] * 9
    lib.gdn_chunk_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_chunk_bwd.argtypes = ([i32] * 7 + [vp, vp, vp, fp, fp, vp, i32, fp, vp, fp]
                                  + [fp] * 6 + [i32, vp, ctypes.c_size_t, vp])
    lib.gdn_chunk_bwd.restype = i32
    _lib = lib
    return lib


def version() -> int:
    return int(load().gdn_version())


def status_string(status: int) -> str:
    return load().gdn_status_string(int(status)).decode()


# ---------------------------------------------------------------------------
# argument marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _check(t, name, shape, dtype=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _fwd_args(q, k, v, alpha, beta, cu_seqlens, h0, o, hT, output_final_state, per_channel=False):
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, T, H, d]")
    B, T, H_qk, d_k = q.shape
    H_v, d_v = v.shape[2], v.shape[3]
    dev = q.device
    _check(q, "q", (B, T, H_qk, d_k), device=dev)
    _check(k, "k", (B, T, H_qk, d_k), q.dtype, dev)
    _check(v, "v", (B, T, H_v, d_v), q.dtype, dev)
    _check(alpha, "alpha", (B, T, H_v, d_k) if per_channel else (B, T, H_v), torch.float32, dev)
    _check(beta, "beta", (B, T, H_v), torch.float32, dev)
    code = _dtype_code(q)
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError("a packed batch (cu_seqlens) needs B == 1")
        _check(cu_seqlens, "cu_seqlens", (cu_seqlens.numel(),), torch.int32, dev)
        n_seqs = cu_seqlens.numel() - 1
        if n_seqs < 0:
            raise ValueError("cu_seqlens needs at least one element")
        N = n_seqs
    else:
        n_seqs = 0
        N = B
    if h0 is not None:
        _check(h0, "h0", (N, H_v, d_k, d_v), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, H_v, d_v), dtype=q.dtype, device=dev)
    else:
        _check(o, "o", (B, T, H_v, d_v), q.dtype, dev)
    if hT is None and output_final_state:
        hT = torch.empty((N, H_v, d_k, d_v), dtype=torch.float32, device=dev)
    elif hT is not None:
        _check(hT, "hT", (N, H_v, d_k, d_v), torch.float32, dev)
    dims = (B, T, H_qk, H_v, d_k, d_v, code)
    return dims, n_seqs, o, hT


def recurrent_fwd(q, k, v, alpha, beta, *, cu_seqlens=None, h0=None, o=None, hT=None,
                  output_final_state: bool = True, stream=None) -> Tuple:
    """Token-by-token gated delta rule.  Returns (o, hT)."""
    dims, n_seqs, o, hT = _fwd_args(q, k, v, alpha, beta, cu_seqlens, h0, o, hT,
                                    output_final_state)
    st = load().gdn_recurrent_fwd(*dims, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                  _ptr(cu_seqlens), n_seqs, _ptr(h0), _ptr(o), _ptr(hT),
                                  _stream(stream))
    if st != GDN_SUCCESS:
        raise GDNError(st, "gdn_recurrent_fwd")
    return o, hT


def chunk_fwd_workspace_bytes(B, T, H_qk, H_v, d_k, d_v, dtype_code, chunk=64, n_seqs=0) -> int:
    return int(load().gdn_chunk_fwd_workspace_bytes(B, T, H_qk, H_v, d_k, d_v, dtype_code, chunk,
                                                    n_seqs))


def chunk_fwd_plan_segments(B, T, H_qk, H_v, d_k, d_v, dtype_code, chunk=64, n_seqs=0) -> int:
    """Chunks per segment that gdn_chunk_fwd uses for these sizes (0: one pass)."""
    n = int(load().gdn_chunk_fwd_plan_segments(B, T, H_qk, H_v, d_k, d_v, dtype_code, chunk, n_seqs))
    if n < 0:
        raise GDNError(2, "gdn_chunk_fwd_plan_segments")
    return n


def chunk_fwd_segmented_workspace_bytes(B, T, H_qk, H_v, d_k, d_v, dtype_code, chunk=64, n_seqs=0,
                                        seg_chunks=0) -> int:
    return int(load().gdn_chunk_fwd_segmented_workspace_bytes(B, T, H_qk, H_v, d_k, d_v, dtype_code,
                                                              chunk, n_seqs, seg_chunks))


def chunk_fwd(q, k, v, alpha, beta, *, chunk: int = 64, cu_seqlens=None, h0=None, o=None,
              hT=None, workspace=None, output_final_state: bool = True, seg_chunks=None,
              stream=None) -> Tuple:
    """Chunked gated delta rule (WY/UT form).  Returns (o, hT).

    ``seg_chunks``: None lets gdn_chunk_fwd choose between one pass and the
    segment-parallel form; 0 forces one pass, n > 0 segments of n chunks
    (gdn_chunk_fwd_segmented).
    ``workspace``: an optional uint8 device tensor of at least the queried
    workspace bytes; allocated per call when omitted.
    """
    torch = _torch()
    dims, n_seqs, o, hT = _fwd_args(q, k, v, alpha, beta, cu_seqlens, h0, o, hT,
                                    output_final_state)
    if seg_chunks is None:
        need = chunk_fwd_workspace_bytes(*dims, chunk, n_seqs)
        where = "gdn_chunk_fwd_workspace_bytes"
    else:
        need = chunk_fwd_segmented_workspace_bytes(*dims, chunk, n_seqs, int(seg_chunks))
        where = "gdn_chunk_fwd_segmented_workspace_bytes"
    if need == 0:
        raise GDNError(2, where)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} "
                         f"bytes, {need} needed")
    args = (*dims, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(cu_seqlens), n_seqs,
            _ptr(h0), _ptr(o), _ptr(hT), chunk)
    ws = (_ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if seg_chunks is None:
        st = load().gdn_chunk_fwd(*args, *ws)
        where = "gdn_chunk_fwd"
    else:
        st = load().gdn_chunk_fwd_segmented(*args, int(seg_chunks), *ws)
        where = "gdn_chunk_fwd_segmented"
    if st != GDN_SUCCESS:
        raise GDNError(st, where)
    return o, hT


def chunk_bwd_workspace_bytes(B, T, H_qk, H_v, d_k, d_v, dtype_code, chunk=64, n_seqs=0) -> int:
    return int(load().gdn_chunk_bwd_workspace_bytes(B, T, H_qk, H_v, d_k, d_v, dtype_code, chunk, n_seqs))


def chunk_bwd(q, k, v, alpha, beta, d_o, *, chunk: int = 64, cu_seqlens=None, h0=None, dhT=None,
              want_dh0: bool = True, out=None, workspace=None, stream=None) -> Tuple:
    """Gradients of L = sum <d_o, o> + <dhT, hT> (gdn_chunk_bwd).

    Returns (dq, dk, dv, dalpha, dbeta, dh0), all float32; dq and dk sum over
    the value heads that read each query/key head; dh0 is None unless
    ``want_dh0``.  ``out`` may hold those six tensors (dh0 may be None),
    written in place; otherwise they are allocated here.
    """
    torch = _torch()
    dims, n_seqs, _, _ = _fwd_args(q, k, v, alpha, beta, cu_seqlens, h0, d_o, None, False)
    B, T, H_qk, H_v, d_k, d_v, code = dims
    N = n_seqs if cu_seqlens is not None else B
    dev = q.device
    if dhT is not None:
        _check(dhT, "dhT", (N, H_v, d_k, d_v), torch.float32, dev)
    shapes = ((B, T, H_qk, d_k), (B, T, H_qk, d_k), (B, T, H_v, d_v), (B, T, H_v), (B, T, H_v),
              (N, H_v, d_k, d_v))
    names = ("dq", "dk", "dv", "dalpha", "dbeta", "dh0")
    if out is None:
        f32 = dict(dtype=torch.float32, device=dev)
        out = [torch.empty(sh, **f32) for sh in shapes[:5]]
        out.append(torch.empty(shapes[5], **f32) if want_dh0 else None)
    else:
        if len(out) != 6:
            raise ValueError("out must hold (dq, dk, dv, dalpha, dbeta, dh0)")
        for t, sh, nm in zip(out, shapes, names):
            if t is not None:
                _check(t, nm, sh, torch.float32, dev)
        if any(t is None for t in out[:5]):
            raise ValueError("out: only dh0 may be None")
    dq, dk, dv, dalpha, dbeta, dh0 = out
    need = chunk_bwd_workspace_bytes(*dims, chunk, n_seqs)
    if need == 0:
        raise GDNError(2, "gdn_chunk_bwd_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} "
                         f"bytes, {need} needed")
    st = load().gdn_chunk_bwd(*dims, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(cu_seqlens),
                              n_seqs, _ptr(h0), _ptr(d_o), _ptr(dhT), _ptr(dq), _ptr(dk), _ptr(dv),
                              _ptr(dalpha), _ptr(dbeta), _ptr(dh0), chunk, _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream))
    if st != GDN_SUCCESS:
        raise GDNError(st, "gdn_chunk_bwd")
    return dq, dk, dv, dalpha, dbeta, dh0


def chunk_fwd_noalloc(q, k, v, alpha, beta, *, chunk: int = 64, cu_seqlens=None, h0=None, o=None,
                      hT=None, output_final_state: bool = True, stream=None) -> Tuple:
    """chunk_fwd without a workspace: the library's static per-GPU scratch
    (32 MiB) serves instead.  Calls that overlap on one GPU race on it.
    Returns (o, hT); ``o`` and ``hT`` are allocated here only when omitted."""
    dims, n_seqs, o, hT = _fwd_args(q, k, v, alpha, beta, cu_seqlens, h0, o, hT,
                                    output_final_state)
    st = load().gdn_chunk_fwd_noalloc(*dims, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                      _ptr(cu_seqlens), n_seqs, _ptr(h0), _ptr(o), _ptr(hT), chunk,
                                      _stream(stream))
    if st != GDN_SUCCESS:
        raise GDNError(st, "gdn_chunk_fwd_noalloc")
    return o, hT


def decode_step(q, k, v, alpha, beta, state, *, o=None, stream=None):
    """One token per sequence; ``state`` [B, H_v, d_k, d_v] is updated in place.  Returns o."""
    torch = _torch()
    if q.dim() != 4 or q.shape[1] != 1:
        raise ValueError("q must be [B, 1, H_qk, d_k]")
    B, _, H_qk, d_k = q.shape
    H_v, d_v = v.shape[2], v.shape[3]
    dev = q.device
    _check(q, "q", (B, 1, H_qk, d_k), device=dev)
    _check(k, "k", (B, 1, H_qk, d_k), q.dtype, dev)
    _check(v, "v", (B, 1, H_v, d_v), q.dtype, dev)
    _check(alpha, "alpha", (B, 1, H_v), torch.float32, dev)
    _check(beta, "beta", (B, 1, H_v), torch.float32, dev)
    _check(state, "state", (B, H_v, d_k, d_v), torch.float32, dev)
    if o is None:
        o = torch.empty((B, 1, H_v, d_v), dtype=q.dtype, device=dev)
    else:
        _check(o, "o", (B, 1, H_v, d_v), q.dtype, dev)
    st = load().gdn_decode_step(B, H_qk, H_v, d_k, d_v, _dtype_code(q), _ptr(q), _ptr(k),
                                _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state), _ptr(o),
                                _stream(stream))
    if st != GDN_SUCCESS:
        raise GDNError(st, "gdn_decode_step")
    return o


def kda_recurrent_fwd(q, k, v, alpha, beta, *, cu_seqlens=None, h0=None, o=None, hT=None,
                      output_final_state: bool = True, stream=None) -> Tuple:
    """Token-by-token delta rule with one decay rate per key channel: alpha is
    [B, T, H_v, d_k] float32.  Returns (o, hT)."""
    dims, n_seqs, o, hT = _fwd_args(q, k, v, alpha, beta, cu_seqlens, h0, o, hT,
                                    output_final_state, per_channel=True)
    st = load().gdn_kda_recurrent_fwd(*dims, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                      _ptr(cu_seqlens), n_seqs, _ptr(h0), _ptr(o), _ptr(hT),
                                      _stream(stream))
    if st != GDN_SUCCESS:
        raise GDNError(st, "gdn_kda_recurrent_fwd")
    return o, hT


def kda_chunk_fwd_workspace_bytes(B, T, H_qk, H_v, d_k, d_v, dtype_code, chunk=64, n_seqs=0) -> int:
    return int(load().gdn_kda_chunk_fwd_workspace_bytes(B, T, H_qk, H_v, d_k, d_v, dtype_code, chunk,
                                                        n_seqs))


def kda_chunk_fwd(q, k, v, alpha, beta, *, chunk: int = 64, cu_seqlens=None, h0=None, o=None, hT=None,
                  workspace=None, output_final_state: bool = True, stream=None) -> Tuple:
    """Chunked delta rule with one decay rate per key channel: alpha is
    [B, T, H_v, d_k] float32.  Returns (o, hT)."""
    torch = _torch()
    dims, n_seqs, o, hT = _fwd_args(q, k, v, alpha, beta, cu_seqlens, h0, o, hT,
                                    output_final_state, per_channel=True)
    need = kda_chunk_fwd_workspace_bytes(*dims, chunk, n_seqs)
    if need == 0:
        raise GDNError(2, "gdn_kda_chunk_fwd_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} "
                         f"bytes, {need} needed")
    st = load().gdn_kda_chunk_fwd(*dims, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                  _ptr(cu_seqlens), n_seqs, _ptr(h0), _ptr(o), _ptr(hT), chunk,
                                  _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(stream))
    if st != GDN_SUCCESS:
        raise GDNError(st, "gdn_kda_chunk_fwd")
    return o, hT


def kda_decode_step(q, k, v, alpha, beta, state, *, o=None, stream=None):
    """One token per sequence with one decay rate per key channel (alpha
    [B, 1, H_v, d_k] float32); ``state`` is updated in place.  Returns o."""
    torch = _torch()
    if q.dim() != 4 or q.shape[1] != 1:
        raise ValueError("q must be [B, 1, H_qk, d_k]")
    B, _, H_qk, d_k = q.shape
    H_v, d_v = v.shape[2], v.shape[3]
    dev = q.device
    _check(q, "q", (B, 1, H_qk, d_k), device=dev)
    _check(k, "k", (B, 1, H_qk, d_k), q.dtype, dev)
    _check(v, "v", (B, 1, H_v, d_v), q.dtype, dev)
    _check(alpha, "alpha", (B, 1, H_v, d_k), torch.float32, dev)
    _check(beta, "beta", (B, 1, H_v), torch.float32, dev)
    _check(state, "state", (B, H_v, d_k, d_v), torch.float32, dev)
    if o is None:
        o = torch.empty((B, 1, H_v, d_v), dtype=q.dtype, device=dev)
    else:
        _check(o, "o", (B, 1, H_v, d_v), q.dtype, dev)
    st = load().gdn_kda_decode_step(B, H_qk, H_v, d_k, d_v, _dtype_code(q), _ptr(q), _ptr(k),
                                    _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state), _ptr(o),
                                    _stream(stream))
    if st != GDN_SUCCESS:
        raise GDNError(st, "gdn_kda_decode_step")
    return o


def block_prologue(q_raw, k_raw, v_raw, conv_q, conv_k, conv_v, a_raw, b_raw, log_A, *,
                   conv_q_bias=None, conv_k_bias=None, conv_v_bias=None, v_norm_weight=None,
                   eps: float = 1e-6, q_scale: float = 1.0, cu_seqlens=None, out=None, stream=None):
    """The GDN block's steps before the recurrence (causal conv + SiLU, unit q/k,
    RMS-normalised v, gate maps) in one kernel.  Returns (q, k, v, alpha, beta),
    the inputs of ``chunk_fwd``; ``out`` may supply those five tensors."""
    torch = _torch()
    if q_raw.dim() != 4 or v_raw.dim() != 4:
        raise ValueError("q_raw, k_raw, v_raw must be [B, T, H, d]")
    B, T, H_qk, d_k = q_raw.shape
    H_v, d_v = v_raw.shape[2], v_raw.shape[3]
    dev, dt = q_raw.device, q_raw.dtype
    f32 = torch.float32
    _check(q_raw, "q_raw", (B, T, H_qk, d_k), device=dev)
    _check(k_raw, "k_raw", (B, T, H_qk, d_k), dt, dev)
    _check(v_raw, "v_raw", (B, T, H_v, d_v), dt, dev)
    _check(conv_q, "conv_q", (H_qk * d_k, 4), f32, dev)
    _check(conv_k, "conv_k", (H_qk * d_k, 4), f32, dev)
    _check(conv_v, "conv_v", (H_v * d_v, 4), f32, dev)
    for t, n, c in ((conv_q_bias, "conv_q_bias", H_qk * d_k), (conv_k_bias, "conv_k_bias", H_qk * d_k),
                    (conv_v_bias, "conv_v_bias", H_v * d_v), (v_norm_weight, "v_norm_weight", d_v)):
        if t is not None:
            _check(t, n, (c,), f32, dev)
    _check(a_raw, "a_raw", (B, T, H_v), f32, dev)
    _check(b_raw, "b_raw", (B, T, H_v), f32, dev)
    _check(log_A, "log_A", (H_v,), f32, dev)
    n_seqs = 0
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError("a packed batch (cu_seqlens) needs B == 1")
        _check(cu_seqlens, "cu_seqlens", (cu_seqlens.numel(),), torch.int32, dev)
        n_seqs = cu_seqlens.numel() - 1
    if out is None:
        out = (torch.empty_like(q_raw), torch.empty_like(k_raw), torch.empty_like(v_raw),
               torch.empty((B, T, H_v), dtype=f32, device=dev), torch.empty((B, T, H_v), dtype=f32, device=dev))
    q, k, v, alpha, beta = out
    for t, n, ref in ((q, "q", q_raw), (k, "k", k_raw), (v, "v", v_raw)):
        _check(t, n, tuple(ref.shape), dt, dev)
    _check(alpha, "alpha", (B, T, H_v), f32, dev)
    _check(beta, "beta", (B, T, H_v), f32, dev)
    st = load().gdn_block_prologue(B, T, H_qk, H_v, d_k, d_v, _dtype_code(q_raw), _ptr(q_raw), _ptr(k_raw),
                                   _ptr(v_raw), _ptr(conv_q), _ptr(conv_k), _ptr(conv_v), _ptr(conv_q_bias),
                                   _ptr(conv_k_bias), _ptr(conv_v_bias), _ptr(a_raw), _ptr(b_raw), _ptr(log_A),
                                   _ptr(v_norm_weight), float(eps), float(q_scale), _ptr(cu_seqlens), n_seqs,
                                   _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _stream(stream))
    if st != GDN_SUCCESS:
        raise GDNError(st, "gdn_block_prologue")
    return q, k, v, alpha, beta


def block_epilogue(o, g, *, o_norm_weight=None, eps: float = 1e-6, y=None, stream=None):
    """The GDN block's steps after the recurrence: RMS normalisation of each
    head's output times SiLU of the output gate's projection ``g``.  Returns y."""
    torch = _torch()
    if o.dim() != 4:
        raise ValueError("o must be [B, T, H_v, d_v]")
    B, T, H_v, d_v = o.shape
    dev = o.device
    _check(o, "o", (B, T, H_v, d_v), device=dev)
    _check(g, "g", (B, T, H_v, d_v), o.dtype, dev)
    if o_norm_weight is not None:
        _check(o_norm_weight, "o_norm_weight", (d_v,), torch.float32, dev)
    if y is None:
        y = torch.empty_like(o)
    else:
        _check(y, "y", (B, T, H_v, d_v), o.dtype, dev)
    st = load().gdn_block_epilogue(B, T, H_v, d_v, _dtype_code(o), _ptr(o), _ptr(g), _ptr(o_norm_weight),
                                   float(eps), _ptr(y), _stream(stream))
    if st != GDN_SUCCESS:
        raise GDNError(st, "gdn_block_epilogue")
    return y
