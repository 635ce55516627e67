"""Float64 CPU oracle of the gated delta rule (test infrastructure).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are the only callers.  The product path never
imports this package, and this package imports nothing from the product.

The arithmetic lives in ``gdn_oracle.c``: a plain token-by-token float64
recurrence of "Linear attention" (arsalanzafar.ai), section "How it works",
Eqs. (1)-(4).  This module only builds that file with gcc and marshals arrays:

* inputs arrive exactly as the library receives them (bf16 or float32 values
  widen to float64 exactly, so input rounding is never counted as error);
* a unit is one (sequence, value head); value head j reads query/key head
  floor(j * H_qk / H_v) (grouped heads: each query/key head serves
  H_v / H_qk consecutive value heads);
* a packed batch restarts the state at every ``cu_seqlens`` boundary;
* a decode step is the one-token case started from the given state.

Pins: every function here is pinned by ``tests/test_oracle_pins.py`` against
values the pages print, closed forms, invariants and library routines.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile
from typing import Dict, Iterable, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def cpu_threads() -> int:
    """Host threads the oracle uses by default (the cores this process may run on)."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def build(out_path: str = _LIB_PATH, mutant: int = 0) -> str:
    """Compile the oracle with gcc (optionally a planted-mistake mutant)."""
    cmd = ["gcc", "-O3", "-fopenmp", "-shared", "-fPIC", "-std=c99",
           f"-DORACLE_MUTANT={int(mutant)}", _SRC, "-o", out_path + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(out_path + ".tmp", out_path)
    return out_path


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    dp = ctypes.POINTER(ctypes.c_double)
    lib.gdn_oracle_forward.argtypes = [ctypes.c_int64] * 4 + [dp] * 6 + [ctypes.c_int, dp, dp,
                                                                       ctypes.c_int]
    lib.gdn_oracle_forward.restype = ctypes.c_int
    lib.gdn_oracle_mutant.argtypes = []
    lib.gdn_oracle_mutant.restype = ctypes.c_int
    return lib


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the built oracle (building it first if needed)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def load_mutant(mutant: int) -> ctypes.CDLL:
    """Build and load a planted-mistake variant into a temporary file."""
    d = tempfile.mkdtemp(prefix="gdn_oracle_mutant_")
    return load(build(os.path.join(d, f"liboracle_m{mutant}.so"), mutant=mutant))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def forward_units(q, k, v, alpha, beta, h0=None, delta: bool = True,
                  threads: Optional[int] = None, lib: Optional[ctypes.CDLL] = None):
    """Run independent units.

    q, k: [U, T, d_k]; v: [U, T, d_v]; alpha, beta: [U, T]; h0: [U, d_k, d_v] or None.
    Returns (o [U, T, d_v], hT [U, d_k, d_v]) in float64.
    """
    lib = lib or load()
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    alpha = np.ascontiguousarray(alpha, dtype=np.float64)
    beta = np.ascontiguousarray(beta, dtype=np.float64)
    U, T, dk = q.shape
    dv = v.shape[2]
    if k.shape != (U, T, dk) or v.shape[:2] != (U, T) or alpha.shape != (U, T) \
            or beta.shape != (U, T):
        raise ValueError("oracle: inconsistent shapes")
    if h0 is not None:
        h0 = np.ascontiguousarray(h0, dtype=np.float64)
        if h0.shape != (U, dk, dv):
            raise ValueError("oracle: h0 shape")
    o = np.empty((U, T, dv), dtype=np.float64)
    hT = np.empty((U, dk, dv), dtype=np.float64)
    rc = lib.gdn_oracle_forward(U, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                _ptr(beta), _ptr(h0), 1 if delta else 0, _ptr(o), _ptr(hT),
                                int(threads or cpu_threads()))
    if rc != 0:
        raise RuntimeError("oracle: gdn_oracle_forward failed")
    return o, hT


def _as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:  # bf16 bit patterns: widen exactly
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def qk_head(j: int, H_qk: int, H_v: int) -> int:
    """Query/key head read by value head j (consecutive grouping)."""
    return (j * H_qk) // H_v


def forward(q, k, v, alpha, beta, *, cu_seqlens=None, h0=None, delta: bool = True,
            units: Optional[Iterable[Tuple[int, int]]] = None, return_o: bool = True,
            threads: Optional[int] = None, lib: Optional[ctypes.CDLL] = None):
    """Oracle forward over a batch laid out as the library receives it.

    q, k: [B, T, H_qk, d_k]; v: [B, T, H_v, d_v]; alpha, beta: [B, T, H_v]
    (float32/float64 values or uint16 bf16 bits).  ``cu_seqlens`` (packed
    batch, B == 1) gives the sequence offsets.  h0: [N, H_v, d_k, d_v] or None.

    With ``units`` None, returns (o [B, T, H_v, d_v], hT [N, H_v, d_k, d_v]) in
    float64.  With ``units`` a list of (sequence, value head) pairs, returns a
    dict mapping each pair to (o [L, d_v], hT [d_k, d_v]) for that unit only.
    ``return_o=False`` skips gathering o (the full result is then (None, hT)).
    """
    B, T, H_qk, dk = q.shape
    H_v, dv = v.shape[2], v.shape[3]
    if cu_seqlens is None:
        seqs = [(b, 0, T) for b in range(B)]
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        if B != 1:
            raise ValueError("oracle: a packed batch has B == 1")
        seqs = [(0, int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)]
    N = len(seqs)
    if units is None:
        want = {i: list(range(H_v)) for i in range(N)}
        o_full = np.zeros((B, T, H_v, dv), dtype=np.float64) if return_o else None
        hT_full = np.zeros((N, H_v, dk, dv), dtype=np.float64)
    else:
        want: Dict[int, list] = {}
        for (i, j) in units:
            want.setdefault(int(i), []).append(int(j))
        out = {}
    for i, heads in sorted(want.items()):
        b, s, e = seqs[i]
        hq = [qk_head(j, H_qk, H_v) for j in heads]
        qs = np.stack([_as_f64(q[b, s:e, h]) for h in hq])
        ks = np.stack([_as_f64(k[b, s:e, h]) for h in hq])
        vs = np.stack([_as_f64(v[b, s:e, j]) for j in heads])
        a_s = np.stack([np.asarray(alpha[b, s:e, j], dtype=np.float64) for j in heads])
        b_s = np.stack([np.asarray(beta[b, s:e, j], dtype=np.float64) for j in heads])
        h0s = None if h0 is None else np.stack([np.asarray(h0[i, j], np.float64) for j in heads])
        o_u, hT_u = forward_units(qs, ks, vs, a_s, b_s, h0=h0s, delta=delta,
                                  threads=threads, lib=lib)
        for n, j in enumerate(heads):
            if units is None:
                if return_o:
                    o_full[b, s:e, j] = o_u[n]
                hT_full[i, j] = hT_u[n]
            else:
                out[(i, j)] = (o_u[n], hT_u[n])
    return (o_full, hT_full) if units is None else out


def decode(state, q, k, v, alpha, beta, threads: Optional[int] = None):
    """One token per sequence from ``state`` [B, H_v, d_k, d_v].

    q, k: [B, 1, H_qk, d_k]; v: [B, 1, H_v, d_v]; alpha, beta: [B, 1, H_v].
    Returns (o [B, 1, H_v, d_v], new state [B, H_v, d_k, d_v]) in float64.
    """
    return forward(q, k, v, alpha, beta, h0=state, threads=threads)
