"""Seeded synthetic inputs for the gated delta rule hot path.

This module draws random numbers and lays them out exactly as the library
receives them.  It holds none of the recurrence's arithmetic: the tests, the
benchmark and the smoke check feed the same arrays to the HIP path and to the
float64 oracle.

Recipe (shared by every workload):

* One ``numpy.random.SeedSequence(seed)`` per workload.  It spawns one child
  stream per sequence plus one "head" stream for per-head constants (and, for
  packed batches, one "lengths" stream).  Each sequence's stream draws, in this
  order: q, k, v (float32 normals), then the two gate normals z_alpha, z_beta
  (float64).  Sequences are therefore independent and are generated on a
  thread pool.
* q and k are scaled to unit length per token and head over d_k, in float32
  ("Linear attention", GDN block walkthrough: F.normalize of queries and
  keys).  The prefill-shaped workloads then multiply q by 1/sqrt(d_k).
* v ~ N(0, 1).
* bf16 workloads round the float32 values to bf16 with round-to-nearest-even;
  the rounded values are what both sides consume.
* Gates are computed in float64 and stored as float32:

  - "tiny":    alpha = sigmoid(N(2, 0.5)),   beta = sigmoid(N(0, 1)).
  - "prefill": log alpha = -softplus(N(0, 1)) * A_h * s with
    A_h = exp(U(-4, 0)) drawn once per value head, s = 1 (or 1/64 for the
    long-memory workload), and beta = sigmoid(N(0, 1)).  This is the gate
    parametrisation of "Linear attention" (the naive PyTorch GDN block:
    alpha = exp(-A * softplus(W_alpha x)), A = exp(log_alpha) per head,
    beta = sigmoid(W_beta x)), with the projections replaced by normals.

* Packed (variable-length) batches draw L = round(exp(U(ln 128, ln 16384)))
  per sequence, clamped to [128, 16384], and pack them along one token axis
  with ``cu_seqlens`` offsets.  Each query/key head serves H_v / H_qk value
  heads.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

__all__ = [
    "Spec",
    "Workload",
    "CONFIGS",
    "config",
    "generate",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
]


# ----------------------------------------------------------------------------
# bf16 storage helpers (bit-level; round to nearest even)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + rounding) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# Workload description
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class Spec:
    """Shape and value distribution of one synthetic workload."""

    name: str
    B: int                      # sequences (1 for a packed batch)
    T: int                      # tokens per sequence (ignored when packed)
    H_qk: int
    H_v: int
    d_k: int
    d_v: int
    dtype: str                  # "f32" or "bf16" for q, k, v and o
    chunk: int
    gates: str = "prefill"      # "tiny" or "prefill"
    q_scale: bool = True        # multiply q by 1/sqrt(d_k)
    log_alpha_scale: float = 1.0
    packed_seqs: int = 0        # >0: variable-length packed batch of this many sequences
    min_len: int = 128
    max_len: int = 16384
    lengths: Optional[tuple] = None  # explicit packed lengths (overrides the draw)
    seed: int = 0


@dataclass
class Workload:
    """Arrays exactly as the library receives them (host copies)."""

    spec: Spec
    q: np.ndarray               # [B, T, H_qk, d_k]  float32, or uint16 bf16 bits
    k: np.ndarray               # [B, T, H_qk, d_k]
    v: np.ndarray               # [B, T, H_v, d_v]
    alpha: np.ndarray           # [B, T, H_v] float32
    beta: np.ndarray            # [B, T, H_v] float32
    cu_seqlens: Optional[np.ndarray] = None   # int32 [n_seqs + 1] for packed batches
    lengths: List[int] = field(default_factory=list)

    @property
    def B(self) -> int:
        return self.q.shape[0]

    @property
    def T(self) -> int:
        return self.q.shape[1]

    @property
    def n_seqs(self) -> int:
        return len(self.lengths)

    @property
    def n_tokens(self) -> int:
        return int(sum(self.lengths))

    def values(self, name: str) -> np.ndarray:
        """float32 view of q, k or v (exact for bf16 storage)."""
        a = getattr(self, name)
        return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a

    def seq_slices(self):
        """(batch index, token start, token end) of every sequence."""
        if self.cu_seqlens is None:
            return [(b, 0, self.T) for b in range(self.B)]
        cu = self.cu_seqlens
        return [(0, int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)]


# ----------------------------------------------------------------------------
# The five workloads named by the hot-path targets
# ----------------------------------------------------------------------------

CONFIGS = {
    1: Spec("tiny", B=1, T=64, H_qk=1, H_v=1, d_k=16, d_v=16, dtype="f32", chunk=16,
            gates="tiny", q_scale=False, seed=101),
    2: Spec("prefill", B=4, T=4096, H_qk=16, H_v=16, d_k=128, d_v=128, dtype="bf16",
            chunk=64, seed=102),
    # Decode: the single new token per sequence.  Its fp32 state comes from a
    # 512-token forward over ``decode_warmup_spec`` drawn from the same seed.
    3: Spec("decode", B=256, T=1, H_qk=32, H_v=32, d_k=128, d_v=128, dtype="bf16",
            chunk=64, seed=103),
    4: Spec("long", B=1, T=65536, H_qk=16, H_v=16, d_k=128, d_v=128, dtype="bf16",
            chunk=64, log_alpha_scale=1.0 / 64.0, seed=104),
    5: Spec("varlen", B=1, T=0, H_qk=16, H_v=32, d_k=128, d_v=128, dtype="bf16",
            chunk=64, packed_seqs=32, seed=105),
}

DECODE_WARMUP_TOKENS = 512


def config(i: int, **overrides) -> Spec:
    """The i-th workload (1-based), optionally with fields replaced."""
    spec = CONFIGS[i]
    if overrides:
        spec = Spec(**{**spec.__dict__, **overrides})
    return spec


def decode_warmup_spec(spec: Spec) -> Spec:
    """Spec of the 512-token forward whose final state seeds a decode step."""
    return Spec(**{**spec.__dict__, "name": spec.name + "-warmup",
                   "T": DECODE_WARMUP_TOKENS, "seed": spec.seed + 1_000_000})


# ----------------------------------------------------------------------------
# Generation
# ----------------------------------------------------------------------------

def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def _draw_sequence(seq_seed, L: int, spec: Spec, A_h: Optional[np.ndarray]):
    rng = np.random.default_rng(seq_seed)
    q = rng.standard_normal((L, spec.H_qk, spec.d_k), dtype=np.float32)
    k = rng.standard_normal((L, spec.H_qk, spec.d_k), dtype=np.float32)
    v = rng.standard_normal((L, spec.H_v, spec.d_v), dtype=np.float32)
    z_a = rng.standard_normal((L, spec.H_v))
    z_b = rng.standard_normal((L, spec.H_v))
    q = _unit_rows(q)
    if spec.q_scale:
        q = (q * np.float32(1.0 / math.sqrt(spec.d_k))).astype(np.float32)
    k = _unit_rows(k)
    if spec.gates == "tiny":
        alpha = _sigmoid(2.0 + 0.5 * z_a)
    else:
        log_alpha = -_softplus(z_a) * A_h[None, :] * spec.log_alpha_scale
        alpha = np.exp(log_alpha)
    beta = _sigmoid(z_b)
    return (_store(q, spec.dtype), _store(k, spec.dtype), _store(v, spec.dtype),
            alpha.astype(np.float32), beta.astype(np.float32))


def packed_lengths(spec: Spec) -> List[int]:
    """Sequence lengths of a packed batch (drawn from the workload's lengths stream)."""
    if spec.lengths is not None:
        return [int(x) for x in spec.lengths]
    root = np.random.SeedSequence(spec.seed)
    lengths_seed = root.spawn(1)[0]
    rng = np.random.default_rng(lengths_seed)
    u = rng.uniform(math.log(spec.min_len), math.log(spec.max_len), size=spec.packed_seqs)
    L = np.clip(np.round(np.exp(u)), spec.min_len, spec.max_len).astype(np.int64)
    return [int(x) for x in L]


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def generate(spec: Spec) -> Workload:
    """Draw the workload described by ``spec``."""
    root = np.random.SeedSequence(spec.seed)
    # Child 0 is reserved for the packed lengths, child 1 for per-head constants,
    # children 2.. for the sequences.
    if spec.packed_seqs or spec.lengths is not None:
        lengths = packed_lengths(spec)
    else:
        lengths = [spec.T] * spec.B
    n_seqs = len(lengths)
    children = root.spawn(2 + n_seqs)
    head_rng = np.random.default_rng(children[1])
    A_h = np.exp(head_rng.uniform(-4.0, 0.0, size=spec.H_v)) if spec.gates != "tiny" else None

    with ThreadPoolExecutor(_threads()) as ex:
        parts = list(ex.map(lambda i: _draw_sequence(children[2 + i], lengths[i], spec, A_h),
                            range(n_seqs)))

    if spec.packed_seqs or spec.lengths is not None:
        cu = np.zeros(n_seqs + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        cat = [np.concatenate([p[j] for p in parts], axis=0)[None] for j in range(5)]
        q, k, v, alpha, beta = cat
        return Workload(spec, q, k, v, alpha, beta, cu_seqlens=cu, lengths=lengths)
    q, k, v, alpha, beta = (np.stack([p[j] for p in parts], axis=0) for j in range(5))
    return Workload(spec, q, k, v, alpha, beta, cu_seqlens=None, lengths=lengths)


def random_state(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    """A seeded float32 N(0, scale^2) array (for initial states h0)."""
    rng = np.random.default_rng(np.random.SeedSequence(seed))
    return (scale * rng.standard_normal(shape, dtype=np.float32)).astype(np.float32)


def channel_rates(B: int, T: int, H_v: int, d_k: int, seed: int, lo: float = 0.8) -> np.ndarray:
    """Seeded float32 decay rates, one per token, value head and key channel,
    uniform in [lo, 1) (the per-channel gate's alpha, [B, T, H_v, d_k])."""
    rng = np.random.default_rng(np.random.SeedSequence(seed))
    return rng.uniform(lo, 1.0, (B, T, H_v, d_k)).astype(np.float32)


def block_inputs(B: int, T: int, H_qk: int, H_v: int, d_k: int, d_v: int, dtype: str, seed: int,
                 lengths: Optional[Sequence[int]] = None) -> dict:
    """Seeded raw inputs of a GDN block's prologue and epilogue: the q, k, v and
    output-gate projections (N(0, 1), stored as ``dtype``), depthwise
    convolution taps (N(0, 0.5^2)) and biases (N(0, 0.1^2)), gate projections
    a, b (N(0, 1)), log A = log U(0.5, 16) per value head, and RMS-norm
    weights 1 + N(0, 0.1^2).  With ``lengths`` the batch is packed (B == 1,
    T = sum of lengths) and ``cu_seqlens`` is included."""
    if lengths is not None:
        B, T = 1, int(sum(lengths))
    rng = np.random.default_rng(np.random.SeedSequence(seed))
    f = lambda *shape: rng.standard_normal(shape, dtype=np.float32)
    out = {
        "q_raw": _store(f(B, T, H_qk, d_k), dtype), "k_raw": _store(f(B, T, H_qk, d_k), dtype),
        "v_raw": _store(f(B, T, H_v, d_v), dtype), "g_raw": _store(f(B, T, H_v, d_v), dtype),
        "conv_q": 0.5 * f(H_qk * d_k, 4), "conv_k": 0.5 * f(H_qk * d_k, 4), "conv_v": 0.5 * f(H_v * d_v, 4),
        "conv_q_bias": 0.1 * f(H_qk * d_k), "conv_k_bias": 0.1 * f(H_qk * d_k),
        "conv_v_bias": 0.1 * f(H_v * d_v),
        "a_raw": f(B, T, H_v), "b_raw": f(B, T, H_v),
        "log_A": np.log(rng.uniform(0.5, 16.0, H_v)).astype(np.float32),
        "v_norm": (1.0 + 0.1 * f(d_v)).astype(np.float32), "o_norm": (1.0 + 0.1 * f(d_v)).astype(np.float32),
        "cu_seqlens": None, "B": B, "T": T,
    }
    if lengths is not None:
        cu = np.zeros(len(lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        out["cu_seqlens"] = cu
    return out
