"""Float64 oracle of the steps around the recurrence in a GDN block (test infrastructure).

TEST INFRASTRUCTURE ONLY, like the rest of this package: the tests, the
smoke check and the benchmark's CPU baseline are the only callers.

"Linear attention" (arsalanzafar.ai), section "A naive PyTorch
implementation", describes what a GDN block does on either side of
Eqs. (1)-(4), after the q, k, v and gate projections and before the output
projection.  Written out here from that description (projections excluded;
they are plain matrix products):

* a causal depthwise convolution of width 4 on every channel of q, k and v,
  left-padded with zeros so the first token sees three zeros, followed by
  SiLU (``causal_conv_silu``);
* q and k scaled to unit length per head; v RMS-normalised per head
  (``unit_rows``, ``rms_norm``);
* alpha = exp(-A softplus(a)) with A = exp(log A) per head, beta =
  sigmoid(b) (``gates``);
* after the recurrence: the output RMS-normalised per head, times SiLU of
  the output gate's projection (``epilogue``).

Readings where the page leaves a detail open are listed in the design notes:
the convolution has a bias (the layer it uses is built without turning its
bias off); a packed batch pads every sequence separately; the unit-length
scaling divides by max(norm, 1e-12); the RMS normalisation divides by
sqrt(mean of squares + eps); ``q_scale`` (1 on the page) multiplies q after
its unit-length scaling.

Pins: ``tests/test_oracle_block_pins.py``.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

from . import _as_f64

CONV_WIDTH = 4


def silu(x: np.ndarray) -> np.ndarray:
    """x times the logistic function of x."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def softplus(x: np.ndarray) -> np.ndarray:
    """log(1 + e^x), evaluated without overflow."""
    x = np.asarray(x, dtype=np.float64)
    return np.logaddexp(0.0, x)


def sigmoid(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def _sequences(B: int, T: int, cu_seqlens) -> Sequence[Tuple[int, int, int]]:
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if B != 1:
        raise ValueError("oracle: a packed batch has B == 1")
    return [(0, int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)]


def causal_conv(x, weight, bias=None, cu_seqlens=None) -> np.ndarray:
    """Depthwise causal convolution of width 4 along the token axis.

    x: [B, T, C] (C channels); weight: [C, 4]; bias: [C] or None.  Output
    token t of channel c is bias[c] + sum_j weight[c, j] * x[t - 3 + j, c],
    where tokens before the start of t's sequence are zeros.
    """
    x = _as_f64(np.asarray(x))
    w = np.asarray(weight, dtype=np.float64)
    B, T, C = x.shape
    out = np.zeros_like(x)
    if bias is not None:
        out += np.asarray(bias, dtype=np.float64)[None, None, :]
    for b, s, e in _sequences(B, T, cu_seqlens):
        seg = x[b, s:e]
        L = e - s
        for j in range(CONV_WIDTH):
            shift = CONV_WIDTH - 1 - j  # tap j reads the token `shift` steps back
            if shift >= L:
                continue
            out[b, s + shift:e] += w[None, :, j] * seg[:L - shift]
    return out


def causal_conv_silu(x, weight, bias=None, cu_seqlens=None) -> np.ndarray:
    return silu(causal_conv(x, weight, bias, cu_seqlens))


def unit_rows(x: np.ndarray, eps: float = 1e-12) -> np.ndarray:
    """Each vector along the last axis divided by max(its Euclidean norm, eps)."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, eps)


def rms_norm(x: np.ndarray, weight=None, eps: float = 1e-6) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) along the last axis, times ``weight``."""
    x = np.asarray(x, dtype=np.float64)
    y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    if weight is not None:
        y = y * np.asarray(weight, dtype=np.float64)
    return y


def gates(a_raw, b_raw, log_A) -> Tuple[np.ndarray, np.ndarray]:
    """alpha = exp(-exp(log_A[h]) * softplus(a_raw)), beta = sigmoid(b_raw).

    a_raw, b_raw: [..., H]; log_A: [H].
    """
    A = np.exp(np.asarray(log_A, dtype=np.float64))
    alpha = np.exp(-A * softplus(a_raw))
    beta = sigmoid(b_raw)
    return alpha, beta


def prologue(q_raw, k_raw, v_raw, conv_q, conv_k, conv_v, a_raw, b_raw, log_A, *,
             conv_q_bias=None, conv_k_bias=None, conv_v_bias=None, norm_weight=None,
             eps: float = 1e-6, q_scale: float = 1.0, cu_seqlens=None):
    """The block's steps between the projections and the recurrence.

    q_raw, k_raw: [B, T, H_qk, d_k]; v_raw: [B, T, H_v, d_v] (float values or
    bf16 bits); conv_*: [H * d, 4] over the flattened (head, feature)
    channels; a_raw, b_raw: [B, T, H_v]; log_A: [H_v]; norm_weight: [d_v].
    Returns q, k, v, alpha, beta in float64, shaped like the recurrence's
    inputs.
    """
    def conv(x, w, bias):
        x = _as_f64(np.asarray(x))
        B, T, H, d = x.shape
        y = causal_conv_silu(x.reshape(B, T, H * d), w, bias, cu_seqlens)
        return y.reshape(B, T, H, d)

    q = unit_rows(conv(q_raw, conv_q, conv_q_bias)) * q_scale
    k = unit_rows(conv(k_raw, conv_k, conv_k_bias))
    v = rms_norm(conv(v_raw, conv_v, conv_v_bias), norm_weight, eps)
    alpha, beta = gates(a_raw, b_raw, log_A)
    return q, k, v, alpha, beta


def epilogue(o, gate_raw, norm_weight=None, eps: float = 1e-6) -> np.ndarray:
    """The block's steps after the recurrence: RMS normalisation of each head's
    output times SiLU of the output gate's projection.

    o: [B, T, H_v, d_v]; gate_raw: [B, T, H_v, d_v] (the projection of the
    token's input, one value per output feature).
    """
    return rms_norm(_as_f64(np.asarray(o)), norm_weight, eps) * silu(_as_f64(np.asarray(gate_raw)))
