"""Oracle for the fused layer prologue and epilogue (fp64, TEST INFRASTRUCTURE).

What the gated entry points compute around the core, written out plainly:
the step size of the Mamba explainer page (a softplus makes it positive;
its training-stability notes, section 5.2, add a learned bias after the
softplus) and the output gate of the SSD theory page's selective-SSM layer
(section 4.1: y * SiLU(z)). Mode 1 puts the bias inside the softplus, the
convention of Mamba-2 implementations outside the pages; mode 2 is the
explainer's order. The same layer (SSD theory page, section 4.1) runs the
scan's input through a causal convolution over time with a 4-token window
and a SiLU first; the explainer's block structure (section 4.1) gives the
window and what it is for. It is read as depthwise (one 4-tap filter and a
bias per channel), with zeros before the first token.
"""
from __future__ import annotations

import numpy as np


def softplus(v):
    """log(1 + e^v), evaluated as log(e^0 + e^v) without overflow."""
    return np.logaddexp(0.0, np.asarray(v, np.float64))


def dt_prologue(dt, bias, mode: int):
    """dt (..., H); bias (H,) or None; mode 0: dt + bias, 1: softplus(dt + bias),
    2: softplus(dt) + bias."""
    dt = np.asarray(dt, np.float64)
    b = 0.0 if bias is None else np.asarray(bias, np.float64)
    if mode == 0:
        return dt + b
    if mode == 1:
        return softplus(dt + b)
    if mode == 2:
        return softplus(dt) + b
    raise ValueError(f"mode {mode}")


def silu(z):
    """z * sigmoid(z) = z / (1 + e^{-z})."""
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(-z))


def gate(y, z):
    """The output gate y * SiLU(z), elementwise."""
    return np.asarray(y, np.float64) * silu(z)


def causal_conv1d(x, w, bias):
    """Depthwise causal convolution over time: x (Bz, T, Cch), w (Cch, K),
    bias (Cch,) -> out[b, t, c] = bias[c] + sum_{k<K} w[c, k] x[b, t - (K-1) + k, c],
    with x = 0 before the first token."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    Bz, T, Cch = x.shape
    K = w.shape[1]
    out = np.broadcast_to(np.asarray(bias, np.float64), (Bz, T, Cch)).copy()
    for k in range(K):
        lag = K - 1 - k            # tap k reads the token `lag` steps back
        if lag < T:
            out[:, lag:, :] += w[None, None, :, k] * x[:, :T - lag, :]
    return out


def conv_silu(x, w, bias):
    """The layer's input activation: SiLU(causal_conv1d(x, w, bias))."""
    return silu(causal_conv1d(x, w, bias))
