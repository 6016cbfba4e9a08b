"""Oracle for the fused layer prologue and epilogue (fp64, TEST INFRASTRUCTURE).

What the gated entry points compute around the core, written out plainly:
the step size of the Mamba explainer page (a softplus makes it positive;
its training-stability notes, section 5.2, add a learned bias after the
softplus) and the output gate of the SSD theory page's selective-SSM layer
(section 4.1: y * SiLU(z)). Mode 1 puts the bias inside the softplus, the
convention of Mamba-2 implementations outside the pages; mode 2 is the
explainer's order.
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
