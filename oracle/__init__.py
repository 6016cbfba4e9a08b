"""CPU oracle for the SSD core (fp64 sequential recurrence + dense dual form).

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package. It shares no code with
the HIP library and never imports it.

Pins (tests/test_oracle.py): the dense dual form, closed forms for a constant
decay, the A = 0 linear-attention special case, the memoryless limit, the
group mapping, causality, linearity, split invariance with an initial state,
step/forward consistency and a hand-derived example under tests/golden/.
The backward oracle (backward.py) is pinned in tests/test_oracle_bwd.py by
finite differences of the forward, homogeneity identities and closed forms.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .backward import bwd  # noqa: F401
from .dual import dual_form, decay_mask  # noqa: F401
from .fused import causal_conv1d, conv_silu, dt_prologue, gate, silu, softplus  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libssd_oracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(
            os.path.join(_HERE, "ssd_oracle.c")):
        from .build import build
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_ssd_fwd.restype = ctypes.c_int
    lib.oracle_ssd_fwd.argtypes = [_D] * 9 + [_D, _I] + [_I] * 6
    lib.oracle_ssd_step.restype = ctypes.c_int
    lib.oracle_ssd_step.argtypes = [_D] * 8 + [_I] * 5
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    _lib = lib
    return lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    return None if a is None else a.ctypes.data_as(_D)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def fwd(X, dt, A, B, C, D, ngroups: int, init_state=None, trace_every: int = 0):
    """Sequential fp64 recurrence over a whole sequence.

    X (Bz,T,H,P), dt (Bz,T,H), A (H,), B/C (Bz,T,G,N), D (H,), init_state
    (Bz,H,P,N) or None. Returns (Y, final_state, trace) where trace is None
    unless trace_every > 0; then trace[:, k] is the state after token
    (k + 1) * trace_every - 1.
    """
    lib = _load()
    X, dt, A, B, C, D = map(_f64, (X, dt, A, B, C, D))
    Bz, T, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    assert dt.shape == (Bz, T, H) and B.shape == (Bz, T, G, N) and C.shape == B.shape
    assert A.shape == (H,) and D.shape == (H,)
    init = None if init_state is None else _f64(init_state)
    if init is not None:
        assert init.shape == (Bz, H, P, N)
    Y = np.empty_like(X)
    final = np.empty((Bz, H, P, N), dtype=np.float64)
    trace = None
    if trace_every > 0:
        trace = np.empty((Bz, T // trace_every, H, P, N), dtype=np.float64)
    rc = lib.oracle_ssd_fwd(_p(X), _p(dt), _p(A), _p(B), _p(C), _p(D), _p(init), _p(Y),
                            _p(final), _p(trace), trace_every, Bz, T, H, P, N, G)
    if rc != 0:
        raise ValueError(f"oracle_ssd_fwd rejected its arguments (rc={rc})")
    return Y, final, trace


def step(state, x, dt, A, B, C, D, ngroups: int):
    """One decode step. state (Bz,H,P,N) fp64 is updated IN PLACE; returns y (Bz,H,P)."""
    lib = _load()
    assert state.dtype == np.float64 and state.flags.c_contiguous
    x, dt, A, B, C, D = map(_f64, (x, dt, A, B, C, D))
    Bz, H, P, N = state.shape
    G = B.shape[1]
    assert x.shape == (Bz, H, P) and dt.shape == (Bz, H) and B.shape == (Bz, G, N)
    y = np.empty((Bz, H, P), dtype=np.float64)
    rc = lib.oracle_ssd_step(_p(state), _p(x), _p(dt), _p(A), _p(B), _p(C), _p(D), _p(y),
                             Bz, H, P, N, G)
    if rc != 0:
        raise ValueError(f"oracle_ssd_step rejected its arguments (rc={rc})")
    return y
