"""CPU pin of the oracle against an independent Mamba-2 implementation.

The transformers package in this image carries a PyTorch Mamba-2 whose
chunked scan (mamba2_chunk_scan) is written independently of this repository.
In float64 it must agree with the oracle's sequential recurrence on
everything the pages leave to convention and that implementation fixes by
data: the contiguous head -> group mapping (head h reads group h // (H / G)),
softplus(raw + bias) as the step-size prologue (dt_softplus = True), the
zero-order-hold decay exp(dt A), dt on the input term, the diagonal of the
mask, the D skip, a partial last chunk, a carried initial state and the
final state. It runs offline (no kernel is fetched; the PyTorch path runs).
"""
from __future__ import annotations

import os

import numpy as np
import pytest

os.environ.setdefault("HF_HUB_OFFLINE", "1")

torch = pytest.importorskip("torch")
mamba2 = pytest.importorskip("transformers.models.mamba2.modeling_mamba2")

import oracle  # noqa: E402
from oracle.fused import dt_prologue  # noqa: E402

# its chunked evaluation keeps the chunk states in float32 even for float64
# inputs (its final states come back as float32), so it agrees with the fp64
# recurrence to ~1e-6 relative; a dropped term, a wrong group or a misplaced
# bias moves the result by O(1)
TOL = 1e-5


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


def _case(seed, b, T, H, P, N, G):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((b, T, H, P))
    raw = rng.standard_normal((b, T, H)) - 2.0
    A = -np.exp(rng.uniform(0.0, np.log(16.0), H))
    B = rng.standard_normal((b, T, G, N)) / np.sqrt(N)
    C = rng.standard_normal((b, T, G, N)) / np.sqrt(N)
    D = rng.standard_normal(H)
    bias = 0.5 * rng.standard_normal(H)
    h0 = rng.standard_normal((b, H, P, N))
    return X, raw, A, B, C, D, bias, h0


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


@pytest.mark.parametrize("b,T,H,P,N,G,chunk", [
    (2, 100, 4, 8, 16, 2, 32),    # groups, ragged last chunk
    (1, 64, 6, 4, 8, 1, 16),      # one group shared by all heads
    (2, 37, 4, 8, 8, 4, 16),      # one group per head
])
def test_oracle_matches_transformers_chunk_scan(b, T, H, P, N, G, chunk):
    X, raw, A, B, C, D, bias, _ = _case(7 + T, b, T, H, P, N, G)
    dt = dt_prologue(raw, bias, 1)
    Y, F, _ = oracle.fwd(X, dt, A, B, C, D, G)
    y, f = mamba2.mamba2_chunk_scan(_t(X), _t(raw), _t(A), _t(B), _t(C), chunk, D=_t(D), dt_bias=_t(bias),
                                    dt_softplus=True, return_final_states=True)
    assert _rel(y.numpy(), Y) < TOL
    assert _rel(f.numpy(), F) < TOL


def test_oracle_matches_transformers_from_initial_state():
    b, T, H, P, N, G = 2, 70, 4, 8, 16, 2
    X, raw, A, B, C, D, bias, h0 = _case(99, b, T, H, P, N, G)
    dt = dt_prologue(raw, bias, 1)
    Y, F, _ = oracle.fwd(X, dt, A, B, C, D, G, init_state=h0)
    y, f = mamba2.mamba2_chunk_scan(_t(X), _t(raw), _t(A), _t(B), _t(C), 32, D=_t(D), dt_bias=_t(bias),
                                    initial_states=_t(h0), dt_softplus=True, return_final_states=True)
    assert _rel(y.numpy(), Y) < TOL
    assert _rel(f.numpy(), F) < TOL


def test_a_wrong_group_mapping_is_caught():
    """The pin is sensitive to R3: the oracle under a strided mapping (head h
    reading group h mod G, written here by permuting the heads) disagrees."""
    b, T, H, P, N, G = 1, 50, 4, 4, 8, 2
    X, raw, A, B, C, D, bias, _ = _case(5, b, T, H, P, N, G)
    dt = dt_prologue(raw, bias, 1)
    # heads reordered so that contiguous groups in the permuted order are h mod G in the original
    perm = np.array([0, 2, 1, 3])
    Yp, _, _ = oracle.fwd(X[:, :, perm], dt[:, :, perm], A[perm], B, C, D[perm], G)
    Y_strided = np.empty_like(Yp)
    Y_strided[:, :, perm] = Yp
    y = mamba2.mamba2_chunk_scan(_t(X), _t(raw), _t(A), _t(B), _t(C), 16, D=_t(D), dt_bias=_t(bias),
                                 dt_softplus=True)
    y = y[0] if isinstance(y, tuple) else y
    assert _rel(y.numpy(), Y_strided) > 1e-2
