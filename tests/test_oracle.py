"""CPU tests: the oracle against its pins, and the pins against planted mistakes."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins


def oracle_fwd(X, dt, A, B, C, D, G, init_state=None):
    Y, F, _ = oracle.fwd(X, dt, A, B, C, D, G, init_state=init_state)
    return Y, F


@pytest.mark.parametrize("pin", pins.ALL_FWD_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle_fwd)


def test_oracle_matches_dual_form():
    pins.check_dual_form(oracle_fwd, oracle.dual_form)


def test_dual_form_on_tiny_workload_shape():
    # the tiny fp32 workload's shape (T 256, H 2, P 16, N 16), fp64 values
    pins.check_dual_form(oracle_fwd, oracle.dual_form, seed=11, shapes=((1, 256, 2, 16, 16, 1),))


def test_dual_form_mask_is_product_of_decays():
    # L[i, j] = prod_{t=j+1..i} a_t (reading report, section 2.2), checked by brute force
    rng = np.random.default_rng(1)
    d = rng.uniform(0.01, 0.5, size=12)
    a = -2.3
    L = oracle.decay_mask(d, a)
    for i in range(12):
        for j in range(12):
            ref = float(np.prod(np.exp(a * d[j + 1:i + 1]))) if i >= j else 0.0
            assert abs(L[i, j] - ref) <= 1e-15 * max(1.0, abs(ref))


def test_step_matches_fwd():
    rng = np.random.default_rng(12)
    Bz, T, H, P, N, G = 2, 33, 4, 3, 5, 2
    X, dt, A, B, C, D = pins.rand_inputs(rng, Bz, T, H, P, N, G)
    Y, F = oracle_fwd(X, dt, A, B, C, D, G)
    s = np.zeros((Bz, H, P, N))
    for t in range(T):
        y = oracle.step(s, X[:, t], dt[:, t], A, B[:, t], C[:, t], D, G)
        assert pins.rel_err(y, Y[:, t]) <= 1e-14
    assert pins.rel_err(s, F) <= 1e-14


def test_step_from_nonzero_state_matches_fwd_with_init():
    rng = np.random.default_rng(13)
    Bz, H, P, N, G = 3, 4, 2, 6, 1
    X, dt, A, B, C, D = pins.rand_inputs(rng, Bz, 1, H, P, N, G)
    s0 = rng.standard_normal((Bz, H, P, N))
    Y, F = oracle_fwd(X, dt, A, B, C, D, G, init_state=s0)
    s = s0.copy()
    y = oracle.step(s, X[:, 0], dt[:, 0], A, B[:, 0], C[:, 0], D, G)
    assert pins.rel_err(y, Y[:, 0]) <= 1e-15
    assert pins.rel_err(s, F) <= 1e-15


def test_trace_states_are_prefix_final_states():
    rng = np.random.default_rng(14)
    Bz, T, H, P, N, G = 1, 40, 2, 3, 4, 1
    X, dt, A, B, C, D = pins.rand_inputs(rng, Bz, T, H, P, N, G)
    _, _, trace = oracle.fwd(X, dt, A, B, C, D, G, trace_every=16)
    assert trace.shape == (1, 2, H, P, N)
    for k in range(2):
        t_end = (k + 1) * 16
        _, Fk = oracle_fwd(X[:, :t_end], dt[:, :t_end], A, B[:, :t_end], C[:, :t_end], D, G)
        assert np.array_equal(trace[:, k], Fk)


def test_oracle_rejects_bad_shapes():
    rng = np.random.default_rng(0)
    X, dt, A, B, C, D = pins.rand_inputs(rng, 1, 4, 3, 2, 2, 1)
    with pytest.raises(ValueError):
        # 3 heads cannot be split into 2 groups
        oracle.fwd(X, dt, A, np.concatenate([B, B], 2), np.concatenate([C, C], 2), D, 2)


def test_empty_sequence():
    X = np.zeros((1, 0, 2, 3))
    dt = np.zeros((1, 0, 2))
    B = np.zeros((1, 0, 1, 4))
    Y, F = oracle_fwd(X, dt, np.array([-1.0, -2.0]), B, B, np.array([1.0, 1.0]), 1)
    assert Y.shape == (1, 0, 2, 3) and not np.any(F)


# ----------------------------------------------------------------------------
# Planted mistakes: each wrong recurrence must fail at least one pin.
# ----------------------------------------------------------------------------
def _mutant(kind):
    def fwd(X, dt, A, B, C, D, G, init_state=None):
        Bz, T, H, P = X.shape
        N = B.shape[-1]
        Y = np.zeros_like(X)
        F = np.zeros((Bz, H, P, N))
        for b in range(Bz):
            for h in range(H):
                g = (h % G) if kind == "groups_mod" else (h * G) // H
                s = np.zeros((P, N)) if init_state is None else init_state[b, h].copy()
                for t in range(T):
                    d = dt[b, t, h]
                    a = 1.0 + d * A[h] if kind == "euler" else math.exp(d * A[h])
                    if kind == "decay_sign":
                        a = math.exp(-d * A[h]) if d * A[h] > -50 else 0.0
                    x = X[b, t, h]
                    bi, ci = B[b, t, g], C[b, t, g]
                    if kind == "swap_bc":
                        bi, ci = ci, bi
                    u = x if kind == "no_dt_input" else d * x
                    prev = s.copy()
                    if kind == "decay_after_input":
                        s = a * (s + np.outer(u, bi))
                    else:
                        s = a * s + np.outer(u, bi)
                    readout = prev if kind == "strict_lower" else s
                    skip = 0.0 if kind == "no_skip" else D[h] * x
                    if kind == "skip_scaled_dt":
                        skip = D[h] * d * x
                    Y[b, t, h] = readout @ ci + skip
                F[b, h] = s
        return Y, F
    return fwd


MUTANTS = ("euler", "decay_sign", "swap_bc", "no_dt_input", "decay_after_input",
           "strict_lower", "no_skip", "skip_scaled_dt", "groups_mod")


def test_reference_mutant_harness_passes_pins():
    # the unmutated Python recurrence passes every pin (the harness is fair)
    good = _mutant("none")
    for pin in pins.ALL_FWD_PINS:
        pin(good)


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_is_caught(kind):
    bad = _mutant(kind)
    failed = []
    for pin in pins.ALL_FWD_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(bad)
        except (AssertionError, FloatingPointError, OverflowError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {kind!r} passed every pin"


# ---- the fused prologue / epilogue (oracle.fused) ----

def test_softplus_pins():
    import oracle
    assert oracle.softplus(0.0) == np.log(2.0)
    x = np.linspace(-30, 30, 601)
    sp = oracle.softplus(x)
    # softplus(x) - softplus(-x) = x (log(1+e^x) - log(1+e^-x) = log e^x), and it stays above max(x, 0)
    assert np.max(np.abs(sp - oracle.softplus(-x) - x)) < 1e-12
    assert np.all(sp > np.maximum(x, 0.0))
    # far out it is e^x (left) and x + e^-x (right) to first order
    assert abs(oracle.softplus(-30.0) / np.exp(-30.0) - 1) < 1e-12
    assert abs(oracle.softplus(30.0) - 30.0 - np.exp(-30.0)) < 1e-14
    assert oracle.softplus(800.0) == 800.0  # no overflow


def test_dt_prologue_modes():
    import oracle
    dt = np.array([[-1.0, 0.5, 2.0]])
    bias = np.array([0.25, -0.5, 1.0])
    assert np.array_equal(oracle.dt_prologue(dt, None, 0), dt)
    assert np.allclose(oracle.dt_prologue(dt, bias, 0), dt + bias)
    assert np.allclose(oracle.dt_prologue(dt, bias, 1), np.log1p(np.exp(dt + bias)))
    assert np.allclose(oracle.dt_prologue(dt, bias, 2), np.log1p(np.exp(dt)) + bias)
    # the two orders differ unless the bias is zero
    assert not np.allclose(oracle.dt_prologue(dt, bias, 1), oracle.dt_prologue(dt, bias, 2))
    assert np.allclose(oracle.dt_prologue(dt, None, 1), oracle.dt_prologue(dt, None, 2))


def test_silu_gate_pins():
    import oracle
    z = np.linspace(-40, 40, 801)
    s = oracle.silu(z)
    assert oracle.silu(0.0) == 0.0
    # sigmoid(z) + sigmoid(-z) = 1, so silu(z) - silu(-z) = z
    assert np.max(np.abs(s - oracle.silu(-z) - z)) < 1e-12
    assert abs(oracle.silu(40.0) - 40.0) < 1e-15 * 40 + 40 * np.exp(-40.0) * 2
    assert abs(oracle.silu(-40.0)) < 40 * np.exp(-40.0) * 1.01
    y = np.array([1.5, -2.0, 3.0])
    assert np.allclose(oracle.gate(y, np.zeros(3)), 0.0)
    # for large z the gate passes y * z (sigmoid -> 1), for very negative z it closes
    assert np.allclose(oracle.gate(y, np.full(3, 50.0)), 50.0 * y)
    assert np.max(np.abs(oracle.gate(y, np.full(3, -50.0)))) < 1e-19


def test_causal_conv1d_pins():
    import oracle
    rng = np.random.default_rng(40)
    x = rng.standard_normal((2, 13, 5))
    w = rng.standard_normal((5, 4))
    bias = rng.standard_normal(5)
    out = oracle.causal_conv1d(x, w, bias)
    # each channel is numpy's full convolution with the reversed taps, first T samples
    for b in range(2):
        for c in range(5):
            ref = np.convolve(x[b, :, c], w[c, ::-1])[:13] + bias[c]
            assert np.max(np.abs(out[b, :, c] - ref)) < 1e-12
    # the last tap alone is the identity; the first alone a 3-token delay
    e = np.zeros((5, 4)); e[:, 3] = 1.0
    assert np.allclose(oracle.causal_conv1d(x, e, np.zeros(5)), x)
    d = np.zeros((5, 4)); d[:, 0] = 1.0
    sh = oracle.causal_conv1d(x, d, np.zeros(5))
    assert np.allclose(sh[:, 3:], x[:, :-3]) and not np.any(sh[:, :3])
    # causal: changing token 7 leaves outputs before it unchanged
    x2 = x.copy(); x2[:, 7] += 1.0
    assert np.array_equal(oracle.causal_conv1d(x2, w, bias)[:, :7], out[:, :7])
    # conv_silu is SiLU of it
    assert np.allclose(oracle.conv_silu(x, w, bias), out / (1 + np.exp(-out)))
