"""CPU tests: the backward oracle against pins that do not use its own code.

- central finite differences of the forward oracle (the C recurrence),
- homogeneity identities of the forward map (Euler's theorem),
- the A = 0 case as a dense linear map, differentiated by hand,
- the one-token case in closed form,
- linearity in the incoming gradients,
and planted mistakes, each of which must fail at least one of them.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from oracle.backward import bwd as oracle_bwd
from tests.oracle_pins import rand_inputs, rel_err

KEYS = ("dX", "ddt", "dA", "dB", "dC", "dD", "dinit")


def loss(X, dt, A, B, C, D, G, dY, init, dF):
    Y, F, _ = oracle.fwd(X, dt, A, B, C, D, G, init_state=init)
    return float(np.sum(dY * Y) + (0.0 if dF is None else np.sum(dF * F)))


def setup(seed, Bz, T, H, P, N, G, with_init=True, with_dF=True, dt_shift=-1.0):
    rng = np.random.default_rng(seed)
    X, dt, A, B, C, D = rand_inputs(rng, Bz, T, H, P, N, G, dt_shift=dt_shift)
    dY = rng.standard_normal(X.shape)
    init = rng.standard_normal((Bz, H, P, N)) if with_init else None
    dF = rng.standard_normal((Bz, H, P, N)) if with_dF else None
    return X, dt, A, B, C, D, dY, init, dF


# --- pin 1: finite differences of the forward oracle ----------------------------------
def check_finite_differences(bwd, G, seed=11):
    X, dt, A, B, C, D, dY, init, dF = setup(seed, 2, 6, 2, 3, 4, G)
    g = bwd(X, dt, A, B, C, D, G, dY, init, dF)
    args = {"X": X, "dt": dt, "A": A, "B": B, "C": C, "D": D, "init": init}
    names = {"X": "dX", "dt": "ddt", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "init": "dinit"}
    for name, arr in args.items():
        fd = np.empty_like(arr)
        for idx in np.ndindex(arr.shape):
            v = arr[idx]
            eps = 1e-5 * max(1.0, abs(v))
            arr[idx] = v + eps
            lp = loss(X, dt, A, B, C, D, G, dY, init, dF)
            arr[idx] = v - eps
            lm = loss(X, dt, A, B, C, D, G, dY, init, dF)
            arr[idx] = v
            fd[idx] = (lp - lm) / (2 * eps)
        err = rel_err(g[names[name]], fd)
        assert err <= 1e-7, (name, err)


# --- pin 2: homogeneity (Euler's theorem) ------------------------------------------
def check_homogeneity(bwd, seed=12):
    """(Y, final) is linear in (X, init) jointly; with init = 0 the SSM part and the
    final state are linear in B, the SSM part in C; scaling dt by s and A by 1/s
    keeps every decay and scales the input terms by s."""
    G = 2
    X, dt, A, B, C, D, dY, init, dF = setup(seed, 2, 40, 4, 8, 8, G)
    Y, F, _ = oracle.fwd(X, dt, A, B, C, D, G, init_state=init)
    g = bwd(X, dt, A, B, C, D, G, dY, init, dF)
    lhs = np.sum(g["dX"] * X) + np.sum(g["dinit"] * init)
    rhs = np.sum(dY * Y) + np.sum(dF * F)
    assert abs(lhs - rhs) <= 1e-11 * (abs(rhs) + np.sum(np.abs(dY * Y))), (lhs, rhs)
    Y0, F0, _ = oracle.fwd(X, dt, A, B, C, D, G)
    g0 = bwd(X, dt, A, B, C, D, G, dY, None, dF)
    ssm = np.sum(dY * (Y0 - D[None, None, :, None] * X))
    fin = np.sum(dF * F0)
    scale = np.sum(np.abs(dY * Y0)) + np.sum(np.abs(dF * F0))
    assert abs(np.sum(g0["dB"] * B) - (ssm + fin)) <= 1e-11 * scale
    assert abs(np.sum(g0["dC"] * C) - ssm) <= 1e-11 * scale
    assert abs(np.sum(g0["ddt"] * dt) - np.sum(g0["dA"] * A) - (ssm + fin)) <= 1e-10 * scale


# --- pin 3: A = 0, a dense linear map -------------------------------------------
def check_no_decay_dense(bwd, seed=13):
    """With A = 0 every decay is 1: per head Y = M X + D X with M = tril(C B^T) diag(dt),
    a plain matrix product; its gradients are written out densely. dA is the
    derivative of exp(A * sum_{t=j+1..i} dt_t) at A = 0."""
    G = 2
    X, dt, A, B, C, D, dY, _, _ = setup(seed, 2, 24, 4, 5, 6, G)
    A = np.zeros_like(A)
    g = bwd(X, dt, A, B, C, D, G, dY, None, None)
    Bz, T, H, P = X.shape
    dX = np.zeros_like(X); ddt = np.zeros_like(dt); dA = np.zeros(H)
    dB = np.zeros_like(B); dC = np.zeros_like(C)
    low = np.tril(np.ones((T, T)))
    csum = np.cumsum(dt, axis=1)
    for b in range(Bz):
        for h in range(H):
            k = (h * G) // H
            CB = C[b, :, k] @ B[b, :, k].T                 # (T,T): C_i . B_j
            K = low * CB                                   # causal
            M = K * dt[b, :, h][None, :]
            dX[b, :, h] += M.T @ dY[b, :, h] + D[h] * dY[b, :, h]
            YX = dY[b, :, h] @ X[b, :, h].T                # (T,T): dY_i . X_j
            W = low * YX                                   # i >= j
            ddt[b, :, h] += np.sum(K * YX, axis=0)
            dC[b, :, k] += (W * dt[b, :, h][None, :]) @ B[b, :, k]
            dB[b, :, k] += dt[b, :, h][:, None] * (W.T @ C[b, :, k])
            span = csum[b, :, h][:, None] - csum[b, :, h][None, :]   # sum_{t=j+1..i} dt_t
            dA[h] += np.sum(M * YX * span * low)
    for name, ref in (("dX", dX), ("ddt", ddt), ("dA", dA), ("dB", dB), ("dC", dC)):
        assert rel_err(g[name], ref) <= 1e-11, (name, rel_err(g[name], ref))
    assert rel_err(g["dD"], np.einsum('bthp,bthp->h', dY, X)) <= 1e-13


# --- pin 4: one token, closed form ------------------------------------------------
def check_one_token(bwd, seed=14):
    X, dt, A, B, C, D, dY, h0, dF = setup(seed, 1, 1, 1, 3, 4, 1)
    g = bwd(X, dt, A, B, C, D, 1, dY, h0, dF)
    x, y, d, al = X[0, 0, 0], dY[0, 0, 0], dt[0, 0, 0], A[0]
    b, c, H0, F = B[0, 0, 0], C[0, 0, 0], h0[0, 0], dF[0, 0]
    a = math.exp(d * al)
    cb = c @ b
    ref = {
        "dX": d * cb * y + D[0] * y + d * (F @ b),
        "dB": d * (y @ x) * c + d * (F.T @ x),
        "dC": a * (H0.T @ y) + d * (y @ x) * b,
        "ddt": al * a * (y @ H0 @ c) + cb * (y @ x) + al * a * np.sum(F * H0) + x @ F @ b,
        "dA": d * a * (y @ H0 @ c + np.sum(F * H0)),
        "dinit": a * (np.outer(y, c) + F),
        "dD": y @ x,
    }
    got = {"dX": g["dX"][0, 0, 0], "dB": g["dB"][0, 0, 0], "dC": g["dC"][0, 0, 0],
           "ddt": g["ddt"][0, 0, 0], "dA": g["dA"][0], "dinit": g["dinit"][0, 0], "dD": g["dD"][0]}
    for k in ref:
        assert np.allclose(got[k], ref[k], rtol=1e-13, atol=1e-13), (k, got[k], ref[k])


# --- pin 5: linear in the incoming gradients ---------------------------------------
def check_linearity(bwd, seed=15):
    X, dt, A, B, C, D, dY, init, dF = setup(seed, 1, 17, 2, 4, 4, 1)
    g1 = bwd(X, dt, A, B, C, D, 1, dY, init, dF)
    g2 = bwd(X, dt, A, B, C, D, 1, -2.5 * dY, init, -2.5 * dF)
    for k in KEYS:
        if k == "dD":
            continue
        assert rel_err(g2[k], -2.5 * g1[k]) <= 1e-13, k


def check_fd_g1(bwd):
    check_finite_differences(bwd, 1)


def check_fd_g2(bwd):
    check_finite_differences(bwd, 2, seed=16)


ALL_BWD_PINS = [check_fd_g1, check_fd_g2, check_homogeneity, check_no_decay_dense, check_one_token,
                check_linearity]


@pytest.mark.parametrize("pin", ALL_BWD_PINS, ids=lambda f: f.__name__)
def test_backward_oracle_pin(pin):
    pin(oracle_bwd)


def test_backward_empty_and_shapes():
    X, dt, A, B, C, D, dY, init, dF = setup(17, 1, 0, 2, 3, 4, 1)
    g = oracle_bwd(X, dt, A, B, C, D, 1, dY, init, dF)
    assert g["dX"].shape == X.shape and np.array_equal(g["dinit"], dF)
    assert not np.any(g["dA"]) and not np.any(g["dD"])


# --- planted mistakes ------------------------------------------------------------
def _mutant(kind):
    """A back-propagation written independently of the oracle's array code (loops over
    b, h), with one mistake planted by `kind` ('none' plants nothing)."""
    def bwd(X, dt, A, B, C, D, G, dY, init, dF):
        Bz, T, H, P = X.shape
        N = B.shape[3]
        out = {"dX": np.zeros_like(X), "ddt": np.zeros_like(dt), "dA": np.zeros(H),
               "dB": np.zeros_like(B), "dC": np.zeros_like(C), "dD": np.zeros(H),
               "dinit": np.zeros((Bz, H, P, N))}
        for b in range(Bz):
            for h in range(H):
                k = (h % G) if kind == "group_mod" else (h * G) // H
                a = np.exp(dt[b, :, h] * A[h])
                s = [np.zeros((P, N)) if init is None else init[b, h].copy()]
                for t in range(T):
                    s.append(a[t] * s[-1] + dt[b, t, h] * np.outer(X[b, t, h], B[b, t, k]))
                ds = np.zeros((P, N)) if dF is None else dF[b, h].copy()
                for t in range(T - 1, -1, -1):
                    if kind == "decay_first":
                        ds = a[t] * ds + np.outer(dY[b, t, h], C[b, t, k])
                    else:
                        ds = ds + np.outer(dY[b, t, h], C[b, t, k])
                    s_t, s_p = s[t + 1], s[t]
                    out["dC"][b, t, k] += (s_p if kind == "dC_prev_state" else s_t).T @ dY[b, t, h]
                    v = ds @ B[b, t, k]
                    out["dX"][b, t, h] = dt[b, t, h] * v + D[h] * dY[b, t, h]
                    wdt = 1.0 if kind == "dB_no_dt" else dt[b, t, h]
                    out["dB"][b, t, k] += wdt * (ds.T @ X[b, t, h])
                    lam = np.sum(ds * a[t] * (s_t if kind == "lam_cur_state" else s_p))
                    out["ddt"][b, t, h] = X[b, t, h] @ v + (0.0 if kind == "ddt_no_decay" else A[h] * lam)
                    out["dA"][h] += dt[b, t, h] * lam
                    if kind != "decay_first":
                        ds = a[t] * ds
                out["dinit"][b, h] = ds / a[0] if (kind == "dinit_no_decay" and T) else ds
                out["dD"][h] += np.sum(dY[b, :, h] * X[b, :, h])
        return out
    return bwd


MUTANTS = ["group_mod", "decay_first", "dC_prev_state", "dB_no_dt", "lam_cur_state", "ddt_no_decay",
           "dinit_no_decay"]


def test_reference_mutant_harness_passes_pins():
    ref = _mutant("none")
    for pin in ALL_BWD_PINS:
        if pin in (check_fd_g1, check_fd_g2):
            continue  # slow through the loop harness; the array oracle covers them
        pin(ref)


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_is_caught(kind):
    bad = _mutant(kind)
    failed = []
    for pin in ALL_BWD_PINS:
        try:
            pin(bad)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {kind} passed every pin"
