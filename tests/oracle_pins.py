"""Pins for the CPU oracle: checks against facts fixed by the pages and by the
mathematics, written so that each takes the forward function under test as an
argument. tests/test_oracle.py runs them on the oracle; the mutation test runs
them on deliberately wrong recurrences to show that each plausible mistake
fails at least one pin.

A forward function has the signature
    fwd(X, dt, A, B, C, D, ngroups, init_state=None) -> (Y, final_state)
with fp64 numpy arrays in the layouts X (Bz,T,H,P), dt (Bz,T,H), A/D (H,),
B/C (Bz,T,G,N), states (Bz,H,P,N).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rel_err(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = float(np.max(np.abs(b))) if b.size else 0.0
    num = float(np.max(np.abs(a - b))) if a.size else 0.0
    return num / den if den > 0 else num


def rand_inputs(rng, Bz, T, H, P, N, G, dt_shift=-1.0, a_lo=0.0, a_hi=math.log(16.0)):
    X = rng.standard_normal((Bz, T, H, P))
    dt = np.log1p(np.exp(rng.standard_normal((Bz, T, H)) + dt_shift))
    A = -np.exp(rng.uniform(a_lo, a_hi, size=H))
    B = rng.standard_normal((Bz, T, G, N)) / math.sqrt(N)
    C = rng.standard_normal((Bz, T, G, N)) / math.sqrt(N)
    D = rng.standard_normal(H)
    return X, dt, A, B, C, D


# --- pin 1: hand-derived worked example -------------------------------------
def check_golden_hand_example(fwd, tol=1e-13):
    with open(os.path.join(GOLDEN, "hand_example_t4.json")) as f:
        g = json.load(f)
    inp, exp_ = g["inputs"], g["expected"]
    ln2 = math.log(2.0)
    T = len(inp["x"])
    X = np.array(inp["x"], np.float64).reshape(1, T, 1, 1)
    dt = (np.array(inp["dt_over_ln2"], np.float64) * ln2).reshape(1, T, 1)
    B = np.array(inp["B"], np.float64).reshape(1, T, 1, 2)
    C = np.array(inp["C"], np.float64).reshape(1, T, 1, 2)
    A = np.array(inp["A"], np.float64)
    D = np.array(inp["D"], np.float64)
    Y, fin = fwd(X, dt, A, B, C, D, 1)
    y_ref = np.array(exp_["y_coef_ln2"]) * ln2 + np.array(exp_["y_coef_one"])
    f_ref = np.array(exp_["final_state_coef_ln2"]) * ln2
    assert np.max(np.abs(Y.reshape(-1) - y_ref)) <= tol, (Y.reshape(-1), y_ref)
    assert np.max(np.abs(fin.reshape(-1) - f_ref)) <= tol, (fin.reshape(-1), f_ref)


# --- pin 2: dense dual form (masked attention) -------------------------------
def check_dual_form(fwd, dual, seed=0, shapes=((1, 64, 2, 16, 16, 1), (2, 37, 4, 8, 8, 2)),
                    tol=1e-10):
    rng = np.random.default_rng(seed)
    for (Bz, T, H, P, N, G) in shapes:
        X, dt, A, B, C, D = rand_inputs(rng, Bz, T, H, P, N, G)
        Y, fin = fwd(X, dt, A, B, C, D, G)
        Yd, find = dual(X, dt, A, B, C, D, G)
        assert rel_err(Y, Yd) <= tol, ("Y", rel_err(Y, Yd), (Bz, T, H, P, N, G))
        assert rel_err(fin, find) <= tol, ("final", rel_err(fin, find), (Bz, T, H, P, N, G))


# --- pin 3: closed form for a constant decay ---------------------------------
def check_closed_form_constant_decay(fwd, tol=1e-12):
    """dt = delta, A = alpha (a = exp(delta*alpha) < 1), constant b, c, x:
    y_t = delta (c.b) x (1 - a^{t+1}) / (1 - a) + D x,
    final = delta x b^T (1 - a^T) / (1 - a)."""
    T, P, N = 50, 3, 4
    delta, alpha, Dv = 0.3, -0.7, 0.25
    rng = np.random.default_rng(7)
    b = rng.standard_normal(N)
    c = rng.standard_normal(N)
    x = rng.standard_normal(P)
    X = np.broadcast_to(x, (1, T, 1, P)).copy()
    dt = np.full((1, T, 1), delta)
    B = np.broadcast_to(b, (1, T, 1, N)).copy()
    C = np.broadcast_to(c, (1, T, 1, N)).copy()
    Y, fin = fwd(X, dt, np.array([alpha]), B, C, np.array([Dv]), 1)
    a = math.exp(delta * alpha)
    t = np.arange(T)
    geo = (1.0 - a ** (t + 1)) / (1.0 - a)
    y_ref = delta * float(c @ b) * geo[:, None] * x[None, :] + Dv * x[None, :]
    f_ref = delta * np.outer(x, b) * (1.0 - a ** T) / (1.0 - a)
    assert rel_err(Y[0, :, 0, :], y_ref) <= tol, rel_err(Y[0, :, 0, :], y_ref)
    assert rel_err(fin[0, 0], f_ref) <= tol, rel_err(fin[0, 0], f_ref)


# --- pin 4: A = 0 gives a = 1 exactly: a plain running sum -------------------
def check_closed_form_no_decay(fwd, tol=1e-12):
    """A = 0 with constant inputs: y_t = delta (c.b) x (t + 1) + D x."""
    T, P, N = 40, 2, 3
    delta, Dv = 0.2, -1.5
    b = np.array([0.5, -1.0, 2.0])
    c = np.array([1.0, 0.25, -0.5])
    x = np.array([1.5, -0.75])
    X = np.broadcast_to(x, (1, T, 1, P)).copy()
    dt = np.full((1, T, 1), delta)
    B = np.broadcast_to(b, (1, T, 1, N)).copy()
    C = np.broadcast_to(c, (1, T, 1, N)).copy()
    Y, fin = fwd(X, dt, np.array([0.0]), B, C, np.array([Dv]), 1)
    t = np.arange(T)
    y_ref = delta * float(c @ b) * (t + 1)[:, None] * x[None, :] + Dv * x[None, :]
    assert rel_err(Y[0, :, 0, :], y_ref) <= tol
    assert rel_err(fin[0, 0], delta * T * np.outer(x, b)) <= tol


# --- pin 5: A = 0 with varying inputs is causal linear attention -------------
def check_linear_attention(fwd, seed=3, tol=1e-11):
    """With A = 0 every decay is 1 and the map is unnormalised causal linear
    attention (linear attention is a special case of the SSM: 'Transformer vs
    Mamba/SSM', core concepts): Y = tril(C B^T) diag(dt) X + D X."""
    rng = np.random.default_rng(seed)
    Bz, T, H, P, N, G = 2, 45, 2, 5, 6, 1
    X, dt, _, B, C, D = rand_inputs(rng, Bz, T, H, P, N, G)
    A = np.zeros(H)
    Y, fin = fwd(X, dt, A, B, C, D, G)
    for b in range(Bz):
        for h in range(H):
            S = np.tril(C[b, :, 0, :] @ B[b, :, 0, :].T)
            ref = S @ (dt[b, :, h, None] * X[b, :, h, :]) + D[h] * X[b, :, h, :]
            assert rel_err(Y[b, :, h, :], ref) <= tol
            fref = (dt[b, :, h, None] * X[b, :, h, :]).T @ B[b, :, 0, :]
            assert rel_err(fin[b, h], fref) <= tol


# --- pin 6: the memoryless limit --------------------------------------------
def check_memoryless(fwd, seed=4, tol=1e-13):
    """dt*A <= -800 underflows the decay to exactly 0: each output sees only
    its own token, y_t = dt_t (C_t . B_t) x_t + D x_t (pins L_ii = 1)."""
    rng = np.random.default_rng(seed)
    Bz, T, H, P, N, G = 1, 20, 2, 3, 4, 1
    X, dt, _, B, C, D = rand_inputs(rng, Bz, T, H, P, N, G)
    dt = dt + 1.0
    A = np.full(H, -1000.0)
    Y, fin = fwd(X, dt, A, B, C, D, G)
    cb = np.einsum("tn,tn->t", C[0, :, 0, :], B[0, :, 0, :])
    for h in range(H):
        ref = (dt[0, :, h] * cb)[:, None] * X[0, :, h, :] + D[h] * X[0, :, h, :]
        assert rel_err(Y[0, :, h, :], ref) <= tol
        fref = dt[0, -1, h] * np.outer(X[0, -1, h, :], B[0, -1, 0, :])
        assert rel_err(fin[0, h], fref) <= tol


# --- pin 7: contiguous group mapping ----------------------------------------
def check_group_mapping(fwd, seed=5):
    """G = 8, H = 16: with B zero in every group but k, only heads with
    floor(h * G / H) == k get an SSM term; all others output exactly D x."""
    rng = np.random.default_rng(seed)
    Bz, T, H, P, N, G = 1, 16, 16, 2, 4, 8
    X, dt, A, B, C, D = rand_inputs(rng, Bz, T, H, P, N, G)
    for k in (0, 3, 7):
        Bk = np.zeros_like(B)
        Bk[:, :, k, :] = B[:, :, k, :]
        Y, fin = fwd(X, dt, A, Bk, C, D, G)
        for h in range(H):
            skip = D[h] * X[0, :, h, :]
            if (h * G) // H == k:
                assert np.max(np.abs(Y[0, :, h, :] - skip)) > 1e-6, (k, h)
                assert np.max(np.abs(fin[0, h])) > 1e-6
            else:
                assert np.array_equal(Y[0, :, h, :], skip), (k, h)
                assert not np.any(fin[0, h])


# --- pin 8: causality ---------------------------------------------------------
def check_causality(fwd, seed=6):
    rng = np.random.default_rng(seed)
    Bz, T, H, P, N, G = 1, 30, 2, 3, 4, 1
    X, dt, A, B, C, D = rand_inputs(rng, Bz, T, H, P, N, G)
    Y0, _ = fwd(X, dt, A, B, C, D, G)
    t0 = 17
    X2, B2, C2, dt2 = X.copy(), B.copy(), C.copy(), dt.copy()
    X2[:, t0:] += 1.0
    B2[:, t0:] *= -2.0
    C2[:, t0:] += 0.5
    dt2[:, t0:] *= 3.0
    Y1, _ = fwd(X2, dt2, A, B2, C2, D, G)
    assert np.array_equal(Y0[:, :t0], Y1[:, :t0])
    assert not np.array_equal(Y0[:, t0:], Y1[:, t0:])


# --- pin 9: linearity in X ----------------------------------------------------
def check_linearity(fwd, seed=8, tol=1e-12):
    rng = np.random.default_rng(seed)
    Bz, T, H, P, N, G = 1, 40, 2, 3, 5, 1
    X1, dt, A, B, C, D = rand_inputs(rng, Bz, T, H, P, N, G)
    X2 = rng.standard_normal(X1.shape)
    al, be = 1.7, -0.6
    Y1, F1 = fwd(X1, dt, A, B, C, D, G)
    Y2, F2 = fwd(X2, dt, A, B, C, D, G)
    Y3, F3 = fwd(al * X1 + be * X2, dt, A, B, C, D, G)
    assert rel_err(Y3, al * Y1 + be * Y2) <= tol
    assert rel_err(F3, al * F1 + be * F2) <= tol


# --- pin 10: splitting a sequence and carrying the state ---------------------
def check_split_invariance(fwd, seed=9, tol=1e-12):
    """Running [0, T1) then [T1, T) from the carried state equals one run,
    the block-decomposition fact that chunk-end states are passed on as the
    next chunk's initial state (reading report, section 3.1)."""
    rng = np.random.default_rng(seed)
    Bz, T, H, P, N, G = 2, 50, 2, 3, 4, 1
    X, dt, A, B, C, D = rand_inputs(rng, Bz, T, H, P, N, G)
    h0 = rng.standard_normal((Bz, H, P, N))
    Y, F = fwd(X, dt, A, B, C, D, G, init_state=h0)
    T1 = 23
    Ya, Fa = fwd(X[:, :T1], dt[:, :T1], A, B[:, :T1], C[:, :T1], D, G, init_state=h0)
    Yb, Fb = fwd(X[:, T1:], dt[:, T1:], A, B[:, T1:], C[:, T1:], D, G, init_state=Fa)
    assert rel_err(np.concatenate([Ya, Yb], axis=1), Y) <= tol
    assert rel_err(Fb, F) <= tol


ALL_FWD_PINS = (
    check_golden_hand_example, check_closed_form_constant_decay, check_closed_form_no_decay,
    check_linear_attention, check_memoryless, check_group_mapping, check_causality,
    check_linearity, check_split_invariance,
)
