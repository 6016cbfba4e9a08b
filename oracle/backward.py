"""Oracle for the backward pass of the SSD core (fp64, TEST INFRASTRUCTURE).

The pages' speed claims are about training (the reading report's summary;
the SSD theory page, section 6.1, compares training throughput), which needs
the gradients of the forward. Nothing on the pages spells the backward out,
so the oracle is the plain definition: the chain rule applied to the
recurrence (back-propagation through the time steps), for the loss

    L = <dY, Y> + <dF, final_state>

so that the returned arrays are dL/d(input) for every input. With

    a_t = exp(dt_t A_h),  s_t = a_t s_{t-1} + dt_t x_t B_t^T,  y_t = s_t C_t + D_h x_t

the adjoint of s_t is ds_t = dy_t C_t^T + a_{t+1} ds_{t+1} (ds_{T-1} also gets
dF), and

    dx_t  = dt_t ds_t B_t + D_h dy_t
    dB_t += dt_t ds_t^T x_t            (summed over the heads of B's group)
    dC_t += s_t^T dy_t                 (likewise)
    ddt_t = x_t^T ds_t B_t + A_h a_t <ds_t, s_{t-1}>
    dA_h  = sum_t dt_t a_t <ds_t, s_{t-1}>
    dD_h  = sum_t <dy_t, x_t>
    d s_{-1} = a_0 ds_0                (the initial state's gradient)

The states s_t are kept for the whole sequence, so this is for test sizes.
Pins (tests/test_oracle_bwd.py): central finite differences of the forward
oracle, homogeneity identities, the A = 0 dense closed form and the
one-token closed form.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def bwd(X, dt, A, B, C, D, ngroups: int, dY, init_state=None, d_final=None):
    """Gradients of <dY, Y> + <dF, final> for one forward over whole sequences.

    Shapes as the forward oracle: X, dY (Bz,T,H,P); dt (Bz,T,H); A, D (H,);
    B, C (Bz,T,G,N); init_state, d_final (Bz,H,P,N) or None (zero).
    Returns a dict with dX, ddt, dA, dB, dC, dD, dinit (all fp64), and lam
    (Bz,T,H): Lambda_t = a_t <ds_t, s_{t-1}>, whose dt-weighted sum is dA.
    """
    X, dt, A, B, C, D, dY = map(_f64, (X, dt, A, B, C, D, dY))
    Bz, T, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    assert G == ngroups and H % G == 0
    assert dt.shape == (Bz, T, H) and B.shape == (Bz, T, G, N) and C.shape == B.shape
    assert dY.shape == X.shape and A.shape == (H,) and D.shape == (H,)
    grp = (np.arange(H) * G) // H               # contiguous head -> group map
    Bh, Ch = B[:, :, grp, :], C[:, :, grp, :]   # (Bz,T,H,N)
    a = np.exp(dt * A[None, None, :])           # (Bz,T,H)

    # forward, keeping every state: S[t + 1] is s_t, S[0] the initial state
    S = np.empty((T + 1, Bz, H, P, N))
    S[0] = 0.0 if init_state is None else _f64(init_state)
    for t in range(T):
        S[t + 1] = (a[:, t, :, None, None] * S[t]
                    + (dt[:, t, :, None, None] * X[:, t, :, :, None]) * Bh[:, t, :, None, :])

    dX = np.empty_like(X)
    ddt = np.empty_like(dt)
    dBh = np.empty((Bz, T, H, N))
    dCh = np.empty((Bz, T, H, N))
    dA = np.zeros(H)
    lams = np.empty((Bz, T, H))
    ds = np.zeros((Bz, H, P, N)) if d_final is None else _f64(d_final).copy()
    for t in range(T - 1, -1, -1):
        ds += dY[:, t, :, :, None] * Ch[:, t, :, None, :]           # ds_t
        dCh[:, t] = np.einsum('bhpn,bhp->bhn', S[t + 1], dY[:, t])
        v = np.einsum('bhpn,bhn->bhp', ds, Bh[:, t])                # ds_t B_t
        dX[:, t] = dt[:, t, :, None] * v + D[None, :, None] * dY[:, t]
        dBh[:, t] = dt[:, t, :, None] * np.einsum('bhpn,bhp->bhn', ds, X[:, t])
        lam = np.einsum('bhpn,bhpn->bh', ds, a[:, t, :, None, None] * S[t])
        lams[:, t] = lam
        ddt[:, t] = np.einsum('bhp,bhp->bh', X[:, t], v) + A[None, :] * lam
        dA += (dt[:, t] * lam).sum(axis=0)
        ds = a[:, t, :, None, None] * ds                            # adjoint entering s_{t-1}
    dB = np.zeros((Bz, T, G, N))
    dC = np.zeros((Bz, T, G, N))
    for h in range(H):
        dB[:, :, grp[h]] += dBh[:, :, h]
        dC[:, :, grp[h]] += dCh[:, :, h]
    dD = np.einsum('bthp,bthp->h', dY, X)
    return {"dX": dX, "ddt": ddt, "dA": dA, "dB": dB, "dC": dC, "dD": dD, "dinit": ds, "lam": lams}
