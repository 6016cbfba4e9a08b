"""GPU parity of the fused prologue/epilogue entry points (ssd_chunk_scan_fwd_gated,
ssd_step_gated) against the oracle: oracle.dt_prologue on the stored dt bits,
the pinned fp64 recurrence, then oracle.gate with the stored z bits.

Tolerances as in test_gpu_fwd (2e-2 bf16 storage, 1e-4 fp32) on Y, on the
final state, and on Y with D = 0 and no gate (the SSM part alone).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import oracle
import ssd_inputs as si
from tests.gpu_util import TOL, log, rel, to_dev, to_np

pytestmark = pytest.mark.gpu


def raw_inputs(cfg, seed):
    """The workload's inputs, with dt replaced by a raw pre-activation ~ N(-3, 1)
    (so that softplus gives the workload's step-size range), a per-head bias
    and a gate z ~ N(0, 1), all rounded to the storage type like the rest."""
    inp = si.make_fwd_inputs(cfg)
    rng = np.random.default_rng(seed)
    raw = (rng.standard_normal(inp["dt32"].shape) - 3.0).astype(np.float32)
    z = rng.standard_normal(inp["X32"].shape).astype(np.float32)
    bias = (0.5 * rng.standard_normal(cfg.nheads)).astype(np.float32)
    if cfg.dtype == "bf16":
        rb, zb = si.bf16_round_bits(raw), si.bf16_round_bits(z)
        inp["dtraw"], inp["dtraw32"] = rb, si.bf16_bits_to_f32(rb)
        inp["z"], inp["z32"] = zb, si.bf16_bits_to_f32(zb)
    else:
        inp["dtraw"] = inp["dtraw32"] = raw
        inp["z"] = inp["z32"] = z
    inp["bias"] = bias
    return inp


def oracle_gated(inp, G, mode, use_bias, use_gate, D_zero=False):
    dt = oracle.dt_prologue(inp["dtraw32"], inp["bias"] if use_bias else None, mode)
    D = np.zeros_like(inp["D"]) if D_zero else inp["D"]
    Y, F, _ = oracle.fwd(inp["X32"], dt, inp["A"], inp["B32"], inp["C32"], D, G)
    if use_gate:
        Y = oracle.gate(Y, inp["z32"])
    return Y, F


def gpu_gated(ssd, inp, chunk, mode, use_bias, use_gate, D_zero=False):
    import torch
    X, dt, B, C = (to_dev(inp[k]) for k in ("X", "dtraw", "B", "C"))
    A = to_dev(inp["A"])
    D = torch.zeros_like(A) if D_zero else to_dev(inp["D"])
    bias = to_dev(inp["bias"]) if use_bias else None
    z = to_dev(inp["z"]) if use_gate else None
    Y, F = ssd.ssd_chunk_scan_fwd_gated(X, dt, A, B, C, D, chunk, dt_bias=bias, dt_softplus=mode, z=z)
    torch.cuda.synchronize()
    return to_np(Y), F.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype,mode,use_bias,use_gate", [
    ("bf16", 1, True, True), ("bf16", 2, True, True), ("bf16", 1, False, False),
    ("f32", 1, True, True), ("f32", 2, True, False), ("f32", 0, True, True),
])
def test_gated_forward(ssd, dtype, mode, use_bias, use_gate):
    base = si.CONFIGS["l1p3b_bf16"] if dtype == "bf16" else si.CONFIGS["tiny_f32"]
    cfg = dataclasses.replace(base, name="gated", batch=2, seqlen=333, nheads=4, headdim=32, dstate=64,
                              ngroups=2, seed=70)
    inp = raw_inputs(cfg, 71)
    if mode == 0:  # no softplus: keep dt positive
        inp["dtraw32"] = np.abs(inp["dtraw32"]) * 0.05
        inp["dtraw"] = si.bf16_round_bits(inp["dtraw32"]) if dtype == "bf16" else inp["dtraw32"]
        if dtype == "bf16":
            inp["dtraw32"] = si.bf16_bits_to_f32(inp["dtraw"])
        inp["bias"] = np.abs(inp["bias"]) * 0.01
    if mode == 2:  # bias added after softplus: keep the step sizes positive
        inp["bias"] = np.abs(inp["bias"])
    chunk = 128
    log(f"[gated] {dtype} mode={mode} bias={use_bias} gate={use_gate}")
    tol = TOL[dtype]
    Yg, Fg = gpu_gated(ssd, inp, chunk, mode, use_bias, use_gate)
    Yr, Fr = oracle_gated(inp, cfg.ngroups, mode, use_bias, use_gate)
    Yg0, _ = gpu_gated(ssd, inp, chunk, mode, use_bias, False, D_zero=True)
    Yr0, _ = oracle_gated(inp, cfg.ngroups, mode, use_bias, False, D_zero=True)
    e = (rel(Yg, Yr), rel(Yg0, Yr0), rel(Fg, Fr))
    log(f"    rel err Y={e[0]:.2e} Y(D=0, no gate)={e[1]:.2e} final={e[2]:.2e} (tol {tol})")
    assert np.all(np.isfinite(Yg))
    assert e[0] <= tol and e[1] <= tol and e[2] <= tol, e


def test_gated_without_options_is_the_plain_forward(ssd):
    import torch
    cfg = dataclasses.replace(si.CONFIGS["l1p3b_bf16"], name="gated_id", batch=2, seqlen=300, nheads=8, seed=72)
    inp = si.make_fwd_inputs(cfg)
    X, dt, B, C = (to_dev(inp[k]) for k in ("X", "dt", "B", "C"))
    A, D = to_dev(inp["A"]), to_dev(inp["D"])
    Y1, F1 = ssd.ssd_chunk_scan_fwd(X, dt, A, B, C, D, 256)
    Y2, F2 = ssd.ssd_chunk_scan_fwd_gated(X, dt, A, B, C, D, 256)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2) and torch.equal(F1, F2)


def test_gated_padding_keeps_zero_steps(ssd):
    """softplus(0 + bias) > 0, but tokens past seqlen must still add nothing:
    the final state of a ragged sequence matches the oracle's."""
    cfg = dataclasses.replace(si.CONFIGS["l1p3b_bf16"], name="gated_pad", batch=1, seqlen=70, nheads=2,
                              headdim=16, dstate=16, ngroups=1, seed=73)
    inp = raw_inputs(cfg, 74)
    Yg, Fg = gpu_gated(ssd, inp, 64, 1, True, True)
    Yr, Fr = oracle_gated(inp, 1, 1, True, True)
    assert rel(Fg, Fr) <= TOL["bf16"] and rel(Yg, Yr) <= TOL["bf16"]


@pytest.mark.parametrize("dtype,mode", [("bf16", 1), ("bf16", 2), ("f32", 1)])
def test_gated_step(ssd, dtype, mode):
    import torch
    rng = np.random.default_rng(75)
    Bz, H, P, N, G = 3, 4, 16, 32, 2
    state0 = rng.standard_normal((Bz, H, P, N)).astype(np.float32)
    x = rng.standard_normal((Bz, H, P)).astype(np.float32)
    raw = (rng.standard_normal((Bz, H)) - 2.0).astype(np.float32)
    Bm = (rng.standard_normal((Bz, G, N)) / np.sqrt(N)).astype(np.float32)
    Cm = (rng.standard_normal((Bz, G, N)) / np.sqrt(N)).astype(np.float32)
    z = rng.standard_normal((Bz, H, P)).astype(np.float32)
    A = -np.exp(rng.uniform(0, np.log(16), H)).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    bias = (0.5 * rng.standard_normal(H)).astype(np.float32)
    if dtype == "bf16":
        q = lambda a: si.bf16_round_bits(a)  # noqa: E731
        x, raw, Bm, Cm, z = (q(v) for v in (x, raw, Bm, Cm, z))
        f = si.bf16_bits_to_f32
    else:
        f = lambda a: a  # noqa: E731
    dt = oracle.dt_prologue(f(raw), bias, mode)
    s_ref = state0.astype(np.float64)
    y_ref = oracle.step(s_ref, f(x), dt, A, f(Bm), f(Cm), D, G)
    y_ref = oracle.gate(y_ref, f(z))
    st = torch.from_numpy(state0).cuda()
    y = ssd.ssd_step_gated(st, to_dev(x), to_dev(raw), to_dev(A), to_dev(Bm), to_dev(Cm), to_dev(D),
                           dt_bias=to_dev(bias), dt_softplus=mode, z=to_dev(z))
    torch.cuda.synchronize()
    tol = TOL[dtype]
    log(f"[gated step] {dtype} mode={mode}: y {rel(to_np(y), y_ref):.2e} state "
        f"{rel(st.cpu().numpy(), s_ref):.2e}")
    assert rel(to_np(y), y_ref) <= tol and rel(st.cpu().numpy(), s_ref) <= tol
