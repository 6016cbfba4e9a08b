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


def conv_inputs(cfg, seed):
    """Taps ~ N(0, 0.5^2) per channel and bias ~ N(0, 0.1^2): the conv keeps the
    workload's input scale."""
    rng = np.random.default_rng(seed)
    C = cfg.nheads * cfg.headdim
    w = (0.5 * rng.standard_normal((C, 4))).astype(np.float32)
    b = (0.1 * rng.standard_normal(C)).astype(np.float32)
    return w, b


def oracle_conv_x(X32, w, b):
    """oracle.conv_silu over the channels c = h * P + p."""
    Bz, T, H, P = X32.shape
    return oracle.conv_silu(X32.reshape(Bz, T, H * P), w, b).reshape(Bz, T, H, P)


@pytest.mark.parametrize("dtype,chunk,with_bias,gated", [
    ("bf16", 128, True, True), ("bf16", 64, False, False), ("f32", 64, True, False),
])
def test_fused_conv_forward(ssd, dtype, chunk, with_bias, gated):
    import torch
    base = si.CONFIGS["l1p3b_bf16"] if dtype == "bf16" else si.CONFIGS["tiny_f32"]
    cfg = dataclasses.replace(base, name="conv", batch=2, seqlen=333, nheads=4,
                              headdim=64 if dtype == "bf16" else 32, dstate=128 if dtype == "bf16" else 32,
                              ngroups=2, seed=76)
    inp = raw_inputs(cfg, 77)
    w, b = conv_inputs(cfg, 78)
    mode = 1 if gated else 0
    if not gated:
        inp["dtraw"], inp["dtraw32"] = inp["dt"], inp["dt32"]
    log(f"[conv] {dtype} chunk={chunk} bias={with_bias} gated={gated}")
    Xc = oracle_conv_x(inp["X32"], w, b if with_bias else np.zeros_like(b))
    tol = TOL[dtype]
    errs = []
    for D_zero in (False, True):
        Dv = np.zeros_like(inp["D"]) if D_zero else inp["D"]
        dt = oracle.dt_prologue(inp["dtraw32"], inp["bias"] if gated else None, mode)
        Yr, Fr, _ = oracle.fwd(Xc, dt, inp["A"], inp["B32"], inp["C32"], Dv, cfg.ngroups)
        if gated and not D_zero:
            Yr = oracle.gate(Yr, inp["z32"])
        Y, F = ssd.ssd_chunk_scan_fwd_fused(
            to_dev(inp["X"]), to_dev(inp["dtraw"]), to_dev(inp["A"]), to_dev(inp["B"]), to_dev(inp["C"]),
            to_dev(Dv), chunk, conv_w=to_dev(w), conv_b=to_dev(b) if with_bias else None,
            dt_bias=to_dev(inp["bias"]) if gated else None, dt_softplus=mode,
            z=to_dev(inp["z"]) if (gated and not D_zero) else None)
        torch.cuda.synchronize()
        errs += [rel(to_np(Y), Yr), rel(F.cpu().numpy(), Fr)]
    log(f"    rel err Y={errs[0]:.2e} final={errs[1]:.2e} Y(D=0, no gate)={errs[2]:.2e}")
    assert all(np.isfinite(e) and e <= tol for e in errs), errs


def test_fused_conv_full_width_walks(ssd):
    """Batch 4 x 64 heads, P 64, N 128, chunk 256, gated, with bias: one
    work-group per (batch, head) over all 64 columns, the variant timed on the
    1.3B-layer shape (its state waves stage the convolved X)."""
    import torch
    cfg = dataclasses.replace(si.CONFIGS["l1p3b_bf16"], name="conv_full", batch=4, seqlen=200, nheads=64,
                              seed=97)
    inp = raw_inputs(cfg, 98)
    w, b = conv_inputs(cfg, 99)
    Xc = oracle_conv_x(inp["X32"], w, b)
    dt = oracle.dt_prologue(inp["dtraw32"], inp["bias"], 1)
    Yr, Fr, _ = oracle.fwd(Xc, dt, inp["A"], inp["B32"], inp["C32"], inp["D"], cfg.ngroups)
    Yr = oracle.gate(Yr, inp["z32"])
    log("[conv] full-width walks")
    Y, F = ssd.ssd_chunk_scan_fwd_fused(
        to_dev(inp["X"]), to_dev(inp["dtraw"]), to_dev(inp["A"]), to_dev(inp["B"]), to_dev(inp["C"]),
        to_dev(inp["D"]), 256, conv_w=to_dev(w), conv_b=to_dev(b), dt_bias=to_dev(inp["bias"]), dt_softplus=1,
        z=to_dev(inp["z"]))
    torch.cuda.synchronize()
    e = (rel(to_np(Y), Yr), rel(F.cpu().numpy(), Fr))
    log(f"    rel err Y={e[0]:.2e} final={e[1]:.2e}")
    assert e[0] <= TOL["bf16"] and e[1] <= TOL["bf16"], e


def test_fused_conv_split_sequence(ssd):
    """Few heads and a long sequence: the walk splits it into segments, whose
    state-only pass applies the convolution too (tokens before each segment
    come from the previous one)."""
    import torch
    cfg = dataclasses.replace(si.CONFIGS["l1p3b_bf16"], name="conv_seg", batch=1, seqlen=2048, nheads=2,
                              headdim=32, dstate=64, ngroups=1, seed=79)
    inp = si.make_fwd_inputs(cfg)
    w, b = conv_inputs(cfg, 80)
    Xc = oracle_conv_x(inp["X32"], w, b)
    Yr, Fr, _ = oracle.fwd(Xc, inp["dt32"], inp["A"], inp["B32"], inp["C32"], inp["D"], 1)
    log("[conv] split sequence")
    Y, F = ssd.ssd_chunk_scan_fwd_fused(to_dev(inp["X"]), to_dev(inp["dt"]), to_dev(inp["A"]), to_dev(inp["B"]),
                                        to_dev(inp["C"]), to_dev(inp["D"]), 64, conv_w=to_dev(w), conv_b=to_dev(b))
    torch.cuda.synchronize()
    e = (rel(to_np(Y), Yr), rel(F.cpu().numpy(), Fr))
    log(f"    rel err Y={e[0]:.2e} final={e[1]:.2e}")
    assert e[0] <= TOL["bf16"] and e[1] <= TOL["bf16"], e


def test_fused_without_conv_is_the_gated_forward(ssd):
    import torch
    cfg = dataclasses.replace(si.CONFIGS["l1p3b_bf16"], name="fused_id", batch=1, seqlen=200, nheads=4, seed=81)
    inp = raw_inputs(cfg, 82)
    args = [to_dev(inp[k]) for k in ("X", "dtraw", "A", "B", "C", "D")]
    kw = dict(dt_bias=to_dev(inp["bias"]), dt_softplus=1, z=to_dev(inp["z"]))
    Y1, F1 = ssd.ssd_chunk_scan_fwd_gated(*args, 256, **kw)
    Y2, F2 = ssd.ssd_chunk_scan_fwd_fused(*args, 256, **kw)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2) and torch.equal(F1, F2)


def _step_seq_inputs(rng, Bz, T, H, P, N, G, dtype):
    X = rng.standard_normal((Bz, T, H, P)).astype(np.float32)
    raw = rng.standard_normal((Bz, T, H)).astype(np.float32)
    Bm = (rng.standard_normal((Bz, T, G, N)) / np.sqrt(N)).astype(np.float32)
    Cm = (rng.standard_normal((Bz, T, G, N)) / np.sqrt(N)).astype(np.float32)
    z = rng.standard_normal((Bz, T, H, P)).astype(np.float32)
    if dtype == "bf16":
        X, raw, Bm, Cm, z = (si.bf16_round_bits(v) for v in (X, raw, Bm, Cm, z))
    return X, raw, Bm, Cm, z


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fused_step_sequence(ssd, dtype):
    """T fused decode steps from a given SSM state and conv state against the
    oracle: the convolution over (conv state, then the step inputs), SiLU, the
    step prologue, the recurrence and the gate. The conv state must end holding
    the last 3 raw inputs exactly."""
    import torch
    rng = np.random.default_rng(91)
    Bz, T, H, P, N, G = 2, 12, 4, 16, 32, 2
    X, raw, Bm, Cm, z = _step_seq_inputs(rng, Bz, T, H, P, N, G, dtype)
    f = si.bf16_bits_to_f32 if dtype == "bf16" else (lambda a: a)
    A = -np.exp(rng.uniform(0, np.log(16), H)).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    bias = np.full(H, -2.0, dtype=np.float32)
    cfg = dataclasses.replace(si.CONFIGS["tiny_f32"], nheads=H, headdim=P)
    w, b = conv_inputs(cfg, 92)
    state0 = rng.standard_normal((Bz, H, P, N)).astype(np.float32)
    cs0 = rng.standard_normal((Bz, H * P, 3)).astype(np.float32)
    if dtype == "bf16":
        cs0 = si.bf16_round_bits(cs0)
    # oracle: the window runs over the conv state's 3 inputs, then the steps'
    ext = np.concatenate([f(cs0).transpose(0, 2, 1).reshape(Bz, 3, H, P), f(X)], axis=1)
    xa = oracle_conv_x(ext, w, b)[:, 3:]
    dt = oracle.dt_prologue(f(raw), bias, 1)
    s_ref = state0.astype(np.float64)
    y_ref = np.stack([oracle.gate(oracle.step(s_ref, xa[:, t], dt[:, t], A, f(Bm[:, t]), f(Cm[:, t]), D, G),
                                  f(z[:, t])) for t in range(T)], axis=1)
    st = torch.from_numpy(state0).cuda()
    cst = to_dev(cs0)
    ys = []
    for t in range(T):
        ys.append(to_np(ssd.ssd_step_fused(st, cst, to_dev(X[:, t]), to_dev(raw[:, t]), to_dev(A), to_dev(Bm[:, t]),
                                           to_dev(Cm[:, t]), to_dev(D), conv_w=to_dev(w), conv_b=to_dev(b),
                                           dt_bias=to_dev(bias), dt_softplus=1, z=to_dev(z[:, t]))))
    torch.cuda.synchronize()
    y = np.stack(ys, axis=1)
    tol = TOL[dtype]
    log(f"[fused step] {dtype}: y {rel(y, y_ref):.2e} state {rel(st.cpu().numpy(), s_ref):.2e}")
    assert rel(y, y_ref) <= tol and rel(st.cpu().numpy(), s_ref) <= tol
    last3 = X[:, T - 3:].reshape(Bz, 3, H * P).transpose(0, 2, 1)
    got = cst.view(torch.int16).cpu().numpy().view(np.uint16) if dtype == "bf16" else cst.cpu().numpy()
    assert np.array_equal(got, last3)


def test_fused_steps_equal_the_fused_forward(ssd):
    """From zero states, T fused decode steps give what ssd_chunk_scan_fwd_fused
    gives over the same T tokens (both on the GPU, bf16 storage)."""
    import torch
    rng = np.random.default_rng(93)
    Bz, T, H, P, N, G = 2, 40, 4, 32, 64, 2
    X, raw, Bm, Cm, z = _step_seq_inputs(rng, Bz, T, H, P, N, G, "bf16")
    A = to_dev(-np.exp(rng.uniform(0, np.log(16), H)).astype(np.float32))
    D = to_dev(rng.standard_normal(H).astype(np.float32))
    bias = to_dev(np.full(H, -2.0, dtype=np.float32))
    cfg = dataclasses.replace(si.CONFIGS["tiny_f32"], nheads=H, headdim=P)
    w, b = (to_dev(v) for v in conv_inputs(cfg, 94))
    Yf, Ff = ssd.ssd_chunk_scan_fwd_fused(to_dev(X), to_dev(raw), A, to_dev(Bm), to_dev(Cm), D, 64, conv_w=w,
                                          conv_b=b, dt_bias=bias, dt_softplus=1, z=to_dev(z))
    st = torch.zeros((Bz, H, P, N), device="cuda")
    cst = torch.zeros((Bz, H * P, 3), dtype=torch.bfloat16, device="cuda")
    ys = [ssd.ssd_step_fused(st, cst, to_dev(X[:, t]), to_dev(raw[:, t]), A, to_dev(Bm[:, t]), to_dev(Cm[:, t]), D,
                             conv_w=w, conv_b=b, dt_bias=bias, dt_softplus=1, z=to_dev(z[:, t]))
          for t in range(T)]
    torch.cuda.synchronize()
    y = np.stack([to_np(v) for v in ys], axis=1)
    e_y, e_f = rel(y, to_np(Yf)), rel(st.cpu().numpy(), Ff.cpu().numpy())
    log(f"[fused steps vs fused forward] y {e_y:.2e} final state {e_f:.2e}")
    assert e_y <= TOL["bf16"] and e_f <= TOL["bf16"]
