"""GPU parity of ssd_step (the recurrent decode step) against the oracle, and
consistency of the decode step with the chunked forward, through the C ABI."""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import oracle
import ssd_inputs as si
from tests.gpu_util import TOL, log, rel, to_dev, to_np

pytestmark = pytest.mark.gpu


def _sliced_oracle_steps(d, cfg, samples, steps_to_check, nsteps):
    """Runs the oracle for selected (b, h) slices over nsteps steps; returns
    {(b, h): ({step: y}, final_state)} with step numbering from 1."""
    H, G = cfg.nheads, cfg.ngroups
    out = {}
    for (b, h) in samples:
        g = (h * G) // H
        s = d["state0"][b:b + 1, h:h + 1].astype(np.float64).copy()
        ys = {}
        for k in range(nsteps):
            st = d["sets"][k % cfg.nsets]
            y = oracle.step(s, st["x32"][b:b + 1, h:h + 1], st["dt32"][b:b + 1, h:h + 1],
                            d["A"][h:h + 1], st["B32"][b:b + 1, g:g + 1], st["C32"][b:b + 1, g:g + 1],
                            d["D"][h:h + 1], 1)
            if k + 1 in steps_to_check:
                ys[k + 1] = y[0, 0].copy()
        out[(b, h)] = (ys, s[0, 0])
    return out


def run_decode(ssd, cfg, samples, nsteps, check_steps):
    import torch
    log(f"[step] {cfg.name} b{cfg.batch} H{cfg.nheads} P{cfg.headdim} N{cfg.dstate} G{cfg.ngroups}, "
        f"{nsteps} steps, samples {samples}")
    d = si.make_decode_inputs(cfg)
    state = to_dev(d["state0"])
    A, D = to_dev(d["A"]), to_dev(d["D"])
    sets = [{k: to_dev(v) for k, v in st.items() if not k.endswith("32")} for st in d["sets"]]
    y = torch.empty_like(sets[0]["x"])
    got = {}
    for k in range(nsteps):
        st = sets[k % cfg.nsets]
        ssd.ssd_step(state, st["x"], st["dt"], A, st["B"], st["C"], D, y)
        if k + 1 in check_steps:
            got[k + 1] = to_np(y)
    torch.cuda.synchronize()
    fin = state.cpu().numpy().astype(np.float64)
    ref = _sliced_oracle_steps(d, cfg, samples, check_steps, nsteps)
    tol = TOL["bf16"]
    worst_y, worst_s = 0.0, 0.0
    for (b, h), (ys, sref) in ref.items():
        for k, yr in ys.items():
            e = rel(got[k][b, h], yr)
            worst_y = max(worst_y, e)
            assert e <= tol, ((b, h), k, e)
        e = rel(fin[b, h], sref)
        worst_s = max(worst_s, e)
        assert e <= tol, ((b, h), "state", e)
    log(f"    worst rel err y={worst_y:.2e} state={worst_s:.2e} (tol {tol})")
    return worst_y, worst_s


def test_decode_small_many_steps(ssd):
    cfg = si.DecodeConfig("decode_small", 3, 4, 64, 128, 2, 50, 8, 51)
    samples = [(b, h) for b in range(3) for h in range(4)]
    run_decode(ssd, cfg, samples, 50, {1, 2, 10, 50})


@pytest.mark.parametrize("N", [4, 8, 16, 32, 64, 256])
def test_decode_state_sizes(ssd, N):
    cfg = si.DecodeConfig(f"decode_N{N}", 2, 4, 16, N, 1, 5, 3, 52)
    run_decode(ssd, cfg, [(b, h) for b in range(2) for h in range(4)], 5, {1, 5})


def test_decode_full_size_whole_state(ssd):
    """Batch 256: the whole y and the whole state after steps 1 and 10 against
    the oracle run on the whole state."""
    import torch
    cfg = si.DECODE
    log(f"[step] {cfg.name} whole-tensor check at steps 1 and 10")
    d = si.make_decode_inputs(cfg)
    state = to_dev(d["state0"])
    A, D = to_dev(d["A"]), to_dev(d["D"])
    sets = [{k: to_dev(v) for k, v in st.items() if not k.endswith("32")} for st in d["sets"]]
    s_ref = d["state0"].astype(np.float64)
    tol = TOL["bf16"]
    for k in range(10):
        st, hs = sets[k % cfg.nsets], d["sets"][k % cfg.nsets]
        y = ssd.ssd_step(state, st["x"], st["dt"], A, st["B"], st["C"], D)
        y_ref = oracle.step(s_ref, hs["x32"], hs["dt32"], d["A"], hs["B32"], hs["C32"], d["D"], cfg.ngroups)
        if k + 1 in (1, 10):
            torch.cuda.synchronize()
            e = (rel(to_np(y), y_ref), rel(state.cpu().numpy(), s_ref))
            log(f"    step {k + 1}: rel err y={e[0]:.2e} state={e[1]:.2e} (tol {tol})")
            assert e[0] <= tol and e[1] <= tol, (k + 1, e)


def test_decode_full_size_1000_steps(ssd):
    cfg = si.DECODE
    samples = [(0, 0), (17, 33), (128, 63), (255, 5)]
    run_decode(ssd, cfg, samples, cfg.nsteps, {1, 10, 100, 1000})


def test_decode_f32_storage(ssd):
    import torch
    rng = np.random.default_rng(5)
    Bz, H, P, N, G = 2, 4, 16, 32, 2
    s0 = rng.standard_normal((Bz, H, P, N)).astype(np.float32)
    x = rng.standard_normal((Bz, H, P)).astype(np.float32)
    dt = np.log1p(np.exp(rng.standard_normal((Bz, H)) - 1)).astype(np.float32)
    A = -np.exp(rng.uniform(0, np.log(16), H)).astype(np.float32)
    Bm = (rng.standard_normal((Bz, G, N)) / np.sqrt(N)).astype(np.float32)
    Cm = (rng.standard_normal((Bz, G, N)) / np.sqrt(N)).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    st = to_dev(s0)
    y = ssd.ssd_step(st, *(to_dev(v) for v in (x, dt, A, Bm, Cm, D)))
    torch.cuda.synchronize()
    sr = s0.astype(np.float64)
    yr = oracle.step(sr, x, dt, A, Bm, Cm, D, G)
    assert rel(to_np(y), yr) <= TOL["f32"]
    assert rel(st.cpu().numpy(), sr) <= TOL["f32"]


def test_step_sequence_equals_forward(ssd):
    """T decode steps from a zero state reproduce the chunked forward (the SSM's
    recurrent and chunked forms compute the same map)."""
    import torch
    cfg = dataclasses.replace(si.CONFIGS["l1p3b_bf16"], name="fwd_vs_step", batch=2, seqlen=300,
                              nheads=4, ngroups=2, seed=60)
    inp = si.make_fwd_inputs(cfg)
    X, dt, B, C = (to_dev(inp[k]) for k in ("X", "dt", "B", "C"))
    A, D = to_dev(inp["A"]), to_dev(inp["D"])
    Yf, Ff = ssd.ssd_chunk_scan_fwd(X, dt, A, B, C, D, 128)
    state = torch.zeros_like(Ff)
    ys = []
    for t in range(cfg.seqlen):
        ys.append(ssd.ssd_step(state, X[:, t].contiguous(), dt[:, t].contiguous(), A,
                               B[:, t].contiguous(), C[:, t].contiguous(), D))
    torch.cuda.synchronize()
    Ys = torch.stack(ys, 1)
    e_y, e_s = rel(to_np(Ys), to_np(Yf)), rel(to_np(state), to_np(Ff))
    log(f"[step vs fwd] rel y={e_y:.2e} state={e_s:.2e}")
    assert e_y <= TOL["bf16"] and e_s <= TOL["bf16"]
