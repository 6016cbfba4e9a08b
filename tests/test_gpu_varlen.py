"""GPU parity of ssd_chunk_scan_fwd_varlen (packed variable-length batches)
against the oracle run on each sequence alone (through the C ABI).

A packed batch is one token axis holding several sequences end to end; the
state restarts at every sequence start, so each sequence must equal the
oracle on that sequence by itself (with its own initial state, if given).
Tolerances as in test_gpu_fwd: 2e-2 for bf16 storage, 1e-4 for fp32, on Y, on
Y with D = 0, and on the final states.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import oracle
import ssd_inputs as si
from tests.gpu_util import TOL, log, rel, to_dev, to_np

pytestmark = pytest.mark.gpu


def packed_inputs(lengths, dtype, H, P, N, G, seed):
    total = int(sum(lengths))
    base = si.CONFIGS["l1p3b_bf16"] if dtype == "bf16" else si.CONFIGS["tiny_f32"]
    cfg = dataclasses.replace(base, name="varlen", batch=1, seqlen=max(total, 1), nheads=H, headdim=P,
                              dstate=N, ngroups=G, seed=seed)
    inp = si.make_fwd_inputs(cfg)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return cfg, inp, cu, total


def run_varlen(ssd, inp, cu, total, chunk, max_seqlen, init=None, D_zero=False):
    import torch
    X, dt, B, C = (to_dev(inp[k][0, :total]) for k in ("X", "dt", "B", "C"))
    A = to_dev(inp["A"])
    D = torch.zeros_like(A) if D_zero else to_dev(inp["D"])
    cu_d = torch.from_numpy(cu).cuda()
    init_d = None if init is None else torch.from_numpy(np.ascontiguousarray(init, np.float32)).cuda()
    Y, F = ssd.ssd_chunk_scan_fwd_varlen(X, dt, A, B, C, D, chunk, cu_d, max_seqlen, initial_state=init_d)
    torch.cuda.synchronize()
    return to_np(Y), F.cpu().numpy().astype(np.float64)


def oracle_varlen(inp, cu, G, init=None, D_zero=False):
    """Each sequence alone through the pinned oracle."""
    D = np.zeros_like(inp["D"]) if D_zero else inp["D"]
    H, P = inp["X32"].shape[2], inp["X32"].shape[3]
    N = inp["B32"].shape[3]
    nseq = len(cu) - 1
    Y = np.zeros((int(cu[-1]), H, P))
    F = np.zeros((nseq, H, P, N))
    for i in range(nseq):
        s0, s1 = int(cu[i]), int(cu[i + 1])
        st = None if init is None else init[i:i + 1].astype(np.float64)
        if s1 == s0:
            F[i] = 0.0 if init is None else init[i]
            continue
        sl = slice(s0, s1)
        y, f, _ = oracle.fwd(inp["X32"][:, sl], inp["dt32"][:, sl], inp["A"], inp["B32"][:, sl],
                             inp["C32"][:, sl], D, G, init_state=st)
        Y[s0:s1] = y[0]
        F[i] = f[0]
    return Y, F


def check_varlen(ssd, lengths, dtype, chunk, H=4, P=64, N=64, G=2, seed=60, with_init=False):
    cfg, inp, cu, total = packed_inputs(lengths, dtype, H, P, N, G, seed)
    max_len = int(max(lengths)) if lengths else 0
    log(f"[varlen] {dtype} chunk={chunk} lengths={list(lengths)} H{H} P{P} N{N} G{G} init={with_init}")
    init = None
    if with_init:
        init = np.random.default_rng(seed + 7).standard_normal((len(lengths), H, P, N)).astype(np.float32)
    tol = TOL[dtype]
    Yg, Fg = run_varlen(ssd, inp, cu, total, chunk, max_len, init)
    Yr, Fr = oracle_varlen(inp, cu, G, init)
    Yg0, _ = run_varlen(ssd, inp, cu, total, chunk, max_len, init, D_zero=True)
    Yr0, _ = oracle_varlen(inp, cu, G, init, D_zero=True)
    e = (rel(Yg, Yr), rel(Yg0, Yr0), rel(Fg, Fr))
    log(f"    rel err Y={e[0]:.2e} Y(D=0)={e[1]:.2e} final={e[2]:.2e} (tol {tol})")
    assert np.all(np.isfinite(Yg)) and np.all(np.isfinite(Fg))
    assert e[0] <= tol and e[1] <= tol and e[2] <= tol, e


@pytest.mark.parametrize("chunk", [64, 256])
def test_varlen_bf16_mixed_lengths(ssd, chunk):
    # empty, one token, chunk and tile boundaries, long
    check_varlen(ssd, [0, 1, 63, 64, 65, 300, 1000, 257], "bf16", chunk)


def test_varlen_f32_with_initial_states(ssd):
    check_varlen(ssd, [5, 200, 0, 129, 64], "f32", 64, H=2, P=16, N=16, G=1, seed=61, with_init=True)


def test_varlen_many_short_sequences(ssd):
    lengths = list(np.random.default_rng(62).integers(0, 40, size=37))
    check_varlen(ssd, lengths, "bf16", 128, H=8, P=32, N=128, G=1, seed=63)


def test_varlen_equal_lengths_match_the_batched_forward(ssd):
    """Equal lengths: the packed call computes what the batched call does, bit for bit."""
    import torch
    lengths = [300] * 4
    cfg, inp, cu, total = packed_inputs(lengths, "bf16", 32, 64, 128, 1, 64)
    log("[varlen] equal lengths vs batched forward")
    Yv, Fv = run_varlen(ssd, inp, cu, total, 128, 300)
    X, dt, B, C = (to_dev(inp[k][0].reshape((4, 300) + inp[k].shape[2:])) for k in ("X", "dt", "B", "C"))
    A, D = to_dev(inp["A"]), to_dev(inp["D"])
    Yb, Fb = ssd.ssd_chunk_scan_fwd(X, dt, A, B, C, D, 128)
    torch.cuda.synchronize()
    assert np.array_equal(Yv.reshape(4, 300, 32, 64), to_np(Yb))
    assert np.array_equal(Fv, Fb.cpu().numpy().astype(np.float64))


def test_varlen_malformed_table_is_clamped(ssd):
    """Entries past the end or going backwards are clamped on the device: with
    total = 400, [0, 200, 500, 300] reads as [0, 200), [200, 400), [400, 400);
    a table ending early leaves the tokens after it unwritten."""
    import torch
    lengths = [200, 200]
    cfg, inp, cu, total = packed_inputs(lengths, "bf16", 4, 64, 64, 1, 65)
    X, dt, B, C = (to_dev(inp[k][0, :total]) for k in ("X", "dt", "B", "C"))
    A, D = to_dev(inp["A"]), to_dev(inp["D"])
    log("[varlen] malformed table")
    bad = torch.tensor([0, 200, 500, 300], dtype=torch.int32, device="cuda")
    Yg, Fg = ssd.ssd_chunk_scan_fwd_varlen(X, dt, A, B, C, D, 64, bad, 256)
    torch.cuda.synchronize()
    Yr, Fr = oracle_varlen(inp, np.array([0, 200, 400], np.int32), 1)
    assert rel(to_np(Yg), Yr) <= TOL["bf16"]
    assert rel(Fg[:2].cpu().numpy(), Fr) <= TOL["bf16"]
    assert not torch.any(Fg[2])
    short = torch.tensor([0, 100], dtype=torch.int32, device="cuda")
    Y = torch.full_like(X, 7.0)
    ssd.ssd_chunk_scan_fwd_varlen(X, dt, A, B, C, D, 64, short, 256, Y=Y)
    torch.cuda.synchronize()
    assert torch.all(Y[100:] == 7.0)
    Yr, _ = oracle_varlen(inp, np.array([0, 100], np.int32), 1)
    assert rel(to_np(Y[:100]), Yr) <= TOL["bf16"]


def test_varlen_no_sequences_and_all_empty(ssd):
    import torch
    X = torch.empty((0, 2, 16), dtype=torch.float32, device="cuda")
    dt = torch.empty((0, 2), dtype=torch.float32, device="cuda")
    B = torch.empty((0, 1, 16), dtype=torch.float32, device="cuda")
    A = torch.full((2,), -1.0, device="cuda")
    D = torch.ones(2, device="cuda")
    cu = torch.zeros(4, dtype=torch.int32, device="cuda")
    init = torch.randn((3, 2, 16, 16), device="cuda")
    Y, F = ssd.ssd_chunk_scan_fwd_varlen(X, dt, A, B, B, D, 64, cu, 0, initial_state=init)
    torch.cuda.synchronize()
    assert torch.equal(F, init)
    Y, F = ssd.ssd_chunk_scan_fwd_varlen(X, dt, A, B, B, D, 64, cu[:1], 0)
    assert F.shape == (0, 2, 16, 16)
