"""GPU parity of ssd_chunk_scan_bwd against the backward oracle (through the C ABI).

Each gradient is compared with the oracle's on the same stored input bits, as
max|g - g_ref| / max|g_ref| per tensor. The GPU keeps the states it hands
between its passes in the storage type and rounds its outputs to it, so the
bound for bf16 storage is the forward's 2e-2; for fp32 storage 1e-4 (ddt and
dA, which are sums over the rest of the sequence, 2e-4).

dA is the exception to the per-tensor relative bound: dA_h = sum over batch and
tokens of dt_t Lambda_t, and these terms cancel (on the workloads here
|dA_h| is 1/30 to 1/700 of sum |dt_t Lambda_t|), so an error bounded relative
to the terms is not bounded relative to the result. Its bound is
|dA_h - ref_h| <= tol * sum_{b,t} |dt_t Lambda_t| (Lambda from the oracle), the
usual bound for a reduction carried out in the storage precision.

At the 1.3B-layer size the oracle runs one head at a time (what a head's dX,
ddt, dA and initial-state gradient depend on is that head alone) and dB, dC
are compared with the sums of the per-head results over the group.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import oracle
import ssd_inputs as si
from tests.gpu_util import TOL, log, rel, to_dev, to_np

pytestmark = pytest.mark.gpu

KEYS = ("dX", "ddt", "dA", "dB", "dC", "dD", "dinit")


def grad_inputs(cfg, seed, with_init, with_dF):
    inp = si.make_fwd_inputs(cfg)
    rng = np.random.default_rng(seed)
    dY = rng.standard_normal(inp["X32"].shape).astype(np.float32)
    if cfg.dtype == "bf16":
        inp["dY"] = si.bf16_round_bits(dY)
        inp["dY32"] = si.bf16_bits_to_f32(inp["dY"])
    else:
        inp["dY"] = inp["dY32"] = dY
    shp = (cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate)
    inp["init"] = rng.standard_normal(shp).astype(np.float32) if with_init else None
    inp["dF"] = rng.standard_normal(shp).astype(np.float32) if with_dF else None
    return inp


def gpu_bwd(ssd, inp, chunk):
    import torch
    X, dt, B, C, dY = (to_dev(inp[k]) for k in ("X", "dt", "B", "C", "dY"))
    A, D = to_dev(inp["A"]), to_dev(inp["D"])
    init = None if inp["init"] is None else to_dev(inp["init"])
    dF = None if inp["dF"] is None else to_dev(inp["dF"])
    out = ssd.ssd_chunk_scan_bwd(X, dt, A, B, C, D, chunk, dY, initial_state=init, d_final_state=dF,
                                 want_initial_grad=True)
    torch.cuda.synchronize()
    return dict(zip(KEYS, (to_np(t) for t in out)))


def oracle_bwd(inp, G):
    return oracle.bwd(inp["X32"], inp["dt32"], inp["A"], inp["B32"], inp["C32"], inp["D"], G, inp["dY32"],
                      inp["init"], inp["dF"])


def tol_for(dtype, key):
    # one bound per storage type for every gradient (dA measured against
    # sum |dt Lambda|, see dA_err)
    return TOL[dtype]


def dA_err(g_dA, ref, dt):
    """max over heads of |dA - ref| / sum_{b,t} |dt Lambda| (see the module docstring)."""
    scale = np.sum(np.abs(dt * ref["lam"]), axis=(0, 1))
    return float(np.max(np.abs(g_dA - ref["dA"]) / scale))


def errors(g, ref, dt):
    e = {k: rel(g[k], ref[k]) for k in KEYS}
    e["dA"] = dA_err(g["dA"], ref, dt)
    return e


def check(ssd, cfg, chunk, with_init, with_dF, seed=80):
    inp = grad_inputs(cfg, seed, with_init, with_dF)
    log(f"[bwd] {cfg.dtype} B{cfg.batch} T{cfg.seqlen} H{cfg.nheads} P{cfg.headdim} N{cfg.dstate} "
        f"G{cfg.ngroups} chunk={chunk} init={with_init} dF={with_dF}")
    g = gpu_bwd(ssd, inp, chunk)
    ref = oracle_bwd(inp, cfg.ngroups)
    errs = errors(g, ref, inp["dt32"])
    log("    " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()) + f" (dA rel to max: {rel(g['dA'], ref['dA']):.2e})")
    for k in KEYS:
        assert np.all(np.isfinite(g[k])), k
        assert errs[k] <= tol_for(cfg.dtype, k), (k, errs[k])


def shape(base, **kw):
    return dataclasses.replace(si.CONFIGS[base], name="bwd", **kw)


@pytest.mark.parametrize("chunk", [64, 256])
def test_bwd_bf16_1p3b_head_shape(ssd, chunk):
    # the 1.3B layer's head shape (P 64, N 128, one group), ragged length
    check(ssd, shape("l1p3b_bf16", batch=2, seqlen=333, nheads=4, seed=81), chunk, False, False)


def test_bwd_bf16_groups_init_and_final_grad(ssd):
    check(ssd, shape("l1p3b_bf16", batch=2, seqlen=200, nheads=4, headdim=32, dstate=64, ngroups=2, seed=82),
          128, True, True)


@pytest.mark.parametrize("P,N", [(32, 32), (64, 32), (64, 64), (32, 128)])
def test_bwd_bf16_head_and_state_sizes(ssd, P, N):
    check(ssd, shape("l1p3b_bf16", batch=1, seqlen=130, nheads=2, headdim=P, dstate=N, seed=83), 64, True,
          True)


@pytest.mark.parametrize("P,N", [(32, 32), (32, 64), (64, 32)])
def test_bwd_f32(ssd, P, N):
    check(ssd, shape("tiny_f32", batch=2, seqlen=150, nheads=2, headdim=P, dstate=N, seed=84), 64, True, True)


@pytest.mark.parametrize("P,N", [(64, 64), (64, 128), (32, 128)])
def test_bwd_f32_n_slices(ssd, P, N):
    """fp32 shapes whose tile kernel takes the n axis in 2 or 4 slices (the
    1.3B layer's head shape among them), the slices' parts of dX, of the
    per-token scalars and of Lambda added afterwards."""
    check(ssd, shape("tiny_f32", batch=2, seqlen=150, nheads=2, headdim=P, dstate=N, seed=94), 64, True, True)


@pytest.mark.parametrize("P", [32, 64])
def test_bwd_bf16_state_size_256(ssd, P):
    """N 256 (the 16K-token workload's state size), two groups, an initial
    state and a final-state gradient, ragged length: the n axis in 2 slices."""
    check(ssd, shape("long16k_bf16", batch=2, seqlen=300, nheads=4, headdim=P, dstate=256, ngroups=2, seed=93),
          128, True, True)


def test_bwd_bf16_state_size_256_head_blocks(ssd):
    """Batch 4, T 2048, 16 heads, P 64, N 256, 2 groups: blocks of 8 heads of
    a group summed in registers together with 2 n slices; every gradient
    element by element."""
    check(ssd, shape("long16k_bf16", batch=4, seqlen=2048, nheads=16, headdim=64, dstate=256, ngroups=2,
                     seed=95), 256, False, True)


@pytest.mark.timeout(600)
def test_bwd_full_size_16k(ssd):
    """The 16K-token workload (batch 1, T 16384, 64 heads, P 64, N 256, 8
    groups, chunk 256): dX, ddt, dA and the initial-state gradient of two heads
    of different groups element by element against the oracle run on those
    heads alone (each depends on its own head only), and every gradient finite.
    dB and dC need all heads of a group; their slices and head blocks are
    checked element by element at N 256 above."""
    cfg = si.CONFIGS["long16k_bf16"]
    inp = grad_inputs(cfg, 96, False, True)
    log("[bwd full size] 16K tokens")
    g = gpu_bwd(ssd, inp, cfg.chunk)
    for k in KEYS:
        assert np.all(np.isfinite(g[k])), k
    HG = cfg.nheads // cfg.ngroups
    for h in (5, 42):
        gr, sl = h // HG, slice(h, h + 1)
        r = oracle.bwd(inp["X32"][:, :, sl], inp["dt32"][:, :, sl], inp["A"][sl], inp["B32"][:, :, gr:gr + 1],
                       inp["C32"][:, :, gr:gr + 1], inp["D"][sl], 1, inp["dY32"][:, :, sl], None, inp["dF"][:, sl])
        e = {"dX": rel(g["dX"][:, :, sl], r["dX"]), "ddt": rel(g["ddt"][:, :, sl], r["ddt"]),
             "dinit": rel(g["dinit"][:, sl], r["dinit"]), "dD": rel(g["dD"][sl], r["dD"]),
             "dA": float(np.abs(g["dA"][h] - r["dA"][0]) / np.sum(np.abs(inp["dt32"][:, :, sl] * r["lam"])))}
        log(f"    head {h}: " + " ".join(f"{k}={v:.2e}" for k, v in e.items()))
        for k, v in e.items():
            assert v <= TOL["bf16"], (h, k, v)


def test_bwd_long_memory(ssd):
    """Small |A|: the adjoint and the states carry across many tiles."""
    cfg = shape("l1p3b_bf16", batch=1, seqlen=700, nheads=2, headdim=32, dstate=32, seed=85)
    inp = grad_inputs(cfg, 86, False, True)
    inp["A"] = (-np.exp(np.random.default_rng(87).uniform(np.log(1e-4), np.log(1e-2), 2))).astype(np.float32)
    g = gpu_bwd(ssd, inp, 256)
    ref = oracle_bwd(inp, 1)
    errs = errors(g, ref, inp["dt32"])
    log("[bwd long memory] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k in KEYS:
        assert errs[k] <= TOL["bf16"], (k, errs[k])


def test_bwd_one_token_and_empty(ssd):
    import torch
    check(ssd, shape("l1p3b_bf16", batch=2, seqlen=1, nheads=2, headdim=32, dstate=32, seed=88), 64, True, True)
    X = torch.empty((2, 0, 2, 32), dtype=torch.bfloat16, device="cuda")
    dt = torch.empty((2, 0, 2), dtype=torch.bfloat16, device="cuda")
    B = torch.empty((2, 0, 1, 32), dtype=torch.bfloat16, device="cuda")
    A = torch.full((2,), -1.0, device="cuda")
    D = torch.ones(2, device="cuda")
    dF = torch.randn((2, 2, 32, 32), device="cuda")
    out = ssd.ssd_chunk_scan_bwd(X, dt, A, B, B, D, 64, X, d_final_state=dF, want_initial_grad=True)
    torch.cuda.synchronize()
    assert not torch.any(out[2]) and not torch.any(out[5]) and torch.equal(out[6], dF)


def test_bwd_deterministic(ssd):
    cfg = shape("l1p3b_bf16", batch=1, seqlen=256, nheads=8, seed=89)
    inp = grad_inputs(cfg, 90, True, True)
    g1, g2 = gpu_bwd(ssd, inp, 128), gpu_bwd(ssd, inp, 128)
    for k in KEYS:
        assert np.array_equal(g1[k], g2[k]), k


@pytest.mark.parametrize("G,P,N", [(1, 32, 32), (2, 64, 64)])
def test_bwd_several_heads_per_block(ssd, G, P, N):
    """Batch 4, T 2048, 16 heads: the backward sums dB and dC over blocks of
    heads of a group in registers (2 blocks of 8 heads with one group, whose
    partials are then added; 1 block of 8 per group with two); every gradient
    is compared element by element."""
    check(ssd, shape("l1p3b_bf16", batch=4, seqlen=2048, nheads=16, headdim=P, dstate=N, ngroups=G,
                     seed=92), 256, False, True)


@pytest.mark.timeout(600)
def test_bwd_full_size_1p3b_layer(ssd):
    """Batch 4, T 2048, 64 heads, P 64, N 128 (32 heads per block): every
    gradient element by element. The oracle runs one head at a time (dX, ddt,
    dA, the initial-state gradient of a head depend on that head alone) and
    dB, dC are the sums of the per-head contributions over the group."""
    cfg = si.CONFIGS["l1p3b_bf16"]
    inp = grad_inputs(cfg, 91, False, True)
    log("[bwd full size] 1.3B layer")
    g = gpu_bwd(ssd, inp, cfg.chunk)
    X, dt, B, C, dY = inp["X32"], inp["dt32"], inp["B32"], inp["C32"], inp["dY32"]
    H = cfg.nheads
    ref = {"dX": np.empty_like(g["dX"]), "ddt": np.empty_like(g["ddt"]), "dA": np.empty(H),
           "dinit": np.empty_like(g["dinit"]), "dB": np.zeros(B.shape), "dC": np.zeros(C.shape),
           "lam": np.empty(dt.shape)}
    for h in range(H):
        sl = slice(h, h + 1)
        r = oracle.bwd(X[:, :, sl], dt[:, :, sl], inp["A"][sl], B, C, inp["D"][sl], 1, dY[:, :, sl], None,
                       inp["dF"][:, sl])
        ref["dX"][:, :, sl], ref["ddt"][:, :, sl], ref["dA"][sl] = r["dX"], r["ddt"], r["dA"]
        ref["dinit"][:, sl], ref["lam"][:, :, sl] = r["dinit"], r["lam"]
        ref["dB"] += r["dB"]
        ref["dC"] += r["dC"]
    e = {k: rel(g[k], ref[k]) for k in ("dX", "ddt", "dB", "dC", "dinit")}
    e["dA"] = dA_err(g["dA"], ref, dt)
    e["dD"] = rel(g["dD"], np.einsum('bthp,bthp->h', dY, X))
    log("    " + " ".join(f"{k}={v:.2e}" for k, v in e.items()))
    for k, v in e.items():
        assert v <= TOL["bf16"], (k, v)
