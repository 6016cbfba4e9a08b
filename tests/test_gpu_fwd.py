"""GPU parity of ssd_chunk_scan_fwd against the oracle (through the C ABI).

Tolerances: max|GPU - oracle| / max|oracle| <= 2e-2 with bf16 storage and
<= 1e-4 with fp32 storage, checked separately on Y, on Y with D = 0 (the SSM
part alone, which the skip term would otherwise dominate) and on the final
state.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import ssd_inputs as si
from tests.gpu_util import TOL, gpu_fwd, log, oracle_fwd, rel, to_dev

pytestmark = pytest.mark.gpu


def check_full(ssd, cfg, chunk=None, tag="", inp=None):
    chunk = chunk or cfg.chunk
    log(f"[fwd full] {cfg.name}{tag} chunk={chunk} shape=(b{cfg.batch},T{cfg.seqlen},H{cfg.nheads},"
        f"P{cfg.headdim},N{cfg.dstate},G{cfg.ngroups}) {cfg.dtype}")
    inp = si.make_fwd_inputs(cfg) if inp is None else inp
    tol = TOL[cfg.dtype]
    Yg, Fg = gpu_fwd(ssd, inp, chunk)
    Yr, Fr = oracle_fwd(inp, cfg.ngroups)
    Yg0, Fg0 = gpu_fwd(ssd, inp, chunk, D_zero=True)
    Yr0, _ = oracle_fwd(inp, cfg.ngroups, D_zero=True)
    e = (rel(Yg, Yr), rel(Yg0, Yr0), rel(Fg, Fr))
    log(f"    rel err Y={e[0]:.2e} Y(D=0)={e[1]:.2e} final={e[2]:.2e} (tol {tol})")
    assert np.all(np.isfinite(Yg)) and np.all(np.isfinite(Fg))
    assert e[0] <= tol and e[1] <= tol and e[2] <= tol, e
    assert np.array_equal(Fg, Fg0)  # the final state does not depend on D
    return e


def test_tiny_f32_workload(ssd):
    check_full(ssd, si.CONFIGS["tiny_f32"])


@pytest.mark.parametrize("chunk", [64, 128, 256])
def test_f32_chunk_invariance_ragged(ssd, chunk):
    cfg = dataclasses.replace(si.CONFIGS["tiny_f32"], name="f32_ragged", batch=2, seqlen=300,
                              nheads=4, ngroups=2, seed=21)
    check_full(ssd, cfg, chunk=chunk)


@pytest.mark.parametrize("chunk", [64, 128, 256])
def test_bf16_chunk_invariance_ragged(ssd, chunk):
    cfg = dataclasses.replace(si.CONFIGS["l1p3b_bf16"], name="bf16_ragged", batch=2, seqlen=600,
                              nheads=4, seed=22)
    check_full(ssd, cfg, chunk=chunk)


@pytest.mark.parametrize("P,N", [(16, 16), (32, 32), (64, 64), (128, 128), (64, 256), (128, 64)])
def test_bf16_head_and_state_sizes(ssd, P, N):
    cfg = dataclasses.replace(si.CONFIGS["l1p3b_bf16"], name=f"bf16_P{P}_N{N}", batch=1,
                              seqlen=320, nheads=4, headdim=P, dstate=N, ngroups=2, seed=23)
    check_full(ssd, cfg, chunk=128)


@pytest.mark.parametrize("P,N", [(32, 64), (64, 128)])
def test_f32_head_and_state_sizes(ssd, P, N):
    cfg = dataclasses.replace(si.CONFIGS["tiny_f32"], name=f"f32_P{P}_N{N}", batch=1, seqlen=200,
                              nheads=2, headdim=P, dstate=N, seed=24)
    check_full(ssd, cfg, chunk=64)


@pytest.mark.parametrize("name", ["s2_a_zero", "s3_ragged", "s4_groups", "s5_large_dt"])
def test_stress_workloads(ssd, name):
    check_full(ssd, si.STRESS[name])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tiles_switching_between_diagonal_forms(ssd, dtype):
    """A 64-token tile whose decay is at most 2^64 takes the factored diagonal
    block, a faster-decaying one the per-element weights. Step sizes that jump
    between small and large inside the sequence make neighbouring tiles, and the
    tiles on either side of a chunk boundary, switch between the two."""
    base = "tiny_f32" if dtype == "f32" else "l1p3b_bf16"
    cfg = dataclasses.replace(si.CONFIGS[base], name=f"mixed_decay_{dtype}", batch=2, seqlen=700, nheads=4,
                              headdim=32, dstate=64, seed=41)
    inp = si.make_fwd_inputs(cfg)
    dt = inp["dt32"].copy()
    for lo, hi in ((70, 150), (250, 262), (400, 600)):
        dt[:, lo:hi, :] = 0.6
    if dtype == "bf16":
        inp["dt"] = si.bf16_round_bits(dt)
        inp["dt32"] = si.bf16_bits_to_f32(inp["dt"])
    else:
        inp["dt"] = inp["dt32"] = dt
    # tile decays (base-2 log units), to show that both forms occur
    dec = -inp["A"][None, None, :] * inp["dt32"] * np.log2(np.e)
    T = cfg.seqlen
    tiles = np.add.reduceat(dec, np.arange(0, T, 64), axis=1)
    n_fast, n_slow = int(np.sum(tiles <= 60)), int(np.sum(tiles > 70))
    log(f"    tiles decaying within 2^60: {n_fast}, beyond 2^70: {n_slow}")
    assert n_fast > 0 and n_slow > 0
    check_full(ssd, cfg, chunk=128, inp=inp)


def test_short_sequences(ssd):
    for T in (1, 2, 63, 65):
        cfg = dataclasses.replace(si.CONFIGS["l1p3b_bf16"], name=f"T{T}", batch=3, seqlen=T,
                                  nheads=2, seed=30 + T)
        check_full(ssd, cfg, chunk=64)


def test_full_size_125m_layer(ssd):
    check_full(ssd, si.CONFIGS["l125m_bf16"])


def test_full_size_1p3b_layer(ssd):
    check_full(ssd, si.CONFIGS["l1p3b_bf16"])


def test_full_size_long_16k(ssd):
    # 64 heads in 8 groups of 8, N 256, one 16K-token sequence (split into segments)
    check_full(ssd, si.CONFIGS["long16k_bf16"])


def test_long_memory_stress_full_size(ssd):
    check_full(ssd, si.STRESS["s1_long_memory"])


def test_group_mapping_probe(ssd):
    """G = 8: B zero in every group but k, so only heads floor(h*G/H) == k get an
    SSM term; the others must equal D x to the output's rounding."""
    import torch
    cfg = si.STRESS["s4_groups"]
    inp = si.make_fwd_inputs(cfg)
    H, G = cfg.nheads, cfg.ngroups
    k = 5
    Bm = inp["B"].copy()
    Bm[:, :, [q for q in range(G) if q != k], :] = 0
    X, dt, C = (to_dev(inp[n]) for n in ("X", "dt", "C"))
    A, D = to_dev(inp["A"]), to_dev(inp["D"])
    Y, F = ssd.ssd_chunk_scan_fwd(X, dt, A, to_dev(Bm), C, D, cfg.chunk)
    torch.cuda.synchronize()
    Y = Y.float().cpu().numpy()
    F = F.cpu().numpy()
    skip = (inp["X32"] * inp["D"][None, None, :, None])
    for h in range(H):
        dev = np.max(np.abs(Y[:, :, h] - skip[:, :, h]))
        if (h * G) // H == k:
            assert dev > 1e-3 and np.max(np.abs(F[:, h])) > 1e-3, h
        else:
            assert not np.any(F[:, h]), h
            assert dev <= 2.0 ** -8 * np.max(np.abs(skip[:, :, h])) + 1e-30, (h, dev)


def test_determinism_and_causality(ssd):
    import torch
    cfg = dataclasses.replace(si.CONFIGS["l1p3b_bf16"], name="det", batch=2, seqlen=1000, nheads=8,
                              seed=40)
    inp = si.make_fwd_inputs(cfg)
    log("[fwd] determinism and causality, T=1000")
    X, dt, B, C = (to_dev(inp[k]) for k in ("X", "dt", "B", "C"))
    A, D = to_dev(inp["A"]), to_dev(inp["D"])
    Y1, F1 = ssd.ssd_chunk_scan_fwd(X, dt, A, B, C, D, 256)
    Y2, F2 = ssd.ssd_chunk_scan_fwd(X, dt, A, B, C, D, 256)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2) and torch.equal(F1, F2)
    t0 = 613
    X2, B2 = X.clone(), B.clone()
    X2[:, t0:] = X2[:, t0:] * -3 + 1
    B2[:, t0:] = B2[:, t0:] * 2
    Y3, _ = ssd.ssd_chunk_scan_fwd(X2, dt, A, B2, C, D, 256)
    torch.cuda.synchronize()
    assert torch.equal(Y1[:, :t0], Y3[:, :t0])
    assert not torch.equal(Y1[:, t0:], Y3[:, t0:])


def test_empty_sequence_zero_final_state(ssd):
    import torch
    X = torch.zeros((2, 0, 4, 64), dtype=torch.bfloat16, device="cuda")
    dt = torch.zeros((2, 0, 4), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((2, 0, 1, 128), dtype=torch.bfloat16, device="cuda")
    A = torch.full((4,), -1.0, device="cuda")
    D = torch.ones(4, device="cuda")
    F = torch.full((2, 4, 64, 128), 7.0, device="cuda")
    Y, F = ssd.ssd_chunk_scan_fwd(X, dt, A, B, B, D, 256, final_state=F)
    torch.cuda.synchronize()
    assert Y.shape == X.shape and not torch.any(F)


def test_prepare_then_walk_is_the_forward(ssd):
    import torch
    cfg = dataclasses.replace(si.CONFIGS["l1p3b_bf16"], name="split", batch=2, seqlen=700, nheads=8,
                              seed=70)
    inp = si.make_fwd_inputs(cfg)
    log("[fwd] prepare + walk == fwd (bitwise)")
    X, dt, B, C = (to_dev(inp[k]) for k in ("X", "dt", "B", "C"))
    A, D = to_dev(inp["A"]), to_dev(inp["D"])
    Y1, F1 = ssd.ssd_chunk_scan_fwd(X, dt, A, B, C, D, 256)
    ws = ssd.ssd_chunk_scan_prepare(dt, A, B, C, 256, cfg.headdim)
    Y2, F2 = ssd.ssd_chunk_scan_walk(X, B, C, D, ws, 256)
    # a second walk over the same preparation with another X: the map is linear
    # in X (skip term included) and scaling by 2 is exact in floating point
    Y3, F3 = ssd.ssd_chunk_scan_walk(X * 2, B, C, D, ws, 256)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2) and torch.equal(F1, F2)
    assert torch.allclose(Y3.float(), 2 * Y1.float(), rtol=2 ** -7, atol=0)
    assert torch.allclose(F3, 2 * F1, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("dtype,chunk", [("bf16", 256), ("bf16", 64), ("f32", 128)])
def test_walk_from_initial_state(ssd, dtype, chunk):
    """A walk from a given initial state matches the oracle run from that state."""
    import torch
    base = si.CONFIGS["l1p3b_bf16"] if dtype == "bf16" else si.CONFIGS["tiny_f32"]
    cfg = dataclasses.replace(base, name=f"init_{dtype}", batch=2, seqlen=333, nheads=4, ngroups=2,
                              seed=71)
    inp = si.make_fwd_inputs(cfg)
    rng = np.random.default_rng(72)
    h0 = rng.standard_normal((cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate)).astype(np.float32)
    log(f"[fwd] walk from initial state {dtype} chunk {chunk}")
    X, dt, B, C = (to_dev(inp[k]) for k in ("X", "dt", "B", "C"))
    A, D = to_dev(inp["A"]), to_dev(inp["D"])
    ws = ssd.ssd_chunk_scan_prepare(dt, A, B, C, chunk, cfg.headdim)
    Y, F = ssd.ssd_chunk_scan_walk(X, B, C, D, ws, chunk, initial_state=to_dev(h0))
    Y0, _ = ssd.ssd_chunk_scan_walk(X, B, C, torch.zeros_like(D), ws, chunk, initial_state=to_dev(h0))
    torch.cuda.synchronize()
    import oracle
    Yr, Fr, _ = oracle.fwd(inp["X32"], inp["dt32"], inp["A"], inp["B32"], inp["C32"], inp["D"],
                           cfg.ngroups, init_state=h0)
    Yr0, _, _ = oracle.fwd(inp["X32"], inp["dt32"], inp["A"], inp["B32"], inp["C32"],
                           np.zeros_like(inp["D"]), cfg.ngroups, init_state=h0)
    e = (rel(Y.float().cpu().numpy(), Yr), rel(Y0.float().cpu().numpy(), Yr0), rel(F.cpu().numpy(), Fr))
    log(f"    rel err Y={e[0]:.2e} Y(D=0)={e[1]:.2e} final={e[2]:.2e}")
    tol = TOL[cfg.dtype]
    assert max(e) <= tol, e


@pytest.mark.parametrize("dtype,T,chunk,init", [("bf16", 1000, 64, False), ("bf16", 950, 64, True),
                                                 ("f32", 1000, 64, True), ("bf16", 2048, 128, False)])
def test_split_sequence_halved_prepass(ssd, dtype, T, chunk, init):
    """Few heads and a long sequence: the walk cuts the sequence into segments
    (8 of 2 chunks at 16 chunks, 4 of 4 at 15 chunks, the last one partial),
    and the end-state pre-pass takes each segment but the last as two halves,
    whose states the scan chains into the segments' entering states; with and
    without an initial state (which enters the first half only)."""
    import torch
    import oracle
    base = si.CONFIGS["l1p3b_bf16"] if dtype == "bf16" else si.CONFIGS["tiny_f32"]
    over = dict(headdim=64, dstate=128) if dtype == "bf16" else dict(headdim=32, dstate=64)
    cfg = dataclasses.replace(base, name=f"split_{dtype}_{T}", batch=1, seqlen=T, nheads=2, ngroups=2,
                              seed=73 + T % 7, **over)
    inp = si.make_fwd_inputs(cfg)
    h0 = np.random.default_rng(74).standard_normal((1, 2, cfg.headdim, cfg.dstate)).astype(np.float32) \
        if init else None
    log(f"[fwd] split sequence {dtype} T {T} chunk {chunk} init {init}")
    X, dt, B, C = (to_dev(inp[k]) for k in ("X", "dt", "B", "C"))
    A, D = to_dev(inp["A"]), to_dev(inp["D"])
    ws = ssd.ssd_chunk_scan_prepare(dt, A, B, C, chunk, cfg.headdim)
    Y, F = ssd.ssd_chunk_scan_walk(X, B, C, D, ws, chunk, initial_state=None if h0 is None else to_dev(h0))
    torch.cuda.synchronize()
    Yr, Fr, _ = oracle.fwd(inp["X32"], inp["dt32"], inp["A"], inp["B32"], inp["C32"], inp["D"], cfg.ngroups,
                           init_state=h0)
    e = (rel(Y.float().cpu().numpy(), Yr), rel(F.cpu().numpy(), Fr))
    log(f"    rel err Y={e[0]:.2e} final={e[1]:.2e}")
    assert max(e) <= TOL[cfg.dtype], e


def test_resume_across_calls(ssd):
    """Forward over [0, T1), then a walk over [T1, T) from the carried final
    state, reproduces one forward over [0, T) to the bf16 tolerance."""
    import torch
    cfg = dataclasses.replace(si.CONFIGS["l1p3b_bf16"], name="resume", batch=2, seqlen=900, nheads=4,
                              seed=73)
    inp = si.make_fwd_inputs(cfg)
    X, dt, B, C = (to_dev(inp[k]) for k in ("X", "dt", "B", "C"))
    A, D = to_dev(inp["A"]), to_dev(inp["D"])
    Yf, Ff = ssd.ssd_chunk_scan_fwd(X, dt, A, B, C, D, 256)
    T1 = 389
    Ya, Fa = ssd.ssd_chunk_scan_fwd(X[:, :T1].contiguous(), dt[:, :T1].contiguous(), A,
                                    B[:, :T1].contiguous(), C[:, :T1].contiguous(), D, 256)
    Xb, dtb, Bb, Cb = (t[:, T1:].contiguous() for t in (X, dt, B, C))
    ws = ssd.ssd_chunk_scan_prepare(dtb, A, Bb, Cb, 256, cfg.headdim)
    Yb, Fb = ssd.ssd_chunk_scan_walk(Xb, Bb, Cb, D, ws, 256, initial_state=Fa)
    torch.cuda.synchronize()
    Ys = torch.cat([Ya, Yb], 1).float().cpu().numpy()
    e = (rel(Ys, Yf.float().cpu().numpy()), rel(Fb.cpu().numpy(), Ff.cpu().numpy()))
    log(f"[fwd] resume across calls: rel Y={e[0]:.2e} final={e[1]:.2e}")
    assert max(e) <= TOL["bf16"], e


@pytest.mark.parametrize("dtype,chunk", [("bf16", 256), ("f32", 64)])
def test_canaries_around_outputs_and_workspace(ssd, dtype, chunk):
    """Y, the final state and the workspace sit inside larger buffers whose
    guard bytes before and after must come back untouched; the results must
    equal those of an ordinary call bit for bit. Ragged T, several heads."""
    import torch
    base = si.CONFIGS["l1p3b_bf16"] if dtype == "bf16" else si.CONFIGS["tiny_f32"]
    cfg = dataclasses.replace(base, name=f"canary_{dtype}", batch=2, seqlen=1000, nheads=8,
                              headdim=64 if dtype == "bf16" else 32, dstate=128 if dtype == "bf16" else 64,
                              ngroups=2, seed=41)
    log(f"[fwd canary] {cfg.name} chunk={chunk}")
    inp = si.make_fwd_inputs(cfg)
    X, dt, B, C = (to_dev(inp[k]) for k in ("X", "dt", "B", "C"))
    A, D = to_dev(inp["A"]), to_dev(inp["D"])
    code = ssd.SSD_BF16 if dtype == "bf16" else ssd.SSD_F32
    Bz, T, H, P, N, G = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups
    need = ssd.ssd_chunk_scan_fwd_workspace_bytes(Bz, T, H, P, N, G, chunk, code)
    Yr, Fr = ssd.ssd_chunk_scan_fwd(X, dt, A, B, C, D, chunk)
    GUARD, MARK = 4096, 0xA5

    def guarded(nbytes):
        return torch.full((GUARD + nbytes + GUARD,), MARK, dtype=torch.uint8, device="cuda")

    y_bytes = X.numel() * X.element_size()
    f_bytes = Bz * H * P * N * 4
    Yb, Fb, Wb = guarded(y_bytes), guarded(f_bytes), guarded(need)
    st = ssd.raw_call("ssd_chunk_scan_fwd", X.data_ptr(), dt.data_ptr(), A.data_ptr(), B.data_ptr(), C.data_ptr(),
                      D.data_ptr(), chunk, Yb.data_ptr() + GUARD, Fb.data_ptr() + GUARD, Bz, T, H, P, N, G, code,
                      Wb.data_ptr() + GUARD, need, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    for buf, n in ((Yb, y_bytes), (Fb, f_bytes), (Wb, need)):
        assert torch.all(buf[:GUARD] == MARK) and torch.all(buf[GUARD + n:] == MARK)
    Y = Yb[GUARD:GUARD + y_bytes].view(X.dtype).view(X.shape)
    F = Fb[GUARD:GUARD + f_bytes].view(torch.float32).view(Fr.shape)
    ints = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(Y.view(ints), Yr.view(ints))
    assert torch.equal(F.view(torch.int32), Fr.view(torch.int32))
