"""GPU tests of ssd_chunk_scan_fwd_noalloc, the forward whose workspace is the
library's static device array: through the C ABI it must give exactly what
ssd_chunk_scan_fwd gives with a caller-allocated workspace (the same kernels
on the same bits), call after call, whatever an earlier call left in the
shared array."""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import ssd_inputs as si
from tests.gpu_util import log, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # the largest workload first (36 MiB of scratch), then smaller ones that
    # find its leftovers in the array
    (si.CONFIGS["long16k_bf16"], None),
    (si.CONFIGS["l1p3b_bf16"], None),
    (dataclasses.replace(si.CONFIGS["l1p3b_bf16"], name="bf16_ragged_small", batch=2, seqlen=1000,
                         nheads=8, dstate=64, ngroups=2, seed=61), 128),
    (dataclasses.replace(si.CONFIGS["tiny_f32"], name="f32_ragged_small", batch=1, seqlen=300,
                         nheads=4, headdim=32, dstate=32, seed=62), 64),
]


def _dev_inputs(cfg):
    inp = si.make_fwd_inputs(cfg)
    return [to_dev(inp[k]) for k in ("X", "dt", "A", "B", "C", "D")]


def _reference(ssd, args, chunk):
    import torch
    Y, F = ssd.ssd_chunk_scan_fwd(*args, chunk)
    torch.cuda.synchronize()
    return Y, F


def _noalloc(ssd, args, chunk):
    import torch
    X = args[0]
    bsz, T, H, P = X.shape
    N = args[3].shape[3]
    Y = torch.full_like(X, float("nan"))
    F = torch.full((bsz, H, P, N), float("nan"), dtype=torch.float32, device=X.device)
    before = torch.cuda.memory_allocated()
    ssd.ssd_chunk_scan_fwd_noalloc(*args, chunk, Y, F)
    assert torch.cuda.memory_allocated() == before
    return Y, F


def test_noalloc_equals_the_workspace_forward_call_after_call(ssd):
    import torch
    for cfg, chunk in CASES:
        chunk = chunk or cfg.chunk
        log(f"[noalloc] {cfg.name} chunk={chunk} shape=(b{cfg.batch},T{cfg.seqlen},H{cfg.nheads},"
            f"P{cfg.headdim},N{cfg.dstate},G{cfg.ngroups}) {cfg.dtype}")
        need = ssd.ssd_chunk_scan_fwd_workspace_bytes(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim,
                                                      cfg.dstate, cfg.ngroups, chunk,
                                                      ssd.SSD_BF16 if cfg.dtype == "bf16" else ssd.SSD_F32)
        assert 0 < need <= ssd.NOALLOC_SCRATCH_BYTES
        args = _dev_inputs(cfg)
        Yr, Fr = _reference(ssd, args, chunk)
        Y, F = _noalloc(ssd, args, chunk)
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16) if Y.dtype == torch.bfloat16 else Y.view(torch.int32),
                           Yr.view(torch.int16) if Yr.dtype == torch.bfloat16 else Yr.view(torch.int32))
        assert torch.equal(F.view(torch.int32), Fr.view(torch.int32))


def test_noalloc_calls_queued_back_to_back_on_one_stream(ssd):
    """Two calls enqueued before any synchronisation: the stream orders them,
    so the second (smaller) one reuses the array only after the first is done."""
    import torch
    (c1, q1), (c2, q2) = CASES[1], CASES[2]
    q1, q2 = q1 or c1.chunk, q2 or c2.chunk
    log(f"[noalloc] back to back: {c1.name} then {c2.name}")
    a1, a2 = _dev_inputs(c1), _dev_inputs(c2)
    r1, r2 = _reference(ssd, a1, q1), _reference(ssd, a2, q2)
    o1 = _noalloc(ssd, a1, q1)
    o2 = _noalloc(ssd, a2, q2)
    torch.cuda.synchronize()
    for (Y, F), (Yr, Fr) in ((o1, r1), (o2, r2)):
        assert torch.equal(Y.view(torch.int16), Yr.view(torch.int16))
        assert torch.equal(F.view(torch.int32), Fr.view(torch.int32))


def test_noalloc_without_final_state_and_empty(ssd):
    import torch
    cfg, chunk = CASES[2]
    args = _dev_inputs(cfg)
    Yr, _ = _reference(ssd, args, chunk)
    Y = torch.empty_like(args[0])
    ssd.ssd_chunk_scan_fwd_noalloc(*args, chunk, Y, None)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Yr.view(torch.int16))
    # zero-length sequences: the final state is zero and nothing else is touched
    X0 = args[0][:, :0].contiguous()
    F0 = torch.full((cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate), 7.0, device=X0.device)
    ssd.ssd_chunk_scan_fwd_noalloc(X0, args[1][:, :0].contiguous(), args[2], args[3][:, :0].contiguous(),
                                   args[4][:, :0].contiguous(), args[5], chunk, torch.empty_like(X0), F0)
    torch.cuda.synchronize()
    assert np.all(F0.cpu().numpy() == 0.0)
