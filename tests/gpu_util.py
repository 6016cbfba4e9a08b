"""Helpers for the GPU parity tests: move the shared seeded inputs to the device,
run the HIP path through the binding, and run the oracle on the same bits."""
from __future__ import annotations

import sys

import numpy as np

import oracle

TOL = {"bf16": 2e-2, "f32": 1e-4}


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_np(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def rel(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = float(np.max(np.abs(b)))
    return float(np.max(np.abs(a - b))) / den if den > 0 else float(np.max(np.abs(a - b)))


def gpu_fwd(ssd, inp, chunk, D_zero=False):
    import torch
    X, dt, B, C = (to_dev(inp[k]) for k in ("X", "dt", "B", "C"))
    A = to_dev(inp["A"])
    D = torch.zeros_like(A) if D_zero else to_dev(inp["D"])
    Y, F = ssd.ssd_chunk_scan_fwd(X, dt, A, B, C, D, chunk)
    torch.cuda.synchronize()
    return to_np(Y), F.cpu().numpy().astype(np.float64)


def oracle_fwd(inp, G, D_zero=False):
    """Oracle on the exact stored values: (Y, final_state) in fp64."""
    X, dt, B, C = inp["X32"], inp["dt32"], inp["B32"], inp["C32"]
    D = np.zeros_like(inp["D"]) if D_zero else inp["D"]
    Y, F, _ = oracle.fwd(X, dt, inp["A"], B, C, D, G)
    return Y, F
