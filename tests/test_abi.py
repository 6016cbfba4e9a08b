"""CPU tests of the C ABI: the library loads, exports every declared entry point,
and every argument check returns its status before anything touches a GPU.

The pointers below are fake (aligned integers): each call is chosen so that a
host-side check fails first, so no kernel is ever launched from these tests.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import ssd_sequence_mixing_amd as ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")

OK, ENULL, ESHAPE, EUNSUP, EWS, EALIGN, EHIP, ETOOLARGE = range(8)
F32, BF16 = ssd.SSD_F32, ssd.SSD_BF16
P16 = 0x10000  # a fake, 16-byte-aligned device address


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(ssd.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ssd.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_library_exports_with_nm():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", ssd.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for name in declared_functions():
        assert name in syms, name


def test_status_strings():
    for code in range(8):
        s = ssd.ssd_status_string(code)
        assert s.startswith("SSD_OK" if code == 0 else "SSD_ERR")
    assert "UNKNOWN" in ssd.ssd_status_string(99)


def ws(*a):
    return ssd.load().ssd_chunk_scan_fwd_workspace_bytes(*a)


def test_workspace_query():
    big = ctypes.c_size_t(-1).value
    n = ws(4, 2048, 64, 64, 128, 1, 256, BF16)
    # two fp32 (b, H, Tpad) arrays plus the bf16 C B^T of every 64-token tile
    assert n == 2 * 4 * 64 * 2048 * 4 + 4 * 1 * 32 * 64 * 64 * 2
    # 16K tokens, 64 heads: the sequence is walked as 4 segments; the end
    # states of the first 3, each in two halves of 8 chunks, take
    # (b, H, 6, P, N) fp32 more
    n = ws(1, 16384, 64, 64, 256, 8, 256, BF16)
    assert n == 2 * 64 * 16384 * 4 + 8 * 16384 * 64 * 2 + 64 * 6 * 64 * 256 * 4
    assert ws(0, 2048, 64, 64, 128, 1, 256, BF16) == 0
    assert ws(4, 0, 64, 64, 128, 1, 256, BF16) == 0
    assert ws(4, 2048, 64, 64, 128, 3, 256, BF16) == big      # H % G
    assert ws(4, 2048, 64, 64, 128, 1, 32, BF16) == big       # chunk
    assert ws(4, 2048, 64, 48, 128, 1, 256, BF16) == big      # headdim
    assert ws(4, 2048, 64, 64, 96, 1, 256, BF16) == big       # dstate
    assert ws(1, 256, 2, 128, 256, 1, 256, F32) == big        # fp32 tiles exceed LDS
    assert ws(4, 2048, 64, 64, 128, 1, 256, 7) == big         # dtype


def fwd(X=P16, dt=P16, A=P16, B=P16, C=P16, D=P16, chunk=256, Y=P16, fin=P16, batch=4, T=2048,
        H=64, P=64, N=128, G=1, dtype=BF16, wsp=P16 * 16, wsb=1 << 40, stream=None):
    return ssd.raw_call("ssd_chunk_scan_fwd", X, dt, A, B, C, D, chunk, Y, fin, batch, T, H, P, N,
                        G, dtype, wsp, wsb, stream)


@pytest.mark.parametrize("field", ["X", "dt", "A", "B", "C", "D", "Y"])
def test_fwd_null(field):
    assert fwd(**{field: None}) == ENULL


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), ESHAPE), (dict(T=-5), ESHAPE), (dict(H=0), ESHAPE), (dict(P=0), ESHAPE),
    (dict(N=-2), ESHAPE), (dict(G=0), ESHAPE), (dict(H=64, G=3), ESHAPE),
    (dict(chunk=32), EUNSUP), (dict(chunk=100), EUNSUP), (dict(chunk=512), EUNSUP),
    (dict(P=48), EUNSUP), (dict(N=100), EUNSUP), (dict(dtype=5), EUNSUP),
    (dict(dtype=F32, P=128, N=256, chunk=256), EUNSUP),
    (dict(T=1 << 40), EUNSUP),
])
def test_fwd_shape_checks(kw, code):
    assert fwd(**kw) == code


@pytest.mark.parametrize("field", ["X", "dt", "A", "B", "C", "D", "Y", "fin"])
def test_fwd_alignment(field):
    assert fwd(**{field: P16 + 4}) == EALIGN


def test_fwd_workspace_checks():
    need = ws(4, 2048, 64, 64, 128, 1, 256, BF16)
    assert fwd(wsp=None) == EWS
    assert fwd(wsb=need - 1) == EWS
    assert fwd(wsp=P16 + 16, wsb=need) == EALIGN  # workspace wants 256-byte alignment


def test_fwd_empty_batch_returns_ok_without_work():
    assert fwd(batch=0, wsp=None, wsb=0) == OK


def fwd_noalloc(X=P16, dt=P16, A=P16, B=P16, C=P16, D=P16, chunk=256, Y=P16, fin=P16, batch=4, T=2048,
                H=64, P=64, N=128, G=1, dtype=BF16, stream=None):
    return ssd.raw_call("ssd_chunk_scan_fwd_noalloc", X, dt, A, B, C, D, chunk, Y, fin, batch, T, H, P, N,
                        G, dtype, stream)


@pytest.mark.parametrize("field", ["X", "dt", "A", "B", "C", "D", "Y"])
def test_fwd_noalloc_null(field):
    assert fwd_noalloc(**{field: None}) == ENULL


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), ESHAPE), (dict(H=64, G=3), ESHAPE), (dict(chunk=32), EUNSUP), (dict(P=48), EUNSUP),
    (dict(dtype=F32, P=128, N=256, chunk=256), EUNSUP),
])
def test_fwd_noalloc_shape_checks(kw, code):
    assert fwd_noalloc(**kw) == code


@pytest.mark.parametrize("field", ["X", "B", "Y", "fin"])
def test_fwd_noalloc_alignment(field):
    assert fwd_noalloc(**{field: P16 + 4}) == EALIGN


def test_fwd_noalloc_rejects_problems_beyond_its_scratch():
    limit = ssd.NOALLOC_SCRATCH_BYTES
    # the 16K-token, N = 256 workload fits (36 MiB); 8 such sequences do not
    assert ws(1, 16384, 64, 64, 256, 8, 256, BF16) <= limit
    assert ws(8, 16384, 64, 64, 256, 8, 256, BF16) > limit
    assert fwd_noalloc(batch=8, T=16384, N=256, G=8) == ETOOLARGE
    # the workspace query decides: a shape just past the limit is refused
    T = 2048
    while ws(4, T, 64, 64, 128, 1, 256, BF16) <= limit:
        T += 2048
    assert fwd_noalloc(T=T) == ETOOLARGE
    assert fwd_noalloc(batch=0) == OK  # nothing to do, nothing looked up


def test_noalloc_limit_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define SSD_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == ssd.NOALLOC_SCRATCH_BYTES


def step(state=P16, x=P16, dt=P16, A=P16, B=P16, C=P16, D=P16, y=P16, batch=256, H=64, P=64,
         N=128, G=1, dtype=BF16, stream=None):
    return ssd.raw_call("ssd_step", state, x, dt, A, B, C, D, y, batch, H, P, N, G, dtype, stream)


@pytest.mark.parametrize("field", ["state", "x", "dt", "A", "B", "C", "D", "y"])
def test_step_null(field):
    assert step(**{field: None}) == ENULL


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), ESHAPE), (dict(H=0), ESHAPE), (dict(P=0), ESHAPE), (dict(N=0), ESHAPE),
    (dict(G=0), ESHAPE), (dict(H=6, G=4), ESHAPE), (dict(N=12), EUNSUP), (dict(N=512), EUNSUP),
    (dict(dtype=9), EUNSUP),
])
def test_step_shape_checks(kw, code):
    assert step(**kw) == code


@pytest.mark.parametrize("field", ["state", "x", "dt", "A", "B", "C", "D", "y"])
def test_step_alignment(field):
    assert step(**{field: P16 + 2}) == EALIGN


def test_step_empty_batch():
    assert step(batch=0) == OK


def test_single_hip_runtime_in_process():
    # torch's HIP runtime and libssd's must be the same library
    ssd.load()
    assert len(ssd._hip_runtimes_mapped()) == 1, ssd._hip_runtimes_mapped()


def prep(dt=P16, A=P16, B=P16, C=P16, chunk=256, batch=4, T=2048, H=64, P=64, N=128, G=1,
         dtype=BF16, wsp=P16 * 16, wsb=1 << 40, stream=None):
    return ssd.raw_call("ssd_chunk_scan_prepare", dt, A, B, C, chunk, batch, T, H, P, N, G, dtype,
                        wsp, wsb, stream)


def walk(X=P16, B=P16, C=P16, D=P16, init=None, chunk=256, Y=P16, fin=P16, batch=4, T=2048, H=64,
         P=64, N=128, G=1, dtype=BF16, wsp=P16 * 16, wsb=1 << 40, stream=None):
    return ssd.raw_call("ssd_chunk_scan_walk", X, B, C, D, init, chunk, Y, fin, batch, T, H, P, N,
                        G, dtype, wsp, wsb, stream)


@pytest.mark.parametrize("field", ["dt", "A", "B", "C"])
def test_prepare_null_and_align(field):
    assert prep(**{field: None}) == ENULL
    assert prep(**{field: P16 + 8}) == EALIGN


@pytest.mark.parametrize("field", ["X", "B", "C", "D", "Y"])
def test_walk_null(field):
    assert walk(**{field: None}) == ENULL


@pytest.mark.parametrize("field", ["X", "B", "C", "D", "Y", "init", "fin"])
def test_walk_alignment(field):
    assert walk(**{field: P16 + 4}) == EALIGN


@pytest.mark.parametrize("kw,code", [
    (dict(H=64, G=3), ESHAPE), (dict(chunk=48), EUNSUP), (dict(N=24), EUNSUP), (dict(wsp=None), EWS),
])
def test_prepare_and_walk_shape_checks(kw, code):
    assert prep(**kw) == code
    assert walk(**kw) == code


def test_prepare_and_walk_empty():
    assert prep(batch=0, wsp=None, wsb=0) == OK
    assert walk(batch=0, wsp=None, wsb=0) == OK


def varlen(X=P16, dt=P16, A=P16, B=P16, C=P16, D=P16, chunk=256, cu=P16, nseq=8, maxlen=2048,
           total=8192, init=None, Y=P16, fin=P16, H=64, P=64, N=128, G=1, dtype=BF16, wsp=P16 * 16,
           wsb=1 << 40, stream=None):
    return ssd.raw_call("ssd_chunk_scan_fwd_varlen", X, dt, A, B, C, D, chunk, cu, nseq, maxlen, total,
                        init, Y, fin, H, P, N, G, dtype, wsp, wsb, stream)


def test_varlen_workspace_query():
    q = ssd.load().ssd_chunk_scan_varlen_workspace_bytes
    # packed batches are never split into segments: no segment states
    assert q(1, 16384, 64, 64, 256, 8, 256, BF16) == 2 * 64 * 16384 * 4 + 8 * 16384 * 64 * 2
    assert q(8, 2048, 64, 64, 128, 1, 256, BF16) == ws(8, 2048, 64, 64, 128, 1, 256, BF16)
    assert q(8, 2048, 64, 64, 96, 1, 256, BF16) == ctypes.c_size_t(-1).value


@pytest.mark.parametrize("field", ["X", "dt", "A", "B", "C", "D", "Y", "cu"])
def test_varlen_null(field):
    assert varlen(**{field: None}) == ENULL


@pytest.mark.parametrize("kw,code", [
    (dict(nseq=-1), ESHAPE), (dict(maxlen=-1), ESHAPE), (dict(total=-3), ESHAPE),
    (dict(H=64, G=3), ESHAPE), (dict(chunk=32), EUNSUP), (dict(total=1 << 40), ESHAPE),
])
def test_varlen_shape_checks(kw, code):
    assert varlen(**kw) == code


@pytest.mark.parametrize("field", ["X", "dt", "B", "Y", "init", "fin"])
def test_varlen_alignment(field):
    assert varlen(**{field: P16 + 4}) == EALIGN


def test_varlen_workspace_and_empty():
    assert varlen(wsp=None) == EWS
    assert varlen(nseq=0, cu=None, wsp=None, wsb=0) == OK


def bwd(X=P16, dt=P16, A=P16, B=P16, C=P16, D=P16, chunk=256, init=None, dY=P16, dF=None, dX=P16, ddt=P16,
        dA=P16, dB=P16, dC=P16, dD=P16, dinit=None, batch=4, T=2048, H=64, P=64, N=128, G=1, dtype=BF16,
        wsp=P16 * 16, wsb=1 << 40, stream=None):
    return ssd.raw_call("ssd_chunk_scan_bwd", X, dt, A, B, C, D, chunk, init, dY, dF, dX, ddt, dA, dB, dC, dD,
                        dinit, batch, T, H, P, N, G, dtype, wsp, wsb, stream)


def bwd_ws(N, dtype, ns):
    """The backward's workspace at batch 4, T 2048, 64 heads, P 64, one group,
    chunk 256, with k_bwd_tile's n axis in `ns` slices."""
    es = 2 if dtype == BF16 else 4
    fwd = ws(4, 2048, 64, 64, N, 1, 256, dtype)
    st = 4 * 64 * 32 * 64 * N * es              # states per 64-token tile, storage type
    lamb = 4 * 64 * 32 * 4
    shares = 8 * ns * lamb                      # Lambda shares: 8 per tile and slice
    tok = 4 * 64 * 2048 * 4
    nblk = 1                                    # 4 x 32 tiles x 1 group x 2 blocks = 256 work-groups
    while 4 * 32 * nblk < 256:
        nblk *= 2
    part = 4 * 2048 * nblk * N * 4
    dxp = ns * 4 * 2048 * 64 * 64 * 4 if ns > 1 else 0
    return fwd + 2 * st + shares + 2 * lamb + 2 * ns * tok + tok + 2 * part + dxp


def test_bwd_workspace_query():
    q = ssd.load().ssd_chunk_scan_bwd_workspace_bytes
    assert q(4, 2048, 64, 64, 128, 1, 256, BF16) == bwd_ws(128, BF16, 1)
    assert q(4, 2048, 64, 64, 256, 1, 256, BF16) == bwd_ws(256, BF16, 2)    # n in 2 slices of 128
    assert q(4, 2048, 64, 64, 128, 1, 256, F32) == bwd_ws(128, F32, 4)      # n in 4 slices of 32
    assert q(4, 2048, 64, 128, 64, 1, 256, BF16) == ctypes.c_size_t(-1).value   # P 128: not covered
    assert q(4, 2048, 64, 64, 256, 1, 256, F32) == ctypes.c_size_t(-1).value    # fp32 N 256: not covered
    assert q(4, 2048, 64, 64, 16, 1, 256, BF16) == ctypes.c_size_t(-1).value    # N 16: not covered
    assert q(2, 100, 4, 32, 64, 1, 64, F32) > 0
    assert q(0, 2048, 64, 64, 128, 1, 256, BF16) == 0


@pytest.mark.parametrize("field", ["X", "dt", "A", "B", "C", "D", "dY", "dX", "ddt", "dA", "dB", "dC", "dD"])
def test_bwd_null(field):
    assert bwd(**{field: None}) == ENULL


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), ESHAPE), (dict(H=64, G=3), ESHAPE), (dict(chunk=32), EUNSUP),
    (dict(N=16), EUNSUP), (dict(P=128), EUNSUP), (dict(dtype=F32, N=256), EUNSUP), (dict(dtype=7), EUNSUP),
])
def test_bwd_shape_checks(kw, code):
    assert bwd(**kw) == code


@pytest.mark.parametrize("field", ["X", "dY", "dX", "ddt", "dA", "dB", "dinit", "dF", "init"])
def test_bwd_alignment(field):
    assert bwd(**{field: P16 + 4}) == EALIGN


def test_bwd_workspace_and_empty():
    assert bwd(wsp=None) == EWS
    assert bwd(wsb=1000) == EWS
    assert bwd(wsp=P16 + 16) == EALIGN
    assert bwd(batch=0, wsp=None, wsb=0) == OK


def fused(X=P16, cw=P16, cb=P16, dt=P16, bias=None, mode=0, A=P16, B=P16, C=P16, D=P16, z=None, chunk=256,
          Y=P16, fin=P16, batch=4, T=2048, H=64, P=64, N=128, G=1, dtype=BF16, wsp=P16 * 16, wsb=1 << 40):
    return ssd.raw_call("ssd_chunk_scan_fwd_fused", X, cw, cb, dt, bias, mode, A, B, C, D, z, chunk, Y, fin,
                        batch, T, H, P, N, G, dtype, wsp, wsb, None)


def test_fused_argument_checks():
    assert fused(cw=None) == ENULL            # a bias without taps
    assert fused(cw=P16 + 4) == EALIGN
    assert fused(cb=P16 + 2) == EALIGN
    assert fused(mode=3) == EUNSUP
    assert fused(X=None) == ENULL
    assert fused(wsp=None) == EWS
    assert fused(batch=0, wsp=None, wsb=0) == OK


def test_binding_rejects_mismatched_tensors():
    """The Python binding checks shapes and dtypes before any C call (the C ABI
    trusts the sizes it is told). CPU tensors suffice: the check comes first."""
    import torch
    X = torch.zeros((2, 8, 4, 16), dtype=torch.bfloat16)
    dt = torch.zeros((2, 8, 4), dtype=torch.bfloat16)
    B = torch.zeros((2, 8, 1, 16), dtype=torch.bfloat16)
    A = torch.zeros(4)
    D = torch.zeros(4)
    bad = [
        ("dt", dict(dt=torch.zeros((2, 8, 3), dtype=torch.bfloat16))),
        ("B", dict(B=torch.zeros((2, 8, 1, 16), dtype=torch.float32))),
        ("A", dict(A=torch.zeros(4, dtype=torch.float64))),
        ("D", dict(D=torch.zeros(5))),
        ("Y", dict(Y=torch.zeros((2, 8, 4, 8), dtype=torch.bfloat16))),
        ("final_state", dict(final_state=torch.zeros((2, 4, 16, 16), dtype=torch.bfloat16))),
    ]
    for name, kw in bad:
        args = dict(X=X, dt=dt, A=A, B=B, C=B, D=D)
        extra = {k: kw.pop(k) for k in list(kw) if k in ("Y", "final_state")}
        args.update(kw)
        with pytest.raises(ValueError, match=f"^{name}:"):
            ssd.ssd_chunk_scan_fwd(args["X"], args["dt"], args["A"], args["B"], args["C"], args["D"], 64,
                                   **extra)
    # the same tensors with consistent shapes pass the check and stop at the device check
    with pytest.raises(ValueError, match="on the GPU"):
        ssd.ssd_chunk_scan_fwd(X, dt, A, B, B, D, 64)
    state = torch.zeros((2, 4, 16, 16))
    x = torch.zeros((2, 4, 16), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="^state:"):
        ssd.ssd_step(state.to(torch.bfloat16), x, dt[:, 0], A, B[:, 0], B[:, 0], D)
    with pytest.raises(ValueError, match="^y:"):
        ssd.ssd_step(state, x, dt[:, 0], A, B[:, 0], B[:, 0], D, y=torch.zeros((2, 4, 8), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="^dY:"):
        ssd.ssd_chunk_scan_bwd(X, dt, A, B, B, D, 64, torch.zeros((2, 8, 4, 16)))
    with pytest.raises(ValueError, match="cu_seqlens"):
        ssd.ssd_chunk_scan_fwd_varlen(X[0], dt[0], A, B[0], B[0], D, 64,
                                      torch.zeros(3, dtype=torch.int64), 8)
