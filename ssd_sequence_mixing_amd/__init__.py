"""Python binding of libssd, the gfx950 SSD core (argument marshalling only).

Every function here forwards to the C ABI declared in include/ssd.h through
ctypes: it checks that tensors are on the GPU and contiguous, allocates outputs
and workspace with torch when the caller gives none, and passes raw device
pointers plus the current HIP stream. All arithmetic runs in the library's
kernels. There is no fallback: if libssd.so is missing, load() raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

__all__ = [
    "SSD_F32", "SSD_BF16", "SSDError", "load", "lib_path", "ssd_status_string",
    "ssd_chunk_scan_fwd_workspace_bytes", "ssd_chunk_scan_fwd", "ssd_chunk_scan_prepare",
    "ssd_chunk_scan_walk", "ssd_step", "ssd_chunk_scan_varlen_workspace_bytes",
    "ssd_chunk_scan_fwd_varlen", "ssd_chunk_scan_fwd_gated", "ssd_step_gated",
    "ssd_chunk_scan_bwd_workspace_bytes", "ssd_chunk_scan_bwd", "ssd_chunk_scan_fwd_fused",
    "ssd_chunk_scan_fwd_noalloc", "ssd_step_fused", "NOALLOC_SCRATCH_BYTES", "EXPORTS",
]

SSD_F32 = 0
SSD_BF16 = 1
_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libssd.so")
_lib = None

# Entry points include/ssd.h declares.
EXPORTS = ("ssd_status_string", "ssd_chunk_scan_fwd_workspace_bytes", "ssd_chunk_scan_fwd",
           "ssd_chunk_scan_prepare", "ssd_chunk_scan_walk", "ssd_step",
           "ssd_chunk_scan_varlen_workspace_bytes", "ssd_chunk_scan_fwd_varlen",
           "ssd_chunk_scan_fwd_gated", "ssd_step_gated", "ssd_chunk_scan_bwd_workspace_bytes",
           "ssd_chunk_scan_bwd", "ssd_chunk_scan_fwd_fused", "ssd_chunk_scan_fwd_noalloc", "ssd_step_fused")

# SSD_NOALLOC_SCRATCH_BYTES: the static workspace of ssd_chunk_scan_fwd_noalloc.
NOALLOC_SCRATCH_BYTES = 64 << 20

_V = ctypes.c_void_p
_I = ctypes.c_int64


class SSDError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {ssd_status_string(code)} (status {code})")


def lib_path() -> str:
    return _LIB_PATH


def _hip_runtimes_mapped():
    """Paths of every libamdhip64 mapped into this process."""
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


def load():
    """Loads libssd.so (built by ssd_sequence_mixing_amd.build); raises if absent.

    torch is imported first on purpose: torch ships its own HIP runtime, whose
    soname (libamdhip64.so.7) is the one libssd.so asks for, so loading torch
    first makes libssd bind to that same runtime. Loading libssd first would
    bring in a second HIP runtime (torch asks for its copy under another
    name), and device memory and streams owned by one runtime are not valid
    in the other."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise FileNotFoundError(
            f"{_LIB_PATH} is missing: build it with `python -m ssd_sequence_mixing_amd.build` "
            "(or __graft_entry__.build()). There is no fallback path.")
    import torch  # noqa: F401  (see the docstring: one HIP runtime per process)
    lib = ctypes.CDLL(_LIB_PATH)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise RuntimeError(f"two HIP runtimes are loaded in this process: {sorted(runtimes)}; "
                           "import torch before loading libssd.so")
    lib.ssd_status_string.restype = ctypes.c_char_p
    lib.ssd_status_string.argtypes = [ctypes.c_int]
    lib.ssd_chunk_scan_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.ssd_chunk_scan_fwd_workspace_bytes.argtypes = [_I] * 7 + [ctypes.c_int]
    lib.ssd_chunk_scan_fwd.restype = ctypes.c_int
    lib.ssd_chunk_scan_fwd.argtypes = [_V] * 6 + [_I, _V, _V] + [_I] * 6 + [ctypes.c_int, _V,
                                                                          ctypes.c_size_t, _V]
    lib.ssd_chunk_scan_prepare.restype = ctypes.c_int
    lib.ssd_chunk_scan_prepare.argtypes = [_V] * 4 + [_I] * 7 + [ctypes.c_int, _V, ctypes.c_size_t, _V]
    lib.ssd_chunk_scan_walk.restype = ctypes.c_int
    lib.ssd_chunk_scan_walk.argtypes = [_V] * 5 + [_I, _V, _V] + [_I] * 6 + [ctypes.c_int, _V,
                                                                           ctypes.c_size_t, _V]
    lib.ssd_step.restype = ctypes.c_int
    lib.ssd_step.argtypes = [_V] * 8 + [_I] * 5 + [ctypes.c_int, _V]
    lib.ssd_chunk_scan_varlen_workspace_bytes.restype = ctypes.c_size_t
    lib.ssd_chunk_scan_varlen_workspace_bytes.argtypes = [_I] * 7 + [ctypes.c_int]
    lib.ssd_chunk_scan_fwd_gated.restype = ctypes.c_int
    lib.ssd_chunk_scan_fwd_gated.argtypes = ([_V, _V, _V, ctypes.c_int] + [_V] * 5 + [_I, _V, _V] + [_I] * 6 +
                                             [ctypes.c_int, _V, ctypes.c_size_t, _V])
    lib.ssd_step_gated.restype = ctypes.c_int
    lib.ssd_step_gated.argtypes = ([_V, _V, _V, _V, ctypes.c_int] + [_V] * 6 + [_I] * 5 +
                                   [ctypes.c_int, _V])
    lib.ssd_chunk_scan_fwd_varlen.restype = ctypes.c_int
    lib.ssd_chunk_scan_fwd_varlen.argtypes = ([_V] * 6 + [_I, _V] + [_I] * 3 + [_V, _V, _V] + [_I] * 4 +
                                              [ctypes.c_int, _V, ctypes.c_size_t, _V])
    lib.ssd_chunk_scan_fwd_fused.restype = ctypes.c_int
    lib.ssd_chunk_scan_fwd_fused.argtypes = ([_V] * 5 + [ctypes.c_int] + [_V] * 5 + [_I, _V, _V] + [_I] * 6 +
                                             [ctypes.c_int, _V, ctypes.c_size_t, _V])
    lib.ssd_step_fused.restype = ctypes.c_int
    lib.ssd_step_fused.argtypes = ([_V] * 7 + [ctypes.c_int] + [_V] * 6 + [_I] * 5 + [ctypes.c_int, _V])
    lib.ssd_chunk_scan_fwd_noalloc.restype = ctypes.c_int
    lib.ssd_chunk_scan_fwd_noalloc.argtypes = [_V] * 6 + [_I, _V, _V] + [_I] * 6 + [ctypes.c_int, _V]
    lib.ssd_chunk_scan_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.ssd_chunk_scan_bwd_workspace_bytes.argtypes = [_I] * 7 + [ctypes.c_int]
    lib.ssd_chunk_scan_bwd.restype = ctypes.c_int
    lib.ssd_chunk_scan_bwd.argtypes = ([_V] * 6 + [_I] + [_V] * 10 + [_I] * 6 +
                                       [ctypes.c_int, _V, ctypes.c_size_t, _V])
    _lib = lib
    return lib


def ssd_status_string(code: int) -> str:
    return load().ssd_status_string(int(code)).decode()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return SSD_BF16
    if t.dtype == torch.float32:
        return SSD_F32
    raise TypeError(f"unsupported storage dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _chk(name: str, t, shape, dtype) -> None:
    """Raises ValueError unless tensor t (when given) has this shape and dtype:
    the C ABI takes raw pointers and trusts the sizes it is told."""
    if t is None:
        return
    if tuple(t.shape) != tuple(int(d) for d in shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(int(d) for d in shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")


def _check_scan(X, dt, A, B, C, D, *, Y=None, final_state=None, initial_state=None, z=None, dY=None,
                packed_seqs: Optional[int] = None):
    """Shapes and dtypes of a forward's (or backward's) tensors against X and B:
    X (b, T, H, P) and B (b, T, G, N), or for a packed batch X (total, H, P) and
    B (total, G, N) with packed_seqs sequences. X, dt, B, C, Y, z, dY share one
    storage dtype; A, D and the states are fp32."""
    import torch
    if packed_seqs is None:
        if X.dim() != 4 or B.dim() != 4:
            raise ValueError("X must be (batch, T, H, P) and B (batch, T, G, N)")
        bsz, T, H, P = X.shape
        G, N = B.shape[2], B.shape[3]
        lead, nst = (bsz, T), bsz
    else:
        if X.dim() != 3 or B.dim() != 3:
            raise ValueError("packed X must be (total, H, P) and B (total, G, N)")
        total, H, P = X.shape
        G, N = B.shape[1], B.shape[2]
        lead, nst = (total,), packed_seqs
    st = X.dtype
    _dtype_code(X)
    _chk("dt", dt, (*lead, H), st)
    _chk("B", B, (*lead, G, N), st)
    _chk("C", C, (*lead, G, N), st)
    _chk("A", A, (H,), torch.float32)
    _chk("D", D, (H,), torch.float32)
    _chk("Y", Y, X.shape, st)
    _chk("z", z, X.shape, st)
    _chk("dY", dY, X.shape, st)
    _chk("final_state", final_state, (nst, H, P, N), torch.float32)
    _chk("initial_state", initial_state, (nst, H, P, N), torch.float32)


def _check_step(state, x, dt, A, B, C, D, y=None, z=None):
    """Shapes and dtypes of a decode step's tensors against state (b, H, P, N)
    and B (b, G, N)."""
    import torch
    if state.dim() != 4 or B.dim() != 3:
        raise ValueError("state must be (batch, H, P, N) and B (batch, G, N)")
    bsz, H, P, N = state.shape
    G = B.shape[1]
    st = x.dtype
    _dtype_code(x)
    _chk("state", state, (bsz, H, P, N), torch.float32)
    _chk("x", x, (bsz, H, P), st)
    _chk("dt", dt, (bsz, H), st)
    _chk("B", B, (bsz, G, N), st)
    _chk("C", C, (bsz, G, N), st)
    _chk("A", A, (H,), torch.float32)
    _chk("D", D, (H,), torch.float32)
    _chk("y", y, (bsz, H, P), st)
    _chk("z", z, (bsz, H, P), st)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def ssd_chunk_scan_fwd_workspace_bytes(batch, seqlen, nheads, headdim, dstate, ngroups, chunk,
                                       dtype: int) -> int:
    n = load().ssd_chunk_scan_fwd_workspace_bytes(batch, seqlen, nheads, headdim, dstate, ngroups,
                                                  chunk, dtype)
    if n == ctypes.c_size_t(-1).value:
        raise SSDError(3, "ssd_chunk_scan_fwd_workspace_bytes")
    return int(n)


def ssd_chunk_scan_fwd(X, dt, A, B, C, D, chunk: int, Y=None, final_state=None, *,
                       want_final: bool = True, workspace=None, stream=None):
    """Chunked SSD forward. Shapes: X (b, T, H, P), dt (b, T, H), A/D (H,) fp32,
    B/C (b, T, G, N); X/dt/B/C share one storage dtype (bf16 or fp32).

    Returns (Y, final_state); final_state is None when want_final is False and
    none was passed in."""
    import torch
    lib = load()
    _check_scan(X, dt, A, B, C, D, Y=Y, final_state=final_state)
    bsz, T, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    code = _dtype_code(X)
    if Y is None:
        Y = torch.empty_like(X)
    if final_state is None and want_final:
        final_state = torch.empty((bsz, H, P, N), dtype=torch.float32, device=X.device)
    need = ssd_chunk_scan_fwd_workspace_bytes(bsz, T, H, P, N, G, chunk, code)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.ssd_chunk_scan_fwd(_ptr(X), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), chunk,
                                _ptr(Y), _ptr(final_state), bsz, T, H, P, N, G, code,
                                _ptr(workspace), ws_bytes, _stream(stream))
    if st != 0:
        raise SSDError(st, "ssd_chunk_scan_fwd")
    return Y, final_state


def ssd_chunk_scan_fwd_noalloc(X, dt, A, B, C, D, chunk: int, Y, final_state=None, *, stream=None):
    """ssd_chunk_scan_fwd with the library's static workspace: the C call
    allocates nothing, so the caller passes Y (and final_state, or None to
    skip it) already allocated. Calls that may overlap on one GPU race on the
    shared workspace. Returns (Y, final_state)."""
    lib = load()
    if Y is None:
        raise ValueError("ssd_chunk_scan_fwd_noalloc allocates nothing: pass Y")
    _check_scan(X, dt, A, B, C, D, Y=Y, final_state=final_state)
    bsz, T, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    st = lib.ssd_chunk_scan_fwd_noalloc(_ptr(X), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), chunk,
                                        _ptr(Y), _ptr(final_state), bsz, T, H, P, N, G, _dtype_code(X),
                                        _stream(stream))
    if st != 0:
        raise SSDError(st, "ssd_chunk_scan_fwd_noalloc")
    return Y, final_state


def ssd_step_fused(state, conv_state, x, dt, A, B, C, D, *, conv_w, conv_b=None, dt_bias=None,
                   dt_softplus: int = 0, z=None, y=None, stream=None):
    """ssd_step_gated with the layer's causal conv1d(4) + SiLU on x: conv_state
    (b, H*P, 3) in x's dtype holds the 3 earlier raw inputs (oldest first) and
    is shifted in place, as is the fp32 state. conv_w (H*P, 4), conv_b (H*P)
    fp32. Returns y."""
    import torch
    lib = load()
    _check_step(state, x, dt, A, B, C, D, y=y, z=z)
    bsz, H, P, N = state.shape
    G = B.shape[1]
    _chk("conv_state", conv_state, (bsz, H * P, 3), x.dtype)
    _chk("conv_w", conv_w, (H * P, 4), torch.float32)
    _chk("conv_b", conv_b, (H * P,), torch.float32)
    _chk("dt_bias", dt_bias, (H,), torch.float32)
    code = _dtype_code(x)
    if y is None:
        y = torch.empty_like(x)
    st = lib.ssd_step_fused(_ptr(state), _ptr(conv_state), _ptr(x), _ptr(conv_w), _ptr(conv_b), _ptr(dt),
                            _ptr(dt_bias), int(dt_softplus), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                            _ptr(y), bsz, H, P, N, G, code, _stream(stream))
    if st != 0:
        raise SSDError(st, "ssd_step_fused")
    return y


def _workspace(workspace, need, device):
    import torch
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return workspace, nbytes


def ssd_chunk_scan_prepare(dt, A, B, C, chunk: int, headdim: int, *, workspace=None, stream=None):
    """Phase 1 of the forward: fills and returns the workspace."""
    import torch
    lib = load()
    if dt.dim() != 3 or B.dim() != 4:
        raise ValueError("dt must be (batch, T, H) and B (batch, T, G, N)")
    bsz, T, H = dt.shape
    G, N = B.shape[2], B.shape[3]
    code = _dtype_code(dt)
    _chk("B", B, (bsz, T, G, N), dt.dtype)
    _chk("C", C, (bsz, T, G, N), dt.dtype)
    _chk("A", A, (H,), torch.float32)
    need = ssd_chunk_scan_fwd_workspace_bytes(bsz, T, H, headdim, N, G, chunk, code)
    workspace, nbytes = _workspace(workspace, need, dt.device)
    st = lib.ssd_chunk_scan_prepare(_ptr(dt), _ptr(A), _ptr(B), _ptr(C), chunk, bsz, T, H, headdim,
                                    N, G, code, _ptr(workspace), nbytes, _stream(stream))
    if st != 0:
        raise SSDError(st, "ssd_chunk_scan_prepare")
    return workspace


def ssd_chunk_scan_walk(X, B, C, D, workspace, chunk: int, initial_state=None, Y=None,
                        final_state=None, *, want_final: bool = True, stream=None):
    """Phase 2 of the forward: the chunk walk over a prepared workspace."""
    import torch
    lib = load()
    if X.dim() != 4 or B.dim() != 4:
        raise ValueError("X must be (batch, T, H, P) and B (batch, T, G, N)")
    bsz, T, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    code = _dtype_code(X)
    _chk("B", B, (bsz, T, G, N), X.dtype)
    _chk("C", C, (bsz, T, G, N), X.dtype)
    _chk("D", D, (H,), torch.float32)
    _chk("Y", Y, X.shape, X.dtype)
    _chk("final_state", final_state, (bsz, H, P, N), torch.float32)
    _chk("initial_state", initial_state, (bsz, H, P, N), torch.float32)
    if Y is None:
        Y = torch.empty_like(X)
    if final_state is None and want_final:
        final_state = torch.empty((bsz, H, P, N), dtype=torch.float32, device=X.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.ssd_chunk_scan_walk(_ptr(X), _ptr(B), _ptr(C), _ptr(D), _ptr(initial_state), chunk,
                                 _ptr(Y), _ptr(final_state), bsz, T, H, P, N, G, code,
                                 _ptr(workspace), nbytes, _stream(stream))
    if st != 0:
        raise SSDError(st, "ssd_chunk_scan_walk")
    return Y, final_state


def ssd_step(state, x, dt, A, B, C, D, y=None, *, stream=None):
    """One decode step; `state` (b, H, P, N) fp32 is updated in place. Returns y."""
    import torch
    lib = load()
    _check_step(state, x, dt, A, B, C, D, y=y)
    bsz, H, P, N = state.shape
    G = B.shape[1]
    code = _dtype_code(x)
    if y is None:
        y = torch.empty_like(x)
    st = lib.ssd_step(_ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(y),
                      bsz, H, P, N, G, code, _stream(stream))
    if st != 0:
        raise SSDError(st, "ssd_step")
    return y


def ssd_chunk_scan_varlen_workspace_bytes(num_seqs, max_seqlen, nheads, headdim, dstate, ngroups,
                                          chunk, dtype: int) -> int:
    n = load().ssd_chunk_scan_varlen_workspace_bytes(num_seqs, max_seqlen, nheads, headdim, dstate,
                                                     ngroups, chunk, dtype)
    if n == ctypes.c_size_t(-1).value:
        raise SSDError(3, "ssd_chunk_scan_varlen_workspace_bytes")
    return int(n)


def ssd_chunk_scan_fwd_varlen(X, dt, A, B, C, D, chunk: int, cu_seqlens, max_seqlen: int,
                              initial_state=None, Y=None, final_state=None, *,
                              want_final: bool = True, workspace=None, stream=None):
    """Forward over a packed variable-length batch. X (total, H, P), dt (total, H),
    B/C (total, G, N); cu_seqlens int32 on the GPU, (num_seqs + 1) cumulative
    lengths; max_seqlen the longest sequence (a host int, so that no device value
    has to be read here). Returns (Y, final_state) with final_state
    (num_seqs, H, P, N) fp32."""
    import torch
    lib = load()
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-d int32 tensor of num_seqs + 1 offsets")
    nseq = cu_seqlens.numel() - 1
    _check_scan(X, dt, A, B, C, D, Y=Y, final_state=final_state, initial_state=initial_state,
                packed_seqs=nseq)
    total, H, P = X.shape
    G, N = B.shape[1], B.shape[2]
    code = _dtype_code(X)
    if Y is None:
        Y = torch.empty_like(X)
    if final_state is None and want_final:
        final_state = torch.empty((nseq, H, P, N), dtype=torch.float32, device=X.device)
    need = ssd_chunk_scan_varlen_workspace_bytes(nseq, max_seqlen, H, P, N, G, chunk, code)
    workspace, nbytes = _workspace(workspace, need, X.device)
    st = lib.ssd_chunk_scan_fwd_varlen(_ptr(X), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), chunk,
                                       _ptr(cu_seqlens), nseq, max_seqlen, total, _ptr(initial_state),
                                       _ptr(Y), _ptr(final_state), H, P, N, G, code, _ptr(workspace),
                                       nbytes, _stream(stream))
    if st != 0:
        raise SSDError(st, "ssd_chunk_scan_fwd_varlen")
    return Y, final_state


def ssd_chunk_scan_fwd_gated(X, dt, A, B, C, D, chunk: int, *, dt_bias=None, dt_softplus: int = 0, z=None,
                             Y=None, final_state=None, want_final: bool = True, workspace=None, stream=None):
    """ssd_chunk_scan_fwd with the fused prologue (dt_bias, dt_softplus: 0 none,
    1 softplus(dt + bias), 2 softplus(dt) + bias) and output gate Y * silu(z)."""
    import torch
    lib = load()
    _check_scan(X, dt, A, B, C, D, Y=Y, final_state=final_state, z=z)
    _chk("dt_bias", dt_bias, (X.shape[2],), torch.float32)
    bsz, T, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    code = _dtype_code(X)
    if Y is None:
        Y = torch.empty_like(X)
    if final_state is None and want_final:
        final_state = torch.empty((bsz, H, P, N), dtype=torch.float32, device=X.device)
    need = ssd_chunk_scan_fwd_workspace_bytes(bsz, T, H, P, N, G, chunk, code)
    workspace, nbytes = _workspace(workspace, need, X.device)
    st = lib.ssd_chunk_scan_fwd_gated(_ptr(X), _ptr(dt), _ptr(dt_bias), int(dt_softplus), _ptr(A), _ptr(B),
                                      _ptr(C), _ptr(D), _ptr(z), chunk, _ptr(Y), _ptr(final_state), bsz, T,
                                      H, P, N, G, code, _ptr(workspace), nbytes, _stream(stream))
    if st != 0:
        raise SSDError(st, "ssd_chunk_scan_fwd_gated")
    return Y, final_state


def ssd_chunk_scan_fwd_fused(X, dt, A, B, C, D, chunk: int, *, conv_w=None, conv_b=None, dt_bias=None,
                             dt_softplus: int = 0, z=None, Y=None, final_state=None, want_final: bool = True,
                             workspace=None, stream=None):
    """ssd_chunk_scan_fwd_gated with the input activation fused in: X is taken before the
    causal 4-tap depthwise convolution (conv_w (H*P, 4), conv_b (H*P) fp32) and SiLU."""
    import torch
    lib = load()
    _check_scan(X, dt, A, B, C, D, Y=Y, final_state=final_state, z=z)
    _chk("dt_bias", dt_bias, (X.shape[2],), torch.float32)
    _chk("conv_w", conv_w, (X.shape[2] * X.shape[3], 4), torch.float32)
    _chk("conv_b", conv_b, (X.shape[2] * X.shape[3],), torch.float32)
    bsz, T, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    code = _dtype_code(X)
    if Y is None:
        Y = torch.empty_like(X)
    if final_state is None and want_final:
        final_state = torch.empty((bsz, H, P, N), dtype=torch.float32, device=X.device)
    need = ssd_chunk_scan_fwd_workspace_bytes(bsz, T, H, P, N, G, chunk, code)
    workspace, nbytes = _workspace(workspace, need, X.device)
    st = lib.ssd_chunk_scan_fwd_fused(_ptr(X), _ptr(conv_w), _ptr(conv_b), _ptr(dt), _ptr(dt_bias),
                                      int(dt_softplus), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), chunk,
                                      _ptr(Y), _ptr(final_state), bsz, T, H, P, N, G, code, _ptr(workspace),
                                      nbytes, _stream(stream))
    if st != 0:
        raise SSDError(st, "ssd_chunk_scan_fwd_fused")
    return Y, final_state


def ssd_step_gated(state, x, dt, A, B, C, D, *, dt_bias=None, dt_softplus: int = 0, z=None, y=None,
                   stream=None):
    """ssd_step with the fused prologue and output gate (see ssd_chunk_scan_fwd_gated)."""
    import torch
    lib = load()
    _check_step(state, x, dt, A, B, C, D, y=y, z=z)
    _chk("dt_bias", dt_bias, (state.shape[1],), torch.float32)
    bsz, H, P, N = state.shape
    G = B.shape[1]
    code = _dtype_code(x)
    if y is None:
        y = torch.empty_like(x)
    st = lib.ssd_step_gated(_ptr(state), _ptr(x), _ptr(dt), _ptr(dt_bias), int(dt_softplus), _ptr(A),
                            _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(y), bsz, H, P, N, G, code,
                            _stream(stream))
    if st != 0:
        raise SSDError(st, "ssd_step_gated")
    return y


def ssd_chunk_scan_bwd_workspace_bytes(batch, seqlen, nheads, headdim, dstate, ngroups, chunk,
                                       dtype=SSD_BF16) -> int:
    n = load().ssd_chunk_scan_bwd_workspace_bytes(batch, seqlen, nheads, headdim, dstate, ngroups, chunk,
                                                  int(dtype))
    if n == ctypes.c_size_t(-1).value:
        raise SSDError(3, "ssd_chunk_scan_bwd_workspace_bytes")
    return int(n)


def ssd_chunk_scan_bwd(X, dt, A, B, C, D, chunk: int, dY, *, initial_state=None, d_final_state=None,
                       want_initial_grad: bool = False, workspace=None, stream=None):
    """Gradients of <dY, Y> + <dF, final_state> for ssd_chunk_scan_fwd(X, dt, A, B, C, D, chunk)
    from initial_state (zero when None). Returns (dX, ddt, dA, dB, dC, dD, d_initial_state);
    the last is None unless want_initial_grad."""
    import torch
    lib = load()
    _check_scan(X, dt, A, B, C, D, dY=dY, final_state=d_final_state, initial_state=initial_state)
    bsz, T, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    code = _dtype_code(X)
    dX, ddt = torch.empty_like(X), torch.empty_like(dt)
    dB, dC = torch.empty_like(B), torch.empty_like(C)
    dA = torch.empty((H,), dtype=torch.float32, device=X.device)
    dD = torch.empty((H,), dtype=torch.float32, device=X.device)
    dinit = (torch.empty((bsz, H, P, N), dtype=torch.float32, device=X.device)
             if want_initial_grad else None)
    nbytes = ssd_chunk_scan_bwd_workspace_bytes(bsz, T, H, P, N, G, chunk, code)
    if workspace is None:
        workspace = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=X.device)
    st = lib.ssd_chunk_scan_bwd(_ptr(X), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), int(chunk),
                                _ptr(initial_state), _ptr(dY), _ptr(d_final_state), _ptr(dX), _ptr(ddt),
                                _ptr(dA), _ptr(dB), _ptr(dC), _ptr(dD), _ptr(dinit), bsz, T, H, P, N, G,
                                code, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(stream))
    if st != 0:
        raise SSDError(st, "ssd_chunk_scan_bwd")
    return dX, ddt, dA, dB, dC, dD, dinit


def raw_call(name: str, *args) -> int:
    """Calls a C entry point with raw integer/pointer arguments; returns its status."""
    return int(getattr(load(), name)(*args))
