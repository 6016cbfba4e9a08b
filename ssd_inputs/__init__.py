"""Seeded synthetic workloads for the SSD core: shapes and input draws only.

This module is shared by the CPU oracle's tests and by the HIP path's tests and
benchmark. It holds no part of the SSD computation itself: it only draws the
inputs (X, dt, A, B, C, D, and for decode an initial state) and rounds them to
the storage dtype. Both sides receive exactly the same stored bits.

Workload shapes follow the pages: sequence lengths 2K and 16K come from the
FlashAttention-2 comparison in the Mamba-2 reading report (section 4 ②); the
125M and 1.3B layer shapes come from its scaling-law study (section 4 ③), with
state size N = 128 (the state-size table in "Mamba 2 state space duality deep
theory", section 6.2) and head dimension P = 64 (reading report, section 2.4).

Distributions (one reading per item):
  X ~ N(0, 1); dt = softplus(z - 4), z ~ N(0, 1) per (b, t, h);
  A = -exp(u), u ~ U(0, ln 16) per head (so A is in [-16, -1]);
  B, C ~ N(0, 1/N) (standard deviation 1/sqrt(N)); D ~ N(0, 1) per head.
Draw order is fixed: X, z, u, B, C, D, all drawn in float32 from numpy's PCG64
with the seed given, then rounded to bfloat16 (round to nearest even) for the
bf16 workloads. A and D stay float32.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

__all__ = [
    "SSDConfig", "DecodeConfig", "CONFIGS", "DECODE", "STRESS",
    "bf16_round_bits", "bf16_bits_to_f32", "make_fwd_inputs", "make_decode_inputs",
]


@dataclasses.dataclass(frozen=True)
class SSDConfig:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    dtype: str            # "f32" or "bf16": storage type of X, dt, B, C and Y
    seed: int
    # distribution knobs for the stress workloads (defaults are the common recipe)
    z_shift: float = -4.0           # dt = softplus(z + z_shift)
    a_log_lo: float = 0.0           # A = -exp(u), u ~ U(a_log_lo, a_log_hi)
    a_log_hi: float = math.log(16.0)
    a_zero: bool = False            # A = 0 exactly (linear-attention special case)

    @property
    def nchunks(self) -> int:
        return -(-self.seqlen // self.chunk)

    def tokens(self) -> int:
        return self.batch * self.seqlen


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    nsteps: int
    nsets: int            # distinct step-input sets; step s uses set s % nsets
    seed: int


# The five workloads the benchmark specification names (index = seed).
CONFIGS: Dict[str, SSDConfig] = {
    "tiny_f32": SSDConfig("tiny_f32", 1, 256, 2, 16, 16, 1, 64, "f32", 0),
    "l125m_bf16": SSDConfig("l125m_bf16", 8, 2048, 24, 64, 128, 1, 256, "bf16", 1),
    "l1p3b_bf16": SSDConfig("l1p3b_bf16", 4, 2048, 64, 64, 128, 1, 256, "bf16", 2),
    "long16k_bf16": SSDConfig("long16k_bf16", 1, 16384, 64, 64, 256, 8, 256, "bf16", 3),
}
DECODE = DecodeConfig("decode_b256", 256, 64, 64, 128, 1, 1000, 8, 4)

# Stress workloads added for coverage of the method's regimes (not benchmark lines).
STRESS: Dict[str, SSDConfig] = {
    # long memory: A close to zero, so cross-chunk terms dominate Y
    "s1_long_memory": SSDConfig("s1_long_memory", 4, 2048, 64, 64, 128, 1, 256, "bf16", 101,
                                a_log_lo=math.log(1e-4), a_log_hi=math.log(1e-2)),
    # A = 0: unnormalised causal linear attention
    "s2_a_zero": SSDConfig("s2_a_zero", 1, 256, 2, 16, 16, 1, 64, "f32", 102, a_zero=True),
    # ragged: T not a multiple of the chunk
    "s3_ragged": SSDConfig("s3_ragged", 2, 1000, 8, 64, 128, 1, 256, "bf16", 103),
    # group mapping probe: eight groups
    "s4_groups": SSDConfig("s4_groups", 1, 512, 16, 64, 128, 8, 128, "bf16", 104),
    # large dt: exercises underflow of the decay and masking
    "s5_large_dt": SSDConfig("s5_large_dt", 2, 512, 8, 64, 128, 1, 256, "bf16", 105, z_shift=1.0),
}


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    r = ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _store(a32: np.ndarray, dtype: str):
    """Returns (stored, as_f32): stored is uint16 bits for bf16, float32 otherwise."""
    a32 = np.ascontiguousarray(a32, dtype=np.float32)
    if dtype == "bf16":
        bits = bf16_round_bits(a32)
        return bits, bf16_bits_to_f32(bits)
    if dtype == "f32":
        return a32, a32
    raise ValueError(f"unknown dtype {dtype!r}")


def _softplus(v: np.ndarray) -> np.ndarray:
    # input-recipe transform (dt arrives already positive); computed in float64
    v = v.astype(np.float64)
    return (np.maximum(v, 0.0) + np.log1p(np.exp(-np.abs(v)))).astype(np.float32)


def make_fwd_inputs(cfg: SSDConfig, seqlen: Optional[int] = None, batch: Optional[int] = None):
    """Draws one forward workload. Returns a dict of numpy arrays.

    Keys X, dt, B, C hold the stored form (uint16 bf16 bits or float32) and
    X32, dt32, B32, C32 the same values as float32 (exact upcast). A and D are
    float32 per head. Layouts: X (batch, T, H, P); dt (batch, T, H);
    B, C (batch, T, G, N); A, D (H,).
    """
    T = cfg.seqlen if seqlen is None else seqlen
    Bsz = cfg.batch if batch is None else batch
    H, P, N, G = cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    X = rng.standard_normal((Bsz, T, H, P), dtype=np.float32)
    z = rng.standard_normal((Bsz, T, H), dtype=np.float32)
    u = rng.uniform(cfg.a_log_lo, cfg.a_log_hi, size=(H,)).astype(np.float32)
    Bm = rng.standard_normal((Bsz, T, G, N), dtype=np.float32) * np.float32(1.0 / math.sqrt(N))
    Cm = rng.standard_normal((Bsz, T, G, N), dtype=np.float32) * np.float32(1.0 / math.sqrt(N))
    D = rng.standard_normal((H,), dtype=np.float32)
    dt = _softplus(z + np.float32(cfg.z_shift))
    A = np.zeros((H,), np.float32) if cfg.a_zero else (-np.exp(u.astype(np.float64))).astype(np.float32)
    out = {"A": A, "D": D}
    for k, v in (("X", X), ("dt", dt), ("B", Bm), ("C", Cm)):
        s, f = _store(v, cfg.dtype)
        out[k] = s
        out[k + "32"] = f
    return out


def make_decode_inputs(cfg: DecodeConfig, batch: Optional[int] = None, with_state: bool = True):
    """Draws the decode workload: an initial state ~ N(0, 1) in float32 of
    shape (batch, H, P, N) and `nsets` step-input sets (x, dt, B, C in bf16).
    Step s of a run uses set s % nsets. A and D are float32 per head.
    """
    Bsz = cfg.batch if batch is None else batch
    H, P, N, G = cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    u = rng.uniform(0.0, math.log(16.0), size=(H,)).astype(np.float32)
    A = (-np.exp(u.astype(np.float64))).astype(np.float32)
    D = rng.standard_normal((H,), dtype=np.float32)
    sets = []
    for _ in range(cfg.nsets):
        x = rng.standard_normal((Bsz, H, P), dtype=np.float32)
        z = rng.standard_normal((Bsz, H), dtype=np.float32)
        Bm = rng.standard_normal((Bsz, G, N), dtype=np.float32) * np.float32(1.0 / math.sqrt(N))
        Cm = rng.standard_normal((Bsz, G, N), dtype=np.float32) * np.float32(1.0 / math.sqrt(N))
        dt = _softplus(z - np.float32(4.0))
        s = {}
        for k, v in (("x", x), ("dt", dt), ("B", Bm), ("C", Cm)):
            st, f = _store(v, "bf16")
            s[k] = st
            s[k + "32"] = f
        sets.append(s)
    out = {"A": A, "D": D, "sets": sets}
    if with_state:
        srng = np.random.Generator(np.random.PCG64(cfg.seed + 1000))
        out["state0"] = srng.standard_normal((Bsz, H, P, N), dtype=np.float32)
    return out
