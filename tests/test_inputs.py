"""CPU tests of the shared seeded input generator (no SSD arithmetic here)."""
import math

import numpy as np

import ssd_inputs as si


def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9, -2.5,
                     3.0e38, 1e-40, 0.0, -0.0], np.float32)
    bits = si.bf16_round_bits(vals)
    back = si.bf16_bits_to_f32(bits)
    # ties go to even mantissa: 1 + 2^-8 -> 1.0 ; 1 + 3*2^-8 -> 1 + 2^-6
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == np.float32(1.0 + 2.0 ** -6)
    assert back[3] == 1.0 and back[4] == -2.5
    assert np.isfinite(back[5]) or back[5] == np.inf
    assert bits[7] == 0 and bits[8] == 0x8000
    nan = si.bf16_round_bits(np.array([np.nan], np.float32))
    assert np.isnan(si.bf16_bits_to_f32(nan))[0]


def test_bf16_round_error_bound():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    y = si.bf16_bits_to_f32(si.bf16_round_bits(x))
    rel = np.abs(y - x) / np.abs(x)
    assert rel.max() <= 2.0 ** -8 + 1e-12


def test_generator_is_deterministic():
    cfg = si.CONFIGS["tiny_f32"]
    a = si.make_fwd_inputs(cfg)
    b = si.make_fwd_inputs(cfg)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_generator_shapes_and_ranges():
    cfg = si.STRESS["s4_groups"]
    d = si.make_fwd_inputs(cfg)
    Bz, T, H, P, N, G = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups
    assert d["X"].shape == (Bz, T, H, P) and d["X"].dtype == np.uint16
    assert d["dt"].shape == (Bz, T, H) and d["B"].shape == (Bz, T, G, N)
    assert d["A"].shape == (H,) and d["A"].dtype == np.float32
    assert np.all(d["dt32"] > 0)
    assert np.all(d["A"] <= -1.0 + 1e-6) and np.all(d["A"] >= -16.0 - 1e-4)
    assert abs(float(np.std(d["B32"])) - 1 / math.sqrt(N)) < 0.01


def test_stress_a_zero_and_long_memory():
    assert not np.any(si.make_fwd_inputs(si.STRESS["s2_a_zero"])["A"])
    A = si.make_fwd_inputs(si.STRESS["s1_long_memory"], seqlen=8, batch=1)["A"]
    assert np.all(A < 0) and np.all(A > -1.01e-2)


def test_decode_inputs():
    cfg = si.DecodeConfig("t", 2, 4, 8, 16, 1, 10, 3, 4)
    d = si.make_decode_inputs(cfg)
    assert d["state0"].shape == (2, 4, 8, 16) and d["state0"].dtype == np.float32
    assert len(d["sets"]) == 3 and d["sets"][0]["x"].shape == (2, 4, 8)
    assert d["sets"][0]["B"].shape == (2, 1, 16) and d["sets"][0]["dt"].shape == (2, 4)
