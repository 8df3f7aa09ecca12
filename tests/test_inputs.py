"""Seeded inputs: determinism, bf16 round-to-nearest-even, workload registry."""

import numpy as np

from exact_attention_flash_amd.inputs import (
    WORKLOADS, bf16_bits_to_f32, default_scale, f32_to_bf16_bits, make_inputs,
)


def test_seed_determinism_and_draw_order():
    a = make_inputs(1, 2, 8, 4, seed=7, with_dout=True)
    b = make_inputs(1, 2, 8, 4, seed=7, with_dout=True)
    for name in ("q", "k", "v", "do"):
        assert a[name].dtype == np.uint16 and a[name].shape == (1, 2, 8, 4)
        assert np.array_equal(a[name], b[name])
    # adding dO does not change Q, K, V (it is drawn last)
    c = make_inputs(1, 2, 8, 4, seed=7)
    for name in ("q", "k", "v"):
        assert np.array_equal(a[name], c[name])
    assert not np.array_equal(a["q"], make_inputs(1, 2, 8, 4, seed=8)["q"])


def test_bf16_round_nearest_even():
    # exactly representable values survive unchanged
    x = np.array([0.0, 1.0, -2.0, 0.5, 3.0, 1.0078125], dtype=np.float32)
    assert np.array_equal(bf16_bits_to_f32(f32_to_bf16_bits(x)), x)
    # ties go to the even mantissa: 1 + 2^-8 lies halfway between 1 and
    # 1 + 2^-7 and rounds down to 1 (even); 1 + 3*2^-8 lies halfway between
    # 1 + 2^-7 (odd) and 1 + 2^-6 (even) and rounds up
    ties = np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8)], dtype=np.float32)
    got = bf16_bits_to_f32(f32_to_bf16_bits(ties))
    assert np.array_equal(got, np.array([1.0, 1 + 2**-6, -1.0], dtype=np.float32))
    # just above a tie rounds up, just below rounds down
    above = np.nextafter(np.float32(1 + 2**-8), np.float32(2))
    below = np.nextafter(np.float32(1 + 2**-8), np.float32(0))
    assert bf16_bits_to_f32(f32_to_bf16_bits(above))[()] == np.float32(1 + 2**-7)
    assert bf16_bits_to_f32(f32_to_bf16_bits(below))[()] == np.float32(1.0)
    # 8 significant bits: relative rounding error is at most 2^-8
    r = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    err = np.abs(bf16_bits_to_f32(f32_to_bf16_bits(r)) - r) / np.abs(r)
    assert err.max() <= 2.0**-8


def test_q_times_eight_is_exact():
    a = make_inputs(2, 1, 16, 8, seed=3)
    b = make_inputs(2, 1, 16, 8, seed=3, q_mult=8.0)
    assert np.array_equal(bf16_bits_to_f32(b["q"]), 8 * bf16_bits_to_f32(a["q"]))
    assert np.array_equal(a["k"], b["k"]) and np.array_equal(a["v"], b["v"])


def test_workloads_and_flop_convention():
    c5 = WORKLOADS["c5"]
    assert (c5.B, c5.H, c5.N, c5.d) == (4, 16, 4096, 128) and c5.backward
    assert c5.flops_fwd(False) == 4.0 * 4 * 16 * 4096**2 * 128
    assert c5.flops_fwd(True) == c5.flops_fwd(False) / 2
    assert c5.flops_bwd(True) == 2.5 * c5.flops_fwd(True)
    assert default_scale(128) == float(np.float32(1 / np.sqrt(128)))
    assert default_scale(64) == 0.125
    assert WORKLOADS["c3"].q_mults == (1.0, 8.0)
    assert WORKLOADS["c4"].N == 16384 and WORKLOADS["c4"].causal == (True,)
