"""Seeded inputs: determinism, bf16 round-to-nearest-even, workload registry."""

import numpy as np
import pytest

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


def _torch_e4m3(x):
    import torch
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_e4m3_encoder_matches_torch():
    import torch
    from exact_attention_flash_amd.inputs import f32_to_e4m3_bits
    # every midpoint between neighbouring finite values (ties to even), both signs
    vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    fin = np.unique(vals[np.isfinite(vals)])
    mids = ((fin[1:] + fin[:-1]) / 2).astype(np.float32)
    for x in (mids, -mids, fin.astype(np.float32)):
        assert np.array_equal(f32_to_e4m3_bits(x), _torch_e4m3(x))
    # random values over many binades, clipped to the finite range
    r = np.random.default_rng(1)
    x = np.concatenate([r.standard_normal(20000) * s for s in (1e-3, 0.05, 1, 30, 300)])
    x = np.clip(x, -448, 448).astype(np.float32)
    assert np.array_equal(f32_to_e4m3_bits(x), _torch_e4m3(x))
    # zeros keep their sign; magnitudes past 448 saturate
    got = f32_to_e4m3_bits(np.array([0.0, -0.0, 500.0, -1e6], dtype=np.float32))
    assert got.tolist() == [0x00, 0x80, 0x7E, 0xFE]


def test_fp8_inputs_share_the_bf16_draws():
    import torch
    from exact_attention_flash_amd.inputs import E4M3_MAX, make_inputs_fp8
    a = make_inputs_fp8(1, 2, 32, 16, seed=9)
    b = make_inputs_fp8(1, 2, 32, 16, seed=9)
    f = make_inputs(1, 2, 32, 16, seed=9)
    for name in ("q", "k", "v"):
        assert a[name].dtype == np.uint8 and np.array_equal(a[name], b[name])
        deq = torch.from_numpy(a[name]).view(torch.float8_e4m3fn).double().numpy() \
            * a["descale_" + name]
        ref = bf16_bits_to_f32(f[name]).astype(np.float64)
        # amax scaling: the largest magnitude lands at the top of the range
        assert np.max(np.abs(deq)) == pytest.approx(np.max(np.abs(ref)), rel=2**-8)
        assert np.max(np.abs(deq / a["descale_" + name])) <= E4M3_MAX
        # E4M3 keeps 4 significant bits (normal range): relative error <= 2^-4,
        # on top of the bf16 rounding of the reference values
        normal = np.abs(deq / a["descale_" + name]) >= 2**-6
        rel = np.abs(deq - ref)[normal] / np.abs(ref)[normal]
        assert rel.max() <= 2**-4 + 2**-7
