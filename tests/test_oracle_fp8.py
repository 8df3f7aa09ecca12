"""Pins of the FP8 (E4M3) oracle to things other than itself.

* the decoder against torch's ``float8_e4m3fn`` conversion (a library
  routine) over all 256 codes, and against values the OCP E4M3 definition
  fixes in closed form;
* the FP8 attention against torch's scaled-dot-product attention in float64
  on torch-decoded inputs, with the descales folded in another way (into the
  softmax scale and onto the output);
* closed-form descale identities.
``test_oracle_mutations.py`` plants slips in the decoder (wrong bias, wrong
subnormal exponent, the other FP8 variant) and shows these pins catch them.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as of8
from exact_attention_flash_amd.inputs import make_inputs_fp8

ALL_CODES = np.arange(256, dtype=np.uint8)


def _torch_decode(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def test_decode_matches_torch_all_codes():
    got = of8.decode_e4m3(ALL_CODES)
    ref = _torch_decode(ALL_CODES)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))


def test_decode_closed_form_values():
    d = of8.decode_e4m3
    c = lambda x: np.array([x], dtype=np.uint8)
    assert d(c(0x38))[0] == 1.0            # exponent field 7 = bias
    assert d(c(0x40))[0] == 2.0 and d(c(0xC0))[0] == -2.0
    assert d(c(0x39))[0] == 1.125          # one mantissa step is 1/8
    assert d(c(0x7E))[0] == 448.0          # largest finite value
    assert d(c(0x08))[0] == 2.0 ** -6      # smallest normal
    assert d(c(0x01))[0] == 2.0 ** -9      # smallest subnormal
    assert d(c(0x07))[0] == 7 * 2.0 ** -9  # largest subnormal
    assert d(c(0x80))[0] == 0.0 and np.signbit(d(c(0x80))[0])
    assert np.isnan(d(c(0x7F))[0]) and np.isnan(d(c(0xFF))[0])
    assert d(c(0x77))[0] == 240.0 and d(c(0x6C))[0] == 96.0
    with pytest.raises(TypeError):
        d(np.zeros(3, dtype=np.int32))


def test_decode_monotone_and_symmetric():
    pos = of8.decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)        # codes 0..0x7E increase strictly
    neg = of8.decode_e4m3(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(neg, -pos)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_attention_matches_torch_sdpa(causal):
    x = make_inputs_fp8(2, 3, 37, 16, seed=11)
    scale = 0.25
    O, L = oracle.attention_forward_fp8(x["q"], x["k"], x["v"], x["descale_q"],
                                        x["descale_k"], x["descale_v"], scale, causal)
    q = torch.from_numpy(_torch_decode(x["q"]))
    k = torch.from_numpy(_torch_decode(x["k"]))
    v = torch.from_numpy(_torch_decode(x["v"]))
    # descales folded into the softmax scale and onto the output instead
    eff = float(np.float32(x["descale_q"])) * float(np.float32(x["descale_k"])) * scale
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=eff)
    ref = ref.numpy() * float(np.float32(x["descale_v"]))
    np.testing.assert_allclose(O, ref, rtol=1e-11, atol=1e-12)
    s = eff * (q @ k.transpose(-1, -2))
    if causal:
        s = s.masked_fill(torch.ones(37, 37, dtype=torch.bool).triu(1), -math.inf)
    np.testing.assert_allclose(L, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


def test_descale_identities():
    x = make_inputs_fp8(1, 2, 20, 8, seed=5)
    args = (x["q"], x["k"], x["v"])
    O, L = oracle.attention_forward_fp8(*args, 0.5, 0.25, 0.75, 0.3, True)
    # doubling the V descale doubles O and leaves LSE
    O2, L2 = oracle.attention_forward_fp8(*args, 0.5, 0.25, 1.5, 0.3, True)
    np.testing.assert_allclose(O2, 2 * O, rtol=1e-14)
    np.testing.assert_array_equal(L2, L)
    # only the product descale_q * descale_k * scale enters the scores
    O3, L3 = oracle.attention_forward_fp8(*args, 0.25, 0.5, 0.75, 0.3, True)
    np.testing.assert_allclose(O3, O, rtol=1e-14)
    np.testing.assert_allclose(L3, L, rtol=1e-14)
    O4, L4 = oracle.attention_forward_fp8(*args, 1.0, 0.25, 0.75, 0.15, True)
    np.testing.assert_allclose(O4, O, rtol=1e-14)
    np.testing.assert_allclose(L4, L, rtol=1e-14)


def test_rows_variant_matches_whole_head():
    x = make_inputs_fp8(1, 1, 50, 16, seed=8)
    O, L = oracle.attention_forward_fp8(x["q"], x["k"], x["v"], x["descale_q"],
                                        x["descale_k"], x["descale_v"], 0.25, True)
    rows = [0, 7, 49]
    Or, Lr = oracle.attention_forward_fp8_rows(x["q"][0, 0], x["k"][0, 0], x["v"][0, 0],
                                               x["descale_q"], x["descale_k"], x["descale_v"],
                                               0.25, True, rows)
    np.testing.assert_allclose(Or, O[0, 0, rows], rtol=1e-13)
    np.testing.assert_allclose(Lr, L[0, 0, rows], rtol=1e-13)


# ---------------------------------------------------------------- incoherent processing
import scipy.linalg


@pytest.mark.parametrize("d", [1, 2, 8, 64, 128])
def test_hadamard_matches_scipy(d):
    assert np.array_equal(of8.hadamard_matrix(d), scipy.linalg.hadamard(d))


def test_rotation_is_orthogonal_and_keeps_scores():
    rng = np.random.default_rng(3)
    for d in (64, 128):
        signs = rng.choice([-1.0, 1.0], d)
        M = of8.incoherent_rotation(np.eye(d), signs)
        np.testing.assert_allclose(M @ M.T, np.eye(d), atol=1e-14)
        q, k = rng.standard_normal((50, d)), rng.standard_normal((40, d))
        qr, kr = of8.incoherent_rotation(q, signs), of8.incoherent_rotation(k, signs)
        np.testing.assert_allclose(qr @ kr.T, q @ k.T, rtol=1e-12, atol=1e-12)
    # spreads a spike: a unit vector becomes +-1/sqrt(d) everywhere
    e = np.zeros(64)
    e[5] = 1.0
    np.testing.assert_allclose(np.abs(of8.incoherent_rotation(e, np.ones(64))), 1 / 8)


def test_encoder_matches_torch():
    vals = _torch_decode(ALL_CODES)
    fin = np.unique(vals[np.isfinite(vals)])
    mids = (fin[1:] + fin[:-1]) / 2
    rng = np.random.default_rng(4)
    x = np.concatenate([fin, mids, -mids, rng.standard_normal(5000) * 30,
                        rng.standard_normal(5000) * 1e-3])
    x = np.clip(x, -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(of8.encode_e4m3(x), ref)
    assert of8.encode_e4m3(np.array([1e6, -1e6])).tolist() == [0x7E, 0xFE]   # saturates


def test_quantize_roundtrip():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((300, 64))
    for signs in (None, rng.choice([-1.0, 1.0], 64)):
        codes, ds = of8.quantize_e4m3(x, signs)
        y = x if signs is None else of8.incoherent_rotation(x, signs)
        back = of8.decode_e4m3(codes) * ds
        assert np.max(np.abs(of8.decode_e4m3(codes))) == 448.0          # amax at the top
        normal = np.abs(y / ds) >= 2 ** -6
        assert np.max(np.abs(back - y)[normal] / np.abs(y)[normal]) <= 2 ** -4 * (1 + 1e-6)


def test_rotation_lowers_quantisation_error_with_outliers():
    """The pages' claim, on the oracle: with a few large channels in Q and K,
    quantising after the rotation gives a much smaller score error."""
    rng = np.random.default_rng(6)
    d, N = 128, 256
    q, k = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    q[:, :4] *= 30
    k[:, :4] *= 30
    ref = q @ k.T
    signs = rng.choice([-1.0, 1.0], d)
    err = {}
    for name, s in (("plain", None), ("rotated", signs)):
        cq, dq = of8.quantize_e4m3(q, s)
        ck, dk = of8.quantize_e4m3(k, s)
        sc = (of8.decode_e4m3(cq) * dq) @ (of8.decode_e4m3(ck) * dk).T
        err[name] = np.sqrt(np.mean((sc - ref) ** 2))
    assert err["rotated"] < 0.5 * err["plain"], err
