"""Plant plausible mistakes in the oracle (on the CPU, via monkeypatch) and
check that the pins catch each of them.  This shows that the pins constrain
the oracle and are not restatements of it."""

import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import oracle.attention as oa
import oracle.fp8 as of8

RNG = np.random.default_rng(99)
B, H, N, d = 1, 1, 6, 3
SCALE = 0.7


def _inputs():
    return tuple(RNG.standard_normal((B, H, N, d)) for _ in range(4))


def _pin_torch_sdpa(causal):
    q, k, v, _ = _inputs()
    O, _ = oracle.attention_forward(q, k, v, SCALE, causal)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        is_causal=causal, scale=SCALE).numpy()
    np.testing.assert_allclose(O, ref, rtol=1e-10, atol=1e-10)


def _pin_causal_row0():
    q, k, v, _ = _inputs()
    O, L = oracle.attention_forward(q, k, v, SCALE, True)
    np.testing.assert_allclose(O[0, 0, 0], v[0, 0, 0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(L[0, 0, 0], SCALE * q[0, 0, 0] @ k[0, 0, 0], rtol=1e-12)


def _pin_logsumexp():
    q, k, _, _ = _inputs()
    q = q * 30  # large logits: a dropped max shows up clearly
    _, L = oracle.attention_forward(q, k, np.zeros_like(q), SCALE, False)
    s = SCALE * q[0, 0] @ k[0, 0].T
    np.testing.assert_allclose(L[0, 0], scipy.special.logsumexp(s, axis=1), rtol=1e-12)


def _pin_finite_difference(causal):
    q, k, v, do = _inputs()
    dQ, dK, dV = oracle.attention_backward(q, k, v, do, SCALE, causal)
    h = 1e-6

    def loss(qq, kk):
        return float(np.sum(oracle.attention_forward(qq, kk, v, SCALE, causal)[0] * do))

    for x, g, is_q in ((q, dQ, True), (k, dK, False)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            fd[idx] = ((loss(xp, k) - loss(xm, k)) if is_q else
                       (loss(q, xp) - loss(q, xm))) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-5, atol=1e-7)


def _no_scale_scores(q, k, scale, causal, row_start=0):
    s = q @ k.T
    if causal:
        rows = np.arange(row_start, row_start + q.shape[0])[:, None]
        s = np.where(np.arange(k.shape[0])[None, :] > rows, -np.inf, s)
    return s


def _shifted_mask_scores(q, k, scale, causal, row_start=0):
    s = (q @ k.T) * scale
    if causal:
        rows = np.arange(row_start, row_start + q.shape[0])[:, None]
        s = np.where(np.arange(k.shape[0])[None, :] > rows + 1, -np.inf, s)
    return s


def _no_max_in_lse(s):
    m = np.max(s, axis=1)
    f = np.exp(s - m[:, None])
    ell = np.sum(f, axis=1)
    return np.zeros_like(m), ell, f / ell[:, None]


def _grad_sign_flip(p, dp):
    return p * dp + p * np.sum(p * dp, axis=1, keepdims=True)


def _grad_dropped_term(p, dp):
    return p * dp


def _grad_transposed(p, dp):
    return (p * dp - p * np.sum(p * dp, axis=1, keepdims=True)).T


def _e4m3_parts(codes):
    c = np.asarray(codes).astype(np.int64)
    return (c >> 7) & 1, (c >> 3) & 0xF, c & 7


def _decode_bias8(codes):  # the other FP8 variant's exponent bias
    s, e, m = _e4m3_parts(codes)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -7), np.ldexp(1.0 + m / 8.0, e - 8))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def _decode_subnormal_exp(codes):  # subnormals scaled by 2^-7 instead of 2^-6
    s, e, m = _e4m3_parts(codes)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -7), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def _decode_mantissa16(codes):  # mantissa step 1/16
    s, e, m = _e4m3_parts(codes)
    mag = np.where(e == 0, np.ldexp(m / 16.0, -6), np.ldexp(1.0 + m / 16.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def _decode_no_nan(codes):  # treats S.1111.111 as 480
    s, e, m = _e4m3_parts(codes)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    return np.where(s == 1, -mag, mag)


def _dequantize_ignores_descale(codes, descale):
    return of8.decode_e4m3(codes)


def _dequantize_squared(codes, descale):
    return of8.decode_e4m3(codes) * np.float64(np.float32(descale)) ** 2


def _pin_fp8_decode_torch():
    from tests.test_oracle_fp8 import test_decode_matches_torch_all_codes
    test_decode_matches_torch_all_codes()


def _pin_fp8_sdpa():
    from tests.test_oracle_fp8 import test_fp8_attention_matches_torch_sdpa
    test_fp8_attention_matches_torch_sdpa(True)


MUTATIONS_FP8 = [
    ("decode_e4m3", _decode_bias8, _pin_fp8_decode_torch),
    ("decode_e4m3", _decode_subnormal_exp, _pin_fp8_decode_torch),
    ("decode_e4m3", _decode_mantissa16, _pin_fp8_decode_torch),
    ("decode_e4m3", _decode_no_nan, _pin_fp8_decode_torch),
    ("decode_e4m3", _decode_bias8, _pin_fp8_sdpa),
    ("dequantize", _dequantize_ignores_descale, _pin_fp8_sdpa),
    ("dequantize", _dequantize_squared, _pin_fp8_sdpa),
]


def _keys_cut_to_queries(q, k, scale, causal, row_start=0, rows=None):
    # a slip that only shows when queries and keys differ in number: the
    # query count taken as the key count (keys past it masked out)
    s = _REAL_SCORES(q, k, scale, causal, row_start, rows)
    s[:, max(1, q.shape[0]):] = -np.inf
    return s


_REAL_SCORES = oa.scores


def _pin_unequal_lengths():
    from tests.test_oracle_forward import test_unequal_lengths_brute_force
    test_unequal_lengths_brute_force(1, 9, 4)


MUTATIONS = [
    ("scores", _keys_cut_to_queries, _pin_unequal_lengths),
    ("scores", _no_scale_scores, lambda: _pin_torch_sdpa(False)),
    ("scores", _shifted_mask_scores, _pin_causal_row0),
    ("softmax_rows", _no_max_in_lse, _pin_logsumexp),
    ("softmax_row_grad", _grad_sign_flip, lambda: _pin_finite_difference(False)),
    ("softmax_row_grad", _grad_dropped_term, lambda: _pin_finite_difference(True)),
    ("softmax_row_grad", _grad_transposed, lambda: _pin_finite_difference(False)),
]


@pytest.mark.parametrize("target,bad,pin", MUTATIONS,
                         ids=[m[1].__name__ for m in MUTATIONS])
def test_pin_catches_planted_mistake(monkeypatch, target, bad, pin):
    pin()  # the unmodified oracle passes the pin
    monkeypatch.setattr(oa, target, bad)
    with pytest.raises(AssertionError):
        pin()


@pytest.mark.parametrize("target,bad,pin", MUTATIONS_FP8,
                         ids=[f"{m[1].__name__}-{m[2].__name__}" for m in MUTATIONS_FP8])
def test_fp8_pin_catches_planted_mistake(monkeypatch, target, bad, pin):
    pin()
    monkeypatch.setattr(of8, target, bad)
    with pytest.raises(AssertionError):
        pin()


# ---------------------------------------------------------------- dropout
import oracle.dropout as odr


def _philox_swapped_multipliers(counter, key, width=32, rounds=10):
    M0, M1, W0, W1 = odr.PHILOX[width]
    mask = (1 << width) - 1
    x = [int(v) & mask for v in counter]
    k = [int(v) & mask for v in key]
    for _ in range(rounds):
        p0 = M1 * x[0]
        p1 = M0 * x[2]
        x = [((p1 >> width) ^ x[1] ^ k[0]) & mask, p1 & mask,
             ((p0 >> width) ^ x[3] ^ k[1]) & mask, p0 & mask]
        k = [(k[0] + W0) & mask, (k[1] + W1) & mask]
    return x


def _philox_seven_rounds(counter, key, width=32, rounds=10):
    return _REAL_PHILOX(counter, key, width, 7)


def _philox_key_bumped_first(counter, key, width=32, rounds=10):
    M0, M1, W0, W1 = odr.PHILOX[width]
    mask = (1 << width) - 1
    k = [(int(key[0]) + W0) & mask, (int(key[1]) + W1) & mask]
    return _REAL_PHILOX(counter, k, width, rounds)


_REAL_PHILOX = odr.philox
_REAL_BYTES = odr.dropout_bytes
_REAL_ARRAY = odr.philox4x32_10_array


def _bytes_big_endian(seed, offset, bh, rows, N):
    rows = np.asarray(rows, dtype=np.int64)
    ng = (N + 15) // 16
    jg = np.arange(ng, dtype=np.int64)
    w = odr.philox4x32_10_array(jg[None, :], rows[:, None], bh, offset,
                                seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    return w.astype(">u4").view(np.uint8).reshape(len(rows), ng * 16)[:, :N]


def _bytes_counter_swapped(seed, offset, bh, rows, N):
    rows = np.asarray(rows, dtype=np.int64)
    ng = (N + 15) // 16
    jg = np.arange(ng, dtype=np.int64)
    w = odr.philox4x32_10_array(rows[:, None], jg[None, :], bh, offset,
                                seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    return w.astype("<u4").view(np.uint8).reshape(len(rows), ng * 16)[:, :N]


def _mask_strict(seed, offset, bh, rows, N, p):
    return _REAL_BYTES(seed, offset, bh, rows, N) > odr.dropout_threshold(p)


def _scale_keep_rate_inverted(p):
    return (256 - odr.dropout_threshold(p)) / 256.0


def _backward_no_mask_in_dp(q, k, v, dout, scale, causal, p, seed, offset=0):
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    B, H, N, d = q.shape
    s = odr.dropout_scale(p)
    dQ, dK, dV = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    for b in range(B):
        for h in range(H):
            P = oa.softmax_rows(oa.scores(q[b, h], k[b, h], scale, causal))[2]
            Zs = odr.dropout_mask(seed, offset, b * H + h, np.arange(N), N, p) * s
            dV[b, h] = (P * Zs).T @ do[b, h]
            dS = oa.softmax_row_grad(P, do[b, h] @ v[b, h].T)
            dQ[b, h] = scale * (dS @ k[b, h])
            dK[b, h] = scale * (dS.T @ q[b, h])
    return dQ, dK, dV


def _pin_numpy_philox():
    from tests.test_oracle_dropout import test_philox4x64_matches_numpy
    test_philox4x64_matches_numpy([5, 0, 0, 0], [7, 9])


def _pin_layout():
    from tests.test_oracle_dropout import test_bytes_and_mask_layout
    test_bytes_and_mask_layout()


def _pin_brute(causal=True):
    from tests.test_oracle_dropout import test_forward_brute_force
    test_forward_brute_force(causal)


def _pin_stats():
    from tests.test_oracle_dropout import test_mask_statistics
    test_mask_statistics()


def _pin_autograd():
    from tests.test_oracle_dropout import test_backward_torch_autograd
    test_backward_torch_autograd(True)


MUTATIONS_DROPOUT = [
    ("philox", _philox_swapped_multipliers, _pin_numpy_philox),
    ("philox", _philox_seven_rounds, _pin_numpy_philox),
    ("philox", _philox_key_bumped_first, _pin_numpy_philox),
    ("dropout_bytes", _bytes_big_endian, _pin_layout),
    ("dropout_bytes", _bytes_counter_swapped, _pin_layout),
    ("dropout_bytes", _bytes_big_endian, _pin_brute),
    ("dropout_mask", _mask_strict, _pin_stats),
    ("dropout_scale", _scale_keep_rate_inverted, _pin_brute),
    ("attention_backward_dropout", _backward_no_mask_in_dp, _pin_autograd),
]


@pytest.mark.parametrize("target,bad,pin", MUTATIONS_DROPOUT,
                         ids=[f"{m[1].__name__}-{m[2].__name__}" for m in MUTATIONS_DROPOUT])
def test_dropout_pin_catches_planted_mistake(monkeypatch, target, bad, pin):
    pin()
    monkeypatch.setattr(odr, target, bad)
    if target == "attention_backward_dropout":
        monkeypatch.setattr(oracle, target, bad)
    with pytest.raises(AssertionError):
        pin()


# ---------------------------------------------------------------- incoherent processing
def _hadamard_other_sylvester(d):
    H = np.ones((1, 1))
    while H.shape[0] < d:
        H = np.block([[H, H], [-H, H]])
    return H


def _rotation_unnormalised(x, signs):
    return (np.asarray(x, dtype=np.float64) * np.asarray(signs, dtype=np.float64)) @ \
        of8.hadamard_matrix(np.asarray(x).shape[-1])


def _encode_ties_to_odd(x):
    pos = of8.decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    v = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(v), pos[-1])
    hi = np.clip(np.searchsorted(pos, a, side="left"), 0, len(pos) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - pos[lo], pos[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 1))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)


def _pin_hadamard_scipy():
    from tests.test_oracle_fp8 import test_hadamard_matches_scipy
    test_hadamard_matches_scipy(8)


def _pin_rotation():
    from tests.test_oracle_fp8 import test_rotation_is_orthogonal_and_keeps_scores
    test_rotation_is_orthogonal_and_keeps_scores()


def _pin_encoder():
    from tests.test_oracle_fp8 import test_encoder_matches_torch
    test_encoder_matches_torch()


MUTATIONS_ROT = [
    ("hadamard_matrix", _hadamard_other_sylvester, _pin_hadamard_scipy),
    ("incoherent_rotation", _rotation_unnormalised, _pin_rotation),
    ("encode_e4m3", _encode_ties_to_odd, _pin_encoder),
]


@pytest.mark.parametrize("target,bad,pin", MUTATIONS_ROT,
                         ids=[m[1].__name__ for m in MUTATIONS_ROT])
def test_rotation_pin_catches_planted_mistake(monkeypatch, target, bad, pin):
    pin()
    monkeypatch.setattr(of8, target, bad)
    with pytest.raises(AssertionError):
        pin()


# ---------------------------------------------------------------- sampled backward
def _sampled_variant(no_scale=False, no_row_term=False, overwrite=False):
    def f(q, k, v, dout, scale, causal, rows, keys, row_chunk=512):
        q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, dout))
        rows, keys = np.asarray(rows), np.asarray(keys)
        N, d = q.shape
        sc = 1.0 if no_scale else scale
        dQ = np.empty((len(rows), d))
        dK = np.zeros((len(keys), d))
        dV = np.zeros((len(keys), d))
        for r0 in range(0, N, row_chunk):
            p = oa.softmax_rows(oa.scores(q[r0:r0 + row_chunk], k, scale, causal, r0))[2]
            dp = do[r0:r0 + row_chunk] @ v.T
            ds = p * dp if no_row_term else oa.softmax_row_grad(p, dp)
            if overwrite:
                dV = p[:, keys].T @ do[r0:r0 + row_chunk]
            else:
                dV += p[:, keys].T @ do[r0:r0 + row_chunk]
            dK += sc * (ds[:, keys].T @ q[r0:r0 + row_chunk])
            for n, i in enumerate(rows):
                if r0 <= i < r0 + row_chunk:
                    dQ[n] = sc * (ds[i - r0] @ k)
        return dQ, dK, dV
    return f


def _pin_sampled():
    from tests.test_oracle_backward import test_sampled_backward_matches_torch_autograd
    test_sampled_backward_matches_torch_autograd(True)


MUTATIONS_SAMPLED = [
    ("dK and dQ without the scale", _sampled_variant(no_scale=True)),
    ("dS without the row term of the softmax Jacobian", _sampled_variant(no_row_term=True)),
    ("dV overwritten by each row chunk", _sampled_variant(overwrite=True)),
]


@pytest.mark.parametrize("name,bad", MUTATIONS_SAMPLED, ids=[m[0] for m in MUTATIONS_SAMPLED])
def test_sampled_backward_pin_catches_planted_mistake(monkeypatch, name, bad):
    _pin_sampled()
    monkeypatch.setattr(oracle, "attention_backward_sampled", bad)
    with pytest.raises(AssertionError):
        _pin_sampled()


# ---------------------------------------------------------------- bf16 widening, Philox4x32
def _widen_byteswapped(bits):
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError(b.dtype)
    return (b.byteswap().astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _widen_low_half(bits):
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError(b.dtype)
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def _pin_widen_torch():
    from tests.test_oracle_forward import test_widen_bf16_matches_torch_on_every_pattern
    test_widen_bf16_matches_torch_on_every_pattern()


def _philox32_swapped_multiplier(counter, key, width=32, rounds=10):
    # only the 32-bit multipliers exchanged (numpy's 4x64 pin cannot see this)
    if width != 32:
        return _REAL_PHILOX(counter, key, width, rounds)
    return _philox_swapped_multipliers(counter, key, width, rounds)


def _pin_rocrand_philox():
    from tests.test_oracle_dropout import test_philox4x32_matches_rocrand
    test_philox4x32_matches_rocrand()


MUTATIONS_BITS = [
    (oa, "widen_bf16", _widen_byteswapped, _pin_widen_torch),
    (oa, "widen_bf16", _widen_low_half, _pin_widen_torch),
    (odr, "philox", _philox32_swapped_multiplier, _pin_rocrand_philox),
    (odr, "philox", _philox_seven_rounds, _pin_rocrand_philox),
]


@pytest.mark.parametrize("mod,target,bad,pin", MUTATIONS_BITS,
                         ids=[f"{m[2].__name__}-{m[3].__name__}" for m in MUTATIONS_BITS])
def test_bits_pin_catches_planted_mistake(monkeypatch, mod, target, bad, pin):
    pin()
    monkeypatch.setattr(mod, target, bad)
    if hasattr(oracle, target):
        monkeypatch.setattr(oracle, target, bad)
    with pytest.raises(AssertionError):
        with np.errstate(all="ignore"):
            pin()
