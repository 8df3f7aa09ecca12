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


MUTATIONS = [
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
