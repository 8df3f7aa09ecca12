"""Pins of the oracle's backward pass: finite differences, autograd through a
library routine, and identities the gradient must satisfy."""

import math

import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(777)


def _rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def _loss(q, k, v, do, scale, causal):
    O, _ = oracle.attention_forward(q, k, v, scale, causal)
    return float(np.sum(O * do))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 2), (4, 3), (6, 4)])
def test_central_finite_differences(N, d, causal):
    """dQ, dK, dV against central differences of L = sum(dO * O)."""
    scale = 0.7
    q, k, v, do = (_rand(1, 1, N, d) for _ in range(4))
    dQ, dK, dV = oracle.attention_backward(q, k, v, do, scale, causal)
    h = 1e-6
    for name, x, g in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], do, scale, causal)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], do, scale, causal)
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_torch_autograd_fp64_cpu(causal):
    B, H, N, d = 1, 2, 33, 8
    scale = 1 / math.sqrt(d)
    q, k, v, do = (_rand(B, H, N, d) for _ in range(4))
    dQ, dK, dV = oracle.attention_backward(q, k, v, do, scale, causal)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=causal, scale=scale)
    out.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dQ, tq.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dK, tk.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dV, tv.grad.numpy(), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_identities(causal):
    N, d = 24, 6
    scale = 0.5
    q, k, v, do = (_rand(1, 1, N, d) for _ in range(4))
    dQ, dK, dV, it = oracle.attention_backward(q, k, v, do, scale, causal,
                                               return_intermediates=True)
    P, dS = it["P"][0, 0], it["dS"][0, 0]
    # softmax rows sum to one, so the row gradients sum to zero
    np.testing.assert_allclose(dS.sum(axis=1), 0.0, atol=1e-13)
    # dV = P^T dO and rows of P sum to one => column sums of dV equal those of dO
    np.testing.assert_allclose(dV[0, 0].sum(axis=0), do[0, 0].sum(axis=0), rtol=1e-12, atol=1e-12)
    # the rowsum(dO o O) term: sum_j P_ij dP_ij equals dO_i . O_i
    O, _ = oracle.attention_forward(q, k, v, scale, causal)
    dP = do[0, 0] @ v[0, 0].T
    np.testing.assert_allclose((P * dP).sum(axis=1), (do[0, 0] * O[0, 0]).sum(axis=1),
                               rtol=1e-11, atol=1e-12)
    # dS written with that term: P o (dP - D)
    D = (do[0, 0] * O[0, 0]).sum(axis=1)
    np.testing.assert_allclose(dS, P * (dP - D[:, None]), rtol=1e-10, atol=1e-12)
    if causal:
        # row 0 only sees key 0, P_00 = 1 whatever Q is: dQ_0 = 0
        np.testing.assert_allclose(dQ[0, 0, 0], 0.0, atol=1e-15)
        # the last key is seen only by the last query
        np.testing.assert_allclose(dK[0, 0, -1], scale * dS[-1, -1] * q[0, 0, -1], rtol=1e-12)


def test_constant_v_gives_zero_dq_dk():
    N, d = 12, 5
    q, k, do = _rand(1, 1, N, d), _rand(1, 1, N, d), _rand(1, 1, N, d)
    v = np.broadcast_to(_rand(d), (1, 1, N, d)).copy()
    for causal in (False, True):
        dQ, dK, _ = oracle.attention_backward(q, k, v, do, 0.9, causal)
        np.testing.assert_allclose(dQ, 0.0, atol=1e-13)
        np.testing.assert_allclose(dK, 0.0, atol=1e-13)


def test_scale_enters_dq_dk_only():
    """Scaling Q by c and the softmax scale by 1/c leaves S unchanged: O and
    dV are unchanged, dQ shrinks by 1/c and dK is unchanged."""
    N, d, c = 10, 4, 4.0
    q, k, v, do = (_rand(1, 1, N, d) for _ in range(4))
    dQ, dK, dV = oracle.attention_backward(q, k, v, do, 0.8, True)
    dQ2, dK2, dV2 = oracle.attention_backward(c * q, k, v, do, 0.8 / c, True)
    np.testing.assert_allclose(dV2, dV, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dK2, dK, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dQ2, dQ / c, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_backward_matches_torch_autograd(causal):
    """The row-chunked backward for a subset of rows and keys (used where a
    whole N x N head would not fit) against torch fp64 autograd on the CPU,
    a library routine, with chunks that split the head unevenly."""
    rng = np.random.default_rng(11 + causal)
    N, d = 37, 8
    q, k, v, do = (rng.standard_normal((N, d)) for _ in range(4))
    scale = 0.3
    rows = np.array([0, 5, 17, 36])
    keys = np.array([0, 1, 20, 36])
    dQ, dK, dV = oracle.attention_backward_sampled(q, k, v, do, scale, causal, rows, keys,
                                                   row_chunk=10)
    qt, kt, vt = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    mask = torch.triu(torch.ones(N, N, dtype=torch.bool), 1) if causal else None
    o = torch.nn.functional.scaled_dot_product_attention(
        qt[None, None], kt[None, None], vt[None, None],
        attn_mask=None if mask is None else ~mask, scale=scale)[0, 0]
    o.backward(torch.tensor(do))
    np.testing.assert_allclose(dQ, qt.grad.numpy()[rows], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dK, kt.grad.numpy()[keys], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dV, vt.grad.numpy()[keys], rtol=1e-10, atol=1e-12)


def test_sampled_backward_equals_whole_head():
    """On a head small enough for the whole-head backward, the sampled one
    gives the same rows and keys for every chunk size, including chunks of
    one row and a single chunk."""
    rng = np.random.default_rng(5)
    N, d = 50, 16
    q, k, v, do = (rng.standard_normal((1, 1, N, d)) for _ in range(4))
    dQ, dK, dV = oracle.attention_backward(q, k, v, do, 0.25, True)
    rows = np.arange(0, N, 7)
    keys = np.arange(3, N, 9)
    for chunk in (1, 7, 50, 64):
        sQ, sK, sV = oracle.attention_backward_sampled(q[0, 0], k[0, 0], v[0, 0], do[0, 0], 0.25,
                                                       True, rows, keys, row_chunk=chunk)
        np.testing.assert_allclose(sQ, dQ[0, 0, rows], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(sK, dK[0, 0, keys], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(sV, dV[0, 0, keys], rtol=1e-12, atol=1e-13)
