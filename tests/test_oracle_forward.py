"""Pins of the oracle's forward pass (O, LSE, P) to things other than itself.

Each check is chosen so that a plausible slip in ``oracle.attention`` (a
missing scale, a shifted mask, a transposed operand, a dropped max in LSE)
fails at least one of them; ``test_oracle_mutations.py`` plants such slips
and confirms it.
"""

import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from exact_attention_flash_amd.inputs import make_inputs

RNG = np.random.default_rng(12345)


def _rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def _brute_head(q, k, v, scale, causal):
    """Per-element sums in pure Python (math.fsum), no max subtraction.

    O_ic = sum_j exp(s_ij) v_jc / sum_j exp(s_ij) over visible j, with
    s_ij = scale * sum_t q_it k_jt.  Only for tiny, well-scaled inputs.
    """
    N, d = len(q), len(q[0])
    O = [[0.0] * len(v[0]) for _ in range(N)]
    lse = [0.0] * N
    for i in range(N):
        vis = range(i + 1) if causal else range(N)
        w = {j: math.exp(scale * math.fsum(q[i][t] * k[j][t] for t in range(d)))
             for j in vis}
        den = math.fsum(w.values())
        for c in range(len(v[0])):
            O[i][c] = math.fsum(w[j] * v[j][c] for j in vis) / den
        lse[i] = math.log(den)
    return np.array(O), np.array(lse)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 1), (2, 3), (5, 4), (8, 2)])
def test_brute_force_tiny(N, d, causal):
    q, k, v = _rand(1, 2, N, d), _rand(1, 2, N, d), _rand(1, 2, N, d)
    scale = 0.7
    O, L = oracle.attention_forward(q, k, v, scale, causal)
    for h in range(2):
        Ob, Lb = _brute_head(q[0, h].tolist(), k[0, h].tolist(),
                             v[0, h].tolist(), scale, causal)
        np.testing.assert_allclose(O[0, h], Ob, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(L[0, h], Lb, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_torch_sdpa_fp64_cpu(causal):
    """Library special case: PyTorch's scaled_dot_product_attention (the
    routine the apxml page calls), run in float64 on the CPU."""
    B, H, N, d = 2, 3, 37, 16
    q, k, v = _rand(B, H, N, d), _rand(B, H, N, d), _rand(B, H, N, d)
    scale = 1 / math.sqrt(d)
    O, _ = oracle.attention_forward(q, k, v, scale, causal)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        is_causal=causal, scale=scale)
    np.testing.assert_allclose(O, ref.numpy(), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- queries != keys (decode)
def _brute_head_lengths(q, k, v, scale):
    """Full attention of len(q) queries over len(k) keys, per element in pure
    Python (math.fsum), no max subtraction."""
    d = len(q[0])
    O, lse = [], []
    for qi in q:
        w = [math.exp(scale * math.fsum(qi[t] * kj[t] for t in range(d))) for kj in k]
        den = math.fsum(w)
        O.append([math.fsum(w[j] * v[j][c] for j in range(len(k))) / den
                  for c in range(len(v[0]))])
        lse.append(math.log(den))
    return np.array(O), np.array(lse)


@pytest.mark.parametrize("Nq,Nk,d", [(1, 1, 3), (1, 9, 4), (3, 7, 2), (6, 2, 3)])
def test_unequal_lengths_brute_force(Nq, Nk, d):
    """A decode step (one query, or a few, against every cached key) and the
    reverse: against per-element sums."""
    q, k, v = _rand(1, 2, Nq, d), _rand(1, 2, Nk, d), _rand(1, 2, Nk, d)
    O, L = oracle.attention_forward(q, k, v, 0.6, False)
    assert O.shape == (1, 2, Nq, d) and L.shape == (1, 2, Nq)
    for h in range(2):
        Ob, Lb = _brute_head_lengths(q[0, h].tolist(), k[0, h].tolist(), v[0, h].tolist(), 0.6)
        np.testing.assert_allclose(O[0, h], Ob, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(L[0, h], Lb, rtol=1e-12, atol=1e-13)


def test_unequal_lengths_torch_sdpa_and_closed_form():
    """torch's fp64 SDPA with queries and keys of different lengths (the
    apxml example's interface), and the closed form for Q = 0: every query
    takes the mean of all N_kv values and LSE = ln N_kv."""
    B, H, Nq, Nk, d = 2, 3, 5, 41, 16
    q, k, v = _rand(B, H, Nq, d), _rand(B, H, Nk, d), _rand(B, H, Nk, d)
    O, _ = oracle.attention_forward(q, k, v, 0.25, False)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=0.25)
    np.testing.assert_allclose(O, ref.numpy(), rtol=1e-12, atol=1e-12)
    O0, L0 = oracle.attention_forward(np.zeros_like(q), k, v, 0.25, False)
    np.testing.assert_allclose(O0, np.broadcast_to(v.mean(axis=2, keepdims=True), O0.shape),
                               rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(L0, np.log(Nk), rtol=1e-15)
    rows = np.array([4, 0, 2])
    Or, Lr = oracle.attention_forward_rows(q[1, 2], k[1, 2], v[1, 2], 0.25, False, rows)
    np.testing.assert_allclose(Or, O[1, 2, rows], rtol=1e-14, atol=1e-14)
    with pytest.raises(ValueError):
        oracle.attention_forward(q, k, v, 0.25, True)   # causal needs equal lengths
    with pytest.raises(ValueError):
        oracle.attention_forward(q, k, v[:, :, :-1], 0.25, False)


@pytest.mark.parametrize("causal", [False, True])
def test_scipy_softmax_and_logsumexp(causal):
    N, d = 23, 8
    q, k = _rand(1, 1, N, d), _rand(1, 1, N, d)
    scale = 0.3
    s = scale * (q[0, 0] @ k[0, 0].T)
    if causal:
        s = np.where(np.tri(N, dtype=bool), s, -np.inf)
    P = oracle.attention_probs(q, k, scale, causal)[0, 0]
    np.testing.assert_allclose(P, scipy.special.softmax(s, axis=1), rtol=1e-13, atol=1e-15)
    _, L = oracle.attention_forward(q, k, np.zeros_like(q), scale, causal)
    np.testing.assert_allclose(L[0, 0], scipy.special.logsumexp(s, axis=1), rtol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_q_closed_form(causal):
    """Q = 0: every visible score is 0, so O_i is the mean of the visible V
    rows and LSE_i = ln(number of visible keys): ln N, or ln(i + 1) causal."""
    N, d = 19, 5
    v = _rand(1, 1, N, d)
    q = np.zeros((1, 1, N, d))
    O, L = oracle.attention_forward(q, _rand(1, 1, N, d), v, 0.5, causal)
    counts = np.arange(1, N + 1) if causal else np.full(N, N)
    means = np.cumsum(v[0, 0], axis=0) / counts[:, None] if causal \
        else np.broadcast_to(v[0, 0].mean(axis=0), (N, d))
    np.testing.assert_allclose(O[0, 0], means, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(L[0, 0], np.log(counts), rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_and_causal_row0(causal):
    N, d = 17, 6
    q, k = _rand(1, 1, N, d, scale=3.0), _rand(1, 1, N, d)
    row = _rand(d)
    v = np.broadcast_to(row, (1, 1, N, d)).copy()
    O, L = oracle.attention_forward(q, k, v, 0.4, causal)
    np.testing.assert_allclose(O[0, 0], np.broadcast_to(row, (N, d)), rtol=1e-13, atol=1e-14)
    if causal:
        v2 = _rand(1, 1, N, d)
        O2, L2 = oracle.attention_forward(q, k, v2, 0.4, True)
        assert np.array_equal(O2[0, 0, 0], v2[0, 0, 0]) or \
            np.allclose(O2[0, 0, 0], v2[0, 0, 0], rtol=1e-15, atol=1e-15)
        np.testing.assert_allclose(L2[0, 0, 0], 0.4 * q[0, 0, 0] @ k[0, 0, 0], rtol=1e-14)


def test_rows_sum_to_one_and_mask_zeros():
    N, d = 29, 7
    q, k = _rand(2, 2, N, d, scale=2.0), _rand(2, 2, N, d)
    for causal in (False, True):
        P = oracle.attention_probs(q, k, 0.9, causal)
        np.testing.assert_allclose(P.sum(-1), 1.0, rtol=0, atol=1e-14)
        if causal:
            upper = np.triu(np.ones((N, N), dtype=bool), 1)
            assert np.all(P[..., upper] == 0.0)
            assert np.all(P[..., ~upper] > 0.0)


def test_permutation_equivariance():
    N, d = 21, 4
    q, k, v = _rand(1, 1, N, d), _rand(1, 1, N, d), _rand(1, 1, N, d)
    O, L = oracle.attention_forward(q, k, v, 0.6, False)
    perm = RNG.permutation(N)
    O2, L2 = oracle.attention_forward(q, k[:, :, perm], v[:, :, perm], 0.6, False)
    np.testing.assert_allclose(O2, O, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(L2, L, rtol=1e-13)
    O3, L3 = oracle.attention_forward(q[:, :, perm], k, v, 0.6, False)
    np.testing.assert_allclose(O3, O[:, :, perm], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(L3, L[:, :, perm], rtol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_row_shift_invariance(causal):
    """Adding u to every key adds scale*q_i.u to row i of S: P and O do not
    change and LSE_i moves by exactly that amount."""
    N, d = 15, 6
    q, k, v = _rand(1, 1, N, d), _rand(1, 1, N, d), _rand(1, 1, N, d)
    u = _rand(d, scale=4.0)
    scale = 0.8
    O, L = oracle.attention_forward(q, k, v, scale, causal)
    O2, L2 = oracle.attention_forward(q, k + u, v, scale, causal)
    np.testing.assert_allclose(O2, O, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(L2[0, 0], L[0, 0] + scale * (q[0, 0] @ u), rtol=1e-12, atol=1e-12)


def test_large_logits_do_not_overflow():
    """Scores far above exp's float64 range (~709) still give finite
    results: the row maximum is subtracted first (CMU notes, safe softmax)."""
    N, d = 9, 4
    q, k, v = _rand(1, 1, N, d, scale=400.0), _rand(1, 1, N, d), _rand(1, 1, N, d)
    O, L = oracle.attention_forward(q, k, v, 1.0, False)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    s = q[0, 0] @ k[0, 0].T
    np.testing.assert_allclose(L[0, 0], scipy.special.logsumexp(s, axis=1), rtol=1e-13)


def test_row_chunking_is_exact():
    N, d = 70, 8
    q, k, v = _rand(1, 2, N, d), _rand(1, 2, N, d), _rand(1, 2, N, d)
    for causal in (False, True):
        O, L = oracle.attention_forward(q, k, v, 0.35, causal)
        Oc, Lc = oracle.attention_forward(q, k, v, 0.35, causal, row_chunk=16)
        assert np.array_equal(O, Oc) and np.array_equal(L, Lc)


def test_bf16_bits_are_widened_exactly():
    x = make_inputs(1, 1, 4, 8, seed=1)
    w = oracle.widen_bf16(x["q"])
    assert w.dtype == np.float64
    # round trip: the float32 of the widened value has zero low half
    assert np.all((w.astype(np.float32).view(np.uint32) & 0xFFFF) == 0)
    O_bits, _ = oracle.attention_forward(x["q"], x["k"], x["v"], 0.125, True)
    O_f, _ = oracle.attention_forward(w, oracle.widen_bf16(x["k"]),
                                      oracle.widen_bf16(x["v"]), 0.125, True)
    assert np.array_equal(O_bits, O_f)
    with pytest.raises(TypeError):
        oracle.widen_bf16(np.zeros(3, dtype=np.int16))


def test_widen_bf16_matches_torch_on_every_pattern():
    """All 65536 bf16 bit patterns widen to the value torch's own bfloat16 ->
    float64 conversion gives (a library routine): same value, same sign of
    zero, NaN exactly where torch has NaN, infinities included."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):  # signalling NaN patterns
        ours = oracle.widen_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert int(nan.sum()) == 2 * 127  # exponent all ones, non-zero mantissa, both signs
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    assert np.isposinf(ours[0x7F80]) and np.isneginf(ours[0xFF80])


@pytest.mark.parametrize("causal", [False, True])
def test_selected_rows_match_whole_head(causal):
    N, d = 40, 8
    q, k, v = _rand(1, 1, N, d), _rand(1, 1, N, d), _rand(1, 1, N, d)
    O, L = oracle.attention_forward(q, k, v, 0.45, causal)
    rows = np.array([0, 39, 7, 8, 20, 1])
    Or, Lr = oracle.attention_forward_rows(q[0, 0], k[0, 0], v[0, 0], 0.45, causal, rows)
    assert np.array_equal(Or, O[0, 0, rows]) or np.allclose(Or, O[0, 0, rows], rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(Lr, L[0, 0, rows], rtol=1e-15, atol=1e-15)
