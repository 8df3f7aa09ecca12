"""The pages' two-block merge identities, and the blockwise FlashAttention-2
loop in float64 against the direct definition."""

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from hypothesis.extra import numpy as hnp

import oracle

finite = st.floats(min_value=-50, max_value=50, allow_nan=False, allow_infinity=False)


@settings(max_examples=200, deadline=None)
@given(x=hnp.arrays(np.float64, st.integers(2, 40), elements=finite),
       cut=st.floats(0.0, 1.0))
def test_merge_matches_whole_vector(x, cut):
    k = min(max(1, int(cut * len(x))), len(x) - 1)
    m, f, ell = oracle.merge_stats(oracle.softmax_stats(x[:k]), oracle.softmax_stats(x[k:]))
    mw, fw, lw = oracle.softmax_stats(x)
    assert m == mw  # the max merges exactly
    # each exponent argument is rounded once per subtraction; with
    # |x - m| <= 100 that is a few 1e-14 relative, hence 1e-13
    np.testing.assert_allclose(f, fw, rtol=1e-13, atol=0)
    np.testing.assert_allclose(ell, lw, rtol=1e-13)
    np.testing.assert_allclose(f / ell, np.exp(x - x.max()) / np.exp(x - x.max()).sum(), rtol=1e-13)


@settings(max_examples=100, deadline=None)
@given(x=hnp.arrays(np.float64, st.integers(1, 60), elements=finite),
       sizes=st.lists(st.integers(1, 9), min_size=1, max_size=12))
def test_left_fold_from_initial_values(x, sizes):
    """Starting from m = -inf, l = 0 and folding block by block gives the
    whole-row statistics; the first step alone is the plain softmax of the
    first block."""
    pieces, i = [], 0
    for s in sizes:
        if i >= len(x):
            break
        pieces.append(x[i:i + s])
        i += s
    if i < len(x):
        pieces.append(x[i:])
    m, f, ell = oracle.fold_blocks(pieces)
    mw, fw, lw = oracle.softmax_stats(x)
    assert m == mw
    np.testing.assert_allclose(ell, lw, rtol=1e-13)
    np.testing.assert_allclose(f, fw, rtol=1e-13, atol=0)
    m1, f1, l1 = oracle.fold_blocks(pieces[:1])
    assert m1 == pieces[0].max()
    np.testing.assert_allclose(f1 / l1, np.exp(pieces[0] - m1) / np.exp(pieces[0] - m1).sum(),
                               rtol=1e-14)


def test_masked_pieces():
    """A piece whose entries are all -inf (a fully masked block) contributes
    nothing, in any position."""
    x = np.array([0.5, -1.0, 2.0])
    blank = np.full(4, -np.inf)
    for pieces in ([blank, x], [x, blank], [x[:1], blank, x[1:]]):
        m, f, ell = oracle.fold_blocks(pieces)
        assert m == 2.0
        np.testing.assert_allclose(ell, np.exp(x - 2.0).sum(), rtol=1e-15)
        assert np.count_nonzero(f) == 3
    m, f, ell = oracle.fold_blocks([blank])
    assert m == -np.inf and ell == 0.0


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,br,bc", [(64, 16, 16), (70, 16, 32), (33, 8, 5), (1, 4, 4), (100, 128, 64)])
def test_blockwise_forward_equals_definition(N, br, bc, causal):
    rng = np.random.default_rng(N * 31 + br)
    d = 8
    q, k, v = (rng.standard_normal((N, d)) * 2 for _ in range(3))
    O, L = oracle.blockwise_forward_head(q, k, v, 0.4, causal, br, bc)
    Od, Ld = oracle.attention_forward(q[None, None], k[None, None], v[None, None], 0.4, causal)
    np.testing.assert_allclose(O, Od[0, 0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(L, Ld[0, 0], rtol=1e-12, atol=1e-13)
