"""The pages' softmax decomposition, in float64, as checkable functions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Transformer、注意力机制与优化" (CMU 15-442/642 notes), section
"安全 Softmax 与在线 Softmax", defines for a vector x

    m(x) = max_i x_i,   f(x) = [exp(x_i - m(x))]_i,   l(x) = sum_i f(x)_i,

and, for x split into two pieces x1, x2, gives the merge

    m(x) = max(m(x1), m(x2)),
    f(x) = [exp(m(x1) - m(x)) f(x1), exp(m(x2) - m(x)) f(x2)],
    l(x) = exp(m(x1) - m(x)) l(x1) + exp(m(x2) - m(x)) l(x2).

The same notes' section "FlashAttention-2 算法" outline the forward pass that
the kernel follows: split Q into row blocks and K, V into column blocks; for
each Q block start from O = 0, l = 0, m = -inf ("FlashAttention 的基本原理",
section 2.3, explains that with these starting values the first update is the
plain softmax of the first block), update the statistics block by block with
the merge rule, accumulate the unnormalised partial output, and write O back
once.  "FlashAttention 系列技术详解", section "具体优化策略", adds that the
division by l happens once, at the end, and that only the log-sum-exp is kept.

``blockwise_forward_head`` is that procedure in float64.  It is not the parity
oracle (``attention.attention_forward`` is); the tests use it to pin the
decomposition against the direct definition.
"""

from __future__ import annotations

import math

import numpy as np


def softmax_stats(x: np.ndarray):
    """(m(x), f(x), l(x)) of a 1-D vector, as defined in the CMU notes."""
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x)
    if m == -np.inf:  # every entry masked: nothing contributes
        f = np.zeros_like(x)
    else:
        f = np.exp(x - m)
    return m, f, float(np.sum(f))


def _rescale(m_part: float, m_all: float) -> float:
    """exp(m_part - m_all), taking exp(-inf - (-inf)) as 0 (empty part)."""
    if m_part == -np.inf:
        return 0.0
    return math.exp(m_part - m_all)


def merge_stats(s1, s2):
    """Two-block merge of (m, f, l) triples, the CMU notes' merge equations."""
    m1, f1, l1 = s1
    m2, f2, l2 = s2
    m = max(m1, m2)
    a1, a2 = _rescale(m1, m), _rescale(m2, m)
    f = np.concatenate([a1 * np.asarray(f1), a2 * np.asarray(f2)])
    return m, f, a1 * l1 + a2 * l2


def fold_blocks(blocks):
    """Left fold of ``merge_stats`` over vector pieces, from m=-inf, l=0, f=[]."""
    acc = (-np.inf, np.zeros(0), 0.0)
    for piece in blocks:
        acc = merge_stats(acc, softmax_stats(piece))
    return acc


def blockwise_forward_head(q, k, v, scale: float, causal: bool,
                           br: int, bc: int):
    """FlashAttention-2 loop order for one head, float64: returns (O, LSE).

    Outer loop over Q blocks of ``br`` rows, inner loop over K/V blocks of
    ``bc`` rows.  Per Q block the running (m, l, O~) start at (-inf, 0, 0);
    each K/V block's scores are merged with the rule above and O~ is
    rescaled by exp(m_old - m_new) before the block's P~ V is added.  One
    division by l at the end; LSE = m + ln l.  Causal masking sets scores of
    keys after the query to -inf; blocks with every score masked contribute
    nothing (their rescale factor is taken as 0, as in ``merge_stats``).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d = q.shape
    O = np.zeros((N, v.shape[1]))
    LSE = np.zeros(N)
    for i0 in range(0, N, br):
        qi = q[i0:i0 + br]
        rows = np.arange(i0, i0 + qi.shape[0])
        m = np.full(qi.shape[0], -np.inf)
        ell = np.zeros(qi.shape[0])
        acc = np.zeros((qi.shape[0], v.shape[1]))
        for j0 in range(0, N, bc):
            s = (qi @ k[j0:j0 + bc].T) * scale
            if causal:
                cols = np.arange(j0, j0 + s.shape[1])
                s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
            m_blk = np.max(s, axis=1)
            m_new = np.maximum(m, m_blk)
            # rows with every score so far masked keep m = -inf; use 0 as the
            # shift there so that no -inf - (-inf) is formed
            shift = np.where(m_new == -np.inf, 0.0, m_new)
            alpha = np.where(m == -np.inf, 0.0, np.exp(m - shift))
            p = np.exp(s - shift[:, None])
            ell = alpha * ell + np.sum(p, axis=1)
            acc = alpha[:, None] * acc + p @ v[j0:j0 + bc]
            m = m_new
        O[i0:i0 + br] = acc / ell[:, None]
        LSE[i0:i0 + br] = m + np.log(ell)
    return O, LSE
