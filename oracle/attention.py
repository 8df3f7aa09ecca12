"""Exact attention written out as its plain definition, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): the HIP library never
imports this module.

The method is *exact* attention: the pages stress that the fused kernel
computes the same mathematical function as the standard pipeline and may
differ only by floating-point rounding order ("优化的注意力实现", section
"注意事项"; "FlashAttention 系列技术详解", section "FlashAttention 的解决方案").
So the oracle is the definition itself, with the N x N score matrix
materialised; no tiling, no online rescaling, no fusion.

Conventions (readings of the pages, also listed in the design notes):

* tensors are ``[B, H, N, d]``; heads are independent (the CMU notes, section
  "多头自注意力机制", apply the same single-head formula per head);
* ``scale`` multiplies Q K^T before masking and softmax; callers pass the
  same float32 value the GPU receives (usually 1/sqrt(d));
* causal: key j is visible to query i iff j <= i (the apxml example builds its
  mask with ``tril(diagonal=0)`` and fills the rest with -inf);
* LSE is the natural-log logsumexp of the *scaled*, masked scores,
  LSE_i = m_i + ln l_i;
* gradients come from direct matrix calculus through the per-row softmax
  Jacobian (no rowsum(dO o O) shortcut), so that the kernel's shortcut is
  checked by something that does not use it.
"""

from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------- inputs
def widen_bf16(bits) -> np.ndarray:
    """Exact float64 values of bf16 bit patterns (uint16 array).

    bf16 is the top half of an IEEE float32, so shifting the 16 bits into the
    high half of a 32-bit word gives the float32 with the same value.
    """
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError(f"expected uint16 bf16 bit patterns, got {b.dtype}")
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _f64(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return widen_bf16(x)
    return x.astype(np.float64, copy=False)


# ---------------------------------------------------------------- forward
def scores(q: np.ndarray, k: np.ndarray, scale: float, causal: bool,
           row_start: int = 0, rows=None) -> np.ndarray:
    """S = scale * Q K^T for one head, masked if causal.

    ``q`` holds query rows ``row_start, row_start + 1, ...`` of the head, or,
    when ``rows`` is given, the rows with those global indices (the mask
    needs the global index of each query).

    Definition: apxml page, equation softmax(QK^T/sqrt(d_k))V and the manual
    fallback in its example (matmul, multiply by the scale factor, add the
    causal bias whose entries above the diagonal are -inf); CMU notes,
    section "计算步骤", steps 2-3 (S = QK^T, then divide by sqrt(d)).
    """
    s = (q @ k.T) * np.float64(scale)
    if causal:
        if rows is None:
            rows = np.arange(row_start, row_start + q.shape[0])
        r = np.asarray(rows)[:, None]
        cols = np.arange(k.shape[0])[None, :]
        s = np.where(cols > r, -np.inf, s)
    return s


def softmax_rows(s: np.ndarray):
    """Row-wise safe softmax of ``s``: returns (m, l, P).

    CMU notes, section "安全 Softmax 与在线 Softmax": m(x) is the row maximum,
    f(x) the exponentials of x - m(x), l(x) their sum, softmax = f / l.
    Entries equal to -inf (masked) give f = 0.
    """
    m = np.max(s, axis=1)
    f = np.exp(s - m[:, None])
    ell = np.sum(f, axis=1)
    return m, ell, f / ell[:, None]


def _heads(q, k, v):
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    return q.shape


def _heads_qkv(q, k, v, causal: bool):
    """Shapes of a forward whose queries and keys may differ in number:
    q [B, H, N_q, d], k and v [B, H, N_kv, d].  The decode step of the CMU
    notes (section "生成式 LLM 推理") attends from one new query to every
    cached key and value, and the apxml example's interface gives queries
    and keys their own sequence lengths.  The causal mask (key j visible to
    query i iff j <= i) is only taken for equal lengths."""
    if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape or q.shape[:2] != k.shape[:2] \
            or q.shape[3] != k.shape[3]:
        raise ValueError("q must be [B, H, N_q, d] and k, v [B, H, N_kv, d]")
    if causal and q.shape[2] != k.shape[2]:
        raise ValueError("the causal mask needs as many queries as keys")
    return q.shape


def attention_probs(q, k, scale: float, causal: bool) -> np.ndarray:
    """P = softmax(scale * Q K^T (masked)) for every head, ``[B, H, N, N]``."""
    q, k = _f64(q), _f64(k)
    B, H, N, _ = q.shape
    out = np.empty((B, H, N, N))
    for b in range(B):
        for h in range(H):
            out[b, h] = softmax_rows(scores(q[b, h], k[b, h], scale, causal))[2]
    return out


def attention_forward(q, k, v, scale: float, causal: bool,
                      row_chunk: int | None = None):
    """O = softmax(scale * Q K^T) V and LSE, both float64.

    Inputs are ``[B, H, N, d]`` arrays (uint16 bf16 bit patterns are widened
    exactly); without the causal mask, k and v may hold another number of
    rows than q (``[B, H, N_kv, d]``, a decode step).  Returns
    ``O [B, H, N, d]`` and ``LSE [B, H, N]`` with LSE_i = m_i + ln l_i.
    ``row_chunk`` bounds the rows of S held at once; every chunk holds
    complete rows, and rows are independent, so chunking changes nothing in
    the arithmetic.

    Follows the apxml manual fallback (scores, causal bias, row softmax, @ V)
    and the CMU notes' steps 2-5; LSE follows the reading that the single
    statistic the FlashAttention-2 forward keeps for the backward pass
    ("FlashAttention 系列技术详解", section "具体优化策略") is the log of the
    per-row sum of exponentials.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = _heads_qkv(q, k, v, causal)
    R = N if row_chunk is None else max(1, int(row_chunk))
    O = np.empty((B, H, N, d))
    LSE = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, R):
                s = scores(q[b, h, r0:r0 + R], k[b, h], scale, causal, r0)
                m, ell, p = softmax_rows(s)
                O[b, h, r0:r0 + R] = p @ v[b, h]
                LSE[b, h, r0:r0 + R] = m + np.log(ell)
    return O, LSE


def attention_forward_rows(q, k, v, scale: float, causal: bool, rows):
    """O and LSE of one head ``[N, d]`` for the query rows listed in ``rows``.

    The same definition as ``attention_forward``: every listed row is
    computed in full against all N keys; rows are independent, so this is
    the whole-head result restricted to those rows.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    if causal and q.shape[0] != k.shape[0]:
        raise ValueError("the causal mask needs as many queries as keys")
    rows = np.asarray(rows, dtype=np.int64)
    s = scores(q[rows], k, scale, causal, rows=rows)
    m, ell, p = softmax_rows(s)
    return p @ v, m + np.log(ell)


# ---------------------------------------------------------------- backward
def softmax_row_grad(p: np.ndarray, dp: np.ndarray) -> np.ndarray:
    """dS for P = softmax(S) row by row: dS_r = (diag(P_r) - P_r P_r^T) dP_r.

    "FlashAttention 的基本原理", section 2.4: softmax acts on each row
    separately, so its gradient is the per-row Jacobian applied to the
    upstream gradient dP.  Written as P_r * dP_r - P_r (P_r . dP_r).
    """
    return p * dp - p * np.sum(p * dp, axis=1, keepdims=True)


def attention_backward(q, k, v, dout, scale: float, causal: bool,
                       return_intermediates: bool = False):
    """dQ, dK, dV of L = sum(dO * O) for O = softmax(scale * Q K^T) V.

    Direct matrix calculus ("FlashAttention 的基本原理", section 2.4):
      dV = P^T dO                     (gradient of the second factor of P V),
      dP = dO V^T                     (gradient of the first factor),
      dS = per-row softmax Jacobian applied to dP,
      dQ = scale * dS K,  dK = scale * dS^T Q   (chain rule through S; the
      CMU notes write the dQ update as dQ_i += dS^(j) K_j, section
      "为什么前向和反向的并行化策略不同").
    The scale factor in dQ and dK comes from S = scale * Q K^T.
    Whole heads are processed at once (no blocking).  With
    ``return_intermediates`` also returns P and dS per head.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, d = _heads(q, k, v)
    if do.shape != q.shape:
        raise ValueError("dout must have the [B, H, N, d] shape of q")
    dQ = np.empty_like(q)
    dK = np.empty_like(k)
    dV = np.empty_like(v)
    inter = {"P": np.empty((B, H, N, N)), "dS": np.empty((B, H, N, N))} \
        if return_intermediates else None
    sc = np.float64(scale)
    for b in range(B):
        for h in range(H):
            s = scores(q[b, h], k[b, h], scale, causal)
            p = softmax_rows(s)[2]
            dV[b, h] = p.T @ do[b, h]
            dp = do[b, h] @ v[b, h].T
            ds = softmax_row_grad(p, dp)
            dQ[b, h] = sc * (ds @ k[b, h])
            dK[b, h] = sc * (ds.T @ q[b, h])
            if inter is not None:
                inter["P"][b, h] = p
                inter["dS"][b, h] = ds
    if return_intermediates:
        return dQ, dK, dV, inter
    return dQ, dK, dV


def attention_backward_sampled(q, k, v, dout, scale: float, causal: bool, rows, keys,
                               row_chunk: int = 512):
    """dQ for the query rows ``rows`` and dK, dV for the keys ``keys`` of one
    head ``[N, d]``, without holding an N x N matrix.

    The same calculus as ``attention_backward``, taken over complete query
    rows a chunk at a time: for each row i, P_i and dP_i = dO_i V^T over all
    N keys, dS_i by the per-row softmax Jacobian; dV_j = sum_i P_ij dO_i and
    dK_j = scale sum_i dS_ij Q_i accumulate over the chunks for the listed
    keys j, and dQ_i = scale dS_i K for the listed rows.  Rows are
    independent and the sums over i only change their order, so this equals
    the whole-head result on those rows and keys up to rounding.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    N, d = q.shape
    sc = np.float64(scale)
    dQ = np.empty((len(rows), d))
    dK = np.zeros((len(keys), d))
    dV = np.zeros((len(keys), d))
    want = {int(r): n for n, r in enumerate(rows)}
    R = max(1, int(row_chunk))
    for r0 in range(0, N, R):
        p = softmax_rows(scores(q[r0:r0 + R], k, scale, causal, r0))[2]
        dp = do[r0:r0 + R] @ v.T
        ds = softmax_row_grad(p, dp)
        dV += p[:, keys].T @ do[r0:r0 + R]
        dK += sc * (ds[:, keys].T @ q[r0:r0 + R])
        for i in range(r0, min(r0 + R, N)):
            if i in want:
                dQ[want[i]] = sc * (ds[i - r0] @ k)
    return dQ, dK, dV
