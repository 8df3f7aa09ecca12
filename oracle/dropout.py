"""Attention with dropout on the probabilities, and its gradients, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): the HIP library never
imports this module.

The pages mention dropout twice: "FlashAttention 的基本原理" (section 2.4)
notes that the paper's backward algorithm also covers masking and dropout,
and the apxml example passes ``dropout_p`` to scaled_dot_product_attention
(zero at inference) and, in its manual fallback, applies dropout to the
attention weights after the softmax.  The readings taken here:

* dropout acts on P = softmax(scale * Q K^T): O = (P o Z * s) V, with a keep
  mask Z and the usual rescale s = 1 / (keep probability); LSE is that of
  the scores (dropout does not change the softmax statistics);
* gradients follow from O = (P o Z * s) V by direct matrix calculus:
  dV = (P o Z * s)^T dO, dP = (dO V^T) o Z * s, dS by the per-row softmax
  Jacobian, dQ = scale dS K, dK = scale dS^T Q;
* the mask is not an input but is drawn from a counter-based generator, so
  that the backward pass can redraw it: Philox4x32-10 (Salmon, Moraes, Dror
  and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011).  Each
  call maps a 128-bit counter and a 64-bit key to 128 bits.  Element
  (b, h, i, j) of the N x N probability matrix (query i, key j) takes byte
  j mod 16 (little-endian within the four 32-bit output words) of the call
  with counter (floor(j / 16), i, b * H + h, offset) and key (seed mod 2^32,
  floor(seed / 2^32));
* the dropout probability is taken in steps of 1/256: t = floor(256 p + 1/2)
  must be at most 255; an element is kept iff its byte is >= t, so the keep
  probability is (256 - t) / 256 and s = 256 / (256 - t) exactly.
"""

from __future__ import annotations

import math

import numpy as np

from .attention import _f64, _heads, scores, softmax_row_grad, softmax_rows

# Philox multipliers and Weyl increments from the SC 2011 paper.  The Weyl
# increments are the leading bits of the golden ratio's fraction and of
# sqrt(3) - 1.
PHILOX = {
    32: (0xD2511F53, 0xCD9E8D57, 0x9E3779B9, 0xBB67AE85),
    64: (0xD2E7470EE14C6C93, 0xCA5A826395121157, 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B),
}


def philox(counter, key, width: int = 32, rounds: int = 10):
    """Philox4xW-R of one counter (4 words) and key (2 words), as Python ints.

    One round maps (x0, x1, x2, x3) to
      (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2), hi(M0 x0) ^ x3 ^ k1, lo(M0 x0)),
    where hi/lo are the upper and lower W bits of the 2W-bit product; the
    key is advanced by the Weyl increments (W0, W1) after every round.
    """
    M0, M1, W0, W1 = PHILOX[width]
    mask = (1 << width) - 1
    x = [int(v) & mask for v in counter]
    k = [int(v) & mask for v in key]
    for _ in range(rounds):
        p0 = M0 * x[0]
        p1 = M1 * x[2]
        x = [((p1 >> width) ^ x[1] ^ k[0]) & mask, p1 & mask,
             ((p0 >> width) ^ x[3] ^ k[1]) & mask, p0 & mask]
        k = [(k[0] + W0) & mask, (k[1] + W1) & mask]
    return x


def philox4x32_10_array(c0, c1, c2, c3, k0: int, k1: int) -> np.ndarray:
    """Philox4x32-10 over arrays of counters (uint32 words), vectorised.

    The same rounds as ``philox`` with width 32, on numpy uint64 arrays (a
    32 x 32-bit product fits in 64 bits).  Returns uint32 [..., 4].
    """
    M0, M1, W0, W1 = PHILOX[32]
    m32 = np.uint64(0xFFFFFFFF)
    sh = np.uint64(32)
    x0, x1, x2, x3 = (np.asarray(v, dtype=np.uint64) & m32 for v in np.broadcast_arrays(c0, c1, c2, c3))
    ka, kb = int(k0) & 0xFFFFFFFF, int(k1) & 0xFFFFFFFF
    for _ in range(10):
        p0 = np.uint64(M0) * x0
        p1 = np.uint64(M1) * x2
        x0, x1, x2, x3 = ((p1 >> sh) ^ x1 ^ np.uint64(ka), p1 & m32,
                          (p0 >> sh) ^ x3 ^ np.uint64(kb), p0 & m32)
        ka = (ka + W0) & 0xFFFFFFFF
        kb = (kb + W1) & 0xFFFFFFFF
    return np.stack([x0, x1, x2, x3], axis=-1).astype(np.uint32)


def dropout_threshold(p: float) -> int:
    """t = floor(256 p + 1/2); ValueError unless 0 <= p and t <= 255."""
    p = float(p)
    if not (p >= 0.0) or math.isnan(p):
        raise ValueError("dropout probability must be >= 0")
    t = math.floor(256.0 * p + 0.5)
    if t > 255:
        raise ValueError("dropout probability rounds to 1")
    return t


def dropout_bytes(seed: int, offset: int, bh: int, rows, N: int) -> np.ndarray:
    """The random byte of every element (i, j), i in ``rows``, j < N, of head
    ``bh``: uint8 [len(rows), N]."""
    rows = np.asarray(rows, dtype=np.int64)
    ngroups = (N + 15) // 16
    jg = np.arange(ngroups, dtype=np.int64)
    words = philox4x32_10_array(jg[None, :], rows[:, None], bh, offset,
                                seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    # little-endian bytes of the four words, in order: byte 4 w + b of a call
    by = words.astype("<u4").view(np.uint8).reshape(len(rows), ngroups * 16)
    return by[:, :N]


def dropout_mask(seed: int, offset: int, bh: int, rows, N: int, p: float) -> np.ndarray:
    """Keep mask Z (bool [len(rows), N]) of head ``bh``."""
    return dropout_bytes(seed, offset, bh, rows, N) >= dropout_threshold(p)


def dropout_scale(p: float) -> float:
    t = dropout_threshold(p)
    return 256.0 / (256 - t)


def attention_forward_dropout(q, k, v, scale: float, causal: bool, p: float,
                              seed: int, offset: int = 0):
    """O = (P o Z * s) V and LSE (of the scores) for every head, float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = _heads(q, k, v)
    s = dropout_scale(p)
    O = np.empty((B, H, N, d))
    LSE = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            sc = scores(q[b, h], k[b, h], scale, causal)
            m, ell, P = softmax_rows(sc)
            Z = dropout_mask(seed, offset, b * H + h, np.arange(N), N, p)
            O[b, h] = (P * Z * s) @ v[b, h]
            LSE[b, h] = m + np.log(ell)
    return O, LSE


def attention_forward_dropout_rows(q, k, v, scale: float, causal: bool, p: float,
                                   seed: int, offset: int, bh: int, rows):
    """O and LSE of one head ``[N, d]`` (head index ``bh``) for the listed rows."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    rows = np.asarray(rows, dtype=np.int64)
    N = k.shape[0]
    sc = scores(q[rows], k, scale, causal, rows=rows)
    m, ell, P = softmax_rows(sc)
    Z = dropout_mask(seed, offset, bh, rows, N, p)
    return (P * Z * dropout_scale(p)) @ v, m + np.log(ell)


def attention_backward_dropout(q, k, v, dout, scale: float, causal: bool, p: float,
                               seed: int, offset: int = 0):
    """dQ, dK, dV of L = sum(dO * O) for O = (P o Z * s) V, float64.

    Direct matrix calculus through the dropped-out probabilities: the mask
    and s are constants, so dV = (P o Z s)^T dO and dP = (dO V^T) o Z s,
    then the per-row softmax Jacobian gives dS, and dQ = scale dS K,
    dK = scale dS^T Q.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, d = _heads(q, k, v)
    dQ, dK, dV = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    for b in range(B):
        for h in range(H):
            dQ[b, h], dK[b, h], dV[b, h] = attention_backward_dropout_head(
                q[b, h], k[b, h], v[b, h], do[b, h], scale, causal, p, seed, offset, b * H + h)
    return dQ, dK, dV


def attention_backward_dropout_head(q, k, v, dout, scale: float, causal: bool, p: float,
                                    seed: int, offset: int, bh: int):
    """The gradients above for one head ``[N, d]`` whose head index is ``bh``."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    N = q.shape[0]
    P = softmax_rows(scores(q, k, scale, causal))[2]
    Zs = dropout_mask(seed, offset, bh, np.arange(N), N, p) * dropout_scale(p)
    dV = (P * Zs).T @ do
    dP = (do @ v.T) * Zs
    dS = softmax_row_grad(P, dP)
    sc_ = np.float64(scale)
    return sc_ * (dS @ k), sc_ * (dS.T @ q), dV
