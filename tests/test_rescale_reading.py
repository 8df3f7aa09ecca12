"""The forward's running-max reading, checked on the CPU by emulating its
roundings (no GPU, no kernel code).

The bf16 forward moves its running max only when a tile raises some row of
a 32-row wave by more than 2^8 (log2 units), and divides O by the row sum
plus, per tile, bf16(p_max) - p_max: the rounding error of the tile's
largest probability in the P V product.  This file emulates that arithmetic
in numpy (fp32 scores and probabilities, bf16-rounded P, fp32 sums, bf16
output) next to the two alternatives, and compares each with the float64
oracle:
  * eager: the max moves whenever a tile raises it (the pages' per-block
    update, where the dominant probability is exactly 1);
  * lazy without the correction: the same stale max, O divided by the
    unrounded sum.
The lazy scheme with the correction must be as accurate as the eager one,
and the constructed stale-max row must come out exactly (the GPU test
``test_fwd_stale_max_rounding`` checks the kernel on the same row).
"""

import math

import numpy as np

import oracle
from exact_attention_flash_amd.inputs import bf16_bits_to_f32, default_scale, f32_to_bf16_bits, make_inputs


def _bf16(x):
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(x, np.float32)))


def _emulate(q, k, v, scale, threshold, corrected):
    """One head of full attention, rows in waves of 32, key tiles of 64."""
    N, d = k.shape
    sl2 = np.float32(scale) * np.float32(1.4426950408889634)
    R = q.shape[0]
    S = (q.astype(np.float64) @ k.T.astype(np.float64)).astype(np.float32)
    m = np.full(R, -np.inf, np.float32)
    l = np.zeros(R, np.float32)
    corr = np.zeros(R, np.float32)
    O = np.zeros((R, d), np.float32)
    wave = np.arange(R) // 32
    for k0 in range(0, N, 64):
        s = S[:, k0:k0 + 64]
        mraw = s.max(axis=1)
        mx = (mraw * sl2).astype(np.float32)
        rise = mx > m + np.float32(threshold)
        fire = np.zeros(R, bool)
        for wv in np.unique(wave):
            sel = wave == wv
            fire[sel] = rise[sel].any()
        m_new = np.where(fire, np.maximum(m, mx), m).astype(np.float32)
        with np.errstate(invalid="ignore"):
            alpha = np.where(fire & (m_new != -np.inf), np.exp2(m - m_new), 1.0).astype(np.float32)
        m = m_new
        l *= alpha
        corr *= alpha
        O *= alpha[:, None]
        m_use = np.where(m == -np.inf, 0.0, m).astype(np.float32)
        p = np.exp2((s * sl2 - m_use[:, None]).astype(np.float32)).astype(np.float32)
        l += p.sum(axis=1, dtype=np.float32)
        if corrected:
            pt = np.exp2((mraw * sl2 - m_use).astype(np.float32)).astype(np.float32)
            corr += _bf16(pt) - pt
        O += (_bf16(p) @ v[k0:k0 + 64]).astype(np.float32)
    den = l + corr if corrected else l
    o = _bf16(O / den[:, None]).astype(np.float64)
    lse = ((m + np.log2(l)) * np.float32(math.log(2))).astype(np.float64)
    return o, lse


def _half_ulp(x):
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 8), 0.0)


def test_lazy_max_with_correction_as_accurate_as_eager():
    """Q x 8 (nearly one-hot rows, the case a stale max hurts) and N(0, 1)."""
    for q_mult in (8.0, 1.0):
        x = make_inputs(1, 2, 1024, 64, seed=3, q_mult=q_mult)
        Q, K, V = (bf16_bits_to_f32(x[n]) for n in "qkv")
        scale = default_scale(64)
        O_ref, L_ref = oracle.attention_forward(x["q"], x["k"], x["v"], scale, False)
        for h in range(2):
            q, k, v = Q[0, h], K[0, h], V[0, h]
            res = {}
            for name, thr, cor in (("eager", 0.0, False), ("lazy", 8.0, True), ("lazy_uncorrected", 8.0, False)):
                o, lse = _emulate(q, k, v, scale, thr, cor)
                err = np.abs(o - O_ref[0, h])
                res[name] = (err.max(), int((err > 1e-2).sum()), np.abs(lse - L_ref[0, h]).max(),
                             bool(np.all(err <= 1e-2 + _half_ulp(O_ref[0, h]))))
            eager, lazy, unc = res["eager"], res["lazy"], res["lazy_uncorrected"]
            assert lazy[0] <= eager[0] + 2.0 ** -10, (q_mult, h, res)
            assert lazy[1] <= eager[1] + 2, (q_mult, h, res)
            assert lazy[2] <= 1e-5 and eager[2] <= 1e-5, (q_mult, h, res)
            assert lazy[3] and eager[3], (q_mult, h, res)
            if q_mult == 8.0:
                # without the correction a stale max leaves more elements past 1e-2
                assert unc[1] > lazy[1], (h, res)


def test_lazy_max_correction_exact_on_stale_one_hot():
    """Key A (score 0, tile 0), key B in tile 3 at probability 2^x in
    [128.3, 128.45] relative to A (below 2^8, so the max stays at A's score;
    bf16 rounds it to 128), 254 keys at -100, every V row equal: the exact O
    is that row.  The correction makes it exact; without it every element is
    one bf16 ulp low."""
    for d in (64, 128):
        scale = default_scale(d)
        sl2 = np.float32(scale) * np.float32(1.4426950408889634)
        best = None
        for a in np.arange(8.0, 16.0, 0.0625, dtype=np.float32):
            for b in _bf16(np.linspace(0.0, 0.5, 257).astype(np.float32)):
                xs = np.float32(np.float32(4.0 * a + b) * sl2)
                if 128.3 <= 2.0 ** float(xs) <= 128.45:
                    best = (float(a), float(b))
                    break
            if best:
                break
        assert best is not None
        N = 256
        q = np.zeros((64, d), np.float32)
        q[:, 0], q[:, 1] = 4.0, 1.0
        k = np.zeros((N, d), np.float32)
        k[:, 0] = -25.0
        k[5, 0] = 0.0
        k[200, 0], k[200, 1] = best
        v_row = (1.875 * 2.0 ** (np.arange(d) % 4 - 2) * (-1.0) ** np.arange(d)).astype(np.float32)
        v = np.broadcast_to(v_row, (N, d)).copy()
        o_cor, _ = _emulate(q, k, v, scale, 8.0, True)
        o_unc, _ = _emulate(q, k, v, scale, 8.0, False)
        assert np.abs(o_cor - v_row).max() == 0.0
        assert np.all(np.abs(o_unc - v_row) == 2.0 * _half_ulp(v_row))
