"""Pins of the dropout oracle (Philox mask, forward, gradients) to things
other than itself.

* The generic Philox is checked against numpy's Philox4x64-10 bit generator
  (a library routine; numpy increments its counter before the first block),
  its Weyl increments against their closed forms, and the vectorised
  4x32 path against the scalar one.
* The mask against statistics it must have (uniform bytes, keep rate) and
  against a per-element scalar recomputation.
* The forward against p = 0 (plain attention) and a brute-force sum; the
  gradients against central finite differences and torch fp64 autograd with
  the same mask given as a tensor.
``test_oracle_mutations.py`` plants slips (byte order, threshold, rescale,
counter layout, a mask missing from dP) and shows these pins catch them.
"""

import math
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import scipy.stats
import torch

import oracle
import oracle.dropout as od

RNG = np.random.default_rng(2024)


def _numpy_philox(counter, key, n_blocks=1):
    # uint64 arrays: numpy would route Python ints above 2^63 through a float cast
    g = np.random.Philox(counter=np.array(counter, dtype=np.uint64),
                         key=np.array(key, dtype=np.uint64))
    assert [int(x) for x in g.state["state"]["counter"]] == list(counter)
    out = [int(x) for x in g.random_raw(4 * n_blocks)]
    return [out[4 * b:4 * b + 4] for b in range(n_blocks)]


@pytest.mark.parametrize("counter,key", [
    ([0, 0, 0, 0], [0, 0]),
    ([5, 0, 0, 0], [7, 9]),
    ([2**64 - 1, 3, 0, 0], [123456789, 987654321]),      # carry into word 1
    ([2**64 - 1, 2**64 - 1, 17, 2**63], [2**64 - 1, 2**64 - 2]),
    ([0x243F6A8885A308D3, 0x13198A2E03707344, 0xA4093822299F31D0, 0x082EFA98EC4E6C89],
     [0x452821E638D01377, 0xBE5466CF34E90C6C]),
])
def test_philox4x64_matches_numpy(counter, key):
    blocks = _numpy_philox(counter, key, n_blocks=3)
    c = list(counter)
    for b in range(3):
        # numpy advances the 256-bit counter by one before each block
        v = (c[0] | c[1] << 64 | c[2] << 128 | c[3] << 192) + 1
        c = [(v >> (64 * i)) & (2**64 - 1) for i in range(4)]
        assert od.philox(c, key, width=64) == blocks[b]


ROCRAND_HEADER = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"
ROCRAND_PROG = os.path.join(os.path.dirname(os.path.abspath(__file__)), "philox_rocrand.cpp")


def rocrand_philox4x32(blocks):
    """Philox4x32-10 output words of each (counter, key) in ``blocks`` from
    rocRAND's header-only engine, compiled for the host with g++ on first use
    (a library implementation written independently of the oracle)."""
    if not os.path.exists(ROCRAND_HEADER) or shutil.which("g++") is None:
        pytest.skip("rocRAND headers or g++ not available")
    exe = os.path.join(tempfile.gettempdir(), f"philox_rocrand_{os.getpid()}")
    if not os.path.exists(exe):
        subprocess.run(["g++", "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                        ROCRAND_PROG, "-o", exe], check=True, capture_output=True)
    text = "".join(" ".join(str(int(x)) for x in (*c, *k)) + "\n" for c, k in blocks)
    out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
    return [[int(w) for w in line.split()] for line in out.strip().splitlines()]


def _philox32_cases():
    rng = np.random.default_rng(321)
    cases = [([0, 0, 0, 0], [0, 0]), ([1, 2, 3, 4], [5, 6]),
             ([2**32 - 1] * 4, [2**32 - 1, 2**32 - 1]),
             # the layout the kernels use: (key group, query, head, offset)
             ([255, 4095, 63, 0], [0x5EED, 0]), ([3, 17, 5, 9], [0xDEADBEEF, 0x01234567])]
    for _ in range(60):
        cases.append(([int(x) for x in rng.integers(0, 2**32, 4)],
                      [int(x) for x in rng.integers(0, 2**32, 2)]))
    return cases


def test_philox4x32_matches_rocrand():
    """The width-32 instance (multipliers, Weyl increments, round structure,
    word order) against rocRAND's philox4x32_10 engine, for the scalar and
    the vectorised oracle paths."""
    cases = _philox32_cases()
    ref = rocrand_philox4x32(cases)
    assert len(ref) == len(cases)
    for (c, k), r in zip(cases, ref):
        assert od.philox(c, k, width=32) == r, (c, k)
    for (cc, k), r in zip(cases[:8], ref[:8]):
        got = od.philox4x32_10_array(cc[0], cc[1], cc[2], cc[3], k[0], k[1])
        assert [int(x) for x in got] == r


def test_weyl_increments_closed_form():
    for w in (32, 64):
        phi_frac = (math.isqrt(5 << (2 * w)) - (1 << w)) >> 1   # floor(2^w (phi - 1))
        sqrt3_m1 = math.isqrt(3 << (2 * w)) - (1 << w)           # floor(2^w (sqrt 3 - 1))
        assert od.PHILOX[w][2] == phi_frac and od.PHILOX[w][3] == sqrt3_m1
    # the 32-bit multipliers and increments are 32-bit odd constants
    assert all(x % 2 == 1 and x < 2**32 for x in od.PHILOX[32])


def test_philox_rounds_structure():
    c, k = [1, 2, 3, 4], [5, 6]
    assert od.philox(c, k, rounds=0) == c
    one = od.philox(c, k, rounds=1)
    assert od.philox(one, [(5 + od.PHILOX[32][2]) % 2**32, (6 + od.PHILOX[32][3]) % 2**32],
                     rounds=9) == od.philox(c, k, rounds=10)


def test_vectorised_matches_scalar():
    c0 = RNG.integers(0, 2**32, 200, dtype=np.uint64)
    c1 = RNG.integers(0, 2**32, 200, dtype=np.uint64)
    k0, k1 = 0xDEADBEEF, 0x01234567
    got = od.philox4x32_10_array(c0, c1, 77, 5, k0, k1)
    for n in range(200):
        assert list(got[n]) == od.philox([c0[n], c1[n], 77, 5], [k0, k1], width=32)


def test_bytes_and_mask_layout():
    seed, off, bh, N = 0x1234567890ABCDEF, 3, 5, 37
    rows = [0, 1, 20]
    by = od.dropout_bytes(seed, off, bh, rows, N)
    for r, i in enumerate(rows):
        for j in range(N):
            w = od.philox([j // 16, i, bh, off], [seed & 0xFFFFFFFF, seed >> 32], width=32)
            assert by[r, j] == (w[(j % 16) // 4] >> (8 * (j % 4))) & 0xFF
    m = od.dropout_mask(seed, off, bh, rows, N, 0.3)
    assert np.array_equal(m, by >= od.dropout_threshold(0.3))


def test_threshold_and_scale():
    assert od.dropout_threshold(0.0) == 0 and od.dropout_scale(0.0) == 1.0
    assert od.dropout_threshold(0.1) == 26 and od.dropout_scale(0.1) == 256 / 230
    assert od.dropout_threshold(0.5) == 128 and od.dropout_scale(0.5) == 2.0
    assert od.dropout_threshold(255.4 / 256) == 255
    for bad in (255.5 / 256, 1.0, -0.01, float("nan")):
        with pytest.raises(ValueError):
            od.dropout_threshold(bad)


def test_mask_statistics():
    by = od.dropout_bytes(99, 0, 0, np.arange(512), 2048).ravel()
    counts = np.bincount(by, minlength=256)
    assert scipy.stats.chisquare(counts).pvalue > 1e-4
    for p in (0.1, 0.25, 0.5):
        keep = od.dropout_mask(99, 0, 0, np.arange(512), 2048, p).mean()
        q = (256 - od.dropout_threshold(p)) / 256
        assert abs(keep - q) < 5 * math.sqrt(q * (1 - q) / by.size)
    # neighbouring counters are uncorrelated
    a = od.dropout_bytes(99, 0, 0, [7], 4096)[0].astype(float)
    assert abs(np.corrcoef(a[:-16], a[16:])[0, 1]) < 0.06
    # different heads, offsets and seeds give different masks
    b0 = od.dropout_bytes(1, 0, 0, [3], 256)
    for other in (od.dropout_bytes(1, 0, 1, [3], 256), od.dropout_bytes(1, 1, 0, [3], 256),
                  od.dropout_bytes(2, 0, 0, [3], 256), od.dropout_bytes(1 << 32, 0, 0, [3], 256)):
        assert (b0 != other).mean() > 0.9


@pytest.mark.parametrize("causal", [False, True])
def test_forward_p0_is_plain_attention(causal):
    q, k, v = (RNG.standard_normal((1, 2, 40, 8)) for _ in range(3))
    O, L = oracle.attention_forward_dropout(q, k, v, 0.3, causal, 0.0, seed=5)
    O0, L0 = oracle.attention_forward(q, k, v, 0.3, causal)
    np.testing.assert_array_equal(O, O0)
    np.testing.assert_array_equal(L, L0)


@pytest.mark.parametrize("causal", [False, True])
def test_forward_brute_force(causal):
    B, H, N, d = 1, 2, 21, 3
    q, k, v = (RNG.standard_normal((B, H, N, d)) for _ in range(3))
    p, seed, off, scale = 0.3, 0xABCDEF0123, 4, 0.6
    O, L = oracle.attention_forward_dropout(q, k, v, scale, causal, p, seed, off)
    t = od.dropout_threshold(p)
    for h in range(H):
        for i in range(N):
            vis = range(i + 1) if causal else range(N)
            w = {j: math.exp(scale * math.fsum(q[0, h, i, c] * k[0, h, j, c] for c in range(d)))
                 for j in vis}
            den = math.fsum(w.values())
            keep = {}
            for j in vis:
                words = od.philox([j // 16, i, h, off], [seed & 0xFFFFFFFF, seed >> 32], width=32)
                keep[j] = ((words[(j % 16) // 4] >> (8 * (j % 4))) & 0xFF) >= t
            for c in range(d):
                ref = math.fsum(w[j] * v[0, h, j, c] for j in vis if keep[j]) / den * 256 / (256 - t)
                assert abs(O[0, h, i, c] - ref) < 1e-12
            assert abs(L[0, h, i] - math.log(den)) < 1e-12


def test_rows_variant_matches():
    q, k, v = (RNG.standard_normal((2, 3, 50, 8)) for _ in range(3))
    O, L = oracle.attention_forward_dropout(q, k, v, 0.4, True, 0.2, seed=11, offset=2)
    rows = [0, 17, 49]
    for b, h in ((0, 0), (1, 2)):
        Or, Lr = oracle.attention_forward_dropout_rows(q[b, h], k[b, h], v[b, h], 0.4, True, 0.2,
                                                       11, 2, b * 3 + h, rows)
        np.testing.assert_allclose(Or, O[b, h, rows], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(Lr, L[b, h, rows], rtol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences(causal):
    B, H, N, d = 1, 1, 18, 3
    q, k, v, do = (RNG.standard_normal((B, H, N, d)) for _ in range(4))
    p, seed, scale = 0.25, 321, 0.7
    dQ, dK, dV = oracle.attention_backward_dropout(q, k, v, do, scale, causal, p, seed)
    h = 1e-6

    def loss(qq, kk, vv):
        return float(np.sum(oracle.attention_forward_dropout(qq, kk, vv, scale, causal, p, seed)[0] * do))

    for x, g, which in ((q, dQ, 0), (k, dK, 1), (v, dV, 2)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_torch_autograd(causal):
    B, H, N, d = 2, 2, 33, 8
    q, k, v, do = (RNG.standard_normal((B, H, N, d)) for _ in range(4))
    p, seed, off, scale = 0.2, 77, 1, 0.35
    dQ, dK, dV = oracle.attention_backward_dropout(q, k, v, do, scale, causal, p, seed, off)
    Z = np.stack([np.stack([od.dropout_mask(seed, off, b * H + hh, np.arange(N), N, p)
                            for hh in range(H)]) for b in range(B)])
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = scale * tq @ tk.transpose(-1, -2)
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), -math.inf)
    P = torch.softmax(s, dim=-1) * torch.tensor(Z, dtype=torch.float64) * od.dropout_scale(p)
    (P @ tv).backward(torch.tensor(do))
    for g, t in ((dQ, tq), (dK, tk), (dV, tv)):
        np.testing.assert_allclose(g, t.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_rowsum_identity_with_dropout():
    """D_i = sum_c dO_ic O_ic equals sum_j P_ij dP_ij with dP = (dO V^T) o Z s."""
    N, d = 30, 6
    q, k, v, do = (RNG.standard_normal((1, 1, N, d)) for _ in range(4))
    p, seed, scale = 0.3, 8, 0.5
    O, _ = oracle.attention_forward_dropout(q, k, v, scale, True, p, seed)
    P = oracle.softmax_rows(oracle.scores(q[0, 0], k[0, 0], scale, True))[2]
    Zs = od.dropout_mask(seed, 0, 0, np.arange(N), N, p) * od.dropout_scale(p)
    dP = (do[0, 0] @ v[0, 0].T) * Zs
    np.testing.assert_allclose(np.sum(do[0, 0] * O[0, 0], axis=1), np.sum(P * dP, axis=1),
                               rtol=1e-12, atol=1e-13)
