"""Parity of the dropout forward and backward with the fp64 oracle, through
the C ABI.

The keep mask is integer work, so it is checked bit-exactly: with Q = 0 every
visible probability is 1/count, and one-hot rows of V (or of dO) make O (or
dV) read out the mask element by element.  The numbers are checked against
``oracle.attention_forward_dropout`` / ``attention_backward_dropout`` with the
bf16 path's bars (O 1e-2 plus half a bf16 ulp, LSE 1e-3, gradients 5e-2 of
each tensor's max).
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from exact_attention_flash_amd import (flash_attn_bwd_dropout, flash_attn_fwd,
                                       flash_attn_fwd_dropout)
from exact_attention_flash_amd.inputs import default_scale, f32_to_bf16_bits, make_inputs

from gpu_util import bf16_to_f64, check_grad, check_lse, check_o, to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _fwd(x, causal, scale, p, seed, offset=0):
    q, k, v = (to_device(x[n]) for n in ("q", "k", "v"))
    o, lse = flash_attn_fwd_dropout(q, k, v, p, seed, offset, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    return (q, k, v), o, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_dropout_mask_exact_forward(d, causal):
    """Q = 0, V one-hot: O[i, c] = Z[i, c] s / count_i for visible c < N."""
    _say(f"dropout mask (forward) d={d} causal={causal}")
    B, H, N = 2, 2, d          # N <= d, so V = I fits
    x = make_inputs(B, H, N, d, seed=41)
    x["q"][:] = 0
    eye = f32_to_bf16_bits(np.eye(N, d, dtype=np.float32))
    x["v"][:] = eye
    p, seed, off = 0.3, 0x0123456789ABCDEF, 7
    _, o, lse = _fwd(x, causal, default_scale(d), p, seed, off)
    og = bf16_to_f64(o)
    for b in range(B):
        for h in range(H):
            Z = oracle.dropout_mask(seed, off, b * H + h, np.arange(N), N, p)
            if causal:
                Z = np.tril(Z)
            got = og[b, h, :, :N] > 0
            assert np.array_equal(got, Z), f"mask mismatch in head {b},{h}: {int((got != Z).sum())}"
    counts = np.arange(1, N + 1) if causal else np.full(N, N)
    check_lse(lse.cpu().numpy().astype(np.float64), np.broadcast_to(np.log(counts), (B, H, N)))


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_mask_exact_dv(causal):
    """Q = 0, dO one-hot: dV[j, i] = P_ij Z_ij s, so dV reads out the mask the
    key-block pass draws."""
    _say(f"dropout mask (dV) causal={causal}")
    B, H, N, d = 1, 3, 128, 128
    x = make_inputs(B, H, N, d, seed=43, with_dout=True)
    x["q"][:] = 0
    x["do"][:] = f32_to_bf16_bits(np.eye(N, d, dtype=np.float32))
    p, seed, off = 0.2, 99, 3
    (q, k, v), o, lse = _fwd(x, causal, 0.125, p, seed, off)
    dout = to_device(x["do"])
    dq, dk, dv = flash_attn_bwd_dropout(dout, q, k, v, o, lse, p, seed, off, causal=causal,
                                        softmax_scale=0.125)
    torch.cuda.synchronize()
    dvg = bf16_to_f64(dv)
    for h in range(H):
        Z = oracle.dropout_mask(seed, off, h, np.arange(N), N, p)
        if causal:
            Z = np.tril(Z)
        got = dvg[0, h, :, :N].T != 0      # dV[j, i] for query i, key j
        assert np.array_equal(got, Z), f"dV mask mismatch in head {h}: {int((got != Z).sum())}"


SMALL = [
    # (B, H, N, d, causal, p)
    (1, 1, 128, 64, False, 0.1),
    (1, 2, 1, 64, True, 0.5),
    (1, 2, 200, 64, True, 0.25),
    (2, 1, 333, 128, False, 0.1),
    (1, 1, 1000, 128, True, 0.3),
    (2, 4, 600, 128, True, 0.15),
    (1, 8, 520, 64, False, 0.4),
]


@pytest.mark.parametrize("B,H,N,d,causal,p", SMALL)
def test_dropout_forward_parity(B, H, N, d, causal, p):
    _say(f"dropout fwd B={B} H={H} N={N} d={d} causal={causal} p={p}")
    x = make_inputs(B, H, N, d, seed=N + d + int(100 * p))
    scale = default_scale(d)
    seed, off = 1234567 + N, 5
    _, o, lse = _fwd(x, causal, scale, p, seed, off)
    O_ref, L_ref = oracle.attention_forward_dropout(x["q"], x["k"], x["v"], scale, causal, p, seed, off)
    check_o(bf16_to_f64(o), O_ref)
    check_lse(lse.cpu().numpy().astype(np.float64), L_ref)


SMALL_BWD = [
    (1, 1, 128, 64, False, 0.1),
    (1, 1, 128, 128, True, 0.3),
    (2, 2, 200, 64, True, 0.2),
    (1, 2, 333, 128, False, 0.25),
    (2, 4, 270, 128, True, 0.1),
    (1, 8, 257, 64, False, 0.5),
]


@pytest.mark.parametrize("B,H,N,d,causal,p", SMALL_BWD)
def test_dropout_backward_parity(B, H, N, d, causal, p):
    _say(f"dropout bwd B={B} H={H} N={N} d={d} causal={causal} p={p}")
    x = make_inputs(B, H, N, d, seed=3 * N + d + int(100 * p), with_dout=True)
    scale = default_scale(d)
    seed, off = 777 + N, 11
    (q, k, v), o, lse = _fwd(x, causal, scale, p, seed, off)
    dout = to_device(x["do"])
    dq, dk, dv = flash_attn_bwd_dropout(dout, q, k, v, o, lse, p, seed, off, causal=causal,
                                        softmax_scale=scale)
    torch.cuda.synchronize()
    dQ, dK, dV = oracle.attention_backward_dropout(x["q"], x["k"], x["v"], x["do"], scale, causal,
                                                   p, seed, off)
    check_grad(bf16_to_f64(dq), dQ, "dQ")
    check_grad(bf16_to_f64(dk), dK, "dK")
    check_grad(bf16_to_f64(dv), dV, "dV")


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_p0_matches_plain(causal):
    _say(f"dropout p=0 equals the plain forward, causal={causal}")
    x = make_inputs(2, 3, 500, 128, seed=8)
    scale = default_scale(128)
    (q, k, v), o, lse = _fwd(x, causal, scale, 0.0, 5)
    o2, l2 = flash_attn_fwd(q, k, v, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, l2)


def test_dropout_deterministic_and_seeded():
    x = make_inputs(1, 4, 700, 64, seed=9)
    (q, k, v), o1, l1 = _fwd(x, True, 0.125, 0.2, 42, 1)
    _, o2, l2 = _fwd(x, True, 0.125, 0.2, 42, 1)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    _, o3, l3 = _fwd(x, True, 0.125, 0.2, 42, 2)       # another offset: another mask
    assert not torch.equal(o1.view(torch.int16), o3.view(torch.int16)) and torch.equal(l1, l3)


FULL = [
    # (name, B, H, N, d, causal, p, seed)
    ("c5-dropout", 4, 16, 4096, 128, True, 0.1, 5200),
    ("c3-dropout", 16, 12, 1024, 64, False, 0.1, 3200),
]


@pytest.mark.parametrize("name,B,H,N,d,causal,p,seed", FULL)
def test_dropout_full_size_sampled(name, B, H, N, d, causal, p, seed):
    """Full-size forward and backward in the bench's configuration; the
    forward checked on sampled rows of sampled heads, the backward through
    properties that hold at any size."""
    _say(f"dropout full size {name}: B={B} H={H} N={N} d={d} causal={causal} p={p}")
    x = make_inputs(B, H, N, d, seed=seed, with_dout=True)
    scale = default_scale(d)
    rs, off = 2**40 + seed, 0
    (q, k, v), o, lse = _fwd(x, causal, scale, p, rs, off)
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, N - 2, N - 1], rng.integers(0, N, 20)]))
    for b, h in ((0, 0), (B - 1, H - 1), (int(rng.integers(B)), int(rng.integers(H)))):
        O_ref, L_ref = oracle.attention_forward_dropout_rows(
            x["q"][b, h], x["k"][b, h], x["v"][b, h], scale, causal, p, rs, off, b * H + h, rows)
        og = bf16_to_f64(o[b, h][torch.as_tensor(rows, device=o.device)])
        check_o(og, O_ref, f"O head {b},{h}")
        check_lse(lse[b, h].cpu().numpy()[rows].astype(np.float64), L_ref)
    dout = to_device(x["do"])
    dq, dk, dv = flash_attn_bwd_dropout(dout, q, k, v, o, lse, p, rs, off, causal=causal,
                                        softmax_scale=scale)
    torch.cuda.synchronize()
    for g in (dq, dk, dv):
        assert bool(torch.isfinite(g.float()).all())
    # one head's gradients in full (the oracle's dense N x N matrices of one
    # head fit comfortably)
    b, h = B - 1, H // 2
    dQ, dK, dV = oracle.attention_backward_dropout_head(
        x["q"][b, h], x["k"][b, h], x["v"][b, h], x["do"][b, h], scale, causal, p, rs, off,
        b * H + h)
    check_grad(bf16_to_f64(dq[b, h]), dQ, "dQ")
    check_grad(bf16_to_f64(dk[b, h]), dK, "dK")
    check_grad(bf16_to_f64(dv[b, h]), dV, "dV")


# Shapes whose persistent dropout forward and key-block pass give some
# workgroup more than one item (snake order and the round-robin fallback).
WALKS_DROPOUT = [
    # (B, H, N, d, causal, p, seed)
    (2, 20, 4096, 128, False, 0.1, 5300),  # forward 640, key blocks 1280 items
    (1, 33, 2100, 128, True, 0.2, 5301),   # forward 297, key blocks 561: round robin
    (2, 20, 4096, 64, True, 0.15, 5302),   # d = 64, causal
]


@pytest.mark.parametrize("B,H,N,d,causal,p,seed", WALKS_DROPOUT)
def test_dropout_walk(B, H, N, d, causal, p, seed):
    _say(f"dropout walk B={B} H={H} N={N} d={d} causal={causal} p={p}")
    from gpu_util import most_items_per_workgroup
    assert most_items_per_workgroup(B * H * -(-N // 256)) > 1
    assert most_items_per_workgroup(B * H * -(-N // 128)) > 1
    x = make_inputs(B, H, N, d, seed=seed, with_dout=True)
    scale = default_scale(d)
    rs, off = 99 + seed, 3
    (q, k, v), o, lse = _fwd(x, causal, scale, p, rs, off)
    dq, dk, dv = flash_attn_bwd_dropout(to_device(x["do"]), q, k, v, o, lse, p, rs, off,
                                        causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, 255, 256, N - 1], rng.integers(0, N, 12)]))
    BH = B * H
    for bh in sorted({0, BH - 1}):
        b, h = divmod(bh, H)
        O_ref, L_ref = oracle.attention_forward_dropout_rows(
            x["q"][b, h], x["k"][b, h], x["v"][b, h], scale, causal, p, rs, off, bh, rows)
        og = bf16_to_f64(o[b, h][torch.as_tensor(rows, device=o.device)])
        check_o(og, O_ref, f"O head {bh}")
        check_lse(lse[b, h].cpu().numpy()[rows].astype(np.float64), L_ref)
    # one whole head's gradients (the last, so a late item of the walk)
    b, h = divmod(BH - 1, H)
    dQ, dK, dV = oracle.attention_backward_dropout_head(
        x["q"][b, h], x["k"][b, h], x["v"][b, h], x["do"][b, h], scale, causal, p, rs, off, BH - 1)
    check_grad(bf16_to_f64(dq[b, h]), dQ, "dQ")
    check_grad(bf16_to_f64(dk[b, h]), dK, "dK")
    check_grad(bf16_to_f64(dv[b, h]), dV, "dV")
