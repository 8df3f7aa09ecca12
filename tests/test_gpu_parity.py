"""Parity of the HIP path with the fp64 oracle, through the C ABI.

Inputs come from ``exact_attention_flash_amd.inputs`` (the same bf16 bits on
both sides).  Small shapes are compared element by element in full; they
span several tiles and ragged tails.  The five named workloads run at their
full sizes in the launch configuration the bench times, and are compared on
sampled heads / rows that the oracle computes one by one, plus properties
that hold at any size.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from exact_attention_flash_amd import flash_attn_bwd, flash_attn_fwd, flash_attn_fwd_splitkv
from exact_attention_flash_amd.inputs import WORKLOADS, default_scale, make_inputs

from gpu_util import (bf16_to_f64, check_grad, check_lse, check_o, most_items_per_workgroup,
                      to_device)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run_fwd(x, causal, scale):
    q, k, v = (to_device(x[n]) for n in ("q", "k", "v"))
    o, lse = flash_attn_fwd(q, k, v, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    return (q, k, v), o, lse


def _run_fwd_split(x, causal, scale, splits):
    q, k, v = (to_device(x[n]) for n in ("q", "k", "v"))
    o, lse = flash_attn_fwd_splitkv(q, k, v, splits, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    return (q, k, v), o, lse


SMALL_FWD = [
    # (B, H, N, d, causal)
    (1, 1, 128, 64, False),
    (1, 1, 1, 64, False),
    (1, 1, 1, 128, True),
    (1, 2, 63, 64, True),
    (2, 1, 127, 128, False),
    (1, 2, 200, 64, True),
    (1, 1, 1000, 128, True),
    (2, 2, 333, 128, False),
    (1, 3, 513, 64, False),
    (1, 1, 256, 128, True),
    # B*H a multiple of 8 (heads grouped per XCD), several 256-row query
    # blocks with a ragged last one
    (2, 4, 600, 128, True),
    (1, 8, 520, 64, False),
]


@pytest.mark.parametrize("B,H,N,d,causal", SMALL_FWD)
def test_fwd_small_full_parity(B, H, N, d, causal):
    _say(f"fwd small B={B} H={H} N={N} d={d} causal={causal}")
    x = make_inputs(B, H, N, d, seed=N * 7 + d + causal)
    scale = default_scale(d)
    _, o, lse = _run_fwd(x, causal, scale)
    O_ref, L_ref = oracle.attention_forward(x["q"], x["k"], x["v"], scale, causal)
    check_o(bf16_to_f64(o), O_ref, strict=True)
    check_lse(lse.cpu().numpy().astype(np.float64), L_ref)


SPLIT_FWD = [
    # (B, H, N, d, causal, num_splits)
    (1, 1, 128, 64, False, 2),
    (1, 2, 200, 64, True, 3),
    (2, 1, 333, 128, False, 4),
    (1, 1, 1000, 128, True, 7),
    (1, 1, 63, 64, True, 5),      # one key tile: four empty ranges
    (1, 1, 1, 128, False, 3),
    (2, 4, 600, 128, True, 16),   # more ranges than some blocks' tiles
    (1, 3, 513, 64, False, 1),
]


@pytest.mark.parametrize("B,H,N,d,causal,splits", SPLIT_FWD)
def test_fwd_splitkv_small_full_parity(B, H, N, d, causal, splits):
    _say(f"fwd split-KV B={B} H={H} N={N} d={d} causal={causal} splits={splits}")
    x = make_inputs(B, H, N, d, seed=N * 5 + d + causal + splits)
    scale = default_scale(d)
    _, o, lse = _run_fwd_split(x, causal, scale, splits)
    O_ref, L_ref = oracle.attention_forward(x["q"], x["k"], x["v"], scale, causal)
    check_o(bf16_to_f64(o), O_ref)
    check_lse(lse.cpu().numpy().astype(np.float64), L_ref)


DECODE = [
    # (B, H, N_q, N_kv, d, num_splits): a decode step (one query, or a short
    # block of them, against a long key/value cache), full attention
    (1, 16, 1, 16384, 128, 16),
    (1, 16, 1, 16384, 128, 1),
    (2, 4, 1, 1000, 64, 8),
    (1, 8, 64, 8192, 128, 32),
    (1, 2, 7, 5003, 128, 5),
    (1, 4, 1, 65536, 128, 64),
    (2, 3, 300, 70, 64, 3),     # more queries than keys
    (1, 1, 1, 1, 128, 4),       # a single key: three empty ranges
    (1, 1, 33, 130, 64, 128),   # more ranges than key tiles
]


@pytest.mark.parametrize("B,H,Nq,Nk,d,splits", DECODE)
def test_fwd_splitkv_decode_parity(B, H, Nq, Nk, d, splits):
    _say(f"split-KV decode B={B} H={H} N_q={Nq} N_kv={Nk} d={d} splits={splits}")
    xq = make_inputs(B, H, Nq, d, seed=31 * Nq + d)
    xk = make_inputs(B, H, Nk, d, seed=17 * Nk + d + 1)
    scale = default_scale(d)
    q, k, v = to_device(xq["q"]), to_device(xk["k"]), to_device(xk["v"])
    o, lse = flash_attn_fwd_splitkv(q, k, v, splits, causal=False, softmax_scale=scale)
    torch.cuda.synchronize()
    assert o.shape == (B, H, Nq, d) and lse.shape == (B, H, Nq)
    O_ref, L_ref = oracle.attention_forward(xq["q"], xk["k"], xk["v"], scale, False)
    check_o(bf16_to_f64(o), O_ref, strict=True)
    check_lse(lse.cpu().numpy().astype(np.float64), L_ref)


def test_fwd_splitkv_deterministic():
    x = make_inputs(1, 2, 700, 128, seed=5)
    scale = default_scale(128)
    _, o1, l1 = _run_fwd_split(x, True, scale, 5)
    _, o2, l2 = _run_fwd_split(x, True, scale, 5)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_closed_forms(d, causal):
    """Q = 0 gives the (prefix) mean of V and LSE = ln(#visible keys);
    constant V rows give O = that row."""
    N = 300
    x = make_inputs(1, 2, N, d, seed=11)
    x["q"][:] = 0
    scale = default_scale(d)
    _, o, lse = _run_fwd(x, causal, scale)
    v = oracle.widen_bf16(x["v"])
    counts = np.arange(1, N + 1) if causal else np.full(N, N)
    mean = (np.cumsum(v, axis=2) / counts[:, None]) if causal else \
        np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
    check_o(bf16_to_f64(o), mean, "O (Q = 0)")
    check_lse(lse.cpu().numpy().astype(np.float64), np.broadcast_to(np.log(counts), (1, 2, N)))
    y = make_inputs(1, 2, N, d, seed=12)
    y["v"][:] = y["v"][:, :, :1, :]
    _, o2, _ = _run_fwd(y, causal, scale)
    check_o(bf16_to_f64(o2), np.broadcast_to(oracle.widen_bf16(y["v"][:, :, :1, :]), (1, 2, N, d)),
            "O (constant V)")


def test_fwd_deterministic():
    x = make_inputs(2, 3, 777, 128, seed=5)
    _, o1, l1 = _run_fwd(x, True, default_scale(128))
    _, o2, l2 = _run_fwd(x, True, default_scale(128))
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


SMALL_BWD = [
    (1, 1, 128, 64, False),
    (1, 1, 128, 128, True),
    (1, 2, 256, 128, True),
    (1, 1, 200, 64, True),
    (2, 1, 190, 128, False),
    (1, 1, 1, 64, True),
    (1, 2, 77, 128, False),
    (1, 1, 300, 64, False),
    # B*H a multiple of 8 (heads grouped per XCD), ragged blocks
    (2, 4, 333, 128, True),
    (1, 8, 270, 64, False),
]


@pytest.mark.parametrize("B,H,N,d,causal", SMALL_BWD)
def test_bwd_small_full_parity(B, H, N, d, causal):
    _say(f"bwd small B={B} H={H} N={N} d={d} causal={causal}")
    x = make_inputs(B, H, N, d, seed=N * 13 + d + causal, with_dout=True)
    scale = default_scale(d)
    (q, k, v), o, lse = _run_fwd(x, causal, scale)
    do = to_device(x["do"])
    dq, dk, dv = flash_attn_bwd(do, q, k, v, o, lse, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    dQ, dK, dV = oracle.attention_backward(x["q"], x["k"], x["v"], x["do"], scale, causal)
    check_grad(bf16_to_f64(dq), dQ, "dQ")
    check_grad(bf16_to_f64(dk), dK, "dK")
    check_grad(bf16_to_f64(dv), dV, "dV")


# ----------------------------------------------------------------- workloads
def _sample_rows(N, rng, n=96):
    edge = list(range(min(32, N))) + list(range(max(0, N - 32), N))
    mid = rng.choice(N, size=min(n, N), replace=False).tolist()
    return np.unique(np.array(edge + mid, dtype=np.int64))


def _fwd_workload(name, causal, q_mult, full_heads_max, splits=None):
    wl = WORKLOADS[name]
    _say(f"workload {name} causal={causal} q_mult={q_mult} splits={splits} "
         f"shape=({wl.B},{wl.H},{wl.N},{wl.d})")
    x = make_inputs(wl.B, wl.H, wl.N, wl.d, seed=wl.seed, q_mult=q_mult)
    if splits is None:
        _, o, lse = _run_fwd(x, causal, wl.scale)
    else:
        _, o, lse = _run_fwd_split(x, causal, wl.scale, splits)
    o64 = bf16_to_f64(o)
    l64 = lse.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(wl.seed)
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    if len(heads) > full_heads_max:
        pick = rng.choice(len(heads), size=full_heads_max, replace=False)
        heads = [heads[i] for i in sorted(set(pick.tolist()) | {0, len(heads) - 1})]
    stats = []
    lse_err = 0.0
    for b, h in heads:
        rows = np.arange(wl.N) if wl.N <= 2048 else _sample_rows(wl.N, rng, n=48)
        Or, Lr = oracle.attention_forward_rows(x["q"][b, h], x["k"][b, h], x["v"][b, h],
                                               wl.scale, causal, rows)
        stats.append(check_o(o64[b, h, rows], Or, f"O[{b},{h}]", strict=q_mult == 1.0))
        lse_err = max(lse_err, check_lse(l64[b, h, rows], Lr, f"LSE[{b},{h}]"))
    # every head, every row: finite, and LSE >= max visible score is implied
    # by LSE >= ln(1) + ... ; check the cheap bound LSE > -inf and O within
    # the convex hull of V columns
    assert np.all(np.isfinite(o64)) and np.all(np.isfinite(l64))
    v = oracle.widen_bf16(x["v"])
    lo = v.min(axis=2, keepdims=True) - 1e-2
    hi = v.max(axis=2, keepdims=True) + 1e-2
    assert np.all(o64 >= lo - np.abs(lo) * 2**-8) and np.all(o64 <= hi + np.abs(hi) * 2**-8)
    _say(f"  max |dO| {max(s['max_abs_err'] for s in stats):.3e}; max |dLSE| {lse_err:.3e}; "
         f"ulp allowance used {sum(s['needed_ulp_allowance'] for s in stats)}")


ALL_HEADS = 1 << 30


def test_workload_c1():
    _fwd_workload("c1", False, 1.0, ALL_HEADS)


def test_workload_c2():
    _fwd_workload("c2", True, 1.0, ALL_HEADS)


def test_workload_c1_splitkv():
    _fwd_workload("c1", False, 1.0, ALL_HEADS, splits=2)


def test_workload_c2_splitkv():
    _fwd_workload("c2", True, 1.0, ALL_HEADS, splits=4)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("q_mult", [1.0, 8.0])
def test_workload_c3(causal, q_mult):
    _fwd_workload("c3", causal, q_mult, ALL_HEADS)


def test_workload_c4():
    _fwd_workload("c4", True, 1.0, ALL_HEADS)


def test_workload_c5_forward():
    _fwd_workload("c5", True, 1.0, ALL_HEADS)


def test_workload_c5_backward():
    """Full-size C5 forward + backward as the bench runs it, compared element
    by element on every one of the 64 heads: dQ on sampled query rows and
    dK, dV on sampled keys (block edges, the ends and random positions,
    different per head), against the oracle's row-chunked backward, which
    takes every query row of the head into the key gradients."""
    wl = WORKLOADS["c5"]
    _say("workload c5 backward (4,16,4096,128) causal")
    x = make_inputs(wl.B, wl.H, wl.N, wl.d, seed=wl.seed, with_dout=True)
    (q, k, v), o, lse = _run_fwd(x, True, wl.scale)
    do = to_device(x["do"])
    dq, dk, dv = flash_attn_bwd(do, q, k, v, o, lse, causal=True, softmax_scale=wl.scale)
    torch.cuda.synchronize()
    dq64, dk64, dv64 = bf16_to_f64(dq), bf16_to_f64(dk), bf16_to_f64(dv)
    assert np.all(np.isfinite(dq64)) and np.all(np.isfinite(dk64)) and np.all(np.isfinite(dv64))
    rng = np.random.default_rng(wl.seed + 1)
    N = wl.N
    fixed = [0, 1, 63, 64, 127, 128, 255, 256, N // 2, N - 129, N - 128, N - 2, N - 1]
    worst = {"dQ": 0.0, "dK": 0.0, "dV": 0.0}
    for b in range(wl.B):
        for h in range(wl.H):
            idx = np.unique(np.concatenate([fixed, rng.choice(N, 12, replace=False)]))
            xs = {n: x[n][b, h] for n in ("q", "k", "v", "do")}
            dQ, dK, dV = oracle.attention_backward_sampled(xs["q"], xs["k"], xs["v"], xs["do"],
                                                           wl.scale, True, idx, idx)
            worst["dQ"] = max(worst["dQ"], check_grad(dq64[b, h, idx], dQ, f"dQ[{b},{h}]"))
            worst["dK"] = max(worst["dK"], check_grad(dk64[b, h, idx], dK, f"dK[{b},{h}]"))
            worst["dV"] = max(worst["dV"], check_grad(dv64[b, h, idx], dV, f"dV[{b},{h}]"))
    _say("  worst relative errors over 64 heads: " +
         ", ".join(f"{n} {e:.2e}" for n, e in worst.items()))


def test_bwd_deterministic_and_staged_equals_one_call():
    """No atomics anywhere: two backward runs give bit-identical dQ, dK, dV,
    and the three staged entry points (in either order of the two passes)
    give exactly what flash_attn_bwd gives."""
    from exact_attention_flash_amd import (flash_attn_bwd_kv_blocks, flash_attn_bwd_preprocess,
                                           flash_attn_bwd_q_blocks, flash_attn_bwd_workspace_bytes)
    B, H, N, d = 2, 3, 333, 128
    x = make_inputs(B, H, N, d, seed=99, with_dout=True)
    scale = default_scale(d)
    (q, k, v), o, lse = _run_fwd(x, True, scale)
    do = to_device(x["do"])
    r1 = flash_attn_bwd(do, q, k, v, o, lse, causal=True, softmax_scale=scale)
    r2 = flash_attn_bwd(do, q, k, v, o, lse, causal=True, softmax_scale=scale)
    ws = torch.empty(flash_attn_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    flash_attn_bwd_preprocess(do, o, lse, ws)
    flash_attn_bwd_q_blocks(do, q, k, v, dq, ws, causal=True, softmax_scale=scale)
    flash_attn_bwd_kv_blocks(do, q, k, v, dk, dv, ws, causal=True, softmax_scale=scale)
    torch.cuda.synchronize()
    for a_, b_, c_ in zip(r1, r2, (dq, dk, dv)):
        assert torch.equal(a_.view(torch.int16), b_.view(torch.int16))
        assert torch.equal(a_.view(torch.int16), c_.view(torch.int16))


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_constant_v_gives_zero_dq_dk(d):
    """Constant V rows make O independent of S, so dQ = dK = 0 exactly in
    exact arithmetic; on the GPU they are tiny relative to dV."""
    N = 260
    x = make_inputs(1, 2, N, d, seed=31, with_dout=True)
    x["v"][:] = x["v"][:, :, :1, :]
    scale = default_scale(d)
    (q, k, v), o, lse = _run_fwd(x, True, scale)
    dq, dk, dv = flash_attn_bwd(to_device(x["do"]), q, k, v, o, lse, causal=True,
                                softmax_scale=scale)
    torch.cuda.synchronize()
    gv = bf16_to_f64(dv)
    assert np.abs(bf16_to_f64(dq)).max() <= 5e-2 * np.abs(gv).max()
    assert np.abs(bf16_to_f64(dk)).max() <= 5e-2 * np.abs(gv).max()


LONG = [
    # (B, H, N, d, causal): a head 1.5 times as long as the longest named
    # workload, and a long ragged one
    (1, 1, 24576, 128, True),
    (1, 1, 20001, 64, False),
]


@pytest.mark.parametrize("B,H,N,d,causal", LONG)
def test_long_sequence_fwd_bwd(B, H, N, d, causal):
    """Forward and backward on one long head, checked on sampled query rows
    (O, LSE, dQ) and keys (dK, dV): block edges, the tail and random
    positions, against the oracle's row-chunked backward."""
    _say(f"long sequence ({B},{H},{N},{d}) causal={causal}")
    x = make_inputs(B, H, N, d, seed=N + d, with_dout=True)
    scale = default_scale(d)
    (q, k, v), o, lse = _run_fwd(x, causal, scale)
    do = to_device(x["do"])
    dq, dk, dv = flash_attn_bwd(do, q, k, v, o, lse, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(N)
    idx = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 255, 256, N // 2, N - 2, N - 1],
                                    rng.choice(N, 29, replace=False)]))
    xs = {n: x[n][0, 0] for n in ("q", "k", "v", "do")}
    Or, Lr = oracle.attention_forward_rows(xs["q"], xs["k"], xs["v"], scale, causal, idx)
    check_o(bf16_to_f64(o)[0, 0, idx], Or, "O")
    check_lse(lse.cpu().numpy().astype(np.float64)[0, 0, idx], Lr, "LSE")
    dQ, dK, dV = oracle.attention_backward_sampled(xs["q"], xs["k"], xs["v"], xs["do"], scale,
                                                   causal, idx, idx)
    check_grad(bf16_to_f64(dq)[0, 0, idx], dQ, "dQ")
    check_grad(bf16_to_f64(dk)[0, 0, idx], dK, "dK")
    check_grad(bf16_to_f64(dv)[0, 0, idx], dV, "dV")


@pytest.mark.parametrize("d", [64, 128])
def test_fwd_stale_max_rounding(d):
    """The forward moves its running max only when a tile raises it by more
    than 2^8 (in log2 units), so a later tile's largest probability can be
    some 2^x > 1 whose bf16 rounding feeds the P V product.  Here every query
    sees key A (score 0, tile 0), key B in tile 3 with probability 2^x in
    [128.3, 128.45] relative to A (rounded to 128 in bf16, 0.3% low), and 254
    keys at score -100; every V row is the same vector v, so the exact O is v
    whatever the weights.  Dividing by the unrounded row sum would put O 0.3%
    low, one bf16 ulp off in every element; with each tile's rounding
    correction in the divisor O comes out as v exactly."""
    from exact_attention_flash_amd.inputs import f32_to_bf16_bits
    _say(f"stale-max rounding d={d}")
    B, H, N = 1, 2, 256
    scale = default_scale(d)
    sl2 = np.float32(scale) * np.float32(1.4426950408889634)
    # key B's score: 4 a + b for bf16 a, b, chosen so that 2^(s sl2) rounds down by ~0.3%
    best = None
    for a in (f32_to_bf16_bits(np.float32(x)) for x in np.arange(8.0, 16.0, 0.0625)):
        af = float(oracle.widen_bf16(np.asarray(a).reshape(1))[0])
        for bb in f32_to_bf16_bits(np.linspace(0.0, 0.5, 257).astype(np.float32)):
            bf = float(oracle.widen_bf16(np.asarray(bb).reshape(1))[0])
            xs = np.float32(np.float32(4.0 * af + bf) * sl2)
            if 128.3 <= 2.0 ** float(xs) <= 128.45:
                best = (af, bf)
                break
        if best:
            break
    assert best is not None
    q = np.zeros((B, H, N, d), np.float32)
    q[..., 0], q[..., 1] = 4.0, 1.0
    k = np.zeros((B, H, N, d), np.float32)
    k[..., 0] = -25.0                  # score -100 for every other key
    k[:, :, 5, 0] = 0.0                # key A, tile 0: score 0
    k[:, :, 200, 0], k[:, :, 200, 1] = best   # key B, tile 3
    v_row = (1.875 * 2.0 ** (np.arange(d) % 4 - 2) * (-1.0) ** np.arange(d)).astype(np.float32)
    v = np.broadcast_to(v_row, (B, H, N, d)).copy()
    x = {"q": f32_to_bf16_bits(q), "k": f32_to_bf16_bits(k), "v": f32_to_bf16_bits(v)}
    (_, _, _), o, lse = _run_fwd(x, False, scale)
    o64 = bf16_to_f64(o)
    err = np.abs(o64 - v_row.astype(np.float64)).max()
    assert err == 0.0, f"O off v by {err:.3e} (the divisor lacks the bf16 rounding of p_max)"
    _, L_ref = oracle.attention_forward(x["q"], x["k"], x["v"], scale, False)
    check_lse(lse.cpu().numpy().astype(np.float64), L_ref)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("pattern", ["rising", "falling", "large"])
def test_fwd_extreme_logits(d, causal, pattern):
    """The lazy running max under stress: scores that rise along the keys by
    more than the rescale threshold per key tile (the max moves on every
    tile), scores that fall along the keys (it never moves after the first),
    and random logits reaching ~350 (Q scaled by 64, exact in bf16); all
    against the oracle."""
    from exact_attention_flash_amd.inputs import f32_to_bf16_bits
    _say(f"extreme logits {pattern} d={d} causal={causal}")
    B, H, N = 1, 2, 700
    x = make_inputs(B, H, N, d, seed=13 + d)
    rng = np.random.default_rng(d + causal)
    scale = default_scale(d)
    if pattern == "large":
        q = oracle.widen_bf16(x["q"]).astype(np.float32) * 64.0
        x["q"] = f32_to_bf16_bits(q)
    else:
        u = rng.standard_normal(d).astype(np.float32)
        u /= np.linalg.norm(u)
        ramp = np.linspace(0.0, 1.0, N, dtype=np.float32)
        if pattern == "falling":
            ramp = ramp[::-1].copy()
        # s_ij = scale * (q_i . u) * c * ramp_j with q_i . u = 1: spans 0 .. 3000
        c = np.float32(3000.0 / scale)
        q = np.broadcast_to(u, (B, H, N, d)) + 0.01 * rng.standard_normal((B, H, N, d))
        k = (c * ramp)[None, None, :, None] * u[None, None, None, :] \
            + 0.01 * rng.standard_normal((B, H, N, d))
        x["q"] = f32_to_bf16_bits(q.astype(np.float32))
        x["k"] = f32_to_bf16_bits(k.astype(np.float32))
    x["do"] = make_inputs(B, H, N, d, seed=77 + d, with_dout=True)["do"]
    (q, k, v), o, lse = _run_fwd(x, causal, scale)
    O_ref, L_ref = oracle.attention_forward(x["q"], x["k"], x["v"], scale, causal)
    check_o(bf16_to_f64(o), O_ref, f"O ({pattern})")
    # Backward on the same inputs.  P is close to one-hot here, so the exact
    # dS = P (dP - D) nearly vanishes while the bf16 rounding of O (which
    # forms D = rowsum(dO * O)) moves it by ~2^-9 |dO . O|: dQ and dK are
    # ill-conditioned against a bar relative to their own maximum and are
    # only checked for finiteness; dV = P^T dO is well-conditioned.
    dq, dk, dv = flash_attn_bwd(to_device(x["do"]), q, k, v, o, lse, causal=causal,
                                softmax_scale=scale)
    torch.cuda.synchronize()
    _, _, dV = oracle.attention_backward(x["q"], x["k"], x["v"], x["do"], scale, causal)
    check_grad(bf16_to_f64(dv), dV, f"dV ({pattern})")
    assert np.all(np.isfinite(bf16_to_f64(dq))) and np.all(np.isfinite(bf16_to_f64(dk)))
    l64 = lse.cpu().numpy().astype(np.float64)
    # Scores reach ~3000 here. Each fp32 rounding on the way to the LSE (the
    # dot product's accumulation, the scale and base-2 conversions, the max
    # and the final log) costs up to 2^-24 of that magnitude: allow 32 of
    # them on top of the usual 1e-3.
    assert np.all(np.isfinite(l64))
    bound = 1e-3 + 32 * 2.0 ** -24 * np.abs(L_ref).max()
    assert np.abs(l64 - L_ref).max() <= bound, (np.abs(l64 - L_ref).max(), bound)


WALKS = [
    # (B, H, N, d, causal) and the walks each gives on a 256-CU device (one
    # workgroup per CU; 256-row forward items, 128-key key-block items):
    (1, 8, 5000, 128, True),    # key blocks: 320 items, snake order, partial second round
    (1, 8, 5000, 64, False),    # the same walk, full attention, d = 64
    (3, 5, 2100, 128, True),    # key blocks: 255 items on 248 workgroups, round robin
    (2, 20, 4096, 64, True),    # key blocks: 1280 items, snake order over five rounds
    (2, 20, 4096, 128, False),  # forward 640 items, key blocks 1280: full attention, d = 128
    (1, 33, 2100, 128, True),   # forward 297 and key blocks 561 items: round robin in both
]


@pytest.mark.parametrize("B,H,N,d,causal", WALKS)
def test_bwd_key_block_walk(B, H, N, d, causal):
    """Backward where the persistent key-block pass gives workgroups several
    items (and an odd number of rounds, a partial last round, or the round
    robin fallback): dK and dV on sampled keys, dQ on sampled rows, of four
    heads, against the oracle's row-chunked backward; O and LSE of the
    persistent forward (several query blocks per workgroup on the largest
    shape) on the same rows."""
    _say(f"key-block walk ({B},{H},{N},{d}) causal={causal}")
    fwd_items = B * H * -(-N // 256)
    kv_items = B * H * -(-N // 128)
    # the case must give some workgroup of the key-block pass (and, where
    # the comment above says so, of the forward) more than one item here
    assert most_items_per_workgroup(kv_items) > 1, kv_items
    _say(f"  forward items {fwd_items} (<= {most_items_per_workgroup(fwd_items)} per workgroup), "
         f"key-block items {kv_items} (<= {most_items_per_workgroup(kv_items)})")
    x = make_inputs(B, H, N, d, seed=7 * N + d, with_dout=True)
    scale = default_scale(d)
    (q, k, v), o, lse = _run_fwd(x, causal, scale)
    dq, dk, dv = flash_attn_bwd(to_device(x["do"]), q, k, v, o, lse, causal=causal,
                                softmax_scale=scale)
    torch.cuda.synchronize()
    dq64, dk64, dv64 = bf16_to_f64(dq), bf16_to_f64(dk), bf16_to_f64(dv)
    o64, lse64 = bf16_to_f64(o), lse.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(N + H)
    idx = np.unique(np.concatenate([[0, 63, 64, 127, 128, N - 1], rng.choice(N, 18, replace=False)]))
    BH = B * H
    for bh in sorted({0, BH - 1, int(rng.integers(BH)), int(rng.integers(BH))}):
        b, h = divmod(bh, H)
        xs = {n: x[n][b, h] for n in ("q", "k", "v", "do")}
        Or, Lr = oracle.attention_forward_rows(xs["q"], xs["k"], xs["v"], scale, causal, idx)
        check_o(o64[b, h, idx], Or, f"O head {bh}")
        check_lse(lse64[b, h, idx], Lr, f"LSE head {bh}")
        dQ, dK, dV = oracle.attention_backward_sampled(xs["q"], xs["k"], xs["v"], xs["do"], scale,
                                                       causal, idx, idx)
        check_grad(dq64[b, h, idx], dQ, f"dQ head {bh}")
        check_grad(dk64[b, h, idx], dK, f"dK head {bh}")
        check_grad(dv64[b, h, idx], dV, f"dV head {bh}")
