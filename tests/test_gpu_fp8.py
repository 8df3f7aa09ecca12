"""Parity of the FP8 (E4M3) forward with the fp64 oracle, through the C ABI.

Inputs are E4M3 codes with per-tensor amax descales from
``exact_attention_flash_amd.inputs.make_inputs_fp8``; the oracle decodes the
same codes exactly.  O is held to the bound derived from the kernel's E4M3
rounding of the probabilities (``gpu_util.check_o_fp8``); LSE, which the
kernel computes from unrounded probabilities, to the bf16 path's 1e-3; and
cases where the rounding is exact (all probabilities equal) to the bf16
path's O bar.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from exact_attention_flash_amd import flash_attn_fwd_fp8
from exact_attention_flash_amd.inputs import default_scale, make_inputs_fp8

from gpu_util import (bf16_to_f64, check_lse, check_o, check_o_fp8, fp8_error_terms,
                      most_items_per_workgroup,
                      fp8_to_device)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(x, causal, scale, **kw):
    q, k, v = (fp8_to_device(x[n]) for n in ("q", "k", "v"))
    o, lse = flash_attn_fwd_fp8(q, k, v, x["descale_q"], x["descale_k"], x["descale_v"],
                                causal=causal, softmax_scale=scale, **kw)
    torch.cuda.synchronize()
    return o, lse


def _deq(x):
    return tuple(oracle.dequantize(x[n], x["descale_" + n]) for n in ("q", "k", "v"))


def _check_full(x, o, lse, causal, scale):
    O_ref, L_ref = oracle.attention_forward_fp8(x["q"], x["k"], x["v"], x["descale_q"],
                                                x["descale_k"], x["descale_v"], scale, causal)
    q, k, v = _deq(x)
    B, H = q.shape[:2]
    terms = [fp8_error_terms(q[b, h], k[b, h], v[b, h], scale, causal)
             for b in range(B) for h in range(H)]
    shape = q.shape
    a_abs, floor, sig2 = (np.stack([t[i] for t in terms]).reshape(shape) for i in range(3))
    res = check_o_fp8(bf16_to_f64(o), O_ref, a_abs, floor, sig2)
    check_lse(lse.cpu().numpy().astype(np.float64), L_ref)
    return res


SMALL_FP8 = [
    # (B, H, N, d, causal, q_mult)
    (1, 1, 128, 64, False, 1.0),
    (1, 1, 1, 64, False, 1.0),
    (1, 1, 1, 128, True, 1.0),
    (1, 2, 63, 64, True, 1.0),
    (2, 1, 127, 128, False, 1.0),
    (1, 2, 200, 64, True, 1.0),
    (1, 1, 1000, 128, True, 1.0),
    (2, 2, 333, 128, False, 1.0),
    (1, 3, 513, 64, False, 1.0),
    (1, 1, 256, 128, True, 1.0),
    # B*H a multiple of 8 (heads grouped per XCD), ragged last query block
    (2, 4, 600, 128, True, 1.0),
    (1, 8, 520, 64, False, 1.0),
    # large logits: Q times 8
    (1, 2, 300, 128, True, 8.0),
    (1, 4, 257, 64, False, 8.0),
]


@pytest.mark.parametrize("B,H,N,d,causal,q_mult", SMALL_FP8)
def test_fwd_fp8_small_full_parity(B, H, N, d, causal, q_mult):
    _say(f"fp8 fwd small B={B} H={H} N={N} d={d} causal={causal} q_mult={q_mult}")
    x = make_inputs_fp8(B, H, N, d, seed=N * 3 + d + causal, q_mult=q_mult)
    scale = default_scale(d)
    o, lse = _run(x, causal, scale)
    res = _check_full(x, o, lse, causal, scale)
    _say(f"  max err {res['max_abs_err']:.3e} rms {res['rms']:.3e} (model {res['rms_pred']:.3e})")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_fp8_equal_probabilities(d, causal):
    """Q = 0: every visible key has the same probability, which E4M3 holds
    exactly, so O is the (prefix) mean of the dequantised V to bf16
    rounding and LSE = ln(#visible keys)."""
    _say(f"fp8 fwd Q=0 d={d} causal={causal}")
    N = 300
    x = make_inputs_fp8(1, 2, N, d, seed=21)
    x["q"][:] = 0
    scale = default_scale(d)
    o, lse = _run(x, causal, scale)
    v = oracle.dequantize(x["v"], x["descale_v"])
    counts = np.arange(1, N + 1) if causal else np.full(N, N)
    mean = (np.cumsum(v, axis=2) / counts[:, None]) if causal else \
        np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
    check_o(bf16_to_f64(o), mean, "O (Q = 0)")
    check_lse(lse.cpu().numpy().astype(np.float64), np.broadcast_to(np.log(counts), (1, 2, N)))


def test_fwd_fp8_descales():
    """O scales with descale_v exactly (a power of two commutes with the
    bf16 rounding); only the product descale_q * descale_k matters."""
    _say("fp8 fwd descale identities")
    x = make_inputs_fp8(2, 2, 400, 128, seed=31)
    scale = default_scale(128)
    o1, l1 = _run(x, True, scale)
    y = dict(x, descale_v=2 * x["descale_v"])
    o2, l2 = _run(y, True, scale)
    assert torch.equal(o2.float(), 2 * o1.float()) and torch.equal(l1, l2)
    z = dict(x, descale_q=x["descale_k"], descale_k=x["descale_q"])
    o3, l3 = _run(z, True, scale)
    assert torch.equal(o3.view(torch.int16), o1.view(torch.int16)) and torch.equal(l3, l1)


def test_fwd_fp8_deterministic():
    x = make_inputs_fp8(2, 3, 777, 128, seed=5)
    o1, l1 = _run(x, True, default_scale(128))
    o2, l2 = _run(x, True, default_scale(128))
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_fwd_fp8_accepts_float8_dtype_and_out_buffers():
    x = make_inputs_fp8(1, 2, 130, 64, seed=7)
    o1, l1 = _run(x, False, 0.125)
    q, k, v = (fp8_to_device(x[n]).view(torch.float8_e4m3fn) for n in ("q", "k", "v"))
    out = torch.full_like(o1, float("nan"))
    lse = torch.full_like(l1, float("nan"))
    flash_attn_fwd_fp8(q, k, v, x["descale_q"], x["descale_k"], x["descale_v"],
                       softmax_scale=0.125, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), o1.view(torch.int16)) and torch.equal(lse, l1)


# Full-size shapes of the long-context and fwd+bwd workloads, in FP8, in the
# configuration the bench times; compared on sampled rows of sampled heads.
FULL_FP8 = [
    # (name, B, H, N, d, causal, seed)
    ("c4-fp8", 1, 16, 16384, 128, True, 4100),
    ("c5-fp8", 4, 16, 4096, 128, True, 5100),
    ("c3-fp8", 16, 12, 1024, 64, False, 3100),
]


@pytest.mark.parametrize("name,B,H,N,d,causal,seed", FULL_FP8)
def test_fwd_fp8_full_size_sampled(name, B, H, N, d, causal, seed):
    _say(f"fp8 fwd full size {name}: B={B} H={H} N={N} d={d} causal={causal}")
    x = make_inputs_fp8(B, H, N, d, seed=seed)
    scale = default_scale(d)
    o, lse = _run(x, causal, scale)
    o_all = o.float()
    assert bool(torch.isfinite(o_all).all()) and bool(torch.isfinite(lse).all())
    rng = np.random.default_rng(seed)
    heads = [(0, 0), (B - 1, H - 1), (int(rng.integers(B)), int(rng.integers(H)))]
    rows = np.unique(np.concatenate([[0, 1, 255, 256, N - 257, N - 2, N - 1],
                                     rng.integers(0, N, 25)]))
    for b, h in heads:
        xs = {n: x[n][b, h] for n in ("q", "k", "v")}
        O_ref, L_ref = oracle.attention_forward_fp8_rows(
            xs["q"], xs["k"], xs["v"], x["descale_q"], x["descale_k"], x["descale_v"],
            scale, causal, rows)
        q = oracle.dequantize(xs["q"], x["descale_q"])
        k = oracle.dequantize(xs["k"], x["descale_k"])
        v = oracle.dequantize(xs["v"], x["descale_v"])
        a_abs, floor, sig2 = fp8_error_terms(q, k, v, scale, causal, rows)
        og = bf16_to_f64(o[b, h][torch.as_tensor(rows, device=o.device)])
        check_o_fp8(og, O_ref, a_abs, floor, sig2, f"O (fp8) head {b},{h}")
        check_lse(lse[b, h].cpu().numpy()[rows].astype(np.float64), L_ref)


# Shapes whose persistent FP8 forward gives some workgroup more than one
# (head, 256-row query block) item: snake order and the round-robin
# fallback (item count not a multiple of 8), both masks, both head dims.
WALKS_FP8 = [
    # (B, H, N, d, causal, seed)
    (2, 20, 4096, 128, False, 6100),   # 640 items
    (1, 33, 2100, 128, True, 6101),    # 297 items: round robin
    (2, 20, 4096, 64, True, 6102),     # 640 items, d = 64
    (1, 33, 2100, 64, False, 6103),    # 297 items, d = 64, full attention
]


@pytest.mark.parametrize("B,H,N,d,causal,seed", WALKS_FP8)
def test_fwd_fp8_walk(B, H, N, d, causal, seed):
    _say(f"fp8 fwd walk B={B} H={H} N={N} d={d} causal={causal}")
    items = B * H * -(-N // 256)
    assert most_items_per_workgroup(items) > 1, items
    x = make_inputs_fp8(B, H, N, d, seed=seed)
    scale = default_scale(d)
    o, lse = _run(x, causal, scale)
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, 255, 256, N - 1], rng.integers(0, N, 12)]))
    BH = B * H
    for bh in sorted({0, BH - 1, int(rng.integers(BH))}):
        b, h = divmod(bh, H)
        xs = {n: x[n][b, h] for n in ("q", "k", "v")}
        O_ref, L_ref = oracle.attention_forward_fp8_rows(
            xs["q"], xs["k"], xs["v"], x["descale_q"], x["descale_k"], x["descale_v"],
            scale, causal, rows)
        q = oracle.dequantize(xs["q"], x["descale_q"])
        k = oracle.dequantize(xs["k"], x["descale_k"])
        v = oracle.dequantize(xs["v"], x["descale_v"])
        a_abs, floor, sig2 = fp8_error_terms(q, k, v, scale, causal, rows)
        og = bf16_to_f64(o[b, h][torch.as_tensor(rows, device=o.device)])
        check_o_fp8(og, O_ref, a_abs, floor, sig2, f"O (fp8) head {bh}")
        check_lse(lse[b, h].cpu().numpy()[rows].astype(np.float64), L_ref)


# ------------------------------------------------- quantisation and incoherent processing
from exact_attention_flash_amd import flash_attn_quantize_fp8
from exact_attention_flash_amd.inputs import f32_to_bf16_bits, make_inputs

from gpu_util import bf16_to_f64 as _bf, to_device as _dev

_E4M3_VALS = np.sort(np.unique(np.abs(oracle.decode_e4m3(np.arange(0x7F, dtype=np.uint8)))))


def _step_distance(c1, c2):
    """Distance between codes in units of representable steps (same sign)."""
    v1, v2 = oracle.decode_e4m3(c1), oracle.decode_e4m3(c2)
    i1 = np.searchsorted(_E4M3_VALS, np.abs(v1)) * np.sign(v1)
    i2 = np.searchsorted(_E4M3_VALS, np.abs(v2)) * np.sign(v2)
    return np.abs(i1 - i2)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("rotate", [False, True])
def test_quantize_parity(d, rotate):
    _say(f"fp8 quantize d={d} rotate={rotate}")
    x = make_inputs(2, 3, 150, d, seed=60 + d + rotate)["q"]
    xt = _dev(x)
    rng = np.random.default_rng(d)
    signs = rng.choice([-1.0, 1.0], d).astype(np.float32) if rotate else None
    codes, ds = flash_attn_quantize_fp8(xt, None if signs is None else torch.from_numpy(signs).cuda())
    torch.cuda.synchronize()
    cg = codes.cpu().numpy()
    dsg = float(ds.item())
    xf = oracle.widen_bf16(x)
    ref_codes, ref_ds = oracle.quantize_e4m3(xf, signs)
    if not rotate:
        assert dsg == ref_ds                  # exact amax, correctly rounded division
    else:
        assert abs(dsg - ref_ds) <= 1e-6 * ref_ds
    # the codes of the oracle's y under the GPU's descale
    y = xf if signs is None else oracle.incoherent_rotation(xf, signs)
    expect = oracle.encode_e4m3(y / dsg)
    dist = _step_distance(cg, expect)
    assert dist.max() <= 1, f"codes off by {dist.max()} steps"
    assert (cg == expect).mean() >= (1.0 if not rotate else 0.999), (cg == expect).mean()
    assert int(np.max(np.abs(oracle.decode_e4m3(cg)))) == 448


@pytest.mark.parametrize("amax", [4.0, 5.3125])
@pytest.mark.parametrize("rotate", [False, True])
def test_quantize_ties_and_grid_stride(amax, rotate):
    """amax with a short mantissa puts x / descale within an fp32 ulp or two
    of a code boundary for whole classes of bf16 mantissas (about 1 % of the
    elements here): the exact path must settle each one.  70001 rows also exceed what one
    pass of either grid covers, so every workgroup strides, and leave a
    ragged last block."""
    d, rows = 128, 70001
    _say(f"fp8 quantize ties amax={amax} rotate={rotate} rows={rows}")
    rng = np.random.default_rng(int(amax * 16) + rotate)
    xf = np.clip(rng.standard_normal((rows, d)), -3.0, 3.0).astype(np.float32)
    xf[rows // 2, 7] = amax                                   # the largest |x|
    x = f32_to_bf16_bits(xf)
    signs = rng.choice([-1.0, 1.0], d).astype(np.float32) if rotate else None
    codes, ds = flash_attn_quantize_fp8(_dev(x), None if signs is None else torch.from_numpy(signs).cuda())
    torch.cuda.synchronize()
    cg = codes.cpu().numpy()
    dsg = float(ds.item())
    xw = oracle.widen_bf16(x)
    ref_codes, ref_ds = oracle.quantize_e4m3(xw, signs)
    if rotate:
        assert abs(dsg - ref_ds) <= 1e-6 * ref_ds
        y = oracle.incoherent_rotation(xw, signs)
        expect = oracle.encode_e4m3(y / dsg)
        assert _step_distance(cg, expect).max() <= 1
        assert (cg == expect).mean() >= 0.999
    else:
        assert dsg == ref_ds
        a = np.abs(xw / dsg).ravel()
        mids = (_E4M3_VALS[1:] + _E4M3_VALS[:-1]) / 2
        i = np.clip(np.searchsorted(mids, a), 1, len(mids) - 1)
        gap = np.minimum(np.abs(a - mids[i - 1]), np.abs(a - mids[i]))
        near = int((gap < a * 2.0 ** -20).sum())             # within a few fp32 ulps of a midpoint
        _say(f"  quotients next to a midpoint: {near}")
        assert near > 1000                                    # the case this test is for
        np.testing.assert_array_equal(cg, ref_codes)


def test_incoherent_processing_lowers_fp8_error():
    """The pages' claim end to end on the GPU: with four large channels in Q
    and K, FP8 attention over rotated-then-quantised Q and K is closer to the
    exact bf16-input attention than over plainly quantised ones."""
    B, H, N, d = 1, 4, 512, 128
    x = make_inputs(B, H, N, d, seed=77)
    for n in ("q", "k"):
        v = oracle.widen_bf16(x[n]).astype(np.float32)
        v[..., :4] *= 32.0                     # a power of two: still exact in bf16
        x[n] = f32_to_bf16_bits(v)
    scale = default_scale(d)
    O_ref, L_ref = oracle.attention_forward(x["q"], x["k"], x["v"], scale, False)
    signs = torch.from_numpy(np.random.default_rng(1).choice([-1.0, 1.0], d).astype(np.float32)).cuda()
    q, k, v = (_dev(x[n]) for n in ("q", "k", "v"))
    v8, dv = flash_attn_quantize_fp8(v)
    err = {}
    for name, sg in (("plain", None), ("rotated", signs)):
        q8, dq = flash_attn_quantize_fp8(q, sg)
        k8, dk = flash_attn_quantize_fp8(k, sg)
        o, lse = flash_attn_fwd_fp8(q8, k8, v8, dq.item(), dk.item(), dv.item(), softmax_scale=scale)
        torch.cuda.synchronize()
        err[name] = (float(np.sqrt(np.mean((_bf(o) - O_ref) ** 2))),
                     float(np.max(np.abs(lse.cpu().numpy() - L_ref))))
    _say(f"  O rms error plain {err['plain'][0]:.3e} rotated {err['rotated'][0]:.3e}; "
         f"LSE max error plain {err['plain'][1]:.3e} rotated {err['rotated'][1]:.3e}")
    assert err["rotated"][0] < 0.6 * err["plain"][0]
    assert err["rotated"][1] < 0.6 * err["plain"][1]
