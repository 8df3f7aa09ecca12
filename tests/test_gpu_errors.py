"""Error paths of the Python binding and the C ABI with real device tensors.

Every call here is rejected on the host before any launch (the binding's
tensor checks or the library's synchronous validation), so nothing runs on
the GPU; a valid call afterwards shows that the library is still usable.
"""

import sys

import pytest
import torch

from exact_attention_flash_amd import (FlashAttnError, flash_attn_bwd, flash_attn_fwd,
                                       flash_attn_fwd_dropout, flash_attn_fwd_fp8,
                                       flash_attn_fwd_splitkv, flash_attn_quantize_fp8)

pytestmark = pytest.mark.gpu

BAD_SHAPE, HEADDIM, BAD_SCALE, WS_SMALL, ALIAS, BAD_SPLITS, BAD_DESCALE, BAD_DROPOUT = \
    2, 3, 5, 6, 8, 9, 10, 11


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _qkv(B=1, H=2, N=40, d=64, dtype=torch.bfloat16):
    return tuple(torch.randn(B, H, N, d, device="cuda").to(dtype) for _ in range(3))


def _status(fn, *a, **kw):
    with pytest.raises(FlashAttnError) as e:
        fn(*a, **kw)
    return e.value.status


def test_binding_tensor_checks():
    _say("binding tensor checks")
    q, k, v = _qkv()
    with pytest.raises(ValueError):                       # not contiguous
        flash_attn_fwd(q.transpose(2, 3), k.transpose(2, 3), v.transpose(2, 3))
    with pytest.raises(ValueError):                       # shapes differ
        flash_attn_fwd(q, k[:, :, :20], v)
    with pytest.raises(TypeError):                        # dtype
        flash_attn_fwd(q.half(), k.half(), v.half())
    with pytest.raises(ValueError):                       # 3-D
        flash_attn_fwd(q[0], k[0], v[0])
    with pytest.raises(ValueError):                       # LSE of the wrong shape
        flash_attn_fwd(q, k, v, lse=torch.empty(1, 2, 39, device="cuda"))
    with pytest.raises(ValueError):                       # seed past 64 bits
        flash_attn_fwd_dropout(q, k, v, 0.1, 1 << 64)
    x = q.reshape(-1, 64).contiguous()
    with pytest.raises(ValueError):                       # signs of the wrong length
        flash_attn_quantize_fp8(x, torch.ones(32, device="cuda"))


def test_library_rejections():
    _say("library rejections")
    q, k, v = _qkv()
    q96, k96, v96 = _qkv(d=96)
    assert _status(flash_attn_fwd, q96, k96, v96) == HEADDIM
    for bad in (float("nan"), 0.0, -1.0, float("inf")):
        assert _status(flash_attn_fwd, q, k, v, softmax_scale=bad) == BAD_SCALE
    assert _status(flash_attn_fwd, q, k, v, out=q) == ALIAS            # output on an input
    for splits in (0, 129):
        assert _status(flash_attn_fwd_splitkv, q, k, v, splits) == BAD_SPLITS
    for p in (1.0, -0.1, float("nan"), 0.999):
        assert _status(flash_attn_fwd_dropout, q, k, v, p, 7) == BAD_DROPOUT
    q8 = torch.zeros(1, 2, 40, 64, dtype=torch.uint8, device="cuda")
    for ds in (0.0, -1.0, float("nan"), float("inf")):
        assert _status(flash_attn_fwd_fp8, q8, q8, q8, ds, 1.0, 1.0) == BAD_DESCALE
    o, lse = flash_attn_fwd(q, k, v)
    do = torch.randn_like(q)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    assert _status(flash_attn_bwd, do, q, k, v, o, lse, workspace=small) == WS_SMALL
    x = q.reshape(-1, 64).contiguous()
    assert _status(flash_attn_quantize_fp8, x, workspace=torch.empty(1, device="cuda")) == WS_SMALL
    torch.cuda.synchronize()
    # the library is still usable after the rejected calls, and equal inputs
    # give equal outputs
    o2, lse2 = flash_attn_fwd(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2)


def test_empty_inputs_return_empty_outputs():
    _say("empty inputs")
    for shape in ((0, 2, 16, 64), (1, 0, 16, 128), (1, 2, 0, 64)):
        q = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        o, lse = flash_attn_fwd(q, q.clone(), q.clone(), causal=True)
        assert o.shape == q.shape and lse.shape == shape[:3]
        dq, dk, dv = flash_attn_bwd(q.clone(), q, q.clone(), q.clone(), o, lse, causal=True)
        assert dq.shape == dk.shape == dv.shape == q.shape
    torch.cuda.synchronize()
