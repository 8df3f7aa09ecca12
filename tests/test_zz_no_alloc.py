"""The allocation-free backward entry point against the one with a caller
workspace, through the C ABI: same kernels, so the outputs must be
bit-identical, on two calls in a row with the second problem smaller (the
static scratch keeps the first call's contents)."""

import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_attention_flash_amd import binding as fa
from exact_attention_flash_amd.inputs import default_scale, make_inputs

from gpu_util import bf16_to_f64, check_grad, to_device

pytestmark = pytest.mark.gpu

SCRATCH_TOO_SMALL = 12


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _noalloc(lib, do, q, k, v, o, lse, dq, dk, dv, causal, scale):
    B, H, N, d = q.shape
    return lib.flash_attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                      lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                      dv.data_ptr(), B, H, N, d, int(causal), scale,
                                      int(torch.cuda.current_stream().cuda_stream))


def test_noalloc_matches_workspace_entry_point():
    lib = fa.load_library()
    # the second problem is smaller than the first
    for B, H, N, d, causal in ((2, 4, 1333, 128, True), (1, 2, 100, 64, False)):
        _say(f"noalloc bwd B={B} H={H} N={N} d={d} causal={causal}")
        x = make_inputs(B, H, N, d, seed=400 + N, with_dout=True)
        scale = default_scale(d)
        q, k, v, do = (to_device(x[n]) for n in ("q", "k", "v", "do"))
        o, lse = fa.flash_attn_fwd(q, k, v, causal=causal, softmax_scale=scale)
        ref = fa.flash_attn_bwd(do, q, k, v, o, lse, causal=causal, softmax_scale=scale)
        dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
        assert _noalloc(lib, do, q, k, v, o, lse, dq, dk, dv, causal, scale) == 0
        torch.cuda.synchronize()
        for r, g in zip(ref, (dq, dk, dv)):
            assert torch.equal(r.view(torch.int16), g.view(torch.int16))
        # and to the parity bar against the oracle (one head)
        b, h = B - 1, H - 1
        dQ, dK, dV = oracle.attention_backward(x["q"][b:b + 1, h:h + 1], x["k"][b:b + 1, h:h + 1],
                                               x["v"][b:b + 1, h:h + 1], x["do"][b:b + 1, h:h + 1],
                                               scale, causal)
        check_grad(bf16_to_f64(dq[b:b + 1, h:h + 1]), dQ, "dQ")
        check_grad(bf16_to_f64(dk[b:b + 1, h:h + 1]), dK, "dK")
        check_grad(bf16_to_f64(dv[b:b + 1, h:h + 1]), dV, "dV")


def test_noalloc_binding_and_limit():
    lib = fa.load_library()
    x = make_inputs(1, 3, 257, 64, seed=9, with_dout=True)
    scale = default_scale(64)
    q, k, v, do = (to_device(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.flash_attn_fwd(q, k, v, causal=True, softmax_scale=scale)
    ref = fa.flash_attn_bwd(do, q, k, v, o, lse, causal=True, softmax_scale=scale)
    got = fa.flash_attn_bwd_noalloc(do, q, k, v, o, lse, torch.empty_like(q), torch.empty_like(k),
                                    torch.empty_like(v), causal=True, softmax_scale=scale)
    torch.cuda.synchronize()
    for r, g in zip(ref, got):
        assert torch.equal(r.view(torch.int16), g.view(torch.int16))
    # a problem whose row vectors exceed the static scratch is refused before
    # any HIP call (the pointers are never touched)
    B, H, N, d = 1, 16, 65537, 64
    assert 2 * B * H * (-(-N // 64) * 64) * 4 > fa.BWD_NOALLOC_SCRATCH_BYTES
    A = 1 << 20
    st = lib.flash_attn_bwd_noalloc(A, 2 * A, 3 * A, 4 * A, 5 * A, 6 * A, 7 * A, 8 * A, 9 * A,
                                    B, H, N, d, 1, 0.125, None)
    assert st == SCRATCH_TOO_SMALL
    assert b"static scratch" in lib.flash_attn_status_string(st)
