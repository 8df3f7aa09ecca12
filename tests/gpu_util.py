"""Helpers for the GPU parity tests: moving bf16 bit patterns to and from the
device, and the tolerance checks of the parity bar.

Tolerances (fixed by the project's acceptance bar):
  * O (bf16 output): |O_gpu - O_ref| <= 1e-2, plus half a bf16 ulp of O_ref
    (a correctly rounded bf16 value with |O| >= 4 can be off by more than
    1e-2 from the exact value; the count of elements that needed the
    allowance is reported);
  * LSE: |LSE_gpu - LSE_ref| <= 1e-3;
  * dQ, dK, dV: max |g_gpu - g_ref| <= 5e-2 * max |g_ref|, per tensor.
"""

from __future__ import annotations

import numpy as np
import torch

from exact_attention_flash_amd.inputs import bf16_bits_to_f32

O_ATOL = 1e-2
LSE_ATOL = 1e-3
GRAD_RTOL = 5e-2


def to_device(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bf16 bit patterns -> contiguous bfloat16 tensor on the GPU."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device).contiguous()


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return bf16_bits_to_f32(bits).astype(np.float64)


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half of one bf16 ulp at |x| (8 significant bits)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 8), 0.0)


def check_o(o_gpu: np.ndarray, o_ref: np.ndarray, what: str = "O") -> dict:
    err = np.abs(o_gpu - o_ref)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite output"
    plain = err <= O_ATOL
    allowed = err <= O_ATOL + half_ulp_bf16(o_ref)
    bad = ~allowed
    assert not np.any(bad), (
        f"{what}: {int(bad.sum())} elements beyond 1e-2 + half ulp; max err {err.max():.3e}")
    return {"max_abs_err": float(err.max()), "needed_ulp_allowance": int((~plain).sum())}


def check_lse(l_gpu: np.ndarray, l_ref: np.ndarray, what: str = "LSE") -> float:
    err = np.abs(l_gpu - l_ref)
    assert np.all(np.isfinite(l_gpu)), f"{what}: non-finite output"
    assert err.max() <= LSE_ATOL, f"{what}: max abs err {err.max():.3e} > {LSE_ATOL}"
    return float(err.max())


def check_grad(g_gpu: np.ndarray, g_ref: np.ndarray, what: str) -> float:
    assert np.all(np.isfinite(g_gpu)), f"{what}: non-finite output"
    scale = np.abs(g_ref).max()
    err = np.abs(g_gpu - g_ref).max()
    rel = err / scale if scale > 0 else err
    assert err <= GRAD_RTOL * scale + 1e-30, f"{what}: max err {err:.3e} = {rel:.3e} x max|ref|"
    return float(rel)
