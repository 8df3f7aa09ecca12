"""Thin ctypes binding over the C ABI in ``include/flash_attn.h``.

Argument marshalling only: tensors are checked (bf16, contiguous, one device,
``[B, H, N, d]``), outputs are allocated with torch when not given, and the
raw device pointers plus the current HIP stream go to the library.  Every
step of the computation runs in the HIP kernels; there is no other path.  If
the shared library is missing the first call raises ``RuntimeError``.
"""

from __future__ import annotations

import ctypes
import math
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libexact_attention_flash_amd.so")

_lib = None
_lock = threading.Lock()


class FlashAttnError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, status: int, message: str):
        super().__init__(f"flash_attn status {status}: {message}")
        self.status = status


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load (once) and return the HIP library, with argument types set."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(
                f"HIP library {p} is not built; run exact_attention_flash_amd.build.build()")
        lib = ctypes.CDLL(p)
        i64, vp, fl, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
        lib.flash_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ci, fl, vp]
        lib.flash_attn_fwd.restype = ci
        lib.flash_attn_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64]
        lib.flash_attn_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.flash_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                       i64, i64, i64, i64, ci, fl, vp]
        lib.flash_attn_bwd.restype = ci
        lib.flash_attn_bwd_preprocess.argtypes = [vp, vp, vp, vp, ctypes.c_size_t,
                                                  i64, i64, i64, i64, vp]
        lib.flash_attn_bwd_preprocess.restype = ci
        lib.flash_attn_bwd_kv_blocks.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                                 i64, i64, i64, i64, ci, fl, vp]
        lib.flash_attn_bwd_kv_blocks.restype = ci
        lib.flash_attn_bwd_q_blocks.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                                i64, i64, i64, i64, ci, fl, vp]
        lib.flash_attn_bwd_q_blocks.restype = ci
        lib.flash_attn_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                               i64, i64, i64, i64, i64, ci, fl, i64, vp]
        lib.flash_attn_fwd_splitkv.restype = ci
        lib.flash_attn_fwd_splitkv_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
        lib.flash_attn_fwd_splitkv_workspace_bytes.restype = ctypes.c_size_t
        lib.flash_attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ci, fl,
                                           fl, fl, fl, vp]
        lib.flash_attn_fwd_fp8.restype = ci
        u64, u32 = ctypes.c_uint64, ctypes.c_uint32
        lib.flash_attn_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ci, fl,
                                               fl, u64, u32, vp]
        lib.flash_attn_fwd_dropout.restype = ci
        lib.flash_attn_bwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                               ctypes.c_size_t, i64, i64, i64, i64, ci, fl,
                                               fl, u64, u32, vp]
        lib.flash_attn_bwd_dropout.restype = ci
        lib.flash_attn_quantize_fp8.argtypes = [vp, vp, vp, vp, ctypes.c_size_t, i64, i64, vp, vp]
        lib.flash_attn_quantize_fp8.restype = ci
        lib.flash_attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                               i64, i64, i64, i64, ci, fl, vp]
        lib.flash_attn_bwd_noalloc.restype = ci
        lib.flash_attn_status_string.argtypes = [ci]
        lib.flash_attn_status_string.restype = ctypes.c_char_p
        _lib = lib
        return lib


def flash_attn_status_string(status: int) -> str:
    return load_library().flash_attn_status_string(int(status)).decode()


def _check(status: int) -> None:
    if status != 0:
        raise FlashAttnError(status, flash_attn_status_string(status))


def _check_tensors(*ts: torch.Tensor, names: str, dtypes=(torch.bfloat16,)) -> tuple:
    ref = ts[0]
    if ref.dim() != 4:
        raise ValueError(f"{names.split(',')[0]} must be [B, H, N, d]")
    for t, n in zip(ts, names.split(",")):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{n} must be a torch.Tensor")
        if t.dtype not in dtypes:
            raise TypeError(f"{n} must be {' or '.join(str(x) for x in dtypes)}, got {t.dtype}")
        if t.shape != ref.shape:
            raise ValueError(f"{n} has shape {tuple(t.shape)}, expected {tuple(ref.shape)}")
        if t.device != ref.device or t.device.type != "cuda":
            raise ValueError(f"{n} must be on the GPU device of {names.split(',')[0]}")
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    return tuple(ref.shape)


def _stream_ptr(device: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream)


def default_scale(d: int) -> float:
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))


def flash_attn_bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(load_library().flash_attn_bwd_workspace_bytes(B, H, N, d))


def flash_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                   softmax_scale: float | None = None, out: torch.Tensor | None = None,
                   lse: torch.Tensor | None = None, stream=None):
    """O and LSE of softmax(scale * Q K^T) V; returns ``(out, lse)``."""
    B, H, N, d = _check_tensors(q, k, v, names="q,k,v")
    scale = default_scale(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensors(q, out, names="q,out")
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    elif lse.dtype != torch.float32 or lse.shape != (B, H, N) or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.flash_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                lse.data_ptr(), B, H, N, d, int(bool(causal)), scale,
                                _stream_ptr(q.device, stream))
    _check(st)
    return out, lse


FP8_DTYPES = (torch.uint8, torch.float8_e4m3fn)


def flash_attn_fwd_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                       descale_q: float, descale_k: float, descale_v: float,
                       causal: bool = False, softmax_scale: float | None = None,
                       out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                       stream=None):
    """FP8 forward over E4M3 codes (uint8 or float8_e4m3fn tensors) with
    per-tensor descales; returns bf16 ``out`` and float32 ``lse``."""
    B, H, N, d = _check_tensors(q, k, v, names="q,k,v", dtypes=FP8_DTYPES)
    scale = default_scale(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q.device)
    else:
        _check_tensors(out, names="out")
        if out.shape != q.shape or out.device != q.device:
            raise ValueError("out must be a bfloat16 tensor of q's shape on q's device")
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    elif lse.dtype != torch.float32 or lse.shape != (B, H, N) or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.flash_attn_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                    lse.data_ptr(), B, H, N, d, int(bool(causal)), scale,
                                    float(descale_q), float(descale_k), float(descale_v),
                                    _stream_ptr(q.device, stream))
    _check(st)
    return out, lse


# Workspace of flash_attn_quantize_fp8 (FA_QUANT_WORKSPACE_BYTES of the C header).
QUANT_WORKSPACE_BYTES = 4096


def flash_attn_quantize_fp8(x: torch.Tensor, signs: torch.Tensor | None = None,
                            codes: torch.Tensor | None = None, descale: torch.Tensor | None = None,
                            workspace: torch.Tensor | None = None, stream=None):
    """E4M3 codes of a bf16 tensor (rows over the last dim, d = 64 or 128),
    rotated by diag(signs) H_d / sqrt(d) first when ``signs`` is given.
    Returns ``(codes, descale)``: uint8 codes of x's shape and a float32
    device tensor [1] holding amax / 448."""
    if not isinstance(x, torch.Tensor) or x.dtype != torch.bfloat16:
        raise TypeError("x must be a bfloat16 tensor")
    if x.device.type != "cuda" or not x.is_contiguous() or x.dim() < 1:
        raise ValueError("x must be a contiguous GPU tensor")
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    if signs is not None and (signs.dtype != torch.float32 or signs.shape != (d,)
                              or signs.device != x.device or not signs.is_contiguous()):
        raise ValueError("signs must be a contiguous float32 [d] tensor on x's device")
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if codes is None else codes
    if codes.dtype not in FP8_DTYPES or codes.shape != x.shape or not codes.is_contiguous() \
            or codes.device != x.device:
        raise ValueError("codes must be a contiguous one-byte tensor of x's shape on x's device")
    descale = torch.empty(1, dtype=torch.float32, device=x.device) if descale is None else descale
    workspace = torch.empty(QUANT_WORKSPACE_BYTES // 4, dtype=torch.float32, device=x.device) \
        if workspace is None else workspace
    lib = load_library()
    with torch.cuda.device(x.device):
        st = lib.flash_attn_quantize_fp8(x.data_ptr(), codes.data_ptr(), descale.data_ptr(),
                                         workspace.data_ptr(),
                                         workspace.numel() * workspace.element_size(), rows, d,
                                         None if signs is None else signs.data_ptr(),
                                         _stream_ptr(x.device, stream))
    _check(st)
    return codes, descale


def flash_attn_fwd_splitkv_workspace_bytes(B: int, H: int, N: int, d: int, num_splits: int) -> int:
    return int(load_library().flash_attn_fwd_splitkv_workspace_bytes(B, H, N, d, num_splits))


def flash_attn_fwd_splitkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                           num_splits: int, causal: bool = False,
                           softmax_scale: float | None = None, out: torch.Tensor | None = None,
                           lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                           stream=None):
    """``flash_attn_fwd`` with each query block's keys cut into ``num_splits``
    ranges and merged; returns ``(out, lse)``.  ``q`` is ``[B, H, N_q, d]``
    and ``k``, ``v`` are ``[B, H, N_kv, d]``; N_q != N_kv (a decode step)
    needs ``causal=False``."""
    _check_tensors(k, v, names="k,v")
    if q.dim() != 4 or tuple(q.shape[:2]) != tuple(k.shape[:2]) or q.shape[3] != k.shape[3]:
        raise ValueError(f"q {tuple(q.shape)} must be [B, H, N_q, d] with k's B, H and d "
                         f"(k is {tuple(k.shape)})")
    B, H, N, d = _check_tensors(q, names="q")
    Nk = int(k.shape[2])
    if q.device != k.device:
        raise ValueError("q and k must be on one device")
    scale = default_scale(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensors(q, out, names="q,out")
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    elif lse.dtype != torch.float32 or lse.shape != (B, H, N) or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, N_q] tensor on q's device")
    lib = load_library()
    need = int(lib.flash_attn_fwd_splitkv_workspace_bytes(B, H, N, d, int(num_splits)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    with torch.cuda.device(q.device):
        st = lib.flash_attn_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                        lse.data_ptr(), workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(),
                                        B, H, N, Nk, d, int(bool(causal)), scale, int(num_splits),
                                        _stream_ptr(q.device, stream))
    _check(st)
    return out, lse


def flash_attn_bwd(dout: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                   out: torch.Tensor, lse: torch.Tensor, causal: bool = False,
                   softmax_scale: float | None = None, dq: torch.Tensor | None = None,
                   dk: torch.Tensor | None = None, dv: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None, stream=None):
    """dQ, dK, dV of the attention whose forward gave ``out`` and ``lse``."""
    B, H, N, d = _check_tensors(q, k, v, out, dout, names="q,k,v,out,dout")
    scale = default_scale(d) if softmax_scale is None else float(softmax_scale)
    if lse.dtype != torch.float32 or lse.shape != (B, H, N) or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_tensors(q, dq, dk, dv, names="q,dq,dk,dv")
    lib = load_library()
    need = int(lib.flash_attn_bwd_workspace_bytes(B, H, N, d))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        st = lib.flash_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                dv.data_ptr(), workspace.data_ptr(), ws_bytes, B, H, N, d,
                                int(bool(causal)), scale, _stream_ptr(q.device, stream))
    _check(st)
    return dq, dk, dv


# Largest workspace the allocation-free backward's static scratch holds
# (FA_BWD_NOALLOC_SCRATCH_BYTES).
BWD_NOALLOC_SCRATCH_BYTES = 8 << 20


def flash_attn_bwd_noalloc(dout: torch.Tensor, q: torch.Tensor, k: torch.Tensor,
                           v: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
                           dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor,
                           causal: bool = False, softmax_scale: float | None = None, stream=None):
    """flash_attn_bwd into the caller's dq, dk, dv with no workspace: the
    library keeps the row vectors in its own static device buffer, so
    nothing is allocated (usable under stream capture).  Calls that overlap
    on one device race on that buffer."""
    B, H, N, d = _check_tensors(q, k, v, out, dout, dq, dk, dv,
                                names="q,k,v,out,dout,dq,dk,dv")
    scale = default_scale(d) if softmax_scale is None else float(softmax_scale)
    if lse.dtype != torch.float32 or lse.shape != (B, H, N) or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.flash_attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                        lse.data_ptr(), dout.data_ptr(), dq.data_ptr(),
                                        dk.data_ptr(), dv.data_ptr(), B, H, N, d,
                                        int(bool(causal)), scale, _stream_ptr(q.device, stream))
    _check(st)
    return dq, dk, dv


def _seed_offset(seed: int, offset: int) -> tuple:
    seed, offset = int(seed), int(offset)
    if not 0 <= seed < 2**64 or not 0 <= offset < 2**32:
        raise ValueError("seed must fit 64 bits and offset 32 bits (unsigned)")
    return seed, offset


def flash_attn_fwd_dropout(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dropout_p: float,
                           seed: int, offset: int = 0, causal: bool = False,
                           softmax_scale: float | None = None, out: torch.Tensor | None = None,
                           lse: torch.Tensor | None = None, stream=None):
    """O = (P o Z s) V with the Philox keep mask Z of (seed, offset); returns ``(out, lse)``."""
    B, H, N, d = _check_tensors(q, k, v, names="q,k,v")
    scale = default_scale(d) if softmax_scale is None else float(softmax_scale)
    seed, offset = _seed_offset(seed, offset)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensors(q, out, names="q,out")
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    elif lse.dtype != torch.float32 or lse.shape != (B, H, N) or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.flash_attn_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                        lse.data_ptr(), B, H, N, d, int(bool(causal)), scale,
                                        float(dropout_p), seed, offset,
                                        _stream_ptr(q.device, stream))
    _check(st)
    return out, lse


def flash_attn_bwd_dropout(dout: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                           out: torch.Tensor, lse: torch.Tensor, dropout_p: float, seed: int,
                           offset: int = 0, causal: bool = False,
                           softmax_scale: float | None = None, dq: torch.Tensor | None = None,
                           dk: torch.Tensor | None = None, dv: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None, stream=None):
    """dQ, dK, dV of flash_attn_fwd_dropout with the same (dropout_p, seed, offset)."""
    B, H, N, d = _check_tensors(q, k, v, out, dout, names="q,k,v,out,dout")
    scale = default_scale(d) if softmax_scale is None else float(softmax_scale)
    seed, offset = _seed_offset(seed, offset)
    if lse.dtype != torch.float32 or lse.shape != (B, H, N) or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_tensors(q, dq, dk, dv, names="q,dq,dk,dv")
    lib = load_library()
    need = int(lib.flash_attn_bwd_workspace_bytes(B, H, N, d))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        st = lib.flash_attn_bwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                        lse.data_ptr(), dout.data_ptr(), dq.data_ptr(),
                                        dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                                        ws_bytes, B, H, N, d, int(bool(causal)), scale,
                                        float(dropout_p), seed, offset,
                                        _stream_ptr(q.device, stream))
    _check(st)
    return dq, dk, dv


def _ws(workspace: torch.Tensor, device) -> tuple:
    if workspace.device != device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def flash_attn_bwd_preprocess(dout: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
                              workspace: torch.Tensor, stream=None) -> None:
    """Stage 1 of the backward pass (row pass into the workspace)."""
    B, H, N, d = _check_tensors(out, dout, names="out,dout")
    wp, wb = _ws(workspace, out.device)
    with torch.cuda.device(out.device):
        st = load_library().flash_attn_bwd_preprocess(
            out.data_ptr(), lse.data_ptr(), dout.data_ptr(), wp, wb, B, H, N, d,
            _stream_ptr(out.device, stream))
    _check(st)


def flash_attn_bwd_kv_blocks(dout: torch.Tensor, q: torch.Tensor, k: torch.Tensor,
                             v: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor,
                             workspace: torch.Tensor, causal: bool = False,
                             softmax_scale: float | None = None, stream=None) -> None:
    """Stage 2 of the backward pass (key-block pass: dK, dV)."""
    B, H, N, d = _check_tensors(q, k, v, dout, dk, dv, names="q,k,v,dout,dk,dv")
    scale = default_scale(d) if softmax_scale is None else float(softmax_scale)
    wp, wb = _ws(workspace, q.device)
    with torch.cuda.device(q.device):
        st = load_library().flash_attn_bwd_kv_blocks(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), dk.data_ptr(),
            dv.data_ptr(), wp, wb, B, H, N, d, int(bool(causal)), scale,
            _stream_ptr(q.device, stream))
    _check(st)


def flash_attn_bwd_q_blocks(dout: torch.Tensor, q: torch.Tensor, k: torch.Tensor,
                            v: torch.Tensor, dq: torch.Tensor, workspace: torch.Tensor,
                            causal: bool = False, softmax_scale: float | None = None,
                            stream=None) -> None:
    """Stage 3 of the backward pass (query-block pass: dQ)."""
    B, H, N, d = _check_tensors(q, k, v, dout, dq, names="q,k,v,dout,dq")
    scale = default_scale(d) if softmax_scale is None else float(softmax_scale)
    wp, wb = _ws(workspace, q.device)
    with torch.cuda.device(q.device):
        st = load_library().flash_attn_bwd_q_blocks(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), dq.data_ptr(), wp, wb,
            B, H, N, d, int(bool(causal)), scale, _stream_ptr(q.device, stream))
    _check(st)
