"""The C ABI library: it loads, exports every entry point the header declares,
and rejects bad arguments on the host, before any HIP call.

The rejection tests pass fake (never dereferenced) pointer values.  They run
only in a process without a GPU, so that a validation bug could at worst get
a launch error from a missing device, never a kernel touching fake memory.
"""

import ctypes
import os
import re
import subprocess

import pytest
import torch

from exact_attention_flash_amd.binding import LIB_PATH, load_library

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flash_attn.h")

FA_OK, NULLP, SHAPE, HEADDIM, MISAL, SCALE, WS, HIPERR, ALIAS, SPLITS, DESCALE, DROPOUT, \
    SCRATCH = range(13)


def test_status_enum_matches_header():
    text = open(HEADER).read()
    enum = dict((n, int(v)) for n, v in re.findall(r"\b(FA_\w+)\s*=\s*(\d+)", text))
    assert enum == {"FA_OK": FA_OK, "FA_ERR_NULL_POINTER": NULLP, "FA_ERR_BAD_SHAPE": SHAPE,
                    "FA_ERR_UNSUPPORTED_HEAD_DIM": HEADDIM, "FA_ERR_MISALIGNED": MISAL,
                    "FA_ERR_BAD_SCALE": SCALE, "FA_ERR_WORKSPACE_TOO_SMALL": WS,
                    "FA_ERR_HIP": HIPERR, "FA_ERR_ALIASING": ALIAS, "FA_ERR_BAD_SPLITS": SPLITS,
                    "FA_ERR_BAD_DESCALE": DESCALE, "FA_ERR_BAD_DROPOUT": DROPOUT,
                    "FA_ERR_SCRATCH_TOO_SMALL": SCRATCH}

no_gpu = pytest.mark.skipif(torch.cuda.is_available(),
                            reason="fake-pointer validation runs only without a GPU")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\w[\w\s\*]*?\b(flash_attn_\w+)\s*\(", text, re.M)))


def test_library_exports_header_symbols():
    lib = load_library()
    names = _declared()
    assert names == sorted(["flash_attn_fwd", "flash_attn_bwd",
                            "flash_attn_bwd_workspace_bytes", "flash_attn_status_string",
                            "flash_attn_bwd_preprocess", "flash_attn_bwd_kv_blocks",
                            "flash_attn_bwd_q_blocks", "flash_attn_fwd_splitkv",
                            "flash_attn_fwd_splitkv_workspace_bytes", "flash_attn_fwd_fp8",
                            "flash_attn_fwd_dropout", "flash_attn_bwd_dropout",
                            "flash_attn_quantize_fp8", "flash_attn_bwd_noalloc"])
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True)
    if out.returncode == 0:
        exported = set(re.findall(r"\bT (flash_attn_\w+)", out.stdout))
        assert set(names) <= exported


def test_status_strings():
    lib = load_library()
    for s in range(13):
        assert lib.flash_attn_status_string(s) not in (None, b"unknown status")
    assert lib.flash_attn_status_string(99) == b"unknown status"


def test_workspace_bytes():
    lib = load_library()
    rows = 4 * 16 * 4096
    assert lib.flash_attn_bwd_workspace_bytes(4, 16, 4096, 128) == 2 * rows * 4
    # two fp32 row vectors, padded to whole 64-row query blocks per head
    assert lib.flash_attn_bwd_workspace_bytes(1, 1, 1, 64) == 2 * 256
    assert lib.flash_attn_bwd_workspace_bytes(1, 3, 100, 128) == 2 * ((3 * 128 * 4 + 255) // 256 * 256)
    assert lib.flash_attn_bwd_workspace_bytes(0, 16, 4096, 128) == 0
    assert lib.flash_attn_bwd_workspace_bytes(1, 1, 10, 96) == 0
    assert lib.flash_attn_bwd_workspace_bytes(-1, 1, 10, 64) == 0


def test_splitkv_workspace_bytes():
    lib = load_library()
    rows = 4 * 2 * 8 * 1024
    # fp32 partial O [S, B*H, N, d], then fp32 m and l [S, B*H, N]
    assert lib.flash_attn_fwd_splitkv_workspace_bytes(2, 8, 1024, 64, 4) == rows * 64 * 4 + 2 * rows * 4
    assert lib.flash_attn_fwd_splitkv_workspace_bytes(1, 1, 3, 128, 1) == 3 * 128 * 4 + 2 * 256
    assert lib.flash_attn_fwd_splitkv_workspace_bytes(1, 1, 16, 64, 0) == 0
    assert lib.flash_attn_fwd_splitkv_workspace_bytes(1, 1, 16, 64, 129) == 0
    assert lib.flash_attn_fwd_splitkv_workspace_bytes(0, 1, 16, 64, 2) == 0
    assert lib.flash_attn_fwd_splitkv_workspace_bytes(1, 1, 16, 96, 2) == 0


A = 1 << 20  # fake, 16-byte-aligned addresses spaced far apart


def _fwd(lib, q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, B=1, H=1, N=16, d=64, causal=0,
         scale=0.125):
    return lib.flash_attn_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, None)


@no_gpu
def test_fwd_validation():
    lib = load_library()
    assert _fwd(lib, B=0) == FA_OK and _fwd(lib, N=0, q=None) == FA_OK  # empty: no-op
    assert _fwd(lib, q=None) == NULLP
    assert _fwd(lib, lse=None) == NULLP
    assert _fwd(lib, N=-1) == SHAPE
    assert _fwd(lib, B=1 << 40, N=1 << 20) == SHAPE
    assert _fwd(lib, d=96) == HEADDIM and _fwd(lib, d=256) == HEADDIM
    assert _fwd(lib, q=A + 8) == MISAL
    assert _fwd(lib, lse=5 * A + 2) == MISAL
    assert _fwd(lib, lse=5 * A + 4) != MISAL
    for bad in (0.0, -0.125, float("nan"), float("inf")):
        assert _fwd(lib, scale=bad) == SCALE
    assert _fwd(lib, o=A) == ALIAS                       # O on top of Q
    assert _fwd(lib, lse=4 * A + 16) == ALIAS            # LSE inside O
    assert _fwd(lib, o=A + 16 * 64 * 2) != ALIAS         # O just after Q


def _fwd_split(lib, ws_bytes=None, q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, ws=6 * A, B=1, H=1,
               N=16, d=64, causal=0, scale=0.125, splits=2, Nk=None):
    need = lib.flash_attn_fwd_splitkv_workspace_bytes(B, H, N, d, splits)
    wsb = need if ws_bytes is None else ws_bytes
    return lib.flash_attn_fwd_splitkv(q, k, v, o, lse, ws, wsb, B, H, N, N if Nk is None else Nk,
                                      d, causal, scale, splits, None)


@no_gpu
def test_fwd_splitkv_validation():
    lib = load_library()
    assert _fwd_split(lib, B=0, ws=None) == FA_OK            # empty: no-op
    assert _fwd_split(lib, splits=0) == SPLITS
    assert _fwd_split(lib, splits=129) == SPLITS
    assert _fwd_split(lib, B=0, splits=0) == SPLITS          # checked even when empty
    assert _fwd_split(lib, ws=None) == NULLP
    assert _fwd_split(lib, q=None) == NULLP
    assert _fwd_split(lib, ws=6 * A + 8) == MISAL
    assert _fwd_split(lib, d=96) == HEADDIM
    assert _fwd_split(lib, scale=float("nan")) == SCALE
    assert _fwd_split(lib, ws_bytes=1024) == WS
    assert _fwd_split(lib, ws=A) == ALIAS                    # workspace on top of Q
    assert _fwd_split(lib, ws=4 * A) == ALIAS                # workspace on top of O
    assert _fwd_split(lib, o=3 * A) == ALIAS                 # O on top of V
    # queries and keys of different lengths (a decode step): full attention only
    assert _fwd_split(lib, N=1, Nk=16, causal=1) == SHAPE
    assert _fwd_split(lib, N=16, Nk=0) == SHAPE               # a query needs a key
    assert _fwd_split(lib, N=16, Nk=-1) == SHAPE
    assert _fwd_split(lib, N=0, Nk=5, ws=None) == FA_OK       # no query: no-op
    assert _fwd_split(lib, N=1, Nk=64, d=96) == HEADDIM
    # the K / V ranges are sized by N_kv (K of 64 Ki keys reaches O at 4 A),
    # the Q / O ranges by N_q (Q of 64 Ki queries reaches O at 3 A + 4096)
    assert _fwd_split(lib, N=1, Nk=64 * 1024, v=3 * A + 16) == ALIAS
    assert _fwd_split(lib, N=64 * 1024, Nk=1, ws_bytes=1 << 30, v=3 * A, o=3 * A + 4096) == ALIAS


def _fwd_fp8(lib, q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, B=1, H=1, N=16, d=64, causal=0,
             scale=0.125, dq=0.01, dk=0.02, dv=0.03):
    return lib.flash_attn_fwd_fp8(q, k, v, o, lse, B, H, N, d, causal, scale, dq, dk, dv, None)


@no_gpu
def test_fwd_fp8_validation():
    lib = load_library()
    assert _fwd_fp8(lib, B=0, q=None) == FA_OK                # empty: no-op
    assert _fwd_fp8(lib, q=None) == NULLP
    assert _fwd_fp8(lib, N=-3) == SHAPE
    assert _fwd_fp8(lib, d=32) == HEADDIM
    assert _fwd_fp8(lib, scale=0.0) == SCALE
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert _fwd_fp8(lib, dq=bad) == DESCALE
        assert _fwd_fp8(lib, dk=bad) == DESCALE
        assert _fwd_fp8(lib, dv=bad) == DESCALE
    assert _fwd_fp8(lib, B=0, dv=-1.0) == DESCALE             # checked even when empty
    # the product scale * dq * dk must stay a positive finite float
    assert _fwd_fp8(lib, dq=1e-30, dk=1e-30) == DESCALE
    assert _fwd_fp8(lib, dq=1e30, dk=1e30) == DESCALE
    assert _fwd_fp8(lib, v=3 * A + 8) == MISAL
    # inputs take one byte per element, O two: O right after a 1-byte Q is fine,
    # O over the second half of its own 2-byte extent is not
    n = 16 * 64
    assert _fwd_fp8(lib, q=A, o=A + n) != ALIAS
    assert _fwd_fp8(lib, q=A + n, o=A) == ALIAS
    assert _fwd_fp8(lib, lse=4 * A + 2 * n - 16) == ALIAS     # LSE inside O


def _fwd_drop(lib, q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, B=1, H=2, N=40, d=64, causal=1,
              scale=0.125, p=0.1, seed=2**64 - 1, offset=2**32 - 1):
    return lib.flash_attn_fwd_dropout(q, k, v, o, lse, B, H, N, d, causal, scale, p, seed, offset,
                                      None)


def _bwd_drop(lib, ws_bytes=None, p=0.1, **kw):
    args = dict(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, do=6 * A, dq=7 * A, dk=8 * A, dv=9 * A,
                ws=10 * A, B=1, H=2, N=16, d=128, causal=1, scale=0.1)
    args.update(kw)
    need = lib.flash_attn_bwd_workspace_bytes(args["B"], args["H"], args["N"], args["d"])
    wsb = need if ws_bytes is None else ws_bytes
    return lib.flash_attn_bwd_dropout(args["q"], args["k"], args["v"], args["o"], args["lse"],
                                      args["do"], args["dq"], args["dk"], args["dv"], args["ws"],
                                      wsb, args["B"], args["H"], args["N"], args["d"],
                                      args["causal"], args["scale"], p, 7, 0, None)


@no_gpu
def test_dropout_validation():
    lib = load_library()
    for bad in (-0.01, float("nan"), 1.0, 255.5 / 256, float("inf")):
        assert _fwd_drop(lib, p=bad) == DROPOUT
        assert _bwd_drop(lib, p=bad) == DROPOUT
    assert _fwd_drop(lib, B=0, p=-1.0) == DROPOUT           # checked even when empty
    assert _fwd_drop(lib, B=0, q=None) == FA_OK              # empty: no-op
    assert _fwd_drop(lib, q=None) == NULLP
    assert _fwd_drop(lib, d=80) == HEADDIM
    assert _fwd_drop(lib, scale=-1.0) == SCALE
    assert _fwd_drop(lib, o=A) == ALIAS
    assert _bwd_drop(lib, ws_bytes=8) == WS
    assert _bwd_drop(lib, dq=8 * A) == ALIAS
    # largest allowed probability (t = 255), and p = 0
    assert _fwd_drop(lib, p=255.4 / 256) == HIPERR
    assert _fwd_drop(lib, p=0.0) == HIPERR
    assert _bwd_drop(lib, p=0.0) == HIPERR


def _quant(lib, x=A, codes=2 * A, ds=3 * A, ws=4 * A, wsb=4096, rows=100, d=128, signs=5 * A):
    return lib.flash_attn_quantize_fp8(x, codes, ds, ws, wsb, rows, d, signs, None)


@no_gpu
def test_quantize_validation():
    lib = load_library()
    assert _quant(lib, rows=0, x=None) == FA_OK
    assert _quant(lib, rows=-1) == SHAPE
    assert _quant(lib, d=96) == HEADDIM
    assert _quant(lib, x=None) == NULLP and _quant(lib, ws=None) == NULLP
    assert _quant(lib, x=A + 8) == MISAL and _quant(lib, signs=5 * A + 4) == MISAL
    assert _quant(lib, wsb=4095) == WS and _quant(lib, ws=4 * A + 4) == MISAL
    assert _quant(lib, ws=3 * A - 4096 + 16) == ALIAS         # workspace runs into descale
    assert _quant(lib, codes=A + 16) == ALIAS                  # codes inside x
    assert _quant(lib, ws=3 * A) == ALIAS                      # workspace on descale
    assert _quant(lib, ds=5 * A) == ALIAS                      # descale on signs
    assert _quant(lib, signs=None) == HIPERR                   # no rotation is allowed
    assert _quant(lib) == HIPERR


def _bwd(lib, ws_bytes=None, **kw):
    args = dict(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, do=6 * A, dq=7 * A, dk=8 * A, dv=9 * A,
                ws=10 * A, B=1, H=2, N=16, d=128, causal=1, scale=0.1)
    args.update(kw)
    need = lib.flash_attn_bwd_workspace_bytes(args["B"], args["H"], args["N"], args["d"])
    wsb = need if ws_bytes is None else ws_bytes
    return lib.flash_attn_bwd(args["q"], args["k"], args["v"], args["o"], args["lse"], args["do"],
                              args["dq"], args["dk"], args["dv"], args["ws"], wsb, args["B"],
                              args["H"], args["N"], args["d"], args["causal"], args["scale"], None)


@no_gpu
def test_bwd_validation():
    lib = load_library()
    assert _bwd(lib, H=0, ws=None) == FA_OK
    assert _bwd(lib, ws=None) == NULLP
    assert _bwd(lib, do=None) == NULLP
    assert _bwd(lib, d=32) == HEADDIM
    assert _bwd(lib, dk=8 * A + 2) == MISAL
    assert _bwd(lib, scale=float("-inf")) == SCALE
    need = lib.flash_attn_bwd_workspace_bytes(1, 2, 16, 128)
    assert _bwd(lib, ws_bytes=need - 1) == WS
    assert _bwd(lib, dq=A) == ALIAS          # dQ on Q
    assert _bwd(lib, dv=8 * A) == ALIAS      # dV on dK
    assert _bwd(lib, ws=6 * A) == ALIAS      # workspace on dO


@no_gpu
def test_bwd_stage_validation():
    lib = load_library()
    need = lib.flash_attn_bwd_workspace_bytes(1, 2, 16, 128)
    # stages check only the pointers they use
    assert lib.flash_attn_bwd_preprocess(None, 5 * A, 6 * A, 10 * A, need, 1, 2, 16, 128,
                                         None) == NULLP
    assert lib.flash_attn_bwd_preprocess(4 * A, 5 * A, 6 * A, 10 * A, need - 4, 1, 2, 16, 128,
                                         None) == WS
    assert lib.flash_attn_bwd_preprocess(4 * A, 5 * A, 6 * A, 4 * A, need, 1, 2, 16, 128,
                                         None) == ALIAS
    assert lib.flash_attn_bwd_kv_blocks(A, 2 * A, 3 * A, 6 * A, 8 * A, 9 * A, 10 * A, need,
                                        1, 2, 16, 96, 1, 0.1, None) == HEADDIM
    assert lib.flash_attn_bwd_kv_blocks(A, 2 * A, 3 * A, 6 * A, 8 * A, 8 * A, 10 * A, need,
                                        1, 2, 16, 128, 1, 0.1, None) == ALIAS
    assert lib.flash_attn_bwd_kv_blocks(A, 2 * A, 3 * A, 6 * A, 8 * A, 9 * A, 10 * A, need,
                                        1, 2, 16, 128, 1, 0.0, None) == SCALE
    assert lib.flash_attn_bwd_q_blocks(A, 2 * A, 3 * A, 6 * A, 7 * A + 4, 10 * A, need,
                                       1, 2, 16, 128, 1, 0.1, None) == MISAL
    assert lib.flash_attn_bwd_q_blocks(A, 2 * A, 3 * A, 6 * A, A, 10 * A, need,
                                       1, 2, 16, 128, 1, 0.1, None) == ALIAS
    assert lib.flash_attn_bwd_q_blocks(A, 2 * A, 3 * A, 6 * A, 7 * A, 10 * A, need,
                                       0, 2, 16, 128, 1, 0.1, None) == FA_OK


def _bwd_noalloc(lib, **kw):
    args = dict(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, do=6 * A, dq=7 * A, dk=8 * A, dv=9 * A,
                B=1, H=2, N=16, d=128, causal=1, scale=0.1)
    args.update(kw)
    return lib.flash_attn_bwd_noalloc(args["q"], args["k"], args["v"], args["o"], args["lse"],
                                      args["do"], args["dq"], args["dk"], args["dv"], args["B"],
                                      args["H"], args["N"], args["d"], args["causal"],
                                      args["scale"], None)


@no_gpu
def test_bwd_noalloc_validation():
    """Same checks as flash_attn_bwd on every caller pointer, plus the size
    limit of the static scratch, all before any HIP call."""
    lib = load_library()
    assert _bwd_noalloc(lib, H=0) == FA_OK
    assert _bwd_noalloc(lib, do=None) == NULLP
    assert _bwd_noalloc(lib, d=32) == HEADDIM
    assert _bwd_noalloc(lib, dk=8 * A + 2) == MISAL
    assert _bwd_noalloc(lib, scale=float("nan")) == SCALE
    assert _bwd_noalloc(lib, dq=A) == ALIAS
    # 2^20 padded rows fit; one more 64-row block does not
    assert _bwd_noalloc(lib, B=1, H=16, N=65536, dq=7 * A) != SCRATCH
    assert _bwd_noalloc(lib, B=1, H=16, N=65537) == SCRATCH
    assert _bwd_noalloc(lib) == HIPERR       # valid: reaches the device, which is absent


@no_gpu
def test_valid_call_without_device_reports_hip_error():
    """All arguments valid: the call reaches the launch, which fails with no
    device present and is reported as FA_ERR_HIP (no fake memory is touched
    because nothing can run)."""
    lib = load_library()
    assert _fwd(lib) == HIPERR
    assert _fwd_split(lib) == HIPERR
    assert _fwd_fp8(lib) == HIPERR
    assert _fwd_drop(lib) == HIPERR
    assert _bwd_drop(lib) == HIPERR


def test_python_binding_rejects_cpu_tensors():
    from exact_attention_flash_amd import flash_attn_fwd
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        flash_attn_fwd(q, q, q)
    with pytest.raises(TypeError):
        flash_attn_fwd(q.float(), q.float(), q.float())
    from exact_attention_flash_amd import flash_attn_fwd_fp8
    q8 = torch.zeros(1, 1, 8, 64, dtype=torch.uint8)
    with pytest.raises(ValueError):
        flash_attn_fwd_fp8(q8, q8, q8, 1.0, 1.0, 1.0)
    with pytest.raises(TypeError):
        flash_attn_fwd_fp8(q, q, q, 1.0, 1.0, 1.0)
