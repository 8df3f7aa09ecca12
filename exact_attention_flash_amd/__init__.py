"""Fused exact attention for AMD MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI declared
in ``include/flash_attn.h``; ``binding`` is a ctypes layer with the same
entry-point names.  Importing this package loads nothing: the shared library
is opened on the first call.
"""

__all__ = [
    "flash_attn_fwd",
    "flash_attn_fwd_splitkv",
    "flash_attn_fwd_fp8",
    "flash_attn_quantize_fp8",
    "QUANT_WORKSPACE_BYTES",
    "flash_attn_fwd_dropout",
    "flash_attn_bwd_dropout",
    "flash_attn_fwd_splitkv_workspace_bytes",
    "flash_attn_bwd",
    "flash_attn_bwd_workspace_bytes",
    "flash_attn_bwd_noalloc",
    "BWD_NOALLOC_SCRATCH_BYTES",
    "flash_attn_bwd_preprocess",
    "flash_attn_bwd_kv_blocks",
    "flash_attn_bwd_q_blocks",
    "flash_attn_status_string",
    "FlashAttnError",
    "load_library",
]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
