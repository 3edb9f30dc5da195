"""Nystrom self-attention forward for AMD MI355X (gfx950).

The compute path is the HIP library libnysattn.so behind the C ABI in
include/nys_attn.h; ``_lib`` is its ctypes binding (loaded on first attribute access,
so ``inputs`` can be imported on machines without the library).
"""
_EXPORTS = {
    "NystromAttention", "NysError", "nys_attn_create", "nys_attn_forward",
    "nys_attn_forward_debug", "nys_attn_workspace_bytes", "nys_attn_profile_enable",
    "nys_attn_profile_read", "nys_attn_destroy", "nys_attn_last_error", "Taps",
    "NYS_F32", "NYS_BF16", "nys_attn_forward_varlen", "nys_proj_qkv", "nys_proj_out",
    "NystromLayer", "nys_attn_backward", "flash_mixed_chunk", "nys_flash_workspace_bytes",
    "nys_flash_states", "nys_flash_attend", "nys_flash_attention", "nys_attn_forward_noalloc",
}


def __getattr__(name):
    if name in _EXPORTS:
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
