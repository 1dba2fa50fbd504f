"""Packed low-bit KV cache and fused single-token decode attention for MI355X.

The computation lives in libkvq.so (hand-written HIP kernels for gfx950, C ABI in
include/kvq.h).  ``api`` marshals torch tensors into those calls.
"""

__all__ = ["Layout", "Stream", "alloc_cache", "alloc_workspace", "kv_quant_pack", "kv_decode_attn", "KvqError"]


def __getattr__(name):
    if name in ("Layout", "Stream", "alloc_cache", "alloc_workspace", "kv_quant_pack", "kv_decode_attn"):
        from . import api
        return getattr(api, name)
    if name == "KvqError":
        from ._lib import KvqError
        return KvqError
    raise AttributeError(name)
