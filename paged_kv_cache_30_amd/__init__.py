"""Paged-KV attention for MI355X (gfx950): a C-ABI HIP library plus a thin
ctypes binding.

Entry points (same names as the C functions in ``include/paged_attn.h``):
``paged_kv_write``, ``paged_attn_decode``, ``paged_attn_prefill``,
``paged_attn_decode_workspace_bytes``, ``paged_attn_decode_workers``.
``BlockAllocator`` is the host-side block allocator that builds the tables.
"""
from .allocator import BlockAllocator, UNMAPPED  # noqa: F401
from ._lib import (  # noqa: F401
    LIB, LIB_PATH, EXPORTS, PagedAttnError, Geometry, geometry,
    PKV_F32, PKV_F16, PKV_BF16, PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EWORKSPACE, PKV_EHIP,
    paged_kv_write, paged_attn_decode, paged_attn_prefill,
    paged_attn_decode_workspace_bytes, paged_attn_decode_workers, decode_workspace,
)
