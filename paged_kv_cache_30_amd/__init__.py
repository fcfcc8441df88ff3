"""Paged-KV attention for MI355X (gfx950): a C-ABI HIP library plus a thin
ctypes binding.

Entry points (same names as the C functions in ``include/paged_attn.h``):
``paged_kv_write``, ``paged_attn_decode``, ``paged_attn_prefill``,
``paged_attn_decode_workspace_bytes``, ``paged_attn_decode_workers``, and for
8-bit (INT8 / FP8 E4M3) pools ``paged_kv_write_quant`` and
``paged_attn_decode_quant``, ``paged_attn_prefill_quant`` and
``paged_attn_mixed_quant``; ``paged_attn_decode_noalloc`` (decode with the
library's fixed scratch instead of a workspace);
``paged_kv_copy_blocks`` (copy-on-write) and
``paged_attn_mixed`` (prefill chunks and decode rows in one call);
``paged_kv_compress`` and ``paged_attn_decode_compressed`` (the compressed-slot
tier: mean-pooled slots of evicted blocks attended next to the recent window).
``PrefixCache`` shares cached prompt blocks between sequences;
``CompressedTier`` keeps the host bookkeeping of the compressed tier.
``BlockAllocator`` is the host-side block allocator that builds the tables.
Every entry point takes ``debug=True`` to check its device-resident indices
on the host first (``validate``; raises ``InvalidContent``).
"""
from .allocator import BlockAllocator, UNMAPPED  # noqa: F401
from .prefix_cache import PrefixCache  # noqa: F401
from .compressed_tier import CompressedTier, CompressOps  # noqa: F401
from .validate import InvalidContent  # noqa: F401
from ._lib import (  # noqa: F401
    LIB, LIB_PATH, EXPORTS, PagedAttnError, Geometry, geometry,
    PKV_F32, PKV_F16, PKV_BF16, PKV_I8, PKV_FP8, PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EWORKSPACE, PKV_EHIP,
    PKV_ESCRATCH, paged_kv_write, paged_attn_decode, paged_attn_decode_noalloc, paged_attn_prefill,
    paged_attn_decode_workspace_bytes, paged_attn_decode_workers, decode_workspace,
    paged_kv_write_quant, paged_attn_decode_quant, bind_kv_write_quant, bind_decode_quant,
    paged_attn_prefill_quant, bind_prefill_quant, paged_attn_mixed_quant, bind_mixed_quant,
    paged_kv_copy_blocks, paged_attn_mixed, bind_mixed,
    paged_kv_compress, paged_attn_decode_compressed, bind_decode_compressed, bind_kv_compress,
)
