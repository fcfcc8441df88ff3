"""ctypes binding of ``libpagedattn.so`` (argument marshalling only).

Every function here takes torch tensors for device memory, reads their data
pointers, shapes and the current HIP stream, and calls the C entry point of
the same name; the computation is entirely in the library's kernels.  A
missing library raises at import time: there is no fallback.

``debug=True`` on a call (or PKV_DEBUG=1 in the environment) adds a host-side
check of its device-resident indices before the C call (``validate``): it
synchronises the device and copies tables and lengths back, so it is for
finding a caller's bug, not for the hot path.

The library is loaded after torch so that the HIP runtime torch already
mapped serves both (same soname).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from . import validate as _val

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PKV_LIBRARY", os.path.join(_HERE, "libpagedattn.so"))

PKV_F32, PKV_F16, PKV_BF16, PKV_I8, PKV_FP8 = 0, 1, 2, 3, 4
PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EWORKSPACE, PKV_EHIP, PKV_ESCRATCH = 0, -1, -2, -3, -4, -5

# 8-bit pools are torch.int8 (INT8 codes) or torch.float8_e4m3fn (FP8 E4M3
# codes); their row scales are separate float32 tensors.
_DTYPES = {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16,
           torch.int8: PKV_I8, torch.float8_e4m3fn: PKV_FP8}
_QUANT = (torch.int8, torch.float8_e4m3fn)

# Every symbol declared in include/paged_attn.h.
EXPORTS = ("paged_kv_write", "paged_attn_decode_workspace_bytes", "paged_attn_decode_workers",
           "paged_attn_decode", "paged_attn_prefill", "paged_kv_write_quant", "paged_attn_decode_quant",
           "paged_attn_prefill_quant", "paged_kv_copy_blocks",
           "paged_attn_mixed_quant", "paged_attn_mixed", "paged_kv_compress",
           "paged_attn_decode_compressed", "paged_attn_decode_noalloc",
           "pkv_status_string", "pkv_last_hip_error", "pkv_version")


class Geometry(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("kv_dtype", ctypes.c_int32)]


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python paged_kv_cache_30_amd/build.py` "
            "(the HIP library is the only implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    G = ctypes.POINTER(Geometry)
    lib.paged_kv_write.argtypes = [G, P, P, P, P, P, P, I32, P, I32, I32, P]
    lib.paged_kv_write.restype = ctypes.c_int
    lib.paged_attn_decode_workspace_bytes.argtypes = [G, I32, I32, I32, I32, I32]
    lib.paged_attn_decode_workspace_bytes.restype = SZ
    lib.paged_attn_decode_workers.argtypes = [G, I32, I32, I32, I32]
    lib.paged_attn_decode_workers.restype = I32
    lib.paged_attn_decode.argtypes = [G, P, P, P, P, P, P, I32, P, I32, I32, I32, I32, F, I32, P, SZ, P]
    lib.paged_attn_decode.restype = ctypes.c_int
    lib.paged_attn_decode_noalloc.argtypes = [G, P, P, P, P, P, P, I32, P, I32, I32, I32, I32, F, I32, P]
    lib.paged_attn_decode_noalloc.restype = ctypes.c_int
    lib.paged_attn_prefill.argtypes = [G, P, P, P, P, P, P, P, I32, P, I32, I32, I32, I32, I32, F, P]
    lib.paged_attn_prefill.restype = ctypes.c_int
    lib.paged_kv_write_quant.argtypes = [G, P, P, P, P, P, P, I32, P, P, I32, P, I32, I32, P]
    lib.paged_kv_write_quant.restype = ctypes.c_int
    lib.paged_attn_decode_quant.argtypes = [G, P, P, P, I32, P, P, P, P, P, I32, P, I32, I32, I32, I32, F, I32, P,
                                            SZ, P]
    lib.paged_attn_decode_quant.restype = ctypes.c_int
    lib.paged_attn_prefill_quant.argtypes = [G, P, P, P, I32, P, P, P, P, P, P, I32, P, I32, I32, I32, I32, I32, F,
                                             P]
    lib.paged_attn_prefill_quant.restype = ctypes.c_int
    lib.paged_attn_mixed_quant.argtypes = [G, P, P, P, I32, P, P, P, P, P, P, I32, P, I32, I32, I32, I32, I32, F,
                                           I32, P, SZ, P]
    lib.paged_attn_mixed_quant.restype = ctypes.c_int
    lib.paged_kv_copy_blocks.argtypes = [G, P, P, P, P, P, P, I32, P]
    lib.paged_kv_copy_blocks.restype = ctypes.c_int
    lib.paged_attn_mixed.argtypes = [G, P, P, P, P, P, P, P, I32, P, I32, I32, I32, I32, I32, F, I32, P, SZ, P]
    lib.paged_attn_mixed.restype = ctypes.c_int
    lib.paged_kv_compress.argtypes = [G, P, P, P, I32, P, P, I32, P]
    lib.paged_kv_compress.restype = ctypes.c_int
    lib.paged_attn_decode_compressed.argtypes = [G, P, P, P, P, P, P, I32, P, P, P, I32, P, I32, I32, I32, F, I32,
                                                 P, SZ, P]
    lib.paged_attn_decode_compressed.restype = ctypes.c_int
    lib.pkv_status_string.argtypes = [ctypes.c_int]
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.pkv_last_hip_error.argtypes = []
    lib.pkv_last_hip_error.restype = ctypes.c_int
    lib.pkv_version.argtypes = []
    lib.pkv_version.restype = ctypes.c_int
    return lib


LIB = _load()


def _debug(flag) -> bool:
    """Debug mode of one call: the flag if given, else PKV_DEBUG=1 in the
    environment."""
    if flag is None:
        return os.environ.get("PKV_DEBUG", "0") not in ("", "0")
    return bool(flag)


def _host(*ts):
    """Host copies of device tensors, after every queued kernel has run
    (debug mode only: it synchronises the device)."""
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in ts]


def _check(status: int, what: str) -> None:
    if status != PKV_OK:
        msg = LIB.pkv_status_string(status).decode()
        if status == PKV_EHIP:
            msg += f" (hipError {LIB.pkv_last_hip_error()})"
        raise PagedAttnError(status, f"{what}: {msg}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev(t: torch.Tensor, name: str, dtype=None, ndim=None) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")
    return t


def geometry(k_pool: torch.Tensor, num_heads: int) -> Geometry:
    """Geometry of a [NB, B, Hkv, D] pool with ``num_heads`` query heads."""
    if k_pool.dim() != 4:
        raise ValueError("pool must be [num_blocks, block_size, num_kv_heads, head_dim]")
    if k_pool.dtype not in _DTYPES:
        raise ValueError(f"unsupported pool dtype {k_pool.dtype}")
    nb, b, hkv, d = k_pool.shape
    return Geometry(nb, b, num_heads, hkv, d, _DTYPES[k_pool.dtype])


def bind_kv_write(k_pool, v_pool, k_new, v_new, seq_idx, pos, block_tables, debug=None):
    """Check and marshal the arguments of ``paged_kv_write`` once; returns a
    callable ``f(stream=None)`` that makes the C call with them.  With
    ``debug`` (default: PKV_DEBUG=1) every call first checks the device-resident
    indices on the host (``validate.check_write``)."""
    _dev(k_pool, "k_pool", ndim=4)
    _dev(v_pool, "v_pool", dtype=k_pool.dtype)
    if v_pool.shape != k_pool.shape:
        raise ValueError("k_pool and v_pool differ in shape")
    _dev(k_new, "k_new", dtype=k_pool.dtype, ndim=3)
    _dev(v_new, "v_new", dtype=k_pool.dtype, ndim=3)
    _dev(seq_idx, "seq_idx", dtype=torch.int32, ndim=1)
    _dev(pos, "pos", dtype=torch.int32, ndim=1)
    _dev(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    T = k_new.shape[0]
    if k_new.shape[1:] != k_pool.shape[2:] or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [T, num_kv_heads, head_dim]")
    if seq_idx.shape[0] != T or pos.shape[0] != T:
        raise ValueError("seq_idx and pos need one entry per token")
    g = geometry(k_pool, k_pool.shape[2])
    args = (ctypes.byref(g), _ptr(k_pool), _ptr(v_pool), _ptr(k_new), _ptr(v_new), _ptr(seq_idx), _ptr(pos), T,
            _ptr(block_tables), block_tables.shape[0], block_tables.shape[1])
    keep = (g, k_pool, v_pool, k_new, v_new, seq_idx, pos, block_tables)
    dbg = _debug(debug)

    def call(stream=None):
        if dbg:
            _val.check_write(*_host(seq_idx, pos, block_tables), num_blocks=g.num_blocks,
                             block_size=g.block_size)
        _check(LIB.paged_kv_write(*args, _stream(stream)), "paged_kv_write")
    call.keep = keep
    return call


def paged_kv_write(k_pool, v_pool, k_new, v_new, seq_idx, pos, block_tables, stream=None, debug=None) -> None:
    """C ``paged_kv_write``: store k_new/v_new [T, Hkv, D] at (seq_idx, pos)."""
    bind_kv_write(k_pool, v_pool, k_new, v_new, seq_idx, pos, block_tables, debug)(stream)


def paged_attn_decode_workspace_bytes(k_pool, num_heads, num_seqs, max_context_len, window=0,
                                      num_workers=0, sinks=0) -> int:
    g = geometry(k_pool, num_heads)
    return int(LIB.paged_attn_decode_workspace_bytes(ctypes.byref(g), num_seqs, max_context_len, window, sinks,
                                                     num_workers))


def paged_attn_decode_workers(k_pool, num_heads, num_seqs, max_context_len, window=0, sinks=0) -> int:
    g = geometry(k_pool, num_heads)
    return int(LIB.paged_attn_decode_workers(ctypes.byref(g), num_seqs, max_context_len, window, sinks))


def decode_workspace(k_pool, num_heads, num_seqs, max_context_len, window=0, num_workers=0, sinks=0):
    """A device workspace tensor of the size paged_attn_decode needs."""
    n = paged_attn_decode_workspace_bytes(k_pool, num_heads, num_seqs, max_context_len, window, num_workers,
                                          sinks)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=k_pool.device)


def bind_decode(out, q, k_pool, v_pool, block_tables, context_lens, max_context_len, *,
                window=0, scale, num_workers=0, workspace=None, lse=None, sinks=0, debug=None):
    """Check and marshal the arguments of ``paged_attn_decode`` once; returns
    a callable ``f(stream=None)`` that makes the C call with them.  With
    ``debug`` every call first checks the tables and lengths on the host
    (``validate.check_decode``)."""
    _dev(q, "q", dtype=k_pool.dtype, ndim=3)
    _dev(out, "out", dtype=torch.float32, ndim=3)
    _dev(k_pool, "k_pool", ndim=4)
    _dev(v_pool, "v_pool", dtype=k_pool.dtype)
    _dev(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _dev(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    S, H, D = q.shape
    if out.shape != q.shape or context_lens.shape[0] != S or block_tables.shape[0] != S:
        raise ValueError("shape mismatch between q, out, context_lens and block_tables")
    if lse is not None:
        _dev(lse, "lse", dtype=torch.float32, ndim=2)
        if lse.shape != (S, H):
            raise ValueError("lse must be [S, H]")
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    g = geometry(k_pool, H)
    args = (ctypes.byref(g), _ptr(out), _ptr(lse), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
            block_tables.shape[1], _ptr(context_lens), S, int(max_context_len), int(window), int(sinks),
            float(scale), int(num_workers), _ptr(workspace), ws_bytes)
    keep = (g, out, q, k_pool, v_pool, block_tables, context_lens, workspace, lse)
    dbg = _debug(debug)

    def call(stream=None):
        if dbg:
            _val.check_decode(*_host(block_tables, context_lens), max_context_len=int(max_context_len),
                              num_blocks=g.num_blocks, block_size=g.block_size, window=int(window),
                              sinks=int(sinks))
        _check(LIB.paged_attn_decode(*args, _stream(stream)), "paged_attn_decode")
    call.keep = keep
    return call


def paged_attn_decode(out, q, k_pool, v_pool, block_tables, context_lens, max_context_len, *,
                      window=0, scale, num_workers=0, workspace=None, lse=None, stream=None, sinks=0,
                      debug=None) -> None:
    """C ``paged_attn_decode``: out[S, H, D] (fp32) for q[S, H, D]."""
    bind_decode(out, q, k_pool, v_pool, block_tables, context_lens, max_context_len, window=window,
                scale=scale, num_workers=num_workers, workspace=workspace, lse=lse, sinks=sinks,
                debug=debug)(stream)


def paged_attn_decode_noalloc(out, q, k_pool, v_pool, block_tables, context_lens, max_context_len, *,
                              window=0, scale, lse=None, num_workers=0, stream=None, sinks=0, debug=None) -> None:
    """C ``paged_attn_decode_noalloc``: ``paged_attn_decode`` with the library's
    fixed per-GPU scratch as its workspace (no allocation in the call; calls
    that can overlap on one GPU race)."""
    _dev(q, "q", dtype=k_pool.dtype, ndim=3)
    _dev(out, "out", dtype=torch.float32, ndim=3)
    _dev(k_pool, "k_pool", ndim=4)
    _dev(v_pool, "v_pool", dtype=k_pool.dtype)
    _dev(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _dev(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    S, H, D = q.shape
    if out.shape != q.shape or context_lens.shape[0] != S or block_tables.shape[0] != S:
        raise ValueError("shape mismatch between q, out, context_lens and block_tables")
    if lse is not None:
        _dev(lse, "lse", dtype=torch.float32, ndim=2)
        if lse.shape != (S, H):
            raise ValueError("lse must be [S, H]")
    g = geometry(k_pool, H)
    if _debug(debug):
        _val.check_decode(*_host(block_tables, context_lens), max_context_len=int(max_context_len),
                          num_blocks=g.num_blocks, block_size=g.block_size, window=int(window), sinks=int(sinks),
                          what="paged_attn_decode_noalloc")
    _check(LIB.paged_attn_decode_noalloc(ctypes.byref(g), _ptr(out), _ptr(lse), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                         _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), S,
                                         int(max_context_len), int(window), int(sinks), float(scale),
                                         int(num_workers), _stream(stream)),
           "paged_attn_decode_noalloc")


def bind_prefill(out, q, q_start, k_pool, v_pool, block_tables, context_lens, max_q_len, max_context_len, *,
                 window=0, scale, lse=None, sinks=0, debug=None):
    """Check and marshal the arguments of ``paged_attn_prefill`` once; returns
    a callable ``f(stream=None)`` that makes the C call with them.  With
    ``debug`` every call first checks q_start, the tables and lengths on the
    host (``validate.check_prefill``)."""
    _dev(q, "q", dtype=k_pool.dtype, ndim=3)
    _dev(out, "out", dtype=torch.float32, ndim=3)
    _dev(q_start, "q_start", dtype=torch.int32, ndim=1)
    _dev(k_pool, "k_pool", ndim=4)
    _dev(v_pool, "v_pool", dtype=k_pool.dtype)
    _dev(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _dev(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    T, H, D = q.shape
    S = context_lens.shape[0]
    if out.shape != q.shape or q_start.shape[0] != S + 1 or block_tables.shape[0] != S:
        raise ValueError("shape mismatch between q, out, q_start, context_lens and block_tables")
    if lse is not None:
        _dev(lse, "lse", dtype=torch.float32, ndim=2)
        if lse.shape != (T, H):
            raise ValueError("lse must be [T, H]")
    g = geometry(k_pool, H)
    args = (ctypes.byref(g), _ptr(out), _ptr(lse), _ptr(q), _ptr(q_start), _ptr(k_pool), _ptr(v_pool),
            _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), S, int(max_q_len), int(max_context_len),
            int(window), int(sinks), float(scale))
    keep = (g, out, q, q_start, k_pool, v_pool, block_tables, context_lens, lse)
    dbg = _debug(debug)

    def call(stream=None):
        if dbg:
            _val.check_prefill(*_host(q_start, block_tables, context_lens), num_rows=T, max_q_len=int(max_q_len),
                               max_context_len=int(max_context_len), num_blocks=g.num_blocks,
                               block_size=g.block_size, window=int(window), sinks=int(sinks))
            _debug_v_range(v_pool, q_start, block_tables, context_lens, window=window, sinks=sinks, min_rows=1,
                           what="paged_attn_prefill")
        _check(LIB.paged_attn_prefill(*args, _stream(stream)), "paged_attn_prefill")
    call.keep = keep
    return call


def _debug_v_range(v_pool, q_start, block_tables, context_lens, *, window, sinks, min_rows, what):
    """Debug mode, bf16 pools: the attended V rows of the chunks the prefill
    kernel computes lie within the range it converts to fp16 exactly."""
    if v_pool.dtype != torch.bfloat16:
        return
    qs, tb, ln = _host(q_start, block_tables, context_lens)
    blk, slot, seq = _val.prefill_v_rows(qs, tb, ln, block_size=v_pool.shape[1], window=int(window),
                                         sinks=int(sinks), min_rows=min_rows)
    if blk.size == 0:
        return
    rows = v_pool[torch.from_numpy(blk).to(v_pool.device), torch.from_numpy(slot).to(v_pool.device)]
    amax = rows.float().abs().amax(dim=(1, 2)).cpu().numpy()
    _val.check_prefill_v_range(amax, seq, _val.PREFILL_BF16_V_LIMIT, what)


def paged_attn_prefill(out, q, q_start, k_pool, v_pool, block_tables, context_lens, max_q_len,
                       max_context_len, *, window=0, scale, lse=None, stream=None, sinks=0, debug=None) -> None:
    """C ``paged_attn_prefill``: out[T, H, D] (fp32) for chunk queries q[T, H, D]."""
    bind_prefill(out, q, q_start, k_pool, v_pool, block_tables, context_lens, max_q_len, max_context_len,
                 window=window, scale=scale, lse=lse, sinks=sinks, debug=debug)(stream)


# ------------------------------------------------------------- 8-bit pools

def _check_quant_pools(k_pool, v_pool, k_scale, v_scale):
    _dev(k_pool, "k_pool", ndim=4)
    if k_pool.dtype not in _QUANT:
        raise ValueError("8-bit pools are torch.int8 (INT8) or torch.float8_e4m3fn (FP8)")
    _dev(v_pool, "v_pool", dtype=k_pool.dtype)
    if v_pool.shape != k_pool.shape:
        raise ValueError("k_pool and v_pool differ in shape")
    nb, b, hkv, _ = k_pool.shape
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        _dev(t, name, dtype=torch.float32, ndim=3)
        if tuple(t.shape) != (nb, hkv, b):
            raise ValueError(f"{name} must be [num_blocks, num_kv_heads, block_size]")


def bind_kv_write_quant(k_pool, v_pool, k_scale, v_scale, k_new, v_new, seq_idx, pos, block_tables, debug=None):
    """Check and marshal the arguments of ``paged_kv_write_quant`` once;
    returns a callable ``f(stream=None)``."""
    _check_quant_pools(k_pool, v_pool, k_scale, v_scale)
    _dev(k_new, "k_new", ndim=3)
    _dev(v_new, "v_new", dtype=k_new.dtype, ndim=3)
    if k_new.dtype not in (torch.float32, torch.float16, torch.bfloat16):
        raise ValueError("k_new/v_new must be float32, float16 or bfloat16")
    _dev(seq_idx, "seq_idx", dtype=torch.int32, ndim=1)
    _dev(pos, "pos", dtype=torch.int32, ndim=1)
    _dev(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    T = k_new.shape[0]
    if k_new.shape[1:] != k_pool.shape[2:] or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [T, num_kv_heads, head_dim]")
    if seq_idx.shape[0] != T or pos.shape[0] != T:
        raise ValueError("seq_idx and pos need one entry per token")
    g = geometry(k_pool, k_pool.shape[2])
    args = (ctypes.byref(g), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(k_new), _ptr(v_new),
            _DTYPES[k_new.dtype], _ptr(seq_idx), _ptr(pos), T, _ptr(block_tables), block_tables.shape[0],
            block_tables.shape[1])
    keep = (g, k_pool, v_pool, k_scale, v_scale, k_new, v_new, seq_idx, pos, block_tables)
    dbg = _debug(debug)

    def call(stream=None):
        if dbg:
            _val.check_write(*_host(seq_idx, pos, block_tables), num_blocks=g.num_blocks,
                             block_size=g.block_size, what="paged_kv_write_quant")
        _check(LIB.paged_kv_write_quant(*args, _stream(stream)), "paged_kv_write_quant")
    call.keep = keep
    return call


def paged_kv_write_quant(k_pool, v_pool, k_scale, v_scale, k_new, v_new, seq_idx, pos, block_tables,
                         stream=None, debug=None) -> None:
    """C ``paged_kv_write_quant``: encode k_new/v_new [T, Hkv, D] into 8-bit pools."""
    bind_kv_write_quant(k_pool, v_pool, k_scale, v_scale, k_new, v_new, seq_idx, pos, block_tables,
                        debug)(stream)


def bind_decode_quant(out, q, k_pool, v_pool, k_scale, v_scale, block_tables, context_lens, max_context_len, *,
                      window=0, scale, num_workers=0, workspace=None, lse=None, sinks=0, debug=None):
    """Check and marshal the arguments of ``paged_attn_decode_quant`` once;
    returns a callable ``f(stream=None)``."""
    _check_quant_pools(k_pool, v_pool, k_scale, v_scale)
    _dev(q, "q", ndim=3)
    if q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("q must be float16 or bfloat16 for 8-bit pools")
    _dev(out, "out", dtype=torch.float32, ndim=3)
    _dev(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _dev(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    S, H, D = q.shape
    if out.shape != q.shape or context_lens.shape[0] != S or block_tables.shape[0] != S:
        raise ValueError("shape mismatch between q, out, context_lens and block_tables")
    if lse is not None:
        _dev(lse, "lse", dtype=torch.float32, ndim=2)
        if lse.shape != (S, H):
            raise ValueError("lse must be [S, H]")
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    g = geometry(k_pool, H)
    args = (ctypes.byref(g), _ptr(out), _ptr(lse), _ptr(q), _DTYPES[q.dtype], _ptr(k_pool), _ptr(v_pool),
            _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), S,
            int(max_context_len), int(window), int(sinks), float(scale), int(num_workers), _ptr(workspace),
            ws_bytes)
    keep = (g, out, q, k_pool, v_pool, k_scale, v_scale, block_tables, context_lens, workspace, lse)
    dbg = _debug(debug)

    def call(stream=None):
        if dbg:
            _val.check_decode(*_host(block_tables, context_lens), max_context_len=int(max_context_len),
                              num_blocks=g.num_blocks, block_size=g.block_size, window=int(window),
                              sinks=int(sinks), what="paged_attn_decode_quant")
        _check(LIB.paged_attn_decode_quant(*args, _stream(stream)), "paged_attn_decode_quant")
    call.keep = keep
    return call


def paged_attn_decode_quant(out, q, k_pool, v_pool, k_scale, v_scale, block_tables, context_lens,
                            max_context_len, *, window=0, scale, num_workers=0, workspace=None, lse=None,
                            stream=None, sinks=0, debug=None) -> None:
    """C ``paged_attn_decode_quant``: decode over 8-bit pools with row scales."""
    bind_decode_quant(out, q, k_pool, v_pool, k_scale, v_scale, block_tables, context_lens, max_context_len,
                      window=window, scale=scale, num_workers=num_workers, workspace=workspace, lse=lse,
                      sinks=sinks, debug=debug)(stream)


def bind_prefill_quant(out, q, q_start, k_pool, v_pool, k_scale, v_scale, block_tables, context_lens, max_q_len,
                       max_context_len, *, window=0, scale, lse=None, sinks=0, debug=None):
    """Check and marshal the arguments of ``paged_attn_prefill_quant`` once;
    returns a callable ``f(stream=None)``."""
    _check_quant_pools(k_pool, v_pool, k_scale, v_scale)
    _dev(q, "q", ndim=3)
    if q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("q must be float16 or bfloat16 for 8-bit pools")
    _dev(out, "out", dtype=torch.float32, ndim=3)
    _dev(q_start, "q_start", dtype=torch.int32, ndim=1)
    _dev(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _dev(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    T, H, D = q.shape
    S = context_lens.shape[0]
    if out.shape != q.shape or q_start.shape[0] != S + 1 or block_tables.shape[0] != S:
        raise ValueError("shape mismatch between q, out, q_start, context_lens and block_tables")
    if lse is not None:
        _dev(lse, "lse", dtype=torch.float32, ndim=2)
        if lse.shape != (T, H):
            raise ValueError("lse must be [T, H]")
    g = geometry(k_pool, H)
    args = (ctypes.byref(g), _ptr(out), _ptr(lse), _ptr(q), _DTYPES[q.dtype], _ptr(q_start), _ptr(k_pool),
            _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), block_tables.shape[1],
            _ptr(context_lens), S, int(max_q_len), int(max_context_len), int(window), int(sinks), float(scale))
    keep = (g, out, q, q_start, k_pool, v_pool, k_scale, v_scale, block_tables, context_lens, lse)
    dbg = _debug(debug)

    def call(stream=None):
        if dbg:
            _val.check_prefill(*_host(q_start, block_tables, context_lens), num_rows=T, max_q_len=int(max_q_len),
                               max_context_len=int(max_context_len), num_blocks=g.num_blocks,
                               block_size=g.block_size, window=int(window), sinks=int(sinks),
                               what="paged_attn_prefill_quant")
        _check(LIB.paged_attn_prefill_quant(*args, _stream(stream)), "paged_attn_prefill_quant")
    call.keep = keep
    return call


def paged_attn_prefill_quant(out, q, q_start, k_pool, v_pool, k_scale, v_scale, block_tables, context_lens,
                             max_q_len, max_context_len, *, window=0, scale, lse=None, stream=None, sinks=0,
                             debug=None) -> None:
    """C ``paged_attn_prefill_quant``: chunked prefill over 8-bit pools with
    row scales."""
    bind_prefill_quant(out, q, q_start, k_pool, v_pool, k_scale, v_scale, block_tables, context_lens, max_q_len,
                       max_context_len, window=window, scale=scale, lse=lse, sinks=sinks, debug=debug)(stream)


# ------------------------------------------------- block copies, mixed batches

def paged_kv_copy_blocks(k_pool, v_pool, src, dst, k_scale=None, v_scale=None, stream=None, debug=None) -> None:
    """C ``paged_kv_copy_blocks``: copy block src[i] to dst[i] in both pools
    (and the row scales of 8-bit pools)."""
    _dev(k_pool, "k_pool", ndim=4)
    _dev(v_pool, "v_pool", dtype=k_pool.dtype)
    if v_pool.shape != k_pool.shape:
        raise ValueError("k_pool and v_pool differ in shape")
    if k_pool.dtype in _QUANT:
        _check_quant_pools(k_pool, v_pool, k_scale, v_scale)
    elif k_scale is not None or v_scale is not None:
        raise ValueError("row scales belong to 8-bit pools only")
    _dev(src, "src", dtype=torch.int32, ndim=1)
    _dev(dst, "dst", dtype=torch.int32, ndim=1)
    if src.shape != dst.shape:
        raise ValueError("src and dst need one entry per pair")
    g = geometry(k_pool, k_pool.shape[2])
    if _debug(debug):
        _val.check_copy_blocks(*_host(src, dst), num_blocks=g.num_blocks)
    _check(LIB.paged_kv_copy_blocks(ctypes.byref(g), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
                                    _ptr(src), _ptr(dst), src.shape[0], _stream(stream)), "paged_kv_copy_blocks")


def bind_mixed(out, q, q_start, k_pool, v_pool, block_tables, context_lens, max_q_len, max_context_len, *,
               window=0, scale, num_workers=0, workspace=None, lse=None, sinks=0, debug=None):
    """Check and marshal the arguments of ``paged_attn_mixed`` once; returns
    a callable ``f(stream=None)``."""
    _dev(q, "q", dtype=k_pool.dtype, ndim=3)
    _dev(out, "out", dtype=torch.float32, ndim=3)
    _dev(q_start, "q_start", dtype=torch.int32, ndim=1)
    _dev(k_pool, "k_pool", ndim=4)
    _dev(v_pool, "v_pool", dtype=k_pool.dtype)
    _dev(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _dev(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    T, H, D = q.shape
    S = context_lens.shape[0]
    if out.shape != q.shape or q_start.shape[0] != S + 1 or block_tables.shape[0] != S:
        raise ValueError("shape mismatch between q, out, q_start, context_lens and block_tables")
    if lse is not None:
        _dev(lse, "lse", dtype=torch.float32, ndim=2)
        if lse.shape != (T, H):
            raise ValueError("lse must be [T, H]")
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    g = geometry(k_pool, H)
    args = (ctypes.byref(g), _ptr(out), _ptr(lse), _ptr(q), _ptr(q_start), _ptr(k_pool), _ptr(v_pool),
            _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), S, int(max_q_len), int(max_context_len),
            int(window), int(sinks), float(scale), int(num_workers), _ptr(workspace), ws_bytes)
    keep = (g, out, q, q_start, k_pool, v_pool, block_tables, context_lens, workspace, lse)
    dbg = _debug(debug)

    def call(stream=None):
        if dbg:
            _val.check_prefill(*_host(q_start, block_tables, context_lens), num_rows=T, max_q_len=int(max_q_len),
                               max_context_len=int(max_context_len), num_blocks=g.num_blocks,
                               block_size=g.block_size, window=int(window), sinks=int(sinks),
                               what="paged_attn_mixed")
            _debug_v_range(v_pool, q_start, block_tables, context_lens, window=window, sinks=sinks, min_rows=2,
                           what="paged_attn_mixed")
        _check(LIB.paged_attn_mixed(*args, _stream(stream)), "paged_attn_mixed")
    call.keep = keep
    return call


def paged_attn_mixed(out, q, q_start, k_pool, v_pool, block_tables, context_lens, max_q_len, max_context_len, *,
                     window=0, scale, num_workers=0, workspace=None, lse=None, stream=None, sinks=0,
                     debug=None) -> None:
    """C ``paged_attn_mixed``: prefill chunks and single decode rows in one call."""
    bind_mixed(out, q, q_start, k_pool, v_pool, block_tables, context_lens, max_q_len, max_context_len,
               window=window, scale=scale, num_workers=num_workers, workspace=workspace, lse=lse,
               sinks=sinks, debug=debug)(stream)


# ------------------------------------------------------- compressed slots

def bind_kv_compress(k_pool, v_pool, src_blocks, dst_block, dst_slot, debug=None):
    """Check and marshal the arguments of ``paged_kv_compress`` once; returns
    a callable ``f(stream=None)``."""
    _dev(k_pool, "k_pool", ndim=4)
    _dev(v_pool, "v_pool", dtype=k_pool.dtype)
    if v_pool.shape != k_pool.shape:
        raise ValueError("k_pool and v_pool differ in shape")
    _dev(src_blocks, "src_blocks", dtype=torch.int32, ndim=2)
    _dev(dst_block, "dst_block", dtype=torch.int32, ndim=1)
    _dev(dst_slot, "dst_slot", dtype=torch.int32, ndim=1)
    n = dst_block.shape[0]
    if dst_slot.shape[0] != n or src_blocks.shape[0] != n:
        raise ValueError("src_blocks, dst_block and dst_slot need one entry (row) per op")
    g = geometry(k_pool, k_pool.shape[2])
    args = (ctypes.byref(g), _ptr(k_pool), _ptr(v_pool), _ptr(src_blocks), max(int(src_blocks.shape[1]), 1),
            _ptr(dst_block), _ptr(dst_slot), n)
    keep = (g, k_pool, v_pool, src_blocks, dst_block, dst_slot)
    dbg = _debug(debug)

    def call(stream=None):
        if dbg:
            _val.check_compress(*_host(src_blocks, dst_block, dst_slot), num_blocks=g.num_blocks,
                                block_size=g.block_size)
        _check(LIB.paged_kv_compress(*args, _stream(stream)), "paged_kv_compress")
    call.keep = keep
    return call


def paged_kv_compress(k_pool, v_pool, src_blocks, dst_block, dst_slot, stream=None, debug=None) -> None:
    """C ``paged_kv_compress``: op i writes the mean of every row of blocks
    src_blocks[i, :] into row dst_slot[i] of block dst_block[i]."""
    bind_kv_compress(k_pool, v_pool, src_blocks, dst_block, dst_slot, debug)(stream)


def bind_decode_compressed(out, q, k_pool, v_pool, block_tables, context_lens, full_start, slot_tables, num_slots,
                           max_context_len, *, window=0, scale, num_workers=0, workspace=None, lse=None,
                           debug=None):
    """Check and marshal the arguments of ``paged_attn_decode_compressed``
    once; returns a callable ``f(stream=None)``."""
    _dev(q, "q", dtype=k_pool.dtype, ndim=3)
    _dev(out, "out", dtype=torch.float32, ndim=3)
    _dev(k_pool, "k_pool", ndim=4)
    _dev(v_pool, "v_pool", dtype=k_pool.dtype)
    _dev(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _dev(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    _dev(full_start, "full_start", dtype=torch.int32, ndim=1)
    _dev(slot_tables, "slot_tables", dtype=torch.int32, ndim=2)
    _dev(num_slots, "num_slots", dtype=torch.int32, ndim=1)
    S, H, D = q.shape
    if (out.shape != q.shape or context_lens.shape[0] != S or block_tables.shape[0] != S
            or full_start.shape[0] != S or slot_tables.shape[0] != S or num_slots.shape[0] != S):
        raise ValueError("shape mismatch between q, out and the per-sequence arrays")
    if lse is not None:
        _dev(lse, "lse", dtype=torch.float32, ndim=2)
        if lse.shape != (S, H):
            raise ValueError("lse must be [S, H]")
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    g = geometry(k_pool, H)
    args = (ctypes.byref(g), _ptr(out), _ptr(lse), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
            block_tables.shape[1], _ptr(context_lens), _ptr(full_start), _ptr(slot_tables), slot_tables.shape[1],
            _ptr(num_slots), S, int(max_context_len), int(window), float(scale), int(num_workers),
            _ptr(workspace), ws_bytes)
    keep = (g, out, q, k_pool, v_pool, block_tables, context_lens, full_start, slot_tables, num_slots, workspace,
            lse)
    dbg = _debug(debug)

    def call(stream=None):
        if dbg:
            _val.check_decode_compressed(*_host(block_tables, context_lens, full_start, slot_tables, num_slots),
                                         max_context_len=int(max_context_len), num_blocks=g.num_blocks,
                                         block_size=g.block_size, window=int(window))
        _check(LIB.paged_attn_decode_compressed(*args, _stream(stream)), "paged_attn_decode_compressed")
    call.keep = keep
    return call


def paged_attn_decode_compressed(out, q, k_pool, v_pool, block_tables, context_lens, full_start, slot_tables,
                                 num_slots, max_context_len, *, window=0, scale, num_workers=0, workspace=None,
                                 lse=None, stream=None, debug=None) -> None:
    """C ``paged_attn_decode_compressed``: decode over compressed slots and
    the full-resolution positions [full_start, L)."""
    bind_decode_compressed(out, q, k_pool, v_pool, block_tables, context_lens, full_start, slot_tables, num_slots,
                           max_context_len, window=window, scale=scale, num_workers=num_workers,
                           workspace=workspace, lse=lse, debug=debug)(stream)


def bind_mixed_quant(out, q, q_start, k_pool, v_pool, k_scale, v_scale, block_tables, context_lens, max_q_len,
                     max_context_len, *, window=0, scale, num_workers=0, workspace=None, lse=None, sinks=0,
                     debug=None):
    """Check and marshal the arguments of ``paged_attn_mixed_quant`` once;
    returns a callable ``f(stream=None)``.  Without ``workspace`` one of the
    size the call needs is allocated here, once."""
    _check_quant_pools(k_pool, v_pool, k_scale, v_scale)
    _dev(q, "q", ndim=3)
    if q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("q must be float16 or bfloat16 for 8-bit pools")
    _dev(out, "out", dtype=torch.float32, ndim=3)
    _dev(q_start, "q_start", dtype=torch.int32, ndim=1)
    _dev(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _dev(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    T, H, D = q.shape
    S = context_lens.shape[0]
    if out.shape != q.shape or q_start.shape[0] != S + 1 or block_tables.shape[0] != S:
        raise ValueError("shape mismatch between q, out, q_start, context_lens and block_tables")
    if lse is not None:
        _dev(lse, "lse", dtype=torch.float32, ndim=2)
        if lse.shape != (T, H):
            raise ValueError("lse must be [T, H]")
    if workspace is None:
        workspace = decode_workspace(k_pool, H, S, max_context_len, window, num_workers, sinks=sinks)
    _dev(workspace, "workspace")
    ws_bytes = workspace.numel() * workspace.element_size()
    g = geometry(k_pool, H)
    args = (ctypes.byref(g), _ptr(out), _ptr(lse), _ptr(q), _DTYPES[q.dtype], _ptr(q_start), _ptr(k_pool),
            _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), block_tables.shape[1],
            _ptr(context_lens), S, int(max_q_len), int(max_context_len), int(window), int(sinks), float(scale),
            int(num_workers), _ptr(workspace), ws_bytes)
    keep = (g, out, q, q_start, k_pool, v_pool, k_scale, v_scale, block_tables, context_lens, workspace, lse)
    dbg = _debug(debug)

    def call(stream=None):
        if dbg:
            _val.check_prefill(*_host(q_start, block_tables, context_lens), num_rows=T, max_q_len=int(max_q_len),
                               max_context_len=int(max_context_len), num_blocks=g.num_blocks,
                               block_size=g.block_size, window=int(window), sinks=int(sinks),
                               what="paged_attn_mixed_quant")
        _check(LIB.paged_attn_mixed_quant(*args, _stream(stream)), "paged_attn_mixed_quant")
    call.keep = keep
    return call


def paged_attn_mixed_quant(out, q, q_start, k_pool, v_pool, k_scale, v_scale, block_tables, context_lens, max_q_len,
                           max_context_len, *, window=0, scale, num_workers=0, workspace=None, lse=None,
                           stream=None, sinks=0, debug=None) -> None:
    """C ``paged_attn_mixed_quant``: prefill chunks and single decode rows in
    one call over 8-bit pools."""
    bind_mixed_quant(out, q, q_start, k_pool, v_pool, k_scale, v_scale, block_tables, context_lens, max_q_len,
                     max_context_len, window=window, scale=scale, num_workers=num_workers, workspace=workspace,
                     lse=lse, sinks=sinks, debug=debug)(stream)
