"""Device staging of a workload for the library: pools, tables, lengths,
queries and the tokens one step writes, as torch device tensors.

Takes host arrays (anything with the fields of ``workloads.Workload``:
storage-dtype numpy arrays, with bfloat16 held as uint16 bit patterns).  The
cached history is written into the pools with the library's own
``paged_kv_write``; one ``step()`` is the hot path: write the step's new
tokens, then attend (decode or chunked prefill).
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch

from . import _lib

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
# 8-bit pool formats: code tensor dtype.
QUANT_DTYPE = {"i8": torch.int8, "fp8": torch.float8_e4m3fn}


def to_device(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Host storage array -> device tensor of the storage dtype (bit copy)."""
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to(device, non_blocking=False)


def from_device(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host storage array (bfloat16 as uint16 bits)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def int_tensor(a, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to(device)


class DeviceWorkload:
    """``kv_format``: "native" (pools in the workload's dtype) or "i8" / "fp8"
    (8-bit pools with row scales; keys and values are encoded on write from
    the workload's 16-bit or fp32 rows; decode and prefill)."""

    def __init__(self, w, device: str = "cuda", poison: bool = True, num_workers: int = 0,
                 with_lse: bool = True, write_history: bool = True, kv_format: str = "native"):
        self.w = w
        self.device = device
        self.kv_format = kv_format
        shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
        fill = math.nan if poison else 0.0
        self.k_scale = self.v_scale = None
        if kv_format == "native":
            dt = TORCH_DTYPE[w.dtype]
            self.k_pool = torch.full(shape, fill, dtype=dt, device=device)
            self.v_pool = torch.full(shape, fill, dtype=dt, device=device)
        else:
            if w.kind not in ("decode", "prefill"):
                raise ValueError("8-bit pools serve decode and prefill workloads")
            # unwritten rows: code 0xFF (NaN for FP8) and scale NaN (or zeros)
            code = 0xFF if poison else 0
            self.k_pool = torch.full(shape, code, dtype=torch.uint8, device=device).view(QUANT_DTYPE[kv_format])
            self.v_pool = torch.full(shape, code, dtype=torch.uint8, device=device).view(QUANT_DTYPE[kv_format])
            sshape = (w.num_blocks, w.num_kv_heads, w.block_size)
            self.k_scale = torch.full(sshape, fill, dtype=torch.float32, device=device)
            self.v_scale = torch.full(sshape, fill, dtype=torch.float32, device=device)
        self.tables = int_tensor(w.block_tables, device)
        self.lens = int_tensor(w.context_lens, device)
        self.q = to_device(w.q, w.dtype, device)
        self.q_start = int_tensor(w.q_start, device) if w.q_start is not None else None
        self.out = torch.empty(self.q.shape, dtype=torch.float32, device=device)
        self.lse = (torch.empty(self.q.shape[:2], dtype=torch.float32, device=device) if with_lse else None)
        si, pos, k, v = w.step_tokens()
        self.step_seq = int_tensor(si, device)
        self.step_pos = int_tensor(pos, device)
        self.step_k = to_device(k, w.dtype, device)
        self.step_v = to_device(v, w.dtype, device)
        self.compressed = getattr(w, "full_start", None) is not None
        if self.compressed:
            if kv_format != "native":
                raise ValueError("compressed slots need 16-bit or fp32 pools")
            self.full_start = int_tensor(w.full_start, device)
            self.slot_tables = int_tensor(w.slot_tables, device)
            self.num_slots = int_tensor(w.num_slots, device)
        self.workspace: Optional[torch.Tensor] = None
        self._bound_write = self._bound_attend = self._bound_compress = None
        self.set_workers(num_workers)
        if write_history:
            self.write_history()

    def set_workers(self, num_workers: int) -> None:
        """Decode worker count (0 = automatic) and a workspace sized for it."""
        self.num_workers = num_workers
        self._bound_attend = None
        w = self.w
        if w.kind == "decode":
            self.workspace = _lib.decode_workspace(self.k_pool, w.num_heads, w.num_seqs, w.max_context_len,
                                                   w.window, num_workers, sinks=w.sinks)
        else:
            self.workspace = None

    def _write(self, k, v, seq, pos):
        if self.kv_format == "native":
            return _lib.bind_kv_write(self.k_pool, self.v_pool, k, v, seq, pos, self.tables)
        return _lib.bind_kv_write_quant(self.k_pool, self.v_pool, self.k_scale, self.v_scale, k, v, seq, pos,
                                        self.tables)

    def write_history(self) -> None:
        w = self.w
        for s, p0, k, v in w.history_tokens():
            n = k.shape[0]
            self._write(to_device(k, w.dtype, self.device), to_device(v, w.dtype, self.device),
                        torch.full((n,), s, dtype=torch.int32, device=self.device),
                        torch.arange(p0, p0 + n, dtype=torch.int32, device=self.device))()
        if self.compressed:
            # slot row r of s is written like position r through the slot table
            for s, e in enumerate(w.slot_kv):
                n = e.k.shape[0]
                if n:
                    _lib.bind_kv_write(self.k_pool, self.v_pool, to_device(e.k, w.dtype, self.device),
                                       to_device(e.v, w.dtype, self.device),
                                       torch.full((n,), s, dtype=torch.int32, device=self.device),
                                       torch.arange(n, dtype=torch.int32, device=self.device), self.slot_tables)()

    def write_step(self, stream=None) -> None:
        if self._bound_write is None:
            self._bound_write = self._write(self.step_k, self.step_v, self.step_seq, self.step_pos)
        self._bound_write(stream)

    def attend(self, stream=None) -> None:
        w = self.w
        if self._bound_attend is None:
            if self.compressed:
                self._bound_attend = _lib.bind_decode_compressed(
                    self.out, self.q, self.k_pool, self.v_pool, self.tables, self.lens, self.full_start,
                    self.slot_tables, self.num_slots, w.max_context_len, window=w.window, scale=w.scale,
                    num_workers=self.num_workers, workspace=self.workspace, lse=self.lse)
            elif w.kind == "decode" and self.kv_format != "native":
                self._bound_attend = _lib.bind_decode_quant(
                    self.out, self.q, self.k_pool, self.v_pool, self.k_scale, self.v_scale, self.tables, self.lens,
                    w.max_context_len, window=w.window, scale=w.scale, num_workers=self.num_workers,
                    workspace=self.workspace, lse=self.lse, sinks=w.sinks)
            elif w.kind == "decode":
                self._bound_attend = _lib.bind_decode(
                    self.out, self.q, self.k_pool, self.v_pool, self.tables, self.lens, w.max_context_len,
                    window=w.window, scale=w.scale, num_workers=self.num_workers, workspace=self.workspace,
                    lse=self.lse, sinks=w.sinks)
            elif self.kv_format != "native":
                self._bound_attend = _lib.bind_prefill_quant(
                    self.out, self.q, self.q_start, self.k_pool, self.v_pool, self.k_scale, self.v_scale,
                    self.tables, self.lens, w.max_q_len, w.max_context_len, window=w.window, scale=w.scale,
                    lse=self.lse, sinks=w.sinks)
            else:
                self._bound_attend = _lib.bind_prefill(
                    self.out, self.q, self.q_start, self.k_pool, self.v_pool, self.tables, self.lens,
                    w.max_q_len, w.max_context_len, window=w.window, scale=w.scale, lse=self.lse, sinks=w.sinks)
        self._bound_attend(stream)

    def set_compress_ops(self, src_blocks, dst_block, dst_slot) -> None:
        """Compressions (``paged_kv_compress``) that every step runs before
        its write: op i averages blocks src_blocks[i] into row dst_slot[i] of
        block dst_block[i] (host int32 arrays)."""
        self.compress_ops = (int_tensor(np.asarray(src_blocks).reshape(len(dst_block), -1), self.device),
                             int_tensor(dst_block, self.device), int_tensor(dst_slot, self.device))
        self._bound_compress = _lib.bind_kv_compress(self.k_pool, self.v_pool, *self.compress_ops)

    def compress_step(self, stream=None) -> None:
        if self._bound_compress is not None:
            self._bound_compress(stream)

    def step(self, stream=None) -> None:
        """One pass of the hot path: compress (if set), write the new tokens,
        then attend."""
        self.compress_step(stream)
        self.write_step(stream)
        self.attend(stream)
