"""Host-side block allocator: hands out physical block ids and builds the
int32 block tables the kernels read.  Plain host bookkeeping, never timed.

Follows "Build a Paged KV Cache in Pure Python", Step 2 (``BlockAllocator``:
a stack of free block ids, pop on allocate and push on free, O(1) each;
``MemoryError`` with the counts when the pool cannot satisfy a request;
``stats``) and Step 3 (``ensure_blocks``: blocks are added as positions grow,
logical block b of a sequence holds positions [b*B, (b+1)*B)), and "Build a
Minimal LLM Inference Engine with Paged Attention and Adaptive KV Cache",
Step 1 and Step 2 (a page's refcount is the number of sequences referencing
it; a page returns to the free pool when its count reaches zero).

Differences from the pages, all deliberate:

* a sequence's logical block b always starts at position b*B (the printed
  ``start_pos`` bookkeeping is not kept);
* blocks can be shared between sequences (``share``) for common prefixes,
  counted by the refcount;
* ``trim_window`` frees the blocks that lie wholly before a sliding window and
  marks their table entries -1 - the block-table alternative to shifting a
  contiguous cache left that "Building a Streaming Sliding-Window Attention
  Engine in Pure Python", Step 2, mentions.
"""
from __future__ import annotations

from typing import Dict, Iterable, List, Optional

import numpy as np

UNMAPPED = -1


class BlockAllocator:
    """LIFO free list of ``num_blocks`` physical blocks of ``block_size``
    positions, per-sequence logical->physical tables and refcounts."""

    def __init__(self, num_blocks: int, block_size: int, order: Optional[Iterable[int]] = None):
        if num_blocks < 0 or block_size <= 0:
            raise ValueError("num_blocks must be >= 0 and block_size > 0")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        # Stack of free ids; allocate pops from the end.  ``order`` lets a
        # caller pre-shuffle the pool (the stack top is the last element).
        self.free_list: List[int] = list(range(num_blocks)) if order is None else [int(i) for i in order]
        if sorted(self.free_list) != list(range(num_blocks)):
            raise ValueError("order must be a permutation of range(num_blocks)")
        self.refcount = np.zeros(num_blocks, dtype=np.int64)
        self.tables: Dict[int, List[int]] = {}
        self.lengths: Dict[int, int] = {}

    # ----------------------------------------------------------- allocation
    def allocate(self, seq_id: int, num_blocks: int = 1) -> List[int]:
        """Append ``num_blocks`` fresh blocks to ``seq_id``'s table."""
        if num_blocks < 0:
            raise ValueError("num_blocks must be >= 0")
        if len(self.free_list) < num_blocks:
            raise MemoryError(
                f"KV cache out of memory: need {num_blocks} blocks, "
                f"only {len(self.free_list)} free of {self.num_blocks} total.")
        got = []
        for _ in range(num_blocks):
            b = self.free_list.pop()
            self.refcount[b] = 1
            got.append(b)
        self.tables.setdefault(seq_id, []).extend(got)
        self.lengths.setdefault(seq_id, 0)
        return got

    def ensure(self, seq_id: int, num_tokens: int) -> None:
        """Make the table cover positions [0, num_tokens)."""
        need = -(-int(num_tokens) // self.block_size)
        have = len(self.tables.get(seq_id, []))
        if have < need:
            self.allocate(seq_id, need - have)
        else:
            self.tables.setdefault(seq_id, [])
            self.lengths.setdefault(seq_id, 0)

    def append_tokens(self, seq_id: int, n: int = 1) -> np.ndarray:
        """Reserve the next ``n`` positions of ``seq_id`` (allocating blocks as
        needed); returns those positions (int32)."""
        L = self.lengths.get(seq_id, 0)
        self.ensure(seq_id, L + n)
        self.lengths[seq_id] = L + n
        return np.arange(L, L + n, dtype=np.int32)

    def share(self, src_seq: int, dst_seq: int, num_blocks: int) -> List[int]:
        """Map the first ``num_blocks`` blocks of ``src_seq`` into a new
        sequence ``dst_seq`` (a common prefix); refcount + 1 for each."""
        if dst_seq in self.tables and self.tables[dst_seq]:
            raise ValueError("share into an empty sequence only")
        src = self.tables[src_seq][:num_blocks]
        if len(src) < num_blocks or any(b == UNMAPPED for b in src):
            raise ValueError("source does not map that many blocks")
        for b in src:
            self.refcount[b] += 1
        self.tables[dst_seq] = list(src)
        self.lengths[dst_seq] = num_blocks * self.block_size
        return list(src)

    def _release(self, b: int) -> None:
        self.refcount[b] -= 1
        if self.refcount[b] < 0:
            raise RuntimeError(f"block {b} released more often than mapped")
        if self.refcount[b] == 0:
            self.free_list.append(b)

    def free(self, seq_id: int) -> None:
        """Drop ``seq_id``: every mapped block loses one reference and returns
        to the free list at zero."""
        for b in self.tables.pop(seq_id, []):
            if b != UNMAPPED:
                self._release(b)
        self.lengths.pop(seq_id, None)

    def trim_window(self, seq_id: int, context_len: int, window: int, sinks: int = 0,
                    chunk_len: int = 1) -> int:
        """Free the blocks that hold no position the next attention call can
        read: its query rows are the last ``chunk_len`` positions of
        ``context_len`` (1 for decode), so the earliest attended position is
        lo = L - chunk_len - window + 1, and with attention sinks positions
        [0, sinks) stay attended too.  Entry b goes when (b + 1) * B <= lo and
        b * B >= sinks.  Returns how many blocks were freed."""
        if window <= 0:
            return 0
        lo = int(context_len) - max(int(chunk_len), 1) - int(window) + 1
        cut = lo // self.block_size
        keep_below = -(-max(int(sinks), 0) // self.block_size)  # blocks holding sink positions
        row = self.tables.get(seq_id, [])
        freed = 0
        for b in range(keep_below, min(max(cut, 0), len(row))):
            if row[b] != UNMAPPED:
                self._release(row[b])
                row[b] = UNMAPPED
                freed += 1
        return freed

    # -------------------------------------------------------------- export
    def table(self, seq_ids: Iterable[int], width: Optional[int] = None) -> np.ndarray:
        """int32 [len(seq_ids), width] block table, -1 past each sequence's
        blocks and where blocks were freed."""
        seq_ids = list(seq_ids)
        rows = [self.tables.get(s, []) for s in seq_ids]
        w = max([len(r) for r in rows] + [1]) if width is None else int(width)
        out = np.full((len(seq_ids), w), UNMAPPED, dtype=np.int32)
        for i, r in enumerate(rows):
            if len(r) > w:
                raise ValueError("table wider than width")
            out[i, :len(r)] = r
        return out

    def context_lens(self, seq_ids: Iterable[int]) -> np.ndarray:
        return np.array([self.lengths.get(s, 0) for s in seq_ids], dtype=np.int32)

    def stats(self) -> dict:
        used = int((self.refcount > 0).sum())
        return {
            "total_blocks": self.num_blocks,
            "free_blocks": len(self.free_list),
            "used_blocks": used,
            "active_sequences": len(self.tables),
            "utilisation": used / self.num_blocks if self.num_blocks else 0.0,
        }
