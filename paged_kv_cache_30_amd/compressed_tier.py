"""Host-side bookkeeping of the compressed-slot tier: which blocks a
sequence's full tier maps, where its slots live, and the compression ops the
device runs (``paged_kv_compress``) before the step's writes.  Plain host
bookkeeping over ``BlockAllocator``, never timed.

Follows "Build a Memory-Compressed Attention Engine with KV Caching from
Scratch", Step 3 (``CompressedKVCache``): a sequence keeps at most ``window``
positions at full resolution; appending a position to a full tier first
compresses the tier's oldest ``window // 2`` positions into one slot (their
mean key and mean value per kv head, Step 2 ``MeanPoolCompression``) and
drops them; at most ``max_slots`` slots are kept, the oldest dropped first.

Paged form:

* ``window // 2`` must be a whole number of blocks; a compressed group is
  those blocks of the block table, which are released afterwards (their
  table entries become -1), so the full tier is positions
  [full_start, length);
* slots are rows of ordinary pool blocks held in a per-sequence slot table;
  the n-th compression of a sequence writes ring index n mod max_slots (row
  r % B of slot block r // B), so the valid slots are always ring indices
  [0, min(n, max_slots)) and dropping the oldest overwrites it in place;
* ``reserve`` returns the compression ops to run on the device before the
  step writes its new positions (same stream): blocks a compression reads
  may be handed out again in the same call, for new positions, and are only
  overwritten by the write that follows.  Destinations of one call are never
  sources of the same call (slot blocks are taken before sources are
  released).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Iterable, List, Optional, Tuple

import numpy as np

from .allocator import UNMAPPED, BlockAllocator


@dataclasses.dataclass
class CompressOps:
    """Arguments of one ``paged_kv_compress`` call: op n averages the blocks
    ``src_blocks[n]`` into row ``dst_slot[n]`` of block ``dst_block[n]``."""
    src_blocks: np.ndarray  # int32 [n, blocks_per_slot]
    dst_block: np.ndarray   # int32 [n]
    dst_slot: np.ndarray    # int32 [n]

    def __len__(self) -> int:
        return len(self.dst_block)


class CompressedTier:
    def __init__(self, allocator: BlockAllocator, window: int, max_slots: int):
        B = allocator.block_size
        if window <= 0 or window % (2 * B):
            raise ValueError(f"window must be a positive multiple of 2 * block_size ({2 * B})")
        if max_slots <= 0:
            raise ValueError("max_slots must be positive")
        self.alloc = allocator
        self.block_size = B
        self.window = int(window)
        self.half = self.window // 2
        self.blocks_per_slot = self.half // B
        self.max_slots = int(max_slots)
        self.full_start: Dict[int, int] = {}
        self.compressions: Dict[int, int] = {}
        self.slot_blocks: Dict[int, List[int]] = {}

    @property
    def slot_table_width(self) -> int:
        return -(-self.max_slots // self.block_size)

    def _take(self, n: int) -> List[int]:
        if len(self.alloc.free_list) < n:
            raise MemoryError(
                f"KV cache out of memory: need {n} blocks, only {len(self.alloc.free_list)} free of "
                f"{self.alloc.num_blocks} total.")
        got = [self.alloc.free_list.pop() for _ in range(n)]
        for b in got:
            self.alloc.refcount[b] = 1
        return got

    def reserve(self, seq_id: int, n: int = 1) -> Tuple[np.ndarray, CompressOps]:
        """Reserve the next ``n`` positions of ``seq_id``, compressing as the
        page's ``append`` does before each one.  Returns the positions
        (int32) and the compression ops to run before writing them.  Raises
        ``ValueError`` when a compression would read a position reserved in
        this same call (reserve fewer positions at a time)."""
        B, half = self.block_size, self.half
        row = self.alloc.tables.setdefault(seq_id, [])
        L0 = self.alloc.lengths.setdefault(seq_id, 0)
        fs = self.full_start.get(seq_id, 0)
        count = self.compressions.get(seq_id, 0)
        slots = self.slot_blocks.setdefault(seq_id, [])
        held = L0 - fs
        src, dst_b, dst_s, released = [], [], [], []
        for _ in range(n):
            if held >= self.window:
                if fs + half > L0:
                    raise ValueError("a compression would read positions reserved in the same call")
                b0 = fs // B
                group = row[b0:b0 + self.blocks_per_slot]
                r = count % self.max_slots
                if r // B >= len(slots):
                    slots.extend(self._take(1))
                src.append(group)
                dst_b.append(slots[r // B])
                dst_s.append(r % B)
                for i in range(b0, b0 + self.blocks_per_slot):
                    released.append(row[i])
                    row[i] = UNMAPPED
                fs += half
                held -= half
                count += 1
            held += 1
        for b in released:
            self.alloc._release(b)
        need = -(-(L0 + n) // B) - len(row)
        if need > 0:
            row.extend(self._take(need))
        self.alloc.lengths[seq_id] = L0 + n
        self.full_start[seq_id] = fs
        self.compressions[seq_id] = count
        k = self.blocks_per_slot
        ops = CompressOps(np.asarray(src, np.int32).reshape(len(src), k), np.asarray(dst_b, np.int32),
                          np.asarray(dst_s, np.int32))
        return np.arange(L0, L0 + n, dtype=np.int32), ops

    def num_slots(self, seq_id: int) -> int:
        return min(self.compressions.get(seq_id, 0), self.max_slots)

    def free(self, seq_id: int) -> None:
        """Drop ``seq_id``: its full-tier and slot blocks lose a reference."""
        self.alloc.free(seq_id)
        for b in self.slot_blocks.pop(seq_id, []):
            self.alloc._release(b)
        self.full_start.pop(seq_id, None)
        self.compressions.pop(seq_id, None)

    def arrays(self, seq_ids: Iterable[int], width: Optional[int] = None):
        """(block_tables [S, width], context_lens [S], full_start [S],
        slot_tables [S, slot_table_width], num_slots [S]), int32, for
        ``paged_attn_decode_compressed``."""
        seq_ids = list(seq_ids)
        tables = self.alloc.table(seq_ids, width)
        lens = self.alloc.context_lens(seq_ids)
        fs = np.array([self.full_start.get(s, 0) for s in seq_ids], np.int32)
        st = np.full((len(seq_ids), self.slot_table_width), UNMAPPED, np.int32)
        for i, s in enumerate(seq_ids):
            blocks = self.slot_blocks.get(s, [])
            st[i, :len(blocks)] = blocks
        ns = np.array([self.num_slots(s) for s in seq_ids], np.int32)
        return tables, lens, fs, st, ns
