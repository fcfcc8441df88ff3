"""Host-side prefix cache over ``BlockAllocator``: prompt blocks shared
between requests by content, refcounted, evicted when the pool runs short,
copied before a sequence writes into a block it shares.  Plain host
bookkeeping, never timed; the device work it asks for is the block copies
it returns (``paged_kv_copy_blocks``).

Follows "Building a Streaming Sliding-Window Attention Engine in Pure
Python", Step 4 (``prefix_index``: a hash of a prompt prefix names cached
state that a later request reuses instead of recomputing it -
``commit_prefix`` / ``reuse_prefix``; the page notes a production system
would share pages through a prefix tree) and "Build a Minimal LLM Inference
Engine with Paged Attention and Adaptive KV Cache", Step 1 and Step 2 (a
page's refcount counts the sequences that reference it; it returns to the
free pool at zero).

Design:

* Only full blocks are cached.  Block b of a token sequence has the key
  H(key of block b-1, tokens of block b), so a key names the whole prefix up
  to the end of that block and equal prefixes map to the same blocks.
* The cache holds one reference to each block it names.  A sequence that
  starts with a cached prefix maps those physical blocks (refcount + 1
  each) and only computes the rest.  Blocks that only the cache still
  references are evictable, least recently released first.
* Copy-on-write: before positions are written into a block another table
  (or the cache) also maps, the sequence gets a private copy; ``reserve``
  returns the (source, destination) block pairs the device must copy
  first.  With full-block prefix sharing this happens after ``fork`` (a
  sequence that continues another one, e.g. a second sample of the same
  prompt), whose partially filled last block is shared.
"""
from __future__ import annotations

import hashlib
from collections import OrderedDict
from typing import Dict, List, Sequence, Tuple

import numpy as np

from .allocator import UNMAPPED, BlockAllocator


class PrefixCache:
    def __init__(self, allocator: BlockAllocator):
        self.alloc = allocator
        self.block_size = allocator.block_size
        self.blocks: Dict[bytes, int] = {}    # key -> physical block
        self.key_of: Dict[int, bytes] = {}    # physical block -> key
        self.idle: "OrderedDict[int, None]" = OrderedDict()  # cached blocks no table maps, oldest first
        self.hits = 0
        self.lookups = 0

    # ------------------------------------------------------------- keys
    def block_keys(self, tokens: Sequence[int]) -> List[bytes]:
        """Chained keys of the full blocks of ``tokens``."""
        B = self.block_size
        toks = np.asarray(tokens, dtype=np.int64)
        keys, h = [], b""
        for b in range(len(toks) // B):
            h = hashlib.blake2b(h + toks[b * B:(b + 1) * B].tobytes(), digest_size=16).digest()
            keys.append(h)
        return keys

    def match(self, tokens: Sequence[int]) -> List[int]:
        """Physical blocks of the longest cached prefix of ``tokens`` (full
        blocks only)."""
        out = []
        for k in self.block_keys(tokens):
            b = self.blocks.get(k)
            if b is None:
                break
            out.append(b)
        return out

    # ------------------------------------------------------- sequences
    def start(self, seq_id: int, tokens: Sequence[int]) -> int:
        """Begin ``seq_id`` with the longest cached prefix of ``tokens``
        mapped (refcount + 1 per block).  Returns the number of positions
        already cached: the caller computes and writes ``tokens[n:]`` only."""
        if self.alloc.tables.get(seq_id):
            raise ValueError(f"sequence {seq_id} already has blocks")
        blocks = self.match(tokens)
        self.lookups += len(tokens) // self.block_size
        self.hits += len(blocks)
        for b in blocks:
            self.alloc.refcount[b] += 1
            self.idle.pop(b, None)
        self.alloc.tables[seq_id] = list(blocks)
        self.alloc.lengths[seq_id] = len(blocks) * self.block_size
        return len(blocks) * self.block_size

    def fork(self, src_seq: int, dst_seq: int) -> None:
        """``dst_seq`` continues ``src_seq``: it maps every block of it
        (refcount + 1 each), its partially filled last block included."""
        if self.alloc.tables.get(dst_seq):
            raise ValueError(f"sequence {dst_seq} already has blocks")
        row = list(self.alloc.tables[src_seq])
        for b in row:
            if b != UNMAPPED:
                self.alloc.refcount[b] += 1
                self.idle.pop(b, None)
        self.alloc.tables[dst_seq] = row
        self.alloc.lengths[dst_seq] = self.alloc.lengths[src_seq]

    def commit(self, seq_id: int, tokens: Sequence[int]) -> int:
        """Name ``seq_id``'s full blocks holding ``tokens`` (already written)
        in the cache; the cache takes one reference to each block it did not
        name before.  Returns how many blocks were added."""
        row = self.alloc.tables[seq_id]
        added = 0
        for i, k in enumerate(self.block_keys(tokens)):
            if i >= len(row) or row[i] == UNMAPPED:
                break
            b = row[i]
            if k in self.blocks or b in self.key_of:
                continue
            self.blocks[k] = b
            self.key_of[b] = k
            self.alloc.refcount[b] += 1
            added += 1
        return added

    def release(self, seq_id: int) -> None:
        """Drop ``seq_id``; its blocks lose one reference; cached blocks that
        no table maps any more become evictable."""
        row = list(self.alloc.tables.get(seq_id, []))
        self.alloc.free(seq_id)
        for b in row:
            if b != UNMAPPED and b in self.key_of and self.alloc.refcount[b] == 1:
                self.idle[b] = None
                self.idle.move_to_end(b)

    def evict(self, n: int) -> int:
        """Return up to ``n`` evictable cached blocks to the free list, least
        recently released first.  Returns how many were freed."""
        freed = 0
        while freed < n and self.idle:
            b, _ = self.idle.popitem(last=False)
            del self.blocks[self.key_of.pop(b)]
            self.alloc._release(b)
            freed += 1
        return freed

    def _take(self, n: int) -> List[int]:
        """n blocks off the free list (refcount 1), evicting cached blocks
        when the list is short."""
        short = n - len(self.alloc.free_list)
        if short > 0:
            self.evict(short)
        if len(self.alloc.free_list) < n:
            raise MemoryError(
                f"KV cache out of memory: need {n} blocks, only {len(self.alloc.free_list)} free of "
                f"{self.alloc.num_blocks} total.")
        got = [self.alloc.free_list.pop() for _ in range(n)]
        for b in got:
            self.alloc.refcount[b] = 1
        return got

    def reserve(self, seq_id: int, n: int = 1) -> Tuple[np.ndarray, List[Tuple[int, int]]]:
        """Reserve the next ``n`` positions of ``seq_id``.  Returns the
        positions (int32) and the (source, destination) block copies to run
        on the device before writing them: a shared, partially filled last
        block is replaced by a private copy (copy-on-write)."""
        B = self.block_size
        row = self.alloc.tables.setdefault(seq_id, [])
        L = self.alloc.lengths.setdefault(seq_id, 0)
        copies: List[Tuple[int, int]] = []
        last = L // B
        if n > 0 and L % B and last < len(row) and row[last] != UNMAPPED and self.alloc.refcount[row[last]] > 1:
            old = row[last]
            new, = self._take(1)
            copies.append((old, new))
            row[last] = new
            self.alloc._release(old)
            if old in self.key_of and self.alloc.refcount[old] == 1:
                self.idle[old] = None
        need = -(-(L + n) // B) - len(row)
        if need > 0:
            row.extend(self._take(need))
        self.alloc.lengths[seq_id] = L + n
        return np.arange(L, L + n, dtype=np.int32), copies

    def stats(self) -> dict:
        s = self.alloc.stats()
        s.update(cached_blocks=len(self.blocks), evictable_blocks=len(self.idle),
                 prefix_hit_rate=self.hits / self.lookups if self.lookups else 0.0)
        return s
