"""Compressed-slot tier: mean-pooled summaries of evicted positions that
decode attends next to the full-resolution tier.  Test infrastructure only
(see ``oracle/__init__.py``).

"Build a Memory-Compressed Attention Engine with KV Caching from Scratch":

* Component Breakdown: two tiers per sequence, a full window of recent
  positions and compressed slots that summarise older ones; attention runs
  over the union of both.
* Step 2 (``MeanPoolCompression``): the summary of a group of positions is
  the mean of their keys and the mean of their values, per head.
* Step 3 (``CompressedKVCache``): ``append`` writes one position into the
  full tier; when the tier already holds ``window`` positions it first
  compresses its oldest half (``window // 2`` positions) into one new slot
  and keeps the newer half (``_compress_and_evict``); at most
  ``max_compressed_slots`` slots are kept, the oldest dropped first.
* Step 4 (``CompressedAttention.forward``): after appending, the query
  attends the full tier's positions and the slots (scores scaled by
  1/sqrt(D), softmax, weighted sum of values), with no mask.

Readings (where the page is silent, contradictory or garbled):

* The value slot is the mean of the values.  The printed eviction stores the
  shifted key window in place of the value window as well (its comment calls
  it a placeholder); that is read as a slip.
* Mean pooling yields one slot per compression.  The printed trim limit
  multiplies by a per-slot query count that only the learned compressor
  defines; for the mean it is read as 1.
* Decode only: the page appends one position per forward call.
* A slot is the exact mean of the stored rows, rounded once to the storage
  dtype (``math.fsum`` per element, divided by the count; exact when the
  count is a power of two).
* Paged form: a group is ``window // 2`` positions = a whole number of blocks
  of the block table; its blocks are freed after compression, so the full
  tier is positions [full_start, L) with full_start = (number of
  compressions) * window // 2.  Slots are rows of ordinary pool blocks: slot
  number n (counting every compression of the sequence) sits at ring index
  r = n mod max_slots, row r % B of block ``slot_table[r // B]``; the newest
  ``min(n, max_slots)`` slots are then exactly ring indices [0, min(n, M)),
  so dropping the oldest moves no data.  Attention over a set of keys does
  not depend on their order, so the ring order is free.

Pinned by ``tests/test_oracle_compressed.py``.
"""
from __future__ import annotations

import math

import numpy as np

from . import ref

# (significant bits, smallest normal exponent) of each storage type.
_FORMAT = {"f32": (24, -126), "f16": (11, -14), "bf16": (8, -126)}


def round_to_storage(x, dtype: str) -> np.ndarray:
    """float64 -> storage dtype, rounded to nearest with ties to even, in one
    step (no intermediate float32 for bfloat16).  bfloat16 is returned as its
    uint16 bit pattern.

    A value of magnitude in [2^(e-1), 2^e) has quantum 2^(e - p) with p
    significant bits, and never below the subnormal quantum 2^(emin - p + 1).
    """
    p, emin = _FORMAT[dtype]
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q_exp = np.maximum(e - p, emin - p + 1)
    y = np.ldexp(np.round(np.ldexp(x, -q_exp)), q_exp)  # np.round: half to even
    with np.errstate(over="ignore"):  # beyond the largest finite value: infinity
        if dtype == "f32":
            return y.astype(np.float32)
        if dtype == "f16":
            return y.astype(np.float16)
        return (y.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def mean_rows(rows, dtype: str) -> np.ndarray:
    """Mean over axis 0 of stored rows [n, ...] (``MeanPoolCompression``),
    exact then rounded to the storage dtype.  n must be positive."""
    r = ref.to_f64(rows, dtype)
    n = r.shape[0]
    if n == 0:
        raise ValueError("mean of no rows")
    flat = r.reshape(n, -1)
    m = np.array([math.fsum(flat[:, j]) / n for j in range(flat.shape[1])])
    return round_to_storage(m.reshape(r.shape[1:]), dtype)


def tier_trace(L: int, window: int, max_slots: int):
    """Run ``CompressedKVCache.append`` for positions 0 .. L-1 on counters
    only.  Returns (groups, kept, full_start): the [start, end) positions of
    every compression in order, the groups still held as slots (the newest
    ``max_slots``), and the first position of the full tier."""
    if window < 2 or window % 2:
        raise ValueError("window must be even and >= 2")
    half = window // 2
    groups, full_start, held = [], 0, 0
    for _ in range(L):
        if held >= window:              # full tier is full: compress its oldest half
            groups.append((full_start, full_start + half))
            full_start += half
            held -= half
        held += 1                        # then append the position
    kept = groups[len(groups) - max_slots:] if len(groups) > max_slots else list(groups)
    return groups, kept, full_start


def compress_blocks(k_pool, v_pool, src_blocks, dst_block, dst_slot, dtype: str):
    """The paged compression step: op n replaces row ``dst_slot[n]`` of block
    ``dst_block[n]`` (every kv head) with the mean of all rows of the blocks
    ``src_blocks[n, :]``.  Source entries outside [0, NB) are left out of the
    mean; an op with no valid source, or a destination block or row out of
    range, writes nothing.  Ops read the input pools (a call's destinations
    are not among its sources).  Returns new pools (inputs untouched)."""
    nk, nv = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    nb, B = k_pool.shape[0], k_pool.shape[1]
    src_blocks = np.asarray(src_blocks).reshape(len(dst_block), -1)
    for n in range(len(dst_block)):
        src = [int(b) for b in src_blocks[n] if 0 <= int(b) < nb]
        db, ds = int(dst_block[n]), int(dst_slot[n])
        if not src or not (0 <= db < nb and 0 <= ds < B):
            continue
        rows_k = np.concatenate([np.asarray(k_pool)[b] for b in src])   # [len(src) * B, Hkv, D]
        rows_v = np.concatenate([np.asarray(v_pool)[b] for b in src])
        nk[db, ds] = mean_rows(rows_k, dtype)
        nv[db, ds] = mean_rows(rows_v, dtype)
    return nk, nv


def decode_compressed(q, k_pool, v_pool, block_tables, context_lens, full_start, slot_tables, num_slots, *,
                      block_size, num_kv_heads, window, scale, dtype):
    """Decode over both tiers, every (seq, head).

    Full tier: positions [max(full_start, L - window), L) through the block
    table (``window`` 0: no sliding window; full_start clamped to [0, L]).
    Slots: ring rows [0, num_slots) through the slot table (num_slots clamped
    to [0, slot table width * B]).  Keys in the page's order, full tier then
    slots.  Returns (out [S, H, D], lse [S, H]) float64.
    """
    S, H, D = q.shape
    B = block_size
    out = np.zeros((S, H, D))
    lse = np.zeros((S, H))
    qf = ref.to_f64(q, dtype)
    width = np.asarray(slot_tables).shape[1]
    for s in range(S):
        L = int(context_lens[s])
        lo, hi = ref.attended_range(L, window)
        lo = max(lo, min(max(int(full_start[s]), 0), L))
        ns = min(max(int(num_slots[s]), 0), width * B)
        pos = np.arange(lo, hi)
        ring = np.arange(ns)
        for h in range(H):
            g = ref.kv_head_of(h, H, num_kv_heads)
            K = np.concatenate([ref.gather(k_pool, block_tables[s], pos, g, B, dtype),
                                ref.gather(k_pool, slot_tables[s], ring, g, B, dtype)])
            V = np.concatenate([ref.gather(v_pool, block_tables[s], pos, g, B, dtype),
                                ref.gather(v_pool, slot_tables[s], ring, g, B, dtype)])
            o, l = ref.attend(qf[s, h:h + 1], K, V, scale)
            out[s, h] = o[0]
            lse[s, h] = l[0]
    return out, lse


def tiered_decode(q_s, k_log, v_log, L: int, *, window: int, max_slots: int, num_kv_heads: int, scale, dtype):
    """The page's cache for one sequence, never paged: the logical rows of
    positions [0, L) (``k_log``/``v_log`` [L, Hkv, D], storage dtype) pass
    through ``tier_trace``; the kept groups become slots (``mean_rows``) and
    the query (q_s [H, D]) attends the full tier then the slots.  This is
    what the paged tier must equal.  Returns (out [H, D], lse [H])."""
    H, D = q_s.shape
    _, kept, full_start = tier_trace(L, window, max_slots)
    qf = ref.to_f64(q_s, dtype)
    out, lse = np.zeros((H, D)), np.zeros(H)
    sk = [ref.to_f64(mean_rows(k_log[a:b], dtype), dtype) for a, b in kept]   # each [Hkv, D]
    sv = [ref.to_f64(mean_rows(v_log[a:b], dtype), dtype) for a, b in kept]
    for h in range(H):
        g = ref.kv_head_of(h, H, num_kv_heads)
        K = np.concatenate([ref.to_f64(k_log[full_start:L, g], dtype), np.array([x[g] for x in sk]).reshape(-1, D)])
        V = np.concatenate([ref.to_f64(v_log[full_start:L, g], dtype), np.array([x[g] for x in sv]).reshape(-1, D)])
        o, l = ref.attend(qf[h:h + 1], K, V, scale)
        out[h], lse[h] = o[0], l[0]
    return out, lse
