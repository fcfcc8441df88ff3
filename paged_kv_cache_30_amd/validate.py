"""Host-side checks of device-resident arguments (the binding's debug mode).

The entry points check sizes and pointers on the host but never read table
entries, lengths or chunk offsets in the hot path: those live in device
memory, and a bad one is the caller's bug (out-of-range entries of attended
blocks are skipped, a length beyond ``max_context_len`` or a chunk offset
past the output is undefined).  With ``debug=True`` the binding copies them
to the host first and calls these checks, which raise ``InvalidContent``
naming the first offending sequence, token or op.  Debug mode is strict: it
also rejects what the kernels define but a correct caller never does (a
token the write would skip, an attended block left unmapped).

All functions take NumPy integer arrays and plain ints; none touches the GPU.
The attended positions follow the same definitions as the kernels: decode
"Build a Paged KV Cache in Pure Python", Step 4, with the window of
"Building a Streaming Sliding-Window Attention Engine in Pure Python",
Step 3; prefill that page's Step 3 causal mask for a chunk ending at the
context length.
"""
from __future__ import annotations

import numpy as np


class InvalidContent(ValueError):
    """A device-resident argument violates the entry point's contract."""


def _blocks_needed(lo: int, L: int, sinks: int, window: int, B: int) -> np.ndarray:
    """Logical block indices holding the attended positions [lo, L) and,
    with a window, the sink positions [0, min(sinks, L))."""
    if L <= lo:
        idx = np.zeros(0, np.int64)
    else:
        idx = np.arange(lo // B, (L - 1) // B + 1)
    if window > 0 and sinks > 0:
        ns = min(sinks, L)
        if ns > 0:
            idx = np.union1d(idx, np.arange(0, (ns - 1) // B + 1))
    return idx


def _check_mapped(tables: np.ndarray, s: int, blocks: np.ndarray, nb: int, what: str) -> None:
    if blocks.size == 0:
        return
    if blocks.max() >= tables.shape[1]:
        raise InvalidContent(f"{what}: sequence {s} needs logical block {int(blocks.max())} but the table has "
                             f"{tables.shape[1]} columns")
    ent = tables[s, blocks]
    bad = (ent < 0) | (ent >= nb)
    if bad.any():
        j = int(np.flatnonzero(bad)[0])
        raise InvalidContent(f"{what}: sequence {s}, logical block {int(blocks[j])} is attended but its table "
                             f"entry {int(ent[j])} is outside [0, {nb})")


def check_lengths(lens: np.ndarray, max_context_len: int, what: str) -> None:
    bad = (lens < 0) | (lens > max_context_len)
    if bad.any():
        s = int(np.flatnonzero(bad)[0])
        raise InvalidContent(f"{what}: context_lens[{s}] = {int(lens[s])} is outside [0, {max_context_len}]")


def check_write(seq_idx, pos, tables, *, num_blocks: int, block_size: int, what="paged_kv_write") -> None:
    """Every token lands in a mapped slot, and no two tokens share a slot
    ("Build a Paged KV Cache in Pure Python", Step 3: block pos // B, offset
    pos % B)."""
    seq_idx = np.asarray(seq_idx, np.int64)
    pos = np.asarray(pos, np.int64)
    tables = np.asarray(tables, np.int64)
    S, MB = tables.shape
    B = block_size
    bad = (seq_idx < 0) | (seq_idx >= S)
    if bad.any():
        n = int(np.flatnonzero(bad)[0])
        raise InvalidContent(f"{what}: token {n} has sequence index {int(seq_idx[n])} outside [0, {S})")
    bad = (pos < 0) | (pos >= MB * B)
    if bad.any():
        n = int(np.flatnonzero(bad)[0])
        raise InvalidContent(f"{what}: token {n} has position {int(pos[n])} outside [0, {MB * B})")
    ent = tables[seq_idx, pos // B]
    bad = (ent < 0) | (ent >= num_blocks)
    if bad.any():
        n = int(np.flatnonzero(bad)[0])
        raise InvalidContent(f"{what}: token {n} (sequence {int(seq_idx[n])}, position {int(pos[n])}) maps to "
                             f"table entry {int(ent[n])} outside [0, {num_blocks})")
    slot = ent * B + pos % B
    uniq, counts = np.unique(slot, return_counts=True)
    if (counts > 1).any():
        dup = uniq[counts > 1][0]
        ns = np.flatnonzero(slot == dup)
        raise InvalidContent(f"{what}: tokens {int(ns[0])} and {int(ns[1])} write the same slot (block "
                             f"{int(dup // B)}, row {int(dup % B)})")


def check_decode(tables, lens, *, max_context_len: int, num_blocks: int, block_size: int, window: int = 0,
                 sinks: int = 0, what="paged_attn_decode") -> None:
    """Lengths in [0, max_context_len]; every block holding an attended
    position mapped."""
    tables = np.asarray(tables, np.int64)
    lens = np.asarray(lens, np.int64)
    check_lengths(lens, max_context_len, what)
    for s in range(lens.shape[0]):
        L = int(lens[s])
        lo = max(0, L - window) if window > 0 else 0
        _check_mapped(tables, s, _blocks_needed(lo, L, sinks, window, block_size), num_blocks, what)


def check_prefill(q_start, tables, lens, *, num_rows: int, max_q_len: int, max_context_len: int,
                  num_blocks: int, block_size: int, window: int = 0, sinks: int = 0,
                  what="paged_attn_prefill") -> None:
    """Chunk offsets start at 0, never decrease and end at the number of
    query rows; each chunk fits max_q_len and its context; every block the
    chunk's rows attend is mapped."""
    q_start = np.asarray(q_start, np.int64)
    tables = np.asarray(tables, np.int64)
    lens = np.asarray(lens, np.int64)
    if q_start[0] != 0:
        raise InvalidContent(f"{what}: q_start[0] = {int(q_start[0])}, must be 0")
    C = np.diff(q_start)
    if (C < 0).any():
        s = int(np.flatnonzero(C < 0)[0])
        raise InvalidContent(f"{what}: q_start decreases at sequence {s}")
    if q_start[-1] != num_rows:
        raise InvalidContent(f"{what}: q_start[num_seqs] = {int(q_start[-1])} but q has {num_rows} rows")
    check_lengths(lens, max_context_len, what)
    for s in range(lens.shape[0]):
        c, L = int(C[s]), int(lens[s])
        if c > max_q_len:
            raise InvalidContent(f"{what}: sequence {s} has {c} query rows, above max_q_len = {max_q_len}")
        if c > L:
            raise InvalidContent(f"{what}: sequence {s} has {c} query rows but context length {L}")
        if c == 0:
            continue
        p0 = L - c  # position of the chunk's first row
        lo = max(0, p0 - window + 1) if window > 0 else 0
        _check_mapped(tables, s, _blocks_needed(lo, L, sinks, window, block_size), num_blocks, what)


# Largest magnitude a bf16 value keeps when the prefill converts V to fp16
# for the matrix cores: bf16 values at or below 65280 are fp16 values; the
# next bf16 value, 65536, is beyond fp16's range (its largest value is 65504).
PREFILL_BF16_V_LIMIT = 65280.0


def prefill_v_rows(q_start, tables, lens, *, block_size: int, window: int = 0, sinks: int = 0,
                   min_rows: int = 1):
    """(physical block, slot) of every cached row a chunk of at least
    ``min_rows`` query rows attends: positions [lo, L) with lo the first
    row's window start (0 without a window), plus the sink positions.
    Returns two int64 arrays and the sequence each row belongs to."""
    q_start = np.asarray(q_start, np.int64)
    tables = np.asarray(tables, np.int64)
    lens = np.asarray(lens, np.int64)
    blk, slot, seq = [], [], []
    for s in range(lens.shape[0]):
        c, L = int(q_start[s + 1] - q_start[s]), int(lens[s])
        if c < min_rows or c == 0 or c > L:
            continue
        lo = max(0, L - c - window + 1) if window > 0 else 0
        pos = np.arange(lo, L)
        if window > 0 and sinks > 0:
            pos = np.union1d(np.arange(0, min(sinks, L)), pos)
        blk.append(tables[s, pos // block_size])
        slot.append(pos % block_size)
        seq.append(np.full(pos.shape, s))
    if not blk:
        z = np.zeros(0, np.int64)
        return z, z, z
    return np.concatenate(blk), np.concatenate(slot), np.concatenate(seq)


def check_prefill_v_range(row_absmax, seq, limit: float, what="paged_attn_prefill") -> None:
    """Every attended V row's largest magnitude within the prefill's limit
    (``row_absmax`` and ``seq`` as given by ``prefill_v_rows``)."""
    row_absmax = np.asarray(row_absmax, np.float64)
    bad = ~(row_absmax <= limit)
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise InvalidContent(f"{what}: sequence {int(seq[i])} attends a V row of largest magnitude "
                             f"{row_absmax[i]:.7g}, beyond the {limit:.7g} that bf16 prefill converts to fp16 "
                             "exactly")


def check_copy_blocks(src, dst, *, num_blocks: int, what="paged_kv_copy_blocks") -> None:
    """Ids in the pool, src != dst, destinations distinct and never a source
    of the same call."""
    src = np.asarray(src, np.int64)
    dst = np.asarray(dst, np.int64)
    for name, a in (("src", src), ("dst", dst)):
        bad = (a < 0) | (a >= num_blocks)
        if bad.any():
            i = int(np.flatnonzero(bad)[0])
            raise InvalidContent(f"{what}: {name}[{i}] = {int(a[i])} is outside [0, {num_blocks})")
    same = src == dst
    if same.any():
        raise InvalidContent(f"{what}: pair {int(np.flatnonzero(same)[0])} copies a block onto itself")
    uniq, counts = np.unique(dst, return_counts=True)
    if (counts > 1).any():
        raise InvalidContent(f"{what}: block {int(uniq[counts > 1][0])} is the destination of two pairs")
    both = np.intersect1d(src, dst)
    if both.size:
        raise InvalidContent(f"{what}: block {int(both[0])} is both a source and a destination")


def check_compress(src_blocks, dst_block, dst_slot, *, num_blocks: int, block_size: int,
                   what="paged_kv_compress") -> None:
    """Every source and destination in the pool, destination rows distinct,
    and no destination row inside a block the call reads."""
    src = np.asarray(src_blocks, np.int64)
    db = np.asarray(dst_block, np.int64)
    ds = np.asarray(dst_slot, np.int64)
    bad = (src < 0) | (src >= num_blocks)
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise InvalidContent(f"{what}: op {int(i)} source {int(j)} = {int(src[i, j])} is outside [0, {num_blocks})")
    for name, a, hi in (("dst_block", db, num_blocks), ("dst_slot", ds, block_size)):
        bad = (a < 0) | (a >= hi)
        if bad.any():
            i = int(np.flatnonzero(bad)[0])
            raise InvalidContent(f"{what}: {name}[{i}] = {int(a[i])} is outside [0, {hi})")
    rows = db * block_size + ds
    uniq, counts = np.unique(rows, return_counts=True)
    if (counts > 1).any():
        r = int(uniq[counts > 1][0])
        raise InvalidContent(f"{what}: two ops write row {r % block_size} of block {r // block_size}")
    both = np.intersect1d(src.ravel(), db)
    if both.size:
        raise InvalidContent(f"{what}: block {int(both[0])} is read and written by the same call")


def check_decode_compressed(tables, lens, full_start, slot_tables, num_slots, *, max_context_len: int,
                            num_blocks: int, block_size: int, window: int = 0,
                            what="paged_attn_decode_compressed") -> None:
    """Lengths as decode; full_start in [0, L]; num_slots in [0, slot rows
    the slot table holds]; every block of an attended full-resolution
    position and of an attended slot row mapped."""
    tables = np.asarray(tables, np.int64)
    lens = np.asarray(lens, np.int64)
    fs = np.asarray(full_start, np.int64)
    st = np.asarray(slot_tables, np.int64)
    ns = np.asarray(num_slots, np.int64)
    B = block_size
    check_lengths(lens, max_context_len, what)
    cap = st.shape[1] * B
    for s in range(lens.shape[0]):
        L = int(lens[s])
        if not 0 <= int(fs[s]) <= L:
            raise InvalidContent(f"{what}: full_start[{s}] = {int(fs[s])} is outside [0, {L}]")
        if not 0 <= int(ns[s]) <= cap:
            raise InvalidContent(f"{what}: num_slots[{s}] = {int(ns[s])} is outside [0, {cap}]")
        lo = max(int(fs[s]), L - window) if window > 0 else int(fs[s])
        _check_mapped(tables, s, _blocks_needed(lo, L, 0, 0, B), num_blocks, what)
        n = int(ns[s])
        if n:
            _check_mapped(st, s, np.arange(0, (n - 1) // B + 1), num_blocks, what + " (slot rows)")
