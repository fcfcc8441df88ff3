"""Seeded synthetic inputs for paged-KV attention.

This module only draws numbers and lays out block tables; it holds none of the
attention arithmetic and none of the write indexing.  Both the fp64 oracle
(via the tests) and the HIP library (via the tests, the smoke check and the
benchmark) consume what it returns, so neither side can feed the other.

What is generated follows the problem statement of the pages:

* a pool of fixed-size blocks and a per-sequence block table of physical block
  ids, with logical block ``b`` of a sequence covering token positions
  ``[b*B, (b+1)*B)`` ("Build a Paged KV Cache in Pure Python", Step 2 and
  Step 3: ``BlockAllocator`` / ``PagedKVCache.append``);
* keys and values per sequence, shape ``(tokens, num_kv_heads, head_dim)``
  (the per-block layout of ``KVCacheBlock`` in the same page, Step 1);
* a query per sequence for decode, or a chunk of queries for prefill
  ("Building a Streaming Sliding-Window Attention Engine in Pure Python",
  Step 3 and Step 4: decode attends with the just-appended token, prefill with
  every prompt token).

Random streams.  Every array comes from its own counter-derived stream
``numpy.random.Generator(PCG64(SeedSequence([seed, tag, index])))`` so that one
sequence's keys/values can be regenerated alone (for sampled parity at full
size) without drawing the rest.  Values are drawn as float32 N(0, 1), scaled,
then rounded to nearest-even into the storage dtype; the rounded values are the
data for both sides.

Storage dtypes: ``"f32"`` -> numpy float32, ``"f16"`` -> numpy float16,
``"bf16"`` -> numpy uint16 holding bfloat16 bit patterns (numpy has no
bfloat16 type).
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Dict, List, Optional, Tuple

import numpy as np

TAG_LENGTHS = 0
TAG_SEQ_KV = 1
TAG_QUERY = 2
TAG_PERM = 3
TAG_PREFIX_KV = 4
TAG_SLOTS = 5

STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def stream(seed: int, tag: int, index: int = 0) -> np.random.Generator:
    """Independent PCG64 stream for (seed, tag, index)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, index])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return the uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # Finite inputs cannot carry past bit 31 (largest finite magnitude bits
    # 0x7F7FFFFF plus the bias stay below 2^31 for each sign); NaNs are set
    # afterwards.
    t = u >> 16
    t &= 1
    t += 0x7FFF
    t += u
    t >>= 16
    out = t.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def to_storage(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round a float32 array into the storage dtype (see module docstring)."""
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "f16":
        return x32.astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(f"unknown dtype {dtype!r}")


def nan_fill(shape, dtype: str) -> np.ndarray:
    """An array of quiet NaNs in the storage dtype (used to poison unused slots)."""
    if dtype == "bf16":
        return np.full(shape, 0x7FC0, dtype=np.uint16)
    return np.full(shape, np.nan, dtype=STORAGE[dtype])


def draw(rng: np.random.Generator, shape, dtype: str, scale: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return to_storage(x, dtype)


@dataclasses.dataclass
class SeqKV:
    """Keys/values of one sequence for positions [start, start + len(k)).
    ``runs``: the position ranges [p0, p1) held in the cache (mapped blocks),
    when not the whole range (attention sinks plus a window)."""
    start: int
    k: np.ndarray  # (n, Hkv, D) storage dtype
    v: np.ndarray
    runs: Optional[List[Tuple[int, int]]] = None


@dataclasses.dataclass
class Workload:
    name: str
    kind: str  # "decode" | "prefill"
    seed: int
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str
    num_blocks: int
    max_blocks_per_seq: int
    window: int
    scale: float
    context_lens: np.ndarray  # int32 [S], includes the query token(s)
    block_tables: np.ndarray  # int32 [S, MB], -1 = unmapped
    q: np.ndarray  # decode: [S, H, D]; prefill: [sum C, H, D]
    seq_kv: List[SeqKV]  # per sequence; for prefill: the chunk tokens only
    q_start: Optional[np.ndarray] = None  # prefill: int32 [S+1]
    prefix: Optional[SeqKV] = None  # prefill: shared prefix tokens [0, P)
    prefix_len: int = 0
    shared_prefix_blocks: int = 0
    sinks: int = 0  # with a window: the first `sinks` positions are attended too
    # Compressed slots (decode only): per sequence the first full-resolution
    # position, the slot table [S, MSB] (slot row r at row r % B of block
    # slot_tables[s, r // B]), the number of slot rows and their K/V rows.
    full_start: Optional[np.ndarray] = None
    slot_tables: Optional[np.ndarray] = None
    num_slots: Optional[np.ndarray] = None
    slot_kv: Optional[List[SeqKV]] = None

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def max_q_len(self) -> int:
        if self.q_start is None:
            return 1
        return int(np.diff(self.q_start).max()) if self.num_seqs else 0

    def logical_kv(self, s: int) -> Tuple[int, np.ndarray, np.ndarray]:
        """(first position, K, V) of every token of sequence s that has data."""
        if self.kind == "prefill" and self.prefix is not None and self.prefix_len > 0:
            k = np.concatenate([self.prefix.k, self.seq_kv[s].k], axis=0)
            v = np.concatenate([self.prefix.v, self.seq_kv[s].v], axis=0)
            return 0, k, v
        e = self.seq_kv[s]
        return e.start, e.k, e.v

    def history_tokens(self):
        """Tokens that are already in the cache before the timed step.

        Yields (seq, first position, K, V) runs.  For decode this is every
        token but the last (the step appends the query token, then attends);
        for prefill it is the common prefix: written once through sequence 0's
        table when its blocks are shared (the other sequences map the same
        physical blocks), else through every sequence's own table.
        """
        if self.kind == "decode":
            for s in range(self.num_seqs):
                e = self.seq_kv[s]
                last = e.start + e.k.shape[0] - 1  # the step writes this one
                for p0, p1 in (e.runs if e.runs is not None else [(e.start, last + 1)]):
                    p1 = min(p1, last)
                    if p1 > p0:
                        yield s, p0, e.k[p0 - e.start:p1 - e.start], e.v[p0 - e.start:p1 - e.start]
        elif self.prefix is not None and self.prefix_len > 0:
            owners = [0] if self.shared_prefix_blocks > 0 else range(self.num_seqs)
            for s in owners:
                yield s, 0, self.prefix.k, self.prefix.v

    def step_tokens(self):
        """Tokens the timed step writes before attending: (seq_idx, pos, K, V)."""
        seq_idx, pos, ks, vs = [], [], [], []
        for s in range(self.num_seqs):
            e = self.seq_kv[s]
            L = int(self.context_lens[s])
            if self.kind == "decode":
                if L == 0:
                    continue
                seq_idx.append(np.array([s], np.int32))
                pos.append(np.array([L - 1], np.int32))
                ks.append(e.k[-1:])
                vs.append(e.v[-1:])
            else:
                c = e.k.shape[0]
                if c == 0:
                    continue
                seq_idx.append(np.full(c, s, np.int32))
                pos.append(np.arange(L - c, L, dtype=np.int32))
                ks.append(e.k)
                vs.append(e.v)
        shape = (0, self.num_kv_heads, self.head_dim)
        if not seq_idx:
            z = np.zeros(shape, STORAGE[self.dtype])
            return np.zeros(0, np.int32), np.zeros(0, np.int32), z, z.copy()
        return (np.concatenate(seq_idx), np.concatenate(pos),
                np.ascontiguousarray(np.concatenate(ks)), np.ascontiguousarray(np.concatenate(vs)))

    def kv_bytes_attended(self) -> int:
        """Algorithmic K+V bytes one decode call must read: each attended
        (token, kv-head) row once, for K and for V."""
        eb = ELEM_BYTES[self.dtype]
        L = self.context_lens.astype(np.int64)
        lo = np.maximum(0, L - self.window) if self.window > 0 else np.zeros_like(L)
        if self.full_start is not None:
            lo = np.maximum(lo, np.minimum(self.full_start.astype(np.int64), L))
            n = (L - lo) + self.num_slots.astype(np.int64)
        elif self.window > 0:
            n = (L - lo) + np.minimum(self.sinks, lo)
        else:
            n = L
        return int(n.sum()) * self.num_kv_heads * self.head_dim * 2 * eb


def _parallel_map(fn, items):
    """Map over independent streams on host threads (NumPy's generators and
    casts release the GIL); results keep their order, so the output does not
    depend on the thread count."""
    items = list(items)
    if len(items) < 2:
        return [fn(i) for i in items]
    workers = min(len(items), max(1, min(16, len(os.sched_getaffinity(0)))))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))


def _deal_tables(rng_perm, blocks_per_seq: List[int], first_block: List[int], mb: int,
                 num_blocks: int, sink_blocks: Optional[List[int]] = None) -> np.ndarray:
    """Hand out shuffled physical ids in sequence order; -1 elsewhere.  A
    sequence's logical blocks [0, sink_blocks[s]) come first, then
    [first_block[s], first_block[s] + blocks_per_seq[s])."""
    perm = rng_perm.permutation(num_blocks).astype(np.int32)
    tables = np.full((len(blocks_per_seq), mb), -1, dtype=np.int32)
    at = 0
    for s, (n, b0) in enumerate(zip(blocks_per_seq, first_block)):
        sb = sink_blocks[s] if sink_blocks is not None else 0
        tables[s, 0:sb] = perm[at:at + sb]
        at += sb
        tables[s, b0:b0 + n] = perm[at:at + n]
        at += n
    return tables


def make_decode(*, lens, num_heads, num_kv_heads, head_dim, block_size, dtype, seed,
                window=0, scale=None, k_scale=1.0, max_blocks_per_seq=None,
                spare_blocks=0, sinks=0, full_start=None, name="decode") -> Workload:
    """A batched single-query decode workload.

    ``lens[s]`` is the context length of sequence s including the query token.
    With ``window > 0`` only blocks that hold a position in ``[L-window, L)``
    are mapped; table entries of blocks that end at or before ``L-window``
    are -1 (freed).  With ``sinks > 0`` as well, the blocks holding the first
    ``sinks`` positions stay mapped too (attention sinks); the blocks between
    them and the window are freed.  ``full_start[s]`` (optional) raises the
    first held position the same way (positions below it were compressed).
    """
    lens = np.asarray(lens, dtype=np.int64)
    S = len(lens)
    B = block_size
    first_block, nblocks, starts, sink_blocks, runs = [], [], [], [], []
    for L in lens:
        L = int(L)
        if L == 0:
            first_block.append(0)
            nblocks.append(0)
            starts.append(0)
            sink_blocks.append(0)
            runs.append(None)
            continue
        lo = max(0, L - window) if window > 0 else 0
        if full_start is not None:
            lo = max(lo, min(int(full_start[len(first_block)]), L))
        b0 = lo // B
        b1 = (L + B - 1) // B
        sb = min((min(sinks, lo) + B - 1) // B, b0) if window > 0 else 0
        first_block.append(b0)
        nblocks.append(b1 - b0)
        sink_blocks.append(sb)
        starts.append(0 if sb else b0 * B)
        runs.append([(0, sb * B), (b0 * B, L)] if sb else None)
    need_mb = max([b + n for b, n in zip(first_block, nblocks)] + [1])
    mb = max_blocks_per_seq if max_blocks_per_seq is not None else need_mb
    if mb < need_mb:
        raise ValueError("max_blocks_per_seq too small")
    nb = int(sum(nblocks)) + int(sum(sink_blocks)) + int(spare_blocks)
    nb = max(nb, 1)
    tables = _deal_tables(stream(seed, TAG_PERM), nblocks, first_block, mb, nb, sink_blocks)
    def one(s):
        n = int(lens[s]) - starts[s]
        rng = stream(seed, TAG_SEQ_KV, s)
        k = draw(rng, (n, num_kv_heads, head_dim), dtype, k_scale)
        v = draw(rng, (n, num_kv_heads, head_dim), dtype)
        return SeqKV(starts[s], k, v, runs[s])

    seq_kv = _parallel_map(one, range(S))
    q = draw(stream(seed, TAG_QUERY), (S, num_heads, head_dim), dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return Workload(name=name, kind="decode", seed=seed, num_seqs=S, num_heads=num_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=B, dtype=dtype,
                    num_blocks=nb, max_blocks_per_seq=mb, window=window, scale=float(scale),
                    context_lens=lens.astype(np.int32), block_tables=tables, q=q, seq_kv=seq_kv,
                    sinks=int(sinks) if window > 0 else 0)


def make_compressed(*, lens, full_start, num_slots, max_slots, num_heads, num_kv_heads, head_dim, block_size,
                    dtype, seed, window=0, scale=None, max_blocks_per_seq=None, spare_blocks=0,
                    name="compressed") -> Workload:
    """A decode workload over two tiers: sequence s holds positions
    [full_start[s], L) at full resolution (blocks below are unmapped) and
    ``num_slots[s]`` slot rows, at most ``max_slots``, in slot blocks of its
    own (ceil(max_slots / B) table entries, mapped as far as the rows
    reach).  Slot rows are drawn like keys and values, scaled by
    1/sqrt(B) (a mean of independent rows is that much narrower).  Slot blocks
    get the pool ids after the full tier's, shuffled."""
    w = make_decode(lens=lens, num_heads=num_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                    block_size=block_size, dtype=dtype, seed=seed, window=window, scale=scale,
                    max_blocks_per_seq=max_blocks_per_seq, spare_blocks=spare_blocks, full_start=full_start,
                    name=name)
    B = block_size
    S = w.num_seqs
    if any(int(f) > max(int(L) - 1, 0) for f, L in zip(full_start, lens)):
        raise ValueError("full_start must leave the step's own position at full resolution (<= L - 1)")
    num_slots = np.asarray(num_slots, np.int64)
    if (num_slots < 0).any() or (num_slots > max_slots).any():
        raise ValueError("num_slots outside [0, max_slots]")
    msb = max(1, -(-int(max_slots) // B))
    used = [-(-int(n) // B) for n in num_slots]
    ids = w.num_blocks + stream(seed, TAG_SLOTS).permutation(max(1, sum(used))).astype(np.int32)
    st = np.full((S, msb), -1, np.int32)
    at = 0
    for s in range(S):
        st[s, :used[s]] = ids[at:at + used[s]]
        at += used[s]

    def one(s):
        rng = stream(seed, TAG_SLOTS, s + 1)
        n = int(num_slots[s])
        k = draw(rng, (n, num_kv_heads, head_dim), dtype, 1.0 / math.sqrt(B))
        v = draw(rng, (n, num_kv_heads, head_dim), dtype, 1.0 / math.sqrt(B))
        return SeqKV(0, k, v)

    w.slot_kv = _parallel_map(one, range(S))
    w.num_blocks += max(1, sum(used))
    w.full_start = np.minimum(np.asarray(full_start, np.int64), w.context_lens).astype(np.int32)
    w.slot_tables = st
    w.num_slots = num_slots.astype(np.int32)
    return w


def make_prefill(*, prefix_len, chunk_lens, num_heads, num_kv_heads, head_dim, block_size,
                 dtype, seed, window=0, scale=None, share_prefix=True, max_blocks_per_seq=None,
                 sinks=0, spare_blocks=0, name="prefill") -> Workload:
    """Chunked prefill: every sequence has a common prefix of ``prefix_len``
    tokens (already cached) followed by its own chunk of ``chunk_lens[s]``
    query tokens.  With ``share_prefix`` the prefix blocks are one set of
    physical blocks mapped by every table (``prefix_len`` must then be a
    multiple of the block size); otherwise each sequence gets private copies.
    ``spare_blocks`` unused blocks widen the pool (the used ids are spread over
    all of it).
    """
    chunk_lens = [int(c) for c in chunk_lens]
    S = len(chunk_lens)
    B = block_size
    if share_prefix and prefix_len % B:
        raise ValueError("a shared prefix must end on a block boundary")
    pb = prefix_len // B if share_prefix else 0
    lens = np.array([prefix_len + c for c in chunk_lens], dtype=np.int64)
    priv = [((int(L) + B - 1) // B) - pb for L in lens]
    need_mb = max([pb + p for p in priv] + [1])
    mb = max_blocks_per_seq if max_blocks_per_seq is not None else need_mb
    nb = max(pb + sum(priv) + int(spare_blocks), 1)
    perm = stream(seed, TAG_PERM).permutation(nb).astype(np.int32)
    tables = np.full((S, mb), -1, dtype=np.int32)
    at = pb
    for s in range(S):
        tables[s, :pb] = perm[:pb]
        tables[s, pb:pb + priv[s]] = perm[at:at + priv[s]]
        at += priv[s]
    rng = stream(seed, TAG_PREFIX_KV)
    prefix = SeqKV(0, draw(rng, (prefix_len, num_kv_heads, head_dim), dtype),
                   draw(rng, (prefix_len, num_kv_heads, head_dim), dtype))
    def one(s):
        rng = stream(seed, TAG_SEQ_KV, s)
        k = draw(rng, (chunk_lens[s], num_kv_heads, head_dim), dtype)
        v = draw(rng, (chunk_lens[s], num_kv_heads, head_dim), dtype)
        return SeqKV(prefix_len, k, v)

    seq_kv = _parallel_map(one, range(S))
    q_start = np.zeros(S + 1, dtype=np.int32)
    q_start[1:] = np.cumsum(chunk_lens)
    q = draw(stream(seed, TAG_QUERY), (int(q_start[-1]), num_heads, head_dim), dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return Workload(name=name, kind="prefill", seed=seed, num_seqs=S, num_heads=num_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=B, dtype=dtype,
                    num_blocks=nb, max_blocks_per_seq=mb, window=window, scale=float(scale),
                    context_lens=lens.astype(np.int32), block_tables=tables, q=q, seq_kv=seq_kv,
                    q_start=q_start, prefix=prefix, prefix_len=prefix_len,
                    shared_prefix_blocks=pb, sinks=int(sinks) if window > 0 else 0)


def private_prefix_copy(w: Workload, seed_perm: int = 7) -> Workload:
    """The same prefill workload with the shared prefix blocks replaced by a
    private copy per sequence (physical ids reshuffled)."""
    assert w.kind == "prefill"
    B = w.block_size
    S = w.num_seqs
    nblk = [int((int(L) + B - 1) // B) for L in w.context_lens]
    nb = sum(nblk)
    mb = max(nblk + [w.max_blocks_per_seq])
    perm = stream(seed_perm, TAG_PERM).permutation(nb).astype(np.int32)
    tables = np.full((S, mb), -1, dtype=np.int32)
    at = 0
    for s in range(S):
        tables[s, :nblk[s]] = perm[at:at + nblk[s]]
        at += nblk[s]
    return dataclasses.replace(w, num_blocks=nb, max_blocks_per_seq=mb, block_tables=tables,
                               shared_prefix_blocks=0)


def repermute(w: Workload, seed_perm: int) -> Workload:
    """The same decode workload with a different physical block assignment."""
    assert w.kind == "decode"
    mapped = w.block_tables >= 0
    ids = w.block_tables[mapped]
    rng = stream(seed_perm, TAG_PERM)
    relabel = rng.permutation(w.num_blocks).astype(np.int32)
    tables = w.block_tables.copy()
    tables[mapped] = relabel[ids]
    return dataclasses.replace(w, block_tables=tables)


# The workloads: a tiny fp32 decode, batched MHA decode, long-context GQA
# decode, sliding-window decode, chunked prefill over a shared prefix, decode
# over a compressed-slot tier and long decode with 8 query heads per kv head.
CONFIG_NAMES = {
    1: "tiny_decode_mha4_d64_b16_L100_f32",
    2: "batched_mha_decode_s32_h32_d128_b16_f16",
    3: "gqa_long_decode_s64_h32kv8_d128_b32_bf16",
    4: "sliding_window_decode_s16_h32kv8_d128_b16_w4096_bf16",
    5: "chunked_prefill_shared_prefix_s8_h32kv8_d128_b16_bf16",
    6: "compressed_tier_decode_s512_h32kv8_d128_b16_w256_m16_bf16",
    7: "gqa8_long_decode_s32_h64kv8_d128_b32_bf16",
}


def config(idx: int, seed: Optional[int] = None) -> Workload:
    """Build one of the workloads by index.  ``seed`` defaults to the index."""
    seed = idx if seed is None else seed
    name = CONFIG_NAMES[idx]
    if idx == 1:
        return make_decode(lens=[100], num_heads=4, num_kv_heads=4, head_dim=64, block_size=16,
                           dtype="f32", seed=seed, scale=1.0 / 8.0, spare_blocks=9, name=name)
    if idx == 2:
        lens = stream(seed, TAG_LENGTHS).integers(512, 4097, size=32)
        return make_decode(lens=lens, num_heads=32, num_kv_heads=32, head_dim=128, block_size=16,
                           dtype="f16", seed=seed, max_blocks_per_seq=256, name=name)
    if idx == 3:
        u = stream(seed, TAG_LENGTHS).uniform(math.log(1024), math.log(32768), size=64)
        lens = np.clip(np.floor(np.exp(u)), 1024, 32768).astype(np.int64)
        return make_decode(lens=lens, num_heads=32, num_kv_heads=8, head_dim=128, block_size=32,
                           dtype="bf16", seed=seed, k_scale=3.0, max_blocks_per_seq=1024,
                           name=name)
    if idx == 4:
        lens = stream(seed, TAG_LENGTHS).integers(16384, 32769, size=16)
        live = sum(((int(L) + 15) // 16) - max(0, int(L) - 4096) // 16 for L in lens)
        return make_decode(lens=lens, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                           dtype="bf16", seed=seed, window=4096, max_blocks_per_seq=2048,
                           spare_blocks=(live + 9) // 10, name=name)
    if idx == 5:
        return make_prefill(prefix_len=2048, chunk_lens=[512] * 8, num_heads=32, num_kv_heads=8,
                            head_dim=128, block_size=16, dtype="bf16", seed=seed,
                            max_blocks_per_seq=160, name=name)
    if idx == 6:
        # Compressed-slot tier with the page's defaults (full window 256,
        # 16 slots, groups of 128 positions): each sequence is in a state the
        # tier reaches, c >= 16 compressions behind it (full tier from
        # c * 128) and 129 .. 256 positions held at full resolution.
        rng = stream(seed, TAG_LENGTHS)
        c = rng.integers(30, 255, size=512)
        held = rng.integers(129, 257, size=512)
        fs = c * 128
        return make_compressed(lens=fs + held, full_start=fs, num_slots=np.full(512, 16), max_slots=16,
                               num_heads=32, num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16", seed=seed,
                               max_blocks_per_seq=2048, name=name)
    if idx == 7:
        # Long-context decode with 8 query heads per kv head (64 query heads
        # over 8 kv heads), otherwise drawn like workload 3.
        u = stream(seed, TAG_LENGTHS).uniform(math.log(1024), math.log(32768), size=32)
        lens = np.clip(np.floor(np.exp(u)), 1024, 32768).astype(np.int64)
        return make_decode(lens=lens, num_heads=64, num_kv_heads=8, head_dim=128, block_size=32,
                           dtype="bf16", seed=seed, k_scale=3.0, max_blocks_per_seq=1024, name=name)
    raise KeyError(idx)
