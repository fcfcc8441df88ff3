"""Vectorised float64 oracle (NumPy).  Test infrastructure only.

Every function states the passage of the pages it writes out.  Notation:
S sequences, H query heads, Hkv key/value heads, G = H // Hkv, D head dim,
B block size, NB pool blocks, MB table width, L_s context length of sequence s
(including the query token(s)), w window (0 = no window).

Pools are ``[NB, B, Hkv, D]`` in the storage dtype ("f32" float32, "f16"
float16, "bf16" uint16 bit patterns).  This is the per-block layout of
``KVCacheBlock`` in "Build a Paged KV Cache in Pure Python", Step 1, with the
K and V arrays of every block stacked into one pool each.
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------- decoding

def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values to float64.  bfloat16 bits are the top
    16 bits of an IEEE float32."""
    if dtype == "bf16":
        a = np.asarray(a, dtype=np.uint16)
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(a).astype(np.float64)


def kv_head_of(h: int, num_heads: int, num_kv_heads: int) -> int:
    """Query head h reads kv head floor(h / G), G = H / Hkv (consecutive query
    heads share one kv head).  The pages are multi-head only; this is the
    grouped reading that reduces to h when G = 1."""
    return h // (num_heads // num_kv_heads)


# ------------------------------------------------------------------- write

def kv_write(k_pool, v_pool, k_new, v_new, seq_idx, pos, block_tables, block_size):
    """Write new tokens' keys/values into their pool slots.

    "Build a Paged KV Cache in Pure Python", Step 3 (``PagedKVCache.append``):
    for a token at logical position p of sequence s, the block is
    ``table[s][p // B]`` and the slot inside it is ``p % B``; the whole
    (Hkv, D) row of keys and of values is stored there.  A byte copy: no
    other byte of either pool changes.  Returns new pools (inputs untouched).
    """
    k_pool = np.array(k_pool, copy=True)
    v_pool = np.array(v_pool, copy=True)
    nb = k_pool.shape[0]
    for n in range(len(seq_idx)):
        s = int(seq_idx[n])
        p = int(pos[n])
        pb = int(block_tables[s, p // block_size])
        if not 0 <= pb < nb:
            raise IndexError(f"token {n}: seq {s} pos {p} maps to block {pb}")
        off = p % block_size
        k_pool[pb, off] = k_new[n]
        v_pool[pb, off] = v_new[n]
    return k_pool, v_pool


def copy_blocks(k_pool, v_pool, src, dst, k_scale=None, v_scale=None):
    """Copy block src[i] to block dst[i] in both pools (every slot and kv
    head), and the rows' scales of 8-bit pools ([NB, Hkv, B]).  The copy of
    copy-on-write: a page shared by several sequences ("Build a Minimal LLM
    Inference Engine ...", Step 1: refcount above one) is duplicated before
    one of them writes into it.  Pairs with an id outside [0, NB) or
    src == dst are skipped.  Returns new arrays (inputs untouched)."""
    out = [np.array(a, copy=True) if a is not None else None for a in (k_pool, v_pool, k_scale, v_scale)]
    nb = out[0].shape[0]
    for a, b in zip(np.asarray(src), np.asarray(dst)):
        a, b = int(a), int(b)
        if not (0 <= a < nb and 0 <= b < nb) or a == b:
            continue
        for arr, orig in zip(out, (k_pool, v_pool, k_scale, v_scale)):
            if arr is not None:
                arr[b] = np.asarray(orig)[a]
    return tuple(out)


# ------------------------------------------------------------------ gather

def gather(pool, table_row, positions, g, block_size, dtype):
    """Rows of kv head g for the given logical positions, as float64 [n, D].

    "Build a Paged KV Cache in Pure Python", Step 3 (``retrieve``) and
    "Build a Minimal LLM Inference Engine ...", Step 4 (``compute_attention``
    walks the block table): position t lives in physical block
    ``table[t // B]`` at slot ``t % B``.
    """
    positions = np.asarray(positions, dtype=np.int64)
    pb = np.asarray(table_row, dtype=np.int64)[positions // block_size]
    if positions.size and (pb < 0).any():
        raise IndexError("attended position maps to an unmapped block")
    return to_f64(pool[pb, positions % block_size, g, :], dtype)


# -------------------------------------------------------------- attention

def attend(q_rows, keys, values, scale):
    """Scaled dot-product attention of query rows over one key/value set.

    "Build a Paged KV Cache in Pure Python", Step 4: scores = q . k_t * scale
    for every key; softmax over the key axis after subtracting the maximum;
    output = sum_t weight_t * v_t.  An empty key set gives zeros (same step)
    and log-sum-exp -inf.

    q_rows [R, D], keys/values [n, D] float64 -> (out [R, D], lse [R]).
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    R, D = q_rows.shape
    if keys.shape[0] == 0:
        return np.zeros((R, values.shape[1] if values.ndim == 2 else D)), np.full(R, -np.inf)
    scores = (q_rows @ keys.T) * scale                   # [R, n]
    m = scores.max(axis=1, keepdims=True)
    e = np.exp(scores - m)
    z = e.sum(axis=1, keepdims=True)
    p = e / z
    if not np.all(np.abs(p.sum(axis=1) - 1.0) < 1e-12):
        raise AssertionError("softmax weights do not sum to 1")
    out = p @ values
    lse = m[:, 0] + np.log(z[:, 0])
    return out, lse


def attended_range(L: int, window: int):
    """Positions a decode query at position L-1 attends: the last ``window``
    positions including itself, or all of [0, L) when window is 0.

    "Building a Streaming Sliding-Window Attention Engine in Pure Python",
    Step 3: query i attends keys in [i - w + 1, i]; at decode time the query is
    the just-appended position T-1 and the window starts at max(0, T - w).
    """
    lo = max(0, L - window) if window > 0 else 0
    return lo, L


def attended_positions(L: int, window: int, sinks: int = 0) -> np.ndarray:
    """Positions a decode query at position L-1 attends, in increasing order:
    ``attended_range`` and, with a window, also the first ``sinks`` positions.

    "Building a Streaming Sliding-Window Attention Engine in Pure Python",
    Step 4 (eviction policies that keep the first few tokens, the "attention
    sinks", when the middle is dropped) and the roadmap's attention-sinks
    item (keep the first 4 tokens regardless of the window).
    """
    lo, hi = attended_range(L, window)
    pos = np.arange(lo, hi)
    if window > 0 and sinks > 0:
        pos = np.union1d(np.arange(min(sinks, L)), pos)
    return pos


def decode(q, k_pool, v_pool, block_tables, context_lens, *, block_size, num_kv_heads,
           window, scale, dtype, seqs=None, heads=None, kv_dtype=None, sinks=0):
    """Single-query decode through the block table, every (seq, head).

    q [S, H, D].  Returns (out [S, H, D], lse [S, H]) float64; with ``seqs`` /
    ``heads`` only those rows are computed (others stay NaN).  ``sinks``: see
    ``attended_positions``.  ``kv_dtype``
    (default ``dtype``) is the storage type of the pools when it differs from
    the queries' ("f64": already decoded values).
    """
    kv_dtype = dtype if kv_dtype is None else kv_dtype
    S, H, D = q.shape
    out = np.full((S, H, D), np.nan)
    lse = np.full((S, H), np.nan)
    qf = to_f64(q, dtype)
    seqs = range(S) if seqs is None else seqs
    heads = range(H) if heads is None else heads
    for s in seqs:
        L = int(context_lens[s])
        pos = attended_positions(L, window, sinks) if sinks else np.arange(*attended_range(L, window))
        by_group = {}
        for h in heads:
            by_group.setdefault(kv_head_of(h, H, num_kv_heads), []).append(h)
        for g, hs in by_group.items():
            K = gather(k_pool, block_tables[s], pos, g, block_size, kv_dtype)
            V = gather(v_pool, block_tables[s], pos, g, block_size, kv_dtype)
            o, l = attend(qf[s, hs], K, V, scale)
            out[s, hs] = o
            lse[s, hs] = l
    return out, lse


def contiguous_decode(q_s, k_log, v_log, first_pos, L, *, num_kv_heads, window, scale, dtype, sinks=0):
    """The same decode over a contiguous (never paged) cache of one sequence.

    "Building a Streaming Sliding-Window Attention Engine in Pure Python",
    Step 2 and Step 3: keys/values of positions [first_pos, L) in one array in
    position order, sliced to the window.  This is what a paged result must
    equal for any physical block assignment.

    q_s [H, D]; k_log/v_log [L - first_pos, Hkv, D].  Returns (out, lse).
    With ``sinks`` the first positions are kept as well (``attended_positions``).
    """
    H, D = q_s.shape
    pos = attended_positions(L, window, sinks)
    if pos.size and pos[0] < first_pos:
        raise ValueError("attended positions reach before the first stored position")
    qf = to_f64(q_s, dtype)
    out = np.zeros((H, D))
    lse = np.zeros(H)
    for h in range(H):
        g = kv_head_of(h, H, num_kv_heads)
        K = to_f64(k_log[pos - first_pos, g], dtype)
        V = to_f64(v_log[pos - first_pos, g], dtype)
        o, l = attend(qf[h:h + 1], K, V, scale)
        out[h] = o[0]
        lse[h] = l[0]
    return out, lse


def prefill_keys(L: int, C: int, window: int, sinks: int = 0):
    """Query row i of a chunk of C rows that ends at position L-1 sits at
    position p = L - C + i; it attends t <= p, and t > p - w when w > 0
    (with ``sinks``, also every t < sinks, t <= p: see ``attended_positions``).

    "Building a Streaming Sliding-Window Attention Engine in Pure Python",
    Step 3 (``prefill_attention``: causal and sliding-window mask); the chunk
    reading (earlier positions are already cached and all visible) extends it
    to a cached prefix.  Returns a boolean mask [C, L].
    """
    p = (L - C) + np.arange(C)[:, None]
    t = np.arange(L)[None, :]
    mask = t <= p
    if window > 0:
        keep = t > p - window
        if sinks > 0:
            keep |= t < sinks
        mask &= keep
    return mask


def prefill(q, q_start, k_pool, v_pool, block_tables, context_lens, *, block_size,
            num_kv_heads, window, scale, dtype, seqs=None, heads=None, sinks=0, kv_dtype=None):
    """Causal chunked prefill through the block table.

    q [sum C, H, D] with sequence s owning rows q_start[s]:q_start[s+1] (its
    chunk = its last C_s positions).  Dense masked attention per (seq, head),
    with the mask of ``prefill_keys``; masked keys are excluded (weight 0).
    ``kv_dtype`` (default ``dtype``) is the pools' storage type when it
    differs from the queries' ("f64": already decoded values).
    Returns (out [sum C, H, D], lse [sum C, H]) float64.
    """
    kv_dtype = dtype if kv_dtype is None else kv_dtype
    T, H, D = q.shape
    out = np.full((T, H, D), np.nan)
    lse = np.full((T, H), np.nan)
    qf = to_f64(q, dtype)
    seqs = range(len(context_lens)) if seqs is None else seqs
    heads = range(H) if heads is None else heads
    for s in seqs:
        r0, r1 = int(q_start[s]), int(q_start[s + 1])
        C = r1 - r0
        L = int(context_lens[s])
        if C == 0:
            continue
        mask = prefill_keys(L, C, window, sinks) if sinks else prefill_keys(L, C, window)
        lo = int(np.argmax(mask[0])) if window > 0 else 0
        pos = np.arange(lo, L)
        mask = mask[:, lo:]
        for h in heads:
            g = kv_head_of(h, H, num_kv_heads)
            K = gather(k_pool, block_tables[s], pos, g, block_size, kv_dtype)
            V = gather(v_pool, block_tables[s], pos, g, block_size, kv_dtype)
            scores = (qf[r0:r1, h] @ K.T) * scale
            scores = np.where(mask, scores, -np.inf)
            m = scores.max(axis=1, keepdims=True)
            e = np.exp(scores - m)
            z = e.sum(axis=1, keepdims=True)
            p = e / z
            if not np.all(np.abs(p.sum(axis=1) - 1.0) < 1e-12):
                raise AssertionError("softmax weights do not sum to 1")
            out[r0:r1, h] = p @ V
            lse[r0:r1, h] = m[:, 0] + np.log(z[:, 0])
    return out, lse


def prefill_attention_single(Q, K, V, window, scale):
    """Dense prefill of n tokens with no cached prefix, one head.

    "Building a Streaming Sliding-Window Attention Engine in Pure Python",
    Step 3 (``prefill_attention``): the (n, n) mask keeps j <= i and
    i - j < w; masked scores are filled with -1e9; softmax is taken per query
    row (the row-wise reading; the printed helper normalises over the whole
    matrix, which would not give a distribution per query).
    """
    Q = np.asarray(Q, np.float64)
    n = Q.shape[0]
    idx = np.arange(n)
    mask = (idx[:, None] - idx[None, :]) < (window if window > 0 else n + 1)
    mask &= idx[None, :] <= idx[:, None]
    scores = (Q @ np.asarray(K, np.float64).T) * scale
    scores = np.where(mask, scores, -1e9)
    m = scores.max(axis=1, keepdims=True)
    e = np.exp(scores - m)
    p = e / e.sum(axis=1, keepdims=True)
    return p @ np.asarray(V, np.float64)


def build_pools(w, *, poison=True, include_step=True):
    """Fill fresh K/V pools for a workload using ``kv_write`` on its history
    tokens (and, with ``include_step``, the step's own tokens), every other
    slot NaN (``poison``) or zero.  Returns (k_pool, v_pool) in the storage
    dtype."""
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    if w.dtype == "bf16":
        fill = np.uint16(0x7FC0) if poison else np.uint16(0)
        k_pool = np.full(shape, fill, np.uint16)
    else:
        st = np.float32 if w.dtype == "f32" else np.float16
        k_pool = np.full(shape, np.nan if poison else 0, st)
    v_pool = k_pool.copy()
    for s, p0, k, v in w.history_tokens():
        n = k.shape[0]
        k_pool, v_pool = kv_write_run(k_pool, v_pool, k, v, s, p0, w.block_tables, w.block_size)
    if include_step:
        si, pos, k, v = w.step_tokens()
        k_pool, v_pool = kv_write(k_pool, v_pool, k, v, si, pos, w.block_tables, w.block_size)
    if getattr(w, "slot_kv", None) is not None:
        # compressed slots: slot row r of s sits where position r would
        # through the slot table (row r % B of block slot_tables[s, r // B])
        for s, e in enumerate(w.slot_kv):
            if e.k.shape[0]:
                k_pool, v_pool = kv_write_run(k_pool, v_pool, e.k, e.v, s, 0, w.slot_tables, w.block_size)
    return k_pool, v_pool


def kv_write_run(k_pool, v_pool, k, v, s, p0, block_tables, block_size):
    """``kv_write`` of a run of consecutive positions p0.. of one sequence,
    in place (a vectorised form of the same per-token rule)."""
    pos = p0 + np.arange(k.shape[0])
    pb = block_tables[s, pos // block_size].astype(np.int64)
    if (pb < 0).any() or (pb >= k_pool.shape[0]).any():
        raise IndexError("write to an unmapped block")
    k_pool[pb, pos % block_size] = k
    v_pool[pb, pos % block_size] = v
    return k_pool, v_pool
