"""Scalar pure-Python oracle for tiny inputs.  Test infrastructure only.

An independent second reading of the same definitions as ``oracle.ref``
(no NumPy arithmetic, no shared helpers): Python floats (IEEE double),
``math.exp``, ``math.log`` and ``math.fsum`` (exactly rounded sums).

"Build a Paged KV Cache in Pure Python", Step 3 and Step 4; "Building a
Streaming Sliding-Window Attention Engine in Pure Python", Step 3.
"""
from __future__ import annotations

import math
import struct


def value(x, dtype: str) -> float:
    """One stored element as a Python float.  bfloat16 is kept as its 16-bit
    pattern, which is the upper half of a float32."""
    if dtype == "bf16":
        return struct.unpack("<f", struct.pack("<I", (int(x) & 0xFFFF) << 16))[0]
    return float(x)


def head_group(h: int, H: int, Hkv: int) -> int:
    group = H // Hkv
    g = 0
    while (g + 1) * group <= h:
        g += 1
    return g


def slot(table_row, t: int, B: int):
    """(physical block, offset) of logical position t."""
    blk = 0
    rem = t
    while rem >= B:
        rem -= B
        blk += 1
    return int(table_row[blk]), rem


def softmax_weighted(q, keys, vals, scale):
    """q: list[D]; keys/vals: lists of list[D].  Returns (out list[D], lse)."""
    D = len(q)
    if not keys:
        return [0.0] * D, -math.inf
    scores = [scale * math.fsum(q[d] * k[d] for d in range(D)) for k in keys]
    m = scores[0]
    for s in scores[1:]:
        if s > m:
            m = s
    e = [math.exp(s - m) for s in scores]
    z = math.fsum(e)
    w = [x / z for x in e]
    out = [math.fsum(w[t] * vals[t][d] for t in range(len(vals))) for d in range(D)]
    return out, m + math.log(z)


def decode(q, k_pool, v_pool, tables, lens, B, Hkv, window, scale, dtype, sinks=0):
    """Nested lists out[s][h][d], lse[s][h].  With a window, positions below
    ``sinks`` are attended as well."""
    S, H, D = len(q), len(q[0]), len(q[0][0])
    out, lse = [], []
    for s in range(S):
        L = int(lens[s])
        lo = 0
        if window > 0 and L - window > 0:
            lo = L - window
        rows, lrow = [], []
        for h in range(H):
            g = head_group(h, H, Hkv)
            keys, vals = [], []
            for t in range(0, L):
                if t < lo and not (window > 0 and t < sinks):
                    continue
                pb, off = slot(tables[s], t, B)
                keys.append([value(k_pool[pb][off][g][d], dtype) for d in range(D)])
                vals.append([value(v_pool[pb][off][g][d], dtype) for d in range(D)])
            qv = [value(q[s][h][d], dtype) for d in range(D)]
            o, l = softmax_weighted(qv, keys, vals, scale)
            rows.append(o)
            lrow.append(l)
        out.append(rows)
        lse.append(lrow)
    return out, lse


def prefill(q, q_start, k_pool, v_pool, tables, lens, B, Hkv, window, scale, dtype, sinks=0):
    """Nested lists out[row][h][d] for every query row of every chunk."""
    H, D = len(q[0]), len(q[0][0])
    out = [None] * len(q)
    for s in range(len(lens)):
        r0, r1 = int(q_start[s]), int(q_start[s + 1])
        L = int(lens[s])
        C = r1 - r0
        for i in range(C):
            p = L - C + i
            rows = []
            for h in range(H):
                g = head_group(h, H, Hkv)
                keys, vals = [], []
                for t in range(0, p + 1):
                    if window > 0 and not (p - t < window) and not t < sinks:
                        continue
                    pb, off = slot(tables[s], t, B)
                    keys.append([value(k_pool[pb][off][g][d], dtype) for d in range(D)])
                    vals.append([value(v_pool[pb][off][g][d], dtype) for d in range(D)])
                qv = [value(q[r0 + i][h][d], dtype) for d in range(D)]
                rows.append(softmax_weighted(qv, keys, vals, scale)[0])
            out[r0 + i] = rows
    return out


def decode_compressed(q, k_pool, v_pool, tables, lens, full_start, slot_tables, num_slots, B, Hkv, window,
                      scale, dtype):
    """Decode over a compressed-slot tier and a full tier: the positions t
    with full_start <= t < L (and inside the window, if any) through the
    block table, plus rows 0 .. num_slots-1 of the slot table (row r at
    offset r % B of its block r // B).  Nested lists out[s][h][d], lse[s][h]."""
    S, H, D = len(q), len(q[0]), len(q[0][0])
    out, lse = [], []
    for s in range(S):
        L = int(lens[s])
        fs = int(full_start[s])
        rows, lrow = [], []
        for h in range(H):
            g = head_group(h, H, Hkv)
            keys, vals = [], []
            for t in range(L):
                if t < fs or (window > 0 and L - t > window):
                    continue
                pb, off = slot(tables[s], t, B)
                keys.append([value(k_pool[pb][off][g][d], dtype) for d in range(D)])
                vals.append([value(v_pool[pb][off][g][d], dtype) for d in range(D)])
            for r in range(int(num_slots[s])):
                pb, off = slot(slot_tables[s], r, B)
                keys.append([value(k_pool[pb][off][g][d], dtype) for d in range(D)])
                vals.append([value(v_pool[pb][off][g][d], dtype) for d in range(D)])
            qv = [value(q[s][h][d], dtype) for d in range(D)]
            o, l = softmax_weighted(qv, keys, vals, scale)
            rows.append(o)
            lrow.append(l)
        out.append(rows)
        lse.append(lrow)
    return out, lse
