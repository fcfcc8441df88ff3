"""Pins of the fp64 oracle against things other than itself: closed forms,
invariants, special cases, a library routine and a scalar brute force.  The
last test plants mistakes in the oracle and checks a pin catches each one.

CPU only.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle.brute as brute
import oracle.ref as ref
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small_decode(seed, *, S=3, H=4, Hkv=2, D=8, B=4, dtype="f32", window=0, lens=None,
                 k_scale=1.0, spare=2):
    if lens is None:
        lens = wl.stream(seed, 99).integers(1, 23, size=S)
    return wl.make_decode(lens=lens, num_heads=H, num_kv_heads=Hkv, head_dim=D, block_size=B,
                          dtype=dtype, seed=seed, window=window, k_scale=k_scale,
                          spare_blocks=spare)


def ref_decode(w, k_pool, v_pool, tables=None):
    return ref.decode(w.q, k_pool, v_pool, w.block_tables if tables is None else tables,
                      w.context_lens, block_size=w.block_size, num_kv_heads=w.num_kv_heads,
                      window=w.window, scale=w.scale, dtype=w.dtype, sinks=w.sinks)


def ref_prefill(w, k_pool, v_pool, window=None, sinks=0):
    return ref.prefill(w.q, w.q_start, k_pool, v_pool, w.block_tables, w.context_lens,
                       block_size=w.block_size, num_kv_heads=w.num_kv_heads,
                       window=w.window if window is None else window, scale=w.scale,
                       dtype=w.dtype, sinks=sinks)


def contiguous(w, s):
    first, k, v = w.logical_kv(s)
    return ref.contiguous_decode(w.q[s], k, v, first, int(w.context_lens[s]),
                                 num_kv_heads=w.num_kv_heads, window=w.window, scale=w.scale,
                                 dtype=w.dtype)


# ---------------------------------------------------------------- the pins
# Each returns True when the oracle passes it; the mutation test reuses them.

def pin_brute_decode():
    ok = True
    cases = [dict(dtype="f32"), dict(dtype="f16", H=4, Hkv=4), dict(dtype="bf16", H=6, Hkv=2),
             dict(dtype="f32", window=5), dict(dtype="bf16", window=1, B=3),
             dict(dtype="f32", H=2, Hkv=1, B=5, window=30)]
    for i, kw in enumerate(cases):
        w = small_decode(100 + i, **kw)
        kp, vp = ref.build_pools(w)
        out, lse = ref_decode(w, kp, vp)
        bo, bl = brute.decode(w.q, kp, vp, w.block_tables, w.context_lens, w.block_size,
                              w.num_kv_heads, w.window, w.scale, w.dtype)
        ok &= np.max(np.abs(out - np.array(bo))) <= 1e-12
        ok &= np.max(np.abs(lse - np.array(bl))) <= 1e-12
    return bool(ok)


def pin_brute_prefill():
    ok = True
    for i, (dtype, window, share) in enumerate([("f32", 0, True), ("bf16", 3, False),
                                                 ("f16", 0, False), ("f32", 6, True)]):
        w = wl.make_prefill(prefix_len=8, chunk_lens=[5, 1, 7], num_heads=4, num_kv_heads=2,
                            head_dim=8, block_size=4, dtype=dtype, seed=200 + i, window=window,
                            share_prefix=share)
        kp, vp = ref.build_pools(w)
        out, _ = ref_prefill(w, kp, vp)
        bo = brute.prefill(w.q, w.q_start, kp, vp, w.block_tables, w.context_lens, w.block_size,
                           w.num_kv_heads, window, w.scale, dtype)
        ok &= np.max(np.abs(out - np.array(bo))) <= 1e-12
    return bool(ok)


def pin_library_sdpa():
    """Contiguous decode and paged prefill vs torch's float64 SDPA (CPU), with
    its own grouped-query convention (enable_gqa)."""
    ok = True
    w = small_decode(7, S=4, H=8, Hkv=2, D=16, B=8, dtype="bf16", k_scale=3.0)
    kp, vp = ref.build_pools(w)
    out, _ = ref_decode(w, kp, vp)
    for s in range(w.num_seqs):
        first, k, v = w.logical_kv(s)
        q = torch.from_numpy(ref.to_f64(w.q[s], w.dtype))[None, :, None, :]
        K = torch.from_numpy(ref.to_f64(k, w.dtype)).permute(1, 0, 2)[None]
        V = torch.from_numpy(ref.to_f64(v, w.dtype)).permute(1, 0, 2)[None]
        lib = torch.nn.functional.scaled_dot_product_attention(q, K, V, scale=w.scale,
                                                               enable_gqa=True)
        ok &= np.max(np.abs(out[s] - lib[0, :, 0].numpy())) <= 1e-12
    p = wl.make_prefill(prefix_len=12, chunk_lens=[6, 9], num_heads=4, num_kv_heads=1, head_dim=8,
                        block_size=4, dtype="f16", seed=9, window=5)
    kp, vp = ref.build_pools(p)
    out, _ = ref_prefill(p, kp, vp)
    for s in range(p.num_seqs):
        r0, r1 = p.q_start[s], p.q_start[s + 1]
        first, k, v = p.logical_kv(s)
        L = int(p.context_lens[s])
        C = r1 - r0
        pos = L - C + np.arange(C)[:, None]
        t = np.arange(L)[None, :]
        mask = torch.from_numpy((t <= pos) & (pos - t < 5))
        q = torch.from_numpy(ref.to_f64(p.q[r0:r1], p.dtype)).permute(1, 0, 2)[None]
        K = torch.from_numpy(ref.to_f64(k, p.dtype)).permute(1, 0, 2)[None]
        V = torch.from_numpy(ref.to_f64(v, p.dtype)).permute(1, 0, 2)[None]
        lib = torch.nn.functional.scaled_dot_product_attention(q, K, V, attn_mask=mask,
                                                               scale=p.scale, enable_gqa=True)
        ok &= np.max(np.abs(out[r0:r1] - lib[0].permute(1, 0, 2).numpy())) <= 1e-12
    return bool(ok)


def pin_closed_forms():
    """L = 1 gives v0 exactly; q = 0 gives the mean of the attended values;
    constant values give that constant; the two-token worked case."""
    g = json.load(open(os.path.join(GOLDEN, "closed_forms.json")))["two_token"]
    ok = True
    # L = 1
    w = small_decode(3, lens=[1, 1], dtype="bf16")
    kp, vp = ref.build_pools(w)
    out, lse = ref_decode(w, kp, vp)
    for s in range(2):
        _, k, v = w.logical_kv(s)
        for h in range(w.num_heads):
            ok &= np.array_equal(out[s, h], ref.to_f64(v[0, ref.kv_head_of(h, 4, 2)], "bf16"))
    # q = 0 -> mean
    w = small_decode(4, dtype="f32")
    w.q[:] = 0
    kp, vp = ref.build_pools(w)
    out, _ = ref_decode(w, kp, vp)
    for s in range(w.num_seqs):
        _, k, v = w.logical_kv(s)
        for h in range(w.num_heads):
            mean = v[:, ref.kv_head_of(h, 4, 2)].astype(np.float64).mean(axis=0)
            ok &= np.max(np.abs(out[s, h] - mean)) <= 1e-14
    # V == c
    w = small_decode(5, dtype="f16")
    for e in w.seq_kv:
        e.v[:] = np.float16(1.5)
    kp, vp = ref.build_pools(w)
    out, _ = ref_decode(w, kp, vp)
    ok &= np.max(np.abs(out - 1.5)) <= 1e-14
    # two tokens, weights 1/4 and 3/4
    D, B = g["head_dim"], g["block_size"]
    w = wl.make_decode(lens=[2], num_heads=1, num_kv_heads=1, head_dim=D, block_size=B,
                       dtype="f32", seed=1, scale=g["scale"])
    w.q[:] = 0
    w.q[0, 0, 0] = g["q_e0"]
    e = w.seq_kv[0]
    e.k[:] = 0
    e.k[1, 0, 0] = np.float32(math.log(3.0))
    e.v[0] = g["v0"]
    e.v[1] = g["v1"]
    kp, vp = ref.build_pools(w)
    out, lse = ref_decode(w, kp, vp)
    k1 = float(np.float32(math.log(3.0)))  # the stored key is float32
    w1 = math.exp(k1) / (1 + math.exp(k1))
    want = g["v0"] * (1 - w1) + g["v1"] * w1
    ok &= abs(w1 - g["weights"][1]) < 1e-7
    ok &= np.max(np.abs(out[0, 0] - want)) <= 1e-14 and abs(want - g["out"]) < 1e-6
    ok &= abs(lse[0, 0] - math.log(1 + math.exp(k1))) <= 1e-14
    return bool(ok)


def pin_permutation_invariance():
    """Paged decode equals contiguous attention for several physical block
    assignments, bit for bit."""
    ok = True
    for window in (0, 7):
        w = small_decode(11, S=4, dtype="bf16", window=window, k_scale=3.0)
        first = None
        for perm_seed in (0, 1, 2):
            wp = wl.repermute(w, perm_seed)
            kp, vp = ref.build_pools(wp)
            out, lse = ref_decode(wp, kp, vp)
            if first is None:
                first = (out, lse)
            ok &= np.array_equal(out, first[0]) and np.array_equal(lse, first[1])
            for s in range(w.num_seqs):
                co, cl = contiguous(wp, s)
                # one head at a time vs a head group at a time: fp64 rounding only
                ok &= np.max(np.abs(out[s] - co)) <= 1e-13 and np.max(np.abs(lse[s] - cl)) <= 1e-13
    return bool(ok)


def pin_window():
    """Window w equals attention over the last w positions only; w = 1 gives
    the query's own value; w >= L equals no window."""
    ok = True
    lens = [9, 20, 4]
    base = wl.make_decode(lens=lens, num_heads=4, num_kv_heads=2, head_dim=8, block_size=4,
                          dtype="f32", seed=12, spare_blocks=2)
    kp, vp = ref.build_pools(base)
    full, _ = ref_decode(base, kp, vp)
    for wsz in (1, 3, 8, 20, 64):
        w = wl.make_decode(lens=lens, num_heads=4, num_kv_heads=2, head_dim=8, block_size=4,
                           dtype="f32", seed=12, window=wsz, spare_blocks=2)
        kpw, vpw = ref.build_pools(w)
        out, _ = ref_decode(w, kpw, vpw)
        for s in range(3):
            L = int(w.context_lens[s])
            first, k, v = w.logical_kv(s)
            lo = max(0, L - wsz)
            for h in range(4):
                g = ref.kv_head_of(h, 4, 2)
                o, _ = ref.attend(ref.to_f64(w.q[s, h:h + 1], "f32"),
                                  k[lo - first:L - first, g].astype(np.float64),
                                  v[lo - first:L - first, g].astype(np.float64), w.scale)
                ok &= np.max(np.abs(out[s, h] - o[0])) <= 1e-13
                if wsz == 1:
                    ok &= np.array_equal(out[s, h], v[L - 1 - first, g].astype(np.float64))
                if wsz >= L:
                    ok &= np.array_equal(out[s, h], full[s, h])
    return bool(ok)


def pin_prefill_rows_are_decodes():
    """Row i of a chunk equals a decode whose context ends at that row's
    position; a chunk of 1 is a decode; with no prefix the chunk equals the
    dense causal (windowed) prefill applied per row."""
    ok = True
    for window in (0, 5):
        p = wl.make_prefill(prefix_len=8, chunk_lens=[6, 1, 4], num_heads=4, num_kv_heads=2,
                            head_dim=8, block_size=4, dtype="f32", seed=21, window=window)
        kp, vp = ref.build_pools(p)
        out, lse = ref_prefill(p, kp, vp)
        for s in range(p.num_seqs):
            r0, r1 = int(p.q_start[s]), int(p.q_start[s + 1])
            L = int(p.context_lens[s])
            C = r1 - r0
            for i in range(C):
                d, dl = ref.decode(p.q[r0 + i][None], kp, vp, p.block_tables[s:s + 1],
                                   np.array([L - C + i + 1]), block_size=4, num_kv_heads=2,
                                   window=window, scale=p.scale, dtype="f32")
                ok &= np.max(np.abs(out[r0 + i] - d[0])) <= 1e-13
                ok &= np.max(np.abs(lse[r0 + i] - dl[0])) <= 1e-13
    for window in (0, 3):
        p = wl.make_prefill(prefix_len=0, chunk_lens=[9], num_heads=2, num_kv_heads=2, head_dim=8,
                            block_size=4, dtype="f32", seed=22, window=window)
        kp, vp = ref.build_pools(p)
        out, _ = ref_prefill(p, kp, vp)
        k, v = p.seq_kv[0].k, p.seq_kv[0].v
        for h in range(2):
            dense = ref.prefill_attention_single(p.q[:, h], k[:, h], v[:, h], window, p.scale)
            ok &= np.max(np.abs(out[:, h] - dense)) <= 1e-13
    return bool(ok)


def pin_shared_prefix():
    """Shared prefix blocks give exactly the result of private copies."""
    p = wl.make_prefill(prefix_len=12, chunk_lens=[5, 7, 3], num_heads=4, num_kv_heads=2,
                        head_dim=8, block_size=4, dtype="bf16", seed=31)
    q = wl.private_prefix_copy(p)
    kp, vp = ref.build_pools(p)
    # Private copies: the prefix is written through every sequence's own table.
    kq, vq = _private_pools(q)
    a, al = ref_prefill(p, kp, vp)
    b, bl = ref_prefill(q, kq, vq)
    return bool(np.array_equal(a, b) and np.array_equal(al, bl))


def _private_pools(q):
    shape = (q.num_blocks, q.block_size, q.num_kv_heads, q.head_dim)
    kp = np.full(shape, 0x7FC0, np.uint16) if q.dtype == "bf16" else np.full(shape, np.nan, np.float32)
    vp = kp.copy()
    for s in range(q.num_seqs):
        first, k, v = q.logical_kv(s)
        kp, vp = ref.kv_write_run(kp, vp, k, v, s, 0, q.block_tables, q.block_size)
    return kp, vp


def pin_gqa_equals_replicated_mha():
    """Grouped heads equal a multi-head run whose kv heads are the grouped
    kv heads repeated G times."""
    w = small_decode(41, S=3, H=6, Hkv=2, D=8, B=4, dtype="f16")
    kp, vp = ref.build_pools(w)
    out, lse = ref_decode(w, kp, vp)
    G = 3
    km = np.repeat(kp, G, axis=2)
    vm = np.repeat(vp, G, axis=2)
    mo, ml = ref.decode(w.q, km, vm, w.block_tables, w.context_lens, block_size=4, num_kv_heads=6,
                        window=0, scale=w.scale, dtype="f16")
    # G heads per matmul vs one: fp64 rounding only
    return bool(np.max(np.abs(out - mo)) <= 1e-13 and np.max(np.abs(lse - ml)) <= 1e-13)


def pin_write_round_trip():
    """35 tokens appended one by one over blocks of 16 read back unchanged;
    no other byte of the pools changes."""
    B, Hkv, D = 16, 8, 64
    rng = np.random.default_rng(5)
    tables = np.array([[5, 0, 9], [1, 2, 3]], dtype=np.int32)
    k_new = rng.standard_normal((35, Hkv, D)).astype(np.float32)
    v_new = rng.standard_normal((35, Hkv, D)).astype(np.float32)
    kp = np.full((10, B, Hkv, D), np.nan, np.float32)
    vp = kp.copy()
    kp2, vp2 = ref.kv_write(kp, vp, k_new, v_new, np.zeros(35, np.int32), np.arange(35),
                            tables, B)
    ok = True
    K = ref.gather(kp2[:, :, :, :], tables[0], np.arange(35), slice(None), B, "f32")
    ok &= K.shape == (35, Hkv, D) and np.array_equal(K, k_new.astype(np.float64))
    V = ref.gather(vp2, tables[0], np.arange(35), slice(None), B, "f32")
    ok &= np.array_equal(V, v_new.astype(np.float64))
    touched = np.zeros(kp.shape[:2], bool)
    for t in range(35):
        touched[tables[0, t // B], t % B] = True
    ok &= bool(np.isnan(kp2[~touched]).all() and np.isnan(vp2[~touched]).all())
    ok &= int(touched.sum()) == 35
    return bool(ok)


def pin_sinks():
    """Window plus attention sinks: attention over exactly the positions
    [0, min(s, L-w)) and [L-w, L) (explicit slices of the contiguous keys),
    the scalar brute force, torch SDPA with the explicit prefill mask, prefill
    rows equal to decodes, and sinks covering everything before the window
    give the unwindowed result.  The generator frees the blocks between the
    sink blocks and the window."""
    ok = True
    lens = [9, 30, 4, 50]
    base = wl.make_decode(lens=lens, num_heads=4, num_kv_heads=2, head_dim=8, block_size=4,
                          dtype="f32", seed=41, spare_blocks=2)
    kpb, vpb = ref.build_pools(base)
    full, _ = ref_decode(base, kpb, vpb)
    for wsz in (3, 8):
        for sk in (1, 4, 6, 64):
            w = wl.make_decode(lens=lens, num_heads=4, num_kv_heads=2, head_dim=8, block_size=4,
                               dtype="f32", seed=41, window=wsz, sinks=sk, spare_blocks=2)
            kp, vp = ref.build_pools(w)
            out, lse = ref_decode(w, kp, vp)
            bo, bl = brute.decode(w.q, kp, vp, w.block_tables, w.context_lens, 4, 2, wsz, w.scale, "f32",
                                  sinks=sk)
            ok &= np.max(np.abs(out - np.array(bo))) <= 1e-12
            for s in range(len(lens)):
                L = int(w.context_lens[s])
                lo = max(0, L - wsz)
                first, k, v = w.logical_kv(s)
                pos = np.concatenate([np.arange(min(sk, lo)), np.arange(lo, L)])
                # freed blocks: nothing between the sink blocks and the window is mapped
                nsb = -(-min(sk, lo) // 4)
                ok &= bool(np.all(w.block_tables[s, nsb:lo // 4] == -1))
                for h in range(4):
                    g = ref.kv_head_of(h, 4, 2)
                    o, _ = ref.attend(ref.to_f64(w.q[s, h:h + 1], "f32"), k[pos - first, g].astype(np.float64),
                                      v[pos - first, g].astype(np.float64), w.scale)
                    ok &= np.max(np.abs(out[s, h] - o[0])) <= 1e-13
                    if sk >= lo:
                        ok &= np.max(np.abs(out[s, h] - full[s, h])) <= 1e-13
    p = wl.make_prefill(prefix_len=12, chunk_lens=[6, 9, 1], num_heads=4, num_kv_heads=2, head_dim=8,
                        block_size=4, dtype="f32", seed=42, window=4)
    kp, vp = ref.build_pools(p)
    for sk in (2, 5):
        out, lse = ref_prefill(p, kp, vp, sinks=sk)
        bo = brute.prefill(p.q, p.q_start, kp, vp, p.block_tables, p.context_lens, 4, 2, 4, p.scale, "f32",
                           sinks=sk)
        ok &= np.max(np.abs(out - np.array(bo))) <= 1e-12
        for s in range(p.num_seqs):
            r0, r1 = int(p.q_start[s]), int(p.q_start[s + 1])
            L = int(p.context_lens[s])
            C = r1 - r0
            first, k, v = p.logical_kv(s)
            pp = L - C + np.arange(C)[:, None]
            t = np.arange(L)[None, :]
            mask = torch.from_numpy((t <= pp) & ((pp - t < 4) | (t < sk)))
            q = torch.from_numpy(ref.to_f64(p.q[r0:r1], "f32")).permute(1, 0, 2)[None]
            K = torch.from_numpy(ref.to_f64(k, "f32")).permute(1, 0, 2)[None]
            V = torch.from_numpy(ref.to_f64(v, "f32")).permute(1, 0, 2)[None]
            lib = torch.nn.functional.scaled_dot_product_attention(q, K, V, attn_mask=mask, scale=p.scale,
                                                                   enable_gqa=True)
            ok &= np.max(np.abs(out[r0:r1] - lib[0].permute(1, 0, 2).numpy())) <= 1e-12
            for i in range(C):
                d, dl = ref.decode(p.q[r0 + i][None], kp, vp, p.block_tables[s:s + 1], np.array([L - C + i + 1]),
                                   block_size=4, num_kv_heads=2, window=4, scale=p.scale, dtype="f32", sinks=sk)
                ok &= np.max(np.abs(out[r0 + i] - d[0])) <= 1e-13
    return bool(ok)


PINS = [pin_brute_decode, pin_brute_prefill, pin_library_sdpa, pin_closed_forms,
        pin_permutation_invariance, pin_window, pin_prefill_rows_are_decodes, pin_shared_prefix,
        pin_gqa_equals_replicated_mha, pin_write_round_trip, pin_sinks]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    assert pin()


def test_empty_context_gives_zeros():
    w = small_decode(51, S=3, lens=[0, 5, 0])
    kp, vp = ref.build_pools(w)
    out, lse = ref_decode(w, kp, vp)
    assert np.array_equal(out[0], np.zeros_like(out[0])) and np.all(np.isneginf(lse[0]))
    assert np.array_equal(out[2], np.zeros_like(out[2])) and np.all(np.isneginf(lse[2]))
    assert np.all(np.isfinite(out[1]))
    bo, bl = brute.decode(w.q, kp, vp, w.block_tables, w.context_lens, 4, 2, 0, w.scale, "f32")
    assert bo[0][0] == [0.0] * 8 and bl[0][0] == -math.inf


def test_softmax_weights_sum_to_one_is_checked():
    # attend() refuses weights that do not sum to one; a NaN key trips it.
    q = np.ones((1, 4))
    k = np.array([[0.0, 0, 0, 0], [np.nan, 0, 0, 0]])
    with pytest.raises(AssertionError):
        ref.attend(q, k, np.ones((2, 4)), 1.0)


def test_tiny_config_layout():
    w = wl.config(1)
    assert w.context_lens.tolist() == [100]
    row = w.block_tables[0]
    assert (row >= 0).sum() == 7 and w.num_blocks == 16
    assert len(set(row.tolist())) == 7
    kp, vp = ref.build_pools(w)
    # the last block holds positions 96..99, slots 4..15 stay poisoned
    last = row[6]
    assert np.isfinite(kp[last, :4]).all() and np.isnan(kp[last, 4:]).all()
    out, _ = ref_decode(w, kp, vp)
    co, _ = contiguous(w, 0)
    assert np.max(np.abs(out[0] - co)) <= 1e-13


def test_bf16_decoding_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F], np.uint16)
    got = ref.to_f64(bits, "bf16")
    assert got[0] == 1.0 and got[1] == -1.0
    assert got[2] == 3.140625
    assert got[3] == 2.0 ** -133
    assert got[4] == (255 / 128) * 2.0 ** 127
    for b in bits:
        assert brute.value(b, "bf16") == ref.to_f64(np.array([b], np.uint16), "bf16")[0]


# ------------------------------------------------- planted mistakes (CPU)

def _mutants():
    orig_attend = ref.attend
    orig_range = ref.attended_range
    orig_keys = ref.prefill_keys

    def kv_head_mod(h, H, Hkv):
        return h % Hkv

    def range_off_by_one(L, window):
        lo, hi = orig_range(L, window)
        return (min(lo + 1, hi - 1) if window > 0 else lo), hi

    def attend_no_scale(q, k, v, scale):
        return orig_attend(q, k, v, 1.0)

    def attend_keys_as_values(q, k, v, scale):
        return orig_attend(q, k, k, scale)

    def gather_swapped(pool, table_row, positions, g, B, dtype):
        positions = np.asarray(positions, np.int64)
        pb = np.asarray(table_row, np.int64)[positions % B]
        return ref.to_f64(pool[pb, positions // B % B, g, :], dtype)

    def keys_strict(L, C, window):
        p = (L - C) + np.arange(C)[:, None]
        t = np.arange(L)[None, :]
        m = t < np.maximum(p, 1)
        if window > 0:
            m &= t > p - window
        return m

    def keys_window_inclusive(L, C, window):
        p = (L - C) + np.arange(C)[:, None]
        t = np.arange(L)[None, :]
        m = t <= p
        if window > 0:
            m &= t >= p - window
        return m

    orig_positions = ref.attended_positions

    def sinks_one_too_many(L, window, sinks=0):
        return orig_positions(L, window, sinks + 1 if sinks else 0)

    def write_off_by_block(k_pool, v_pool, k_new, v_new, seq_idx, pos, tables, B):
        return ref_kv_write(k_pool, v_pool, k_new, v_new, seq_idx, np.asarray(pos) + 1, tables, B)

    ref_kv_write = ref.kv_write
    return {
        "gqa_head_mapping_modulo": ("kv_head_of", kv_head_mod),
        "window_off_by_one": ("attended_range", range_off_by_one),
        "dropped_scale": ("attend", attend_no_scale),
        "keys_used_as_values": ("attend", attend_keys_as_values),
        "block_offset_swapped": ("gather", gather_swapped),
        "causal_excludes_self": ("prefill_keys", keys_strict),
        "window_one_too_wide": ("prefill_keys", keys_window_inclusive),
        "write_shifted": ("kv_write", write_off_by_block),
        "sinks_one_too_many": ("attended_positions", sinks_one_too_many),
    }


@pytest.mark.parametrize("name", sorted(_mutants().keys()))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = _mutants()[name]
    monkeypatch.setattr(ref, attr, fn)
    failed = []
    for pin in PINS:
        try:
            if not pin():
                failed.append(pin.__name__)
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {name}"


def test_copy_blocks_definition():
    """Copied blocks equal their sources byte for byte; every other block is
    untouched; invalid pairs are skipped."""
    rng = np.random.default_rng(3)
    k = rng.standard_normal((6, 4, 2, 8)).astype(np.float32)
    v = rng.standard_normal((6, 4, 2, 8)).astype(np.float32)
    ks = rng.standard_normal((6, 2, 4)).astype(np.float32)
    nk, nv, nks, _ = ref.copy_blocks(k, v, [1, 4, 9, 2], [3, 0, 2, 2], ks, ks.copy())
    assert nk[3].tobytes() == k[1].tobytes() and nv[0].tobytes() == v[4].tobytes()
    assert nks[3].tobytes() == ks[1].tobytes()
    for b in (1, 2, 4, 5):
        assert nk[b].tobytes() == k[b].tobytes() and nv[b].tobytes() == v[b].tobytes()
