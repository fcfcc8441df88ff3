"""Seeded generators: determinism, shapes and the structure of the five
workloads.  CPU only."""
import numpy as np

import workloads as wl


def test_same_seed_same_bytes():
    a = wl.config(1)
    b = wl.config(1)
    assert a.q.tobytes() == b.q.tobytes()
    assert a.block_tables.tobytes() == b.block_tables.tobytes()
    assert a.seq_kv[0].k.tobytes() == b.seq_kv[0].k.tobytes()
    c = wl.config(1, seed=101)
    assert a.q.tobytes() != c.q.tobytes()


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e38], np.float32)
    bits = wl.f32_to_bf16_bits(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: rounds to even (1.0)
    assert bits.tolist()[:2] == [0x3F80, 0x3F80]
    # 1 + 3*2^-8 is a tie between 1+2^-7 and 1+2^-6: rounds to even (1+2^-6)
    assert bits[2] == 0x3F82
    assert bits[3] == 0xC020


def test_config_structures():
    w2 = wl.config(2)
    assert w2.num_seqs == 32 and w2.dtype == "f16" and w2.block_size == 16
    assert (w2.context_lens >= 512).all() and (w2.context_lens <= 4096).all()
    ids = w2.block_tables[w2.block_tables >= 0]
    assert len(ids) == w2.num_blocks and len(np.unique(ids)) == len(ids)
    assert w2.max_blocks_per_seq == 256
    w4 = wl.config(4)
    assert w4.window == 4096
    for s in range(w4.num_seqs):
        L = int(w4.context_lens[s])
        row = w4.block_tables[s]
        first_live = (L - 4096) // 16
        assert (row[:first_live] == -1).all() and (row[first_live:(L + 15) // 16] >= 0).all()
    assert w4.kv_bytes_attended() == 268435456
    live = int((w4.block_tables >= 0).sum())
    assert w4.num_blocks == live + (live + 9) // 10


def test_prefill_config_shares_prefix():
    w = wl.config(5)
    assert w.kind == "prefill" and w.q.shape == (4096, 32, 128)
    assert (w.block_tables[:, :128] == w.block_tables[0, :128]).all()
    priv = w.block_tables[:, 128:160]
    assert len(np.unique(priv)) == 8 * 32 and not np.isin(priv, w.block_tables[0, :128]).any()
    assert w.num_blocks == 384 and w.context_lens.tolist() == [2560] * 8
    assert w.q_start.tolist() == list(range(0, 4097, 512))
