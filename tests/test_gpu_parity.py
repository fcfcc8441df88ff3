"""GPU parity of the HIP library against the fp64 oracle, through the C ABI.

Bars: the write and every table lookup bit-exact; attention outputs within
max-abs 2e-3 for 16-bit K/V and within 1e-5 relative (per output row, against
the row's largest magnitude) for fp32.  Unused pool slots are NaN everywhere.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle.ref as ref
import workloads as wl

pytestmark = pytest.mark.gpu

TOL_ABS_16 = 2e-3
TOL_REL_32 = 1e-5
# lse: decode sums the fp32 weights (1e-4 covers fp32 accumulation); prefill
# sums its weights as rounded to fp16 for the matrix cores, within 2^-11
# relative of the exact sum plus 2^-25 per subnormal weight against a sum of
# at least 1 (a few thousand keys): |error| <= 4.9e-4 + 0.8e-4 < 6e-4.
TOL_LSE = 1e-4
TOL_LSE_PREFILL = 6e-4


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_30_amd as pkv
    from paged_kv_cache_30_amd import session
    return pkv, session


def assert_close(got, want, dtype, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    if dtype == "f32":
        D = got.shape[-1]
        g2 = got.reshape(-1, D)
        w2 = want.reshape(-1, D)
        err = np.abs(g2 - w2).max(axis=1)
        bound = TOL_REL_32 * np.maximum(np.abs(w2).max(axis=1), 1e-30)
        bad = err > bound
        rel = float((err / bound).max()) * TOL_REL_32
        note(f"{what}: fp32 max row-relative err {rel:.3g}")
        assert not bad.any(), f"{what}: fp32 rel err {rel:.3g}"
    else:
        err = float(np.abs(got - want).max())
        note(f"{what}: max abs err {err:.3g}")
        assert err <= TOL_ABS_16, f"{what}: max abs err {err:.3g}"


def oracle_decode(w, kp, vp):
    return ref.decode(w.q, kp, vp, w.block_tables, w.context_lens, block_size=w.block_size,
                      num_kv_heads=w.num_kv_heads, window=w.window, scale=w.scale, dtype=w.dtype)


def oracle_prefill(w, kp, vp):
    return ref.prefill(w.q, w.q_start, kp, vp, w.block_tables, w.context_lens, block_size=w.block_size,
                       num_kv_heads=w.num_kv_heads, window=w.window, scale=w.scale, dtype=w.dtype)


def run(session, w, **kw):
    d = session.DeviceWorkload(w, **kw)
    d.step()
    torch.cuda.synchronize()
    return d


def check_lse(d, want_lse, tol=TOL_LSE):
    got = d.lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(want_lse)
    assert np.array_equal(fin, np.isfinite(got))
    assert np.all(np.isneginf(got[~fin]))
    err = np.abs(got[fin] - want_lse[fin]).max(initial=0)
    note(f"lse max abs err {err:.3g}")
    assert err <= tol


# ------------------------------------------------------------------ write

def pools_bit_exact(session, d, kp, vp, what):
    """Both device pools equal the oracle's pools bit for bit (NaN poison in
    unwritten slots included: compared as raw storage words)."""
    for got, want, name in ((session.from_device(d.k_pool), kp, "K"), (session.from_device(d.v_pool), vp, "V")):
        assert got.shape == want.shape, f"{what}: {name} pool shape"
        gw = got.view(np.uint8).reshape(-1)
        ww = want.view(np.uint8).reshape(-1)
        assert np.array_equal(gw, ww), f"{what}: {name} pool differs at byte {int(np.flatnonzero(gw != ww)[0])}"


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_write_bit_exact_configs(lib, cfg):
    pkv, session = lib
    note(f"write cfg{cfg}")
    w = wl.config(cfg)
    d = run(session, w)
    kp, vp = ref.build_pools(w, poison=True)
    pools_bit_exact(session, d, kp, vp, f"cfg{cfg}")


def test_write_skips_invalid_tokens(lib):
    pkv, session = lib
    note("write invalid tokens")
    B, Hkv, D = 16, 2, 64
    kp = torch.full((4, B, Hkv, D), float("nan"), dtype=torch.float16, device="cuda")
    vp = kp.clone()
    tables = torch.tensor([[2, -1], [7, 1]], dtype=torch.int32, device="cuda")  # 7 is out of range
    kn = torch.ones((5, Hkv, D), dtype=torch.float16, device="cuda")
    seq = torch.tensor([0, 0, 1, 1, 5], dtype=torch.int32, device="cuda")
    pos = torch.tensor([3, 20, 0, 17, 0], dtype=torch.int32, device="cuda")
    pkv.paged_kv_write(kp, vp, kn, kn, seq, pos, tables)
    torch.cuda.synchronize()
    k = kp.float().cpu().numpy()
    written = ~np.isnan(k[:, :, 0, 0])
    assert written.sum() == 2 and written[2, 3] and written[1, 1]


# ----------------------------------------------------------------- decode

DECODE_CASES = [
    # (dtype, H, Hkv, D, B, lens, window, workers)
    ("f32", 4, 4, 64, 16, [100, 1, 33, 0], 0, 0),
    ("f32", 8, 2, 128, 32, [77, 300, 5], 0, 7),
    ("f16", 8, 8, 128, 16, [1, 17, 250, 513, 0], 0, 0),
    ("f16", 8, 8, 128, 16, [1, 17, 250, 513, 1000], 0, 33),
    ("bf16", 16, 4, 128, 32, [31, 32, 33, 640, 2000], 0, 0),
    ("bf16", 16, 4, 128, 32, [31, 32, 33, 640, 2000], 0, 2),
    ("bf16", 8, 1, 64, 16, [5, 64, 700], 0, 48),
    ("f16", 4, 2, 64, 32, [3, 90, 129], 0, 0),
    ("bf16", 16, 2, 128, 16, [40, 600, 1500], 100, 0),
    ("bf16", 16, 2, 128, 16, [40, 600, 1500], 100, 1),
    ("f16", 8, 8, 128, 32, [1, 2, 500], 1, 0),
    ("f32", 4, 2, 64, 16, [10, 70], 16, 3),
    ("bf16", 32, 8, 128, 16, [0, 0, 2000, 0, 4100, 1], 0, 0),
    ("f16", 64, 8, 128, 16, [300, 20000, 7], 0, 0),
    # 4 or more query heads per kv head run on the matrix cores
    ("bf16", 64, 8, 128, 32, [1, 15, 16, 17, 33, 1000, 5000], 0, 0),
    ("bf16", 64, 8, 128, 32, [1, 15, 16, 17, 33, 1000, 5000], 0, 9),
    ("f16", 32, 4, 128, 16, [20, 700, 2100], 300, 0),
    ("bf16", 16, 2, 64, 32, [40, 600, 1500], 0, 0),
    ("f16", 16, 4, 64, 32, [3, 50, 900, 31], 64, 5),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[f"{c[0]}-g{c[1] // c[2]}-d{c[3]}-b{c[4]}-w{c[6]}-p{c[7]}"
                                                    for c in DECODE_CASES])
def test_decode_small(lib, case):
    pkv, session = lib
    dtype, H, Hkv, D, B, lens, window, part = case
    note(f"decode small {case}")
    w = wl.make_decode(lens=lens, num_heads=H, num_kv_heads=Hkv, head_dim=D, block_size=B, dtype=dtype,
                       seed=sum(lens) + H, window=window, k_scale=3.0 if dtype == "bf16" else 1.0,
                       spare_blocks=3)
    d = run(session, w, num_workers=part)
    kp, vp = ref.build_pools(w)
    out, lse = oracle_decode(w, kp, vp)
    assert_close(d.out.cpu().numpy(), out, dtype, str(case))
    check_lse(d, lse)


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_decode_config_full(lib, cfg):
    pkv, session = lib
    note(f"decode cfg{cfg} full")
    w = wl.config(cfg)
    d = run(session, w)
    kp, vp = ref.build_pools(w)
    out, lse = oracle_decode(w, kp, vp)
    assert_close(d.out.cpu().numpy(), out, w.dtype, f"cfg{cfg}")
    check_lse(d, lse)


@pytest.mark.parametrize("cfg", [3, 7])
def test_decode_long_configs_full(lib, cfg):
    """Long-context GQA at full size (4 query heads per kv head, and the
    8-head variant whose scores run on the matrix cores): every sequence and
    head against the paged fp64 oracle, output and lse; the shortest and the
    longest sequence also against the contiguous (never paged) oracle."""
    pkv, session = lib
    note(f"decode cfg{cfg} full")
    w = wl.config(cfg)
    d = run(session, w)
    got = d.out.cpu().numpy()
    kp, vp = ref.build_pools(w)
    out, lse = oracle_decode(w, kp, vp)
    del kp, vp
    assert_close(got, out, "bf16", f"cfg{cfg} all sequences")
    check_lse(d, lse)
    order = np.argsort(w.context_lens)
    for s in (int(order[0]), int(order[-1])):
        first, k, v = w.logical_kv(s)
        o, _ = ref.contiguous_decode(w.q[s], k, v, first, int(w.context_lens[s]), num_kv_heads=w.num_kv_heads,
                                     window=0, scale=w.scale, dtype="bf16")
        assert_close(got[s], o, "bf16", f"cfg{cfg} seq {s} vs contiguous")


def test_decode_config4_contiguous(lib):
    pkv, session = lib
    note("decode cfg4 vs contiguous")
    w = wl.config(4)
    d = run(session, w)
    got = d.out.cpu().numpy()
    for s in range(w.num_seqs):
        first, k, v = w.logical_kv(s)
        o, _ = ref.contiguous_decode(w.q[s], k, v, first, int(w.context_lens[s]), num_kv_heads=8,
                                     window=w.window, scale=w.scale, dtype="bf16")
        assert_close(got[s], o, "bf16", f"cfg4 seq {s}")


def test_decode_permutation_bitwise(lib):
    pkv, session = lib
    note("decode permutation invariance")
    base = wl.make_decode(lens=[50, 300, 1200, 7], num_heads=16, num_kv_heads=4, head_dim=128, block_size=16,
                          dtype="bf16", seed=5, spare_blocks=5)
    outs = []
    for ps in (0, 1, 2):
        w = wl.repermute(base, ps)
        d = run(session, w, num_workers=16)
        outs.append(d.out.cpu().numpy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_decode_split_count_independent(lib):
    pkv, session = lib
    note("decode split count")
    w = wl.make_decode(lens=[900, 2047, 4000], num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                       dtype="bf16", seed=8, k_scale=3.0)
    res = []
    for part in (16, 64, 256, 4096):
        d = run(session, w, num_workers=part)
        res.append(d.out.cpu().numpy())
    for r in res[1:]:
        assert np.abs(r - res[0]).max() <= 1e-5


def test_decode_gqa_equals_replicated_mha(lib):
    pkv, session = lib
    note("decode gqa vs replicated")
    w = wl.make_decode(lens=[70, 513, 1024], num_heads=16, num_kv_heads=4, head_dim=128, block_size=32,
                       dtype="bf16", seed=9)
    G = 4
    d = run(session, w, num_workers=16)
    m = wl.make_decode(lens=[70, 513, 1024], num_heads=16, num_kv_heads=16, head_dim=128, block_size=32,
                       dtype="bf16", seed=9)
    for s in range(3):
        m.seq_kv[s].k = np.repeat(w.seq_kv[s].k, G, axis=1)
        m.seq_kv[s].v = np.repeat(w.seq_kv[s].v, G, axis=1)
    m.q = w.q.copy()
    dm = run(session, m, num_workers=16)
    # Same arithmetic per head; the group kernel may process a partition in
    # smaller chunks (less register state per query), so only the fp32
    # rounding of the online softmax may differ.
    assert np.abs(d.out.cpu().numpy() - dm.out.cpu().numpy()).max() <= 1e-5


def test_decode_unit_cases(lib):
    """L = 1 gives the stored value exactly; constant values give the
    constant; w = 1 gives the query position's own value."""
    pkv, session = lib
    note("decode unit cases")
    w = wl.make_decode(lens=[1, 1, 300], num_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                       dtype="bf16", seed=11, window=0)
    d = run(session, w)
    got = d.out.cpu().numpy()
    for s in range(2):
        for h in range(8):
            assert np.array_equal(got[s, h], ref.to_f64(w.seq_kv[s].v[0, h // 4], "bf16"))
    w1 = wl.make_decode(lens=[9, 300, 1000], num_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                        dtype="bf16", seed=12, window=1)
    d1 = run(session, w1)
    got = d1.out.cpu().numpy()
    for s in range(3):
        for h in range(8):
            assert np.array_equal(got[s, h], ref.to_f64(w1.seq_kv[s].v[-1, h // 4], "bf16"))
    wc = wl.make_decode(lens=[20, 700], num_heads=4, num_kv_heads=4, head_dim=64, block_size=16,
                        dtype="f16", seed=13)
    for e in wc.seq_kv:
        e.v[:] = np.float16(0.75)
    dc = run(session, wc, num_workers=5)
    assert np.abs(dc.out.cpu().numpy() - 0.75).max() <= 1e-6


# ---------------------------------------------------------------- prefill

PREFILL_CASES = [
    # (dtype, H, Hkv, D, B, prefix, chunks, window, share)
    ("bf16", 8, 2, 128, 16, 64, [40, 1, 100], 0, True),
    ("bf16", 4, 4, 128, 32, 0, [70, 33], 0, False),
    ("f16", 8, 1, 128, 16, 32, [130], 0, True),
    ("bf16", 16, 2, 64, 16, 48, [64, 17], 0, True),
    ("bf16", 8, 2, 128, 16, 160, [90, 31], 50, True),
    ("f16", 16, 2, 128, 32, 96, [200, 5], 0, False),
    # two query heads per kv head; head dim 64 with 32-slot blocks (one table
    # entry per wavefront load); 1 to 4 key tiles per workgroup with a window
    ("f16", 8, 4, 64, 32, 64, [33, 64], 0, True),
    ("bf16", 6, 3, 64, 16, 0, [10, 130, 190], 100, False),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[f"{c[0]}-g{c[1] // c[2]}-d{c[3]}-b{c[4]}-P{c[5]}-w{c[7]}"
                                                      for c in PREFILL_CASES])
def test_prefill_small(lib, case):
    pkv, session = lib
    dtype, H, Hkv, D, B, prefix, chunks, window, share = case
    note(f"prefill small {case}")
    w = wl.make_prefill(prefix_len=prefix, chunk_lens=chunks, num_heads=H, num_kv_heads=Hkv, head_dim=D,
                        block_size=B, dtype=dtype, seed=prefix + sum(chunks), window=window, share_prefix=share)
    d = run(session, w)
    kp, vp = ref.build_pools(w)
    out, lse = oracle_prefill(w, kp, vp)
    assert_close(d.out.cpu().numpy(), out, dtype, str(case))
    check_lse(d, lse, TOL_LSE_PREFILL)


def test_prefill_config5(lib):
    """The chunked prefill over a shared prefix at full size: all 4096 rows
    and 32 heads against the fp64 oracle, output and lse."""
    pkv, session = lib
    note("prefill cfg5 full")
    w = wl.config(5)
    d = run(session, w)
    kp, vp = ref.build_pools(w)
    got = d.out.cpu().numpy()
    out, lse = oracle_prefill(w, kp, vp)
    assert_close(got, out, "bf16", "cfg5 all rows and heads")
    check_lse(d, lse, TOL_LSE_PREFILL)


def _plant_v(w, value, seed):
    """Set a few attended V rows of prefill workload w (prefix and chunks)
    to +-value, in the storage type."""
    rng = np.random.default_rng(seed)
    D = w.head_dim
    for arr in [w.prefix.v] + [e.v for e in w.seq_kv]:
        if arr.shape[0] == 0:
            continue
        for _ in range(3):
            t, g = int(rng.integers(arr.shape[0])), int(rng.integers(arr.shape[1]))
            row = np.where(rng.random(D) < 0.5, -value, value).astype(np.float32)
            arr[t, g] = wl.to_storage(row, w.dtype)


def test_prefill_bf16_v_at_fp16_limit(lib, monkeypatch):
    """bf16 prefill multiplies fp16 weights with V converted to fp16, which
    is exact for |v| <= 65280 (the largest bf16 value fp16 holds). V rows at
    +-65280 among N(0,1) rows: parity with the oracle, and the chunk's last
    rows equal decode over the same pages. The bound scales with the values
    averaged: an output is a weighted average of V rows, so its rounding
    error is relative to them (2e-3 of the largest attended |v|, the
    16-bit bar at unit scale). Debug mode accepts these pages."""
    pkv, session = lib
    note("prefill bf16 V at the fp16 limit")
    monkeypatch.setenv("PKV_DEBUG", "1")
    w = wl.make_prefill(prefix_len=64, chunk_lens=[50, 17, 1], num_heads=8, num_kv_heads=2, head_dim=128,
                        block_size=16, dtype="bf16", seed=23)
    _plant_v(w, 65280.0, 23)
    d = run(session, w)
    kp, vp = ref.build_pools(w)
    out, lse = oracle_prefill(w, kp, vp)
    got = d.out.cpu().numpy()
    err = float(np.abs(got - out).max())
    tol = TOL_ABS_16 * 65280.0
    note(f"max abs err {err:.4g} (bound {tol:.4g}, relative {err / 65280.0:.3g})")
    assert np.isfinite(got).all() and err <= tol
    check_lse(d, lse, TOL_LSE_PREFILL)
    for s in range(w.num_seqs):
        i = int(w.q_start[s + 1]) - 1
        L = int(w.context_lens[s])
        qd = d.q[i:i + 1].contiguous()
        outd = torch.empty((1, 8, 128), dtype=torch.float32, device="cuda")
        lens = torch.tensor([L], dtype=torch.int32, device="cuda")
        tab = d.tables[s:s + 1].contiguous()
        ws = pkv.decode_workspace(d.k_pool, 8, 1, L)
        pkv.paged_attn_decode(outd, qd, d.k_pool, d.v_pool, tab, lens, L, scale=w.scale, workspace=ws)
        torch.cuda.synchronize()
        assert np.abs(outd.cpu().numpy()[0] - got[i]).max() <= tol


def test_prefill_bf16_v_beyond_limit_rejected(lib):
    """One attended bf16 V row at 65536 (the next bf16 value, outside fp16's
    range): debug mode rejects the prefill and the mixed call before
    anything is launched, naming the sequence."""
    pkv, session = lib
    note("prefill bf16 V beyond the fp16 limit")
    w = wl.make_prefill(prefix_len=32, chunk_lens=[20, 9], num_heads=4, num_kv_heads=2, head_dim=64,
                        block_size=16, dtype="bf16", seed=29)
    w.seq_kv[1].v[4, 1, 7] = wl.to_storage(np.array([65536.0], np.float32), "bf16")[0]
    d = run(session, w)
    out = torch.full_like(d.out, 7.0)
    kw = dict(window=0, scale=w.scale, debug=True)
    with pytest.raises(pkv.InvalidContent, match="sequence 1"):
        pkv.paged_attn_prefill(out, d.q, d.q_start, d.k_pool, d.v_pool, d.tables, d.lens, w.max_q_len,
                               w.max_context_len, **kw)
    ws = pkv.decode_workspace(d.k_pool, 4, w.num_seqs, w.max_context_len)
    with pytest.raises(pkv.InvalidContent, match="sequence 1"):
        pkv.paged_attn_mixed(out, d.q, d.q_start, d.k_pool, d.v_pool, d.tables, d.lens, w.max_q_len,
                             w.max_context_len, workspace=ws, **kw)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


def test_prefill_shared_prefix_bitwise(lib):
    pkv, session = lib
    note("prefill shared vs private prefix")
    w = wl.make_prefill(prefix_len=256, chunk_lens=[100, 64, 3], num_heads=8, num_kv_heads=2, head_dim=128,
                        block_size=16, dtype="bf16", seed=17)
    p = wl.private_prefix_copy(w)
    a = run(session, w).out.cpu().numpy()
    b = run(session, p).out.cpu().numpy()
    assert np.array_equal(a, b)


def test_prefill_rows_match_decode(lib):
    pkv, session = lib
    note("prefill rows vs decode")
    w = wl.make_prefill(prefix_len=128, chunk_lens=[37], num_heads=8, num_kv_heads=2, head_dim=128,
                        block_size=16, dtype="bf16", seed=19)
    d = run(session, w)
    got = d.out.cpu().numpy()
    L = int(w.context_lens[0])
    C = 37
    for i in (0, 5, 36):
        qd = torch.from_numpy(w.q[i:i + 1].view(np.int16)).view(torch.bfloat16).cuda()
        outd = torch.empty((1, 8, 128), dtype=torch.float32, device="cuda")
        lens = torch.tensor([L - C + i + 1], dtype=torch.int32, device="cuda")
        ws = pkv.decode_workspace(d.k_pool, 8, 1, L)
        pkv.paged_attn_decode(outd, qd, d.k_pool, d.v_pool, d.tables, lens, L, scale=w.scale, workspace=ws)
        torch.cuda.synchronize()
        assert np.abs(outd.cpu().numpy()[0] - got[i]).max() <= TOL_ABS_16


# ------------------------------------------------------------- ABI errors

def test_abi_errors_on_device(lib):
    pkv, session = lib
    note("abi errors")
    w = wl.make_decode(lens=[100, 40], num_heads=8, num_kv_heads=2, head_dim=128, block_size=16, dtype="bf16",
                       seed=1)
    d = session.DeviceWorkload(w, num_workers=16)
    with pytest.raises(pkv.PagedAttnError) as e:
        pkv.paged_attn_decode(d.out, d.q, d.k_pool, d.v_pool, d.tables, d.lens, 100, scale=0.1,
                              num_workers=16, workspace=None)
    assert e.value.status == pkv.PKV_EWORKSPACE
    small = d.workspace[:-16]
    with pytest.raises(pkv.PagedAttnError) as e:
        pkv.paged_attn_decode(d.out, d.q, d.k_pool, d.v_pool, d.tables, d.lens, 100, scale=0.1,
                              num_workers=16, workspace=small)
    assert e.value.status == pkv.PKV_EWORKSPACE
    with pytest.raises(pkv.PagedAttnError) as e:
        pkv.paged_attn_decode(d.out, d.q, d.k_pool, d.v_pool, d.tables, d.lens, 10 ** 6, scale=0.1)
    assert e.value.status == pkv.PKV_EINVAL
    with pytest.raises(ValueError):
        pkv.paged_attn_decode(d.out, d.q.float(), d.k_pool, d.v_pool, d.tables, d.lens, 100, scale=0.1)


def test_debug_mode_checks_device_content(lib):
    """debug=True gives the same result as a plain call on valid input, and
    rejects bad device-resident indices before anything is launched (the
    output and the pools keep their bytes)."""
    pkv, session = lib
    note("debug mode")
    w = wl.make_decode(lens=[700, 33, 1], num_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                       dtype="bf16", seed=21, window=100, sinks=4)
    d = run(session, w, num_workers=24)
    kw = dict(window=w.window, sinks=w.sinks, scale=w.scale, num_workers=24, workspace=d.workspace)
    out = torch.full_like(d.out, 7.0)
    pkv.paged_attn_decode(out, d.q, d.k_pool, d.v_pool, d.tables, d.lens, w.max_context_len, debug=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, d.out)
    bad = d.lens.clone()
    bad[1] = w.max_context_len + 1
    out.fill_(7.0)
    with pytest.raises(pkv.InvalidContent, match=r"context_lens\[1\]"):
        pkv.paged_attn_decode(out, d.q, d.k_pool, d.v_pool, d.tables, bad, w.max_context_len, debug=True, **kw)
    tab = d.tables.clone()
    tab[0, 0] = -1  # a sink block
    with pytest.raises(pkv.InvalidContent, match="logical block 0"):
        pkv.paged_attn_decode(out, d.q, d.k_pool, d.v_pool, tab, d.lens, w.max_context_len, debug=True, **kw)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())

    kp = d.k_pool.clone()
    seq = torch.tensor([0, 0], dtype=torch.int32, device="cuda")
    pos = torch.tensor([699, 699], dtype=torch.int32, device="cuda")
    kn = torch.zeros((2, 2, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pkv.InvalidContent, match="same slot"):
        pkv.paged_kv_write(kp, kp, kn, kn, seq, pos, d.tables, debug=True)
    torch.cuda.synchronize()
    assert torch.equal(kp.view(torch.int16), d.k_pool.view(torch.int16))

    wp = wl.make_prefill(prefix_len=64, chunk_lens=[40, 7], num_heads=8, num_kv_heads=2, head_dim=128,
                         block_size=16, dtype="bf16", seed=22)
    dp = run(session, wp)
    outp = torch.full_like(dp.out, 7.0)
    pkv.paged_attn_prefill(outp, dp.q, dp.q_start, dp.k_pool, dp.v_pool, dp.tables, dp.lens, wp.max_q_len,
                           wp.max_context_len, scale=wp.scale, debug=True)
    torch.cuda.synchronize()
    assert torch.equal(outp, dp.out)
    qs = dp.q_start.clone()
    qs[2] += 1  # one row past the output
    outp.fill_(7.0)
    with pytest.raises(pkv.InvalidContent, match="q_start"):
        pkv.paged_attn_prefill(outp, dp.q, qs, dp.k_pool, dp.v_pool, dp.tables, dp.lens, wp.max_q_len + 1,
                               wp.max_context_len, scale=wp.scale, debug=True)
    torch.cuda.synchronize()
    assert bool((outp == 7.0).all())


# ------------------------------------------------------------ HIP graphs

@pytest.mark.parametrize("kind", ["decode", "prefill", "decode-i8", "prefill-fp8"])
def test_graph_replay_matches_eager(lib, kind):
    """The step's calls captured in a HIP graph: every replay, with eager work
    and synchronisations between replays, gives the eager result bit for bit
    (16-bit pages, and 8-bit pages with their write and prefill)."""
    pkv, session = lib
    note(f"graph replay {kind}")
    kind, _, fmt = kind.partition("-")
    if kind == "decode":
        w = wl.make_decode(lens=[33, 700, 1500, 4], num_heads=16, num_kv_heads=4, head_dim=128, block_size=16,
                           dtype="bf16", seed=23)
    else:
        w = wl.make_prefill(prefix_len=64, chunk_lens=[50, 20], num_heads=8, num_kv_heads=2, head_dim=128,
                            block_size=16, dtype="bf16", seed=24)
    d = session.DeviceWorkload(w, kv_format=fmt or "native")
    d.step()
    torch.cuda.synchronize()
    eager = d.out.clone()
    eager_lse = d.lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d.step()
    torch.cuda.synchronize()
    for i in range(4):
        d.out.zero_()
        d.lse.fill_(1.0)
        junk = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d.out, eager), f"replay {i} differs"
        assert torch.equal(d.lse, eager_lse), f"replay {i} lse differs"
        del junk


# ------------------------------------------------------- attention sinks

SINK_CASES = [
    # (dtype, H, Hkv, D, B, lens, window, sinks, workers)
    ("bf16", 16, 4, 128, 16, [40, 600, 1500, 3], 100, 4, 0),
    ("f16", 8, 8, 128, 32, [70, 1000, 333], 64, 4, 7),
    ("bf16", 8, 1, 64, 16, [5, 64, 700], 30, 20, 3),
    ("f32", 4, 2, 64, 16, [10, 170, 90], 16, 40, 0),
    ("bf16", 32, 8, 128, 16, [2000, 4100, 1], 256, 1, 48),
    ("bf16", 64, 8, 128, 32, [2000, 4100, 1], 256, 4, 0),
]


def poison_freed_middle(w):
    """Point the freed table entries between the sink blocks and the window
    at a spare (never written, NaN) block: reading them would show."""
    used = set(w.block_tables[w.block_tables >= 0].tolist())
    spare = next(i for i in range(w.num_blocks) if i not in used)
    t = w.block_tables.copy()
    for s in range(w.num_seqs):
        L = int(w.context_lens[s])
        lo = max(0, L - w.window)
        sb = min(-(-min(w.sinks, lo) // w.block_size), lo // w.block_size)
        t[s, sb:lo // w.block_size] = spare
    w.block_tables = t


@pytest.mark.parametrize("case", SINK_CASES, ids=[f"{c[0]}-g{c[1] // c[2]}-d{c[3]}-b{c[4]}-w{c[6]}-s{c[7]}-p{c[8]}"
                                                  for c in SINK_CASES])
def test_decode_sinks(lib, case):
    pkv, session = lib
    dtype, H, Hkv, D, B, lens, window, sinks, workers = case
    note(f"decode sinks {case}")
    w = wl.make_decode(lens=lens, num_heads=H, num_kv_heads=Hkv, head_dim=D, block_size=B, dtype=dtype,
                       seed=sum(lens) + sinks, window=window, sinks=sinks, spare_blocks=1)
    poison_freed_middle(w)
    d = run(session, w, num_workers=workers)
    kp, vp = ref.build_pools(w)
    out, lse = ref.decode(w.q, kp, vp, w.block_tables, w.context_lens, block_size=B, num_kv_heads=Hkv,
                          window=window, scale=w.scale, dtype=dtype, sinks=sinks)
    assert_close(d.out.cpu().numpy(), out, dtype, str(case))
    check_lse(d, lse)


@pytest.mark.parametrize("fmt", ["i8", "fp8"])
def test_decode_sinks_8bit(lib, fmt):
    pkv, session = lib
    import oracle.quant as oq
    note(f"decode sinks 8-bit {fmt}")
    w = wl.make_decode(lens=[40, 600, 1500, 3], num_heads=16, num_kv_heads=4, head_dim=128, block_size=16,
                       dtype="bf16", seed=77, window=100, sinks=4, spare_blocks=1)
    poison_freed_middle(w)
    d = session.DeviceWorkload(w, kv_format=fmt)
    d.step()
    torch.cuda.synchronize()
    kp, vp = ref.build_pools(w)
    kc, vc, ks, vs = oq.quantize_pools(kp, vp, "bf16", fmt)
    kd, vd = oq.dequantize_pool(kc, ks, fmt), oq.dequantize_pool(vc, vs, fmt)
    out, _ = ref.decode(w.q, kd, vd, w.block_tables, w.context_lens, block_size=16, num_kv_heads=4, window=100,
                        scale=w.scale, dtype="bf16", kv_dtype="f64", sinks=4)
    assert_close(d.out.cpu().numpy(), out, "bf16", f"sinks {fmt}")


def test_decode_sinks_long_window(lib):
    """Sliding-window sizes (contexts 16K-32K, window 4096) with 4 sinks,
    against the contiguous oracle over the sink and window positions."""
    pkv, session = lib
    note("decode sinks long window")
    w = wl.make_decode(lens=[16384, 20001, 32768, 24577], num_heads=32, num_kv_heads=8, head_dim=128,
                       block_size=16, dtype="bf16", seed=78, window=4096, sinks=4, spare_blocks=1)
    poison_freed_middle(w)
    d = run(session, w)
    got = d.out.cpu().numpy()
    for s in range(w.num_seqs):
        first, k, v = w.logical_kv(s)
        o, _ = ref.contiguous_decode(w.q[s], k, v, first, int(w.context_lens[s]), num_kv_heads=8, window=4096,
                                     scale=w.scale, dtype="bf16", sinks=4)
        assert_close(got[s], o, "bf16", f"sinks long seq {s}")


PREFILL_SINK_CASES = [
    # (dtype, H, Hkv, D, B, prefix, chunks, window, sinks)
    ("bf16", 8, 2, 128, 16, 160, [90, 31], 50, 4),
    ("f16", 16, 2, 128, 32, 96, [200, 5], 64, 70),
    ("bf16", 4, 4, 64, 16, 64, [130, 64], 17, 1),
]


@pytest.mark.parametrize("case", PREFILL_SINK_CASES,
                         ids=[f"{c[0]}-g{c[1] // c[2]}-d{c[3]}-w{c[7]}-s{c[8]}" for c in PREFILL_SINK_CASES])
def test_prefill_sinks(lib, case):
    pkv, session = lib
    dtype, H, Hkv, D, B, prefix, chunks, window, sinks = case
    note(f"prefill sinks {case}")
    w = wl.make_prefill(prefix_len=prefix, chunk_lens=chunks, num_heads=H, num_kv_heads=Hkv, head_dim=D,
                        block_size=B, dtype=dtype, seed=prefix + sinks, window=window, sinks=sinks)
    d = run(session, w)
    kp, vp = ref.build_pools(w)
    out, lse = ref.prefill(w.q, w.q_start, kp, vp, w.block_tables, w.context_lens, block_size=B,
                           num_kv_heads=Hkv, window=window, scale=w.scale, dtype=dtype, sinks=sinks)
    assert_close(d.out.cpu().numpy(), out, dtype, str(case))
    check_lse(d, lse, TOL_LSE_PREFILL)


# ----------------------------------------------------- batch and length limits

def test_decode_many_sequences_plan_launch(lib):
    """More than 4096 sequences: the prefix of attended blocks comes from the
    separate one-workgroup launch. Ragged short contexts (0..40, some empty);
    the first, the last, the empty and 60 random sequences against the oracle."""
    pkv, session = lib
    note("decode 5000 sequences")
    rng = np.random.default_rng(50)
    lens = rng.integers(0, 41, 5000)
    lens[::97] = 0
    w = wl.make_decode(lens=lens, num_heads=8, num_kv_heads=2, head_dim=64, block_size=16, dtype="bf16", seed=50)
    d = run(session, w)
    kp, vp = ref.build_pools(w)
    empty = [int(i) for i in np.where(lens == 0)[0][:3]]
    pick = sorted(set([0, 1, 4998, 4999] + empty + [int(i) for i in rng.choice(5000, 60, replace=False)]))
    out, lse = ref.decode(w.q, kp, vp, w.block_tables, w.context_lens, block_size=16, num_kv_heads=2, window=0,
                          scale=w.scale, dtype="bf16", seqs=pick)
    assert_close(d.out.cpu().numpy()[pick], out[pick], "bf16", "5000 sequences")
    got_lse = d.lse.cpu().numpy()[pick]
    fin = np.isfinite(lse[pick])
    assert np.array_equal(fin, np.isfinite(got_lse))
    assert np.abs(got_lse[fin] - lse[pick][fin]).max() <= 1e-4


def test_decode_128k_context(lib):
    """One 131072-token context next to a 5-token one (GQA, logits std ~3):
    the long sequence is split over every wavefront; against attention over
    its logical rows."""
    pkv, session = lib
    note("decode 128K context")
    w = wl.make_decode(lens=[131072, 5], num_heads=8, num_kv_heads=2, head_dim=128, block_size=32, dtype="bf16",
                       seed=51, k_scale=3.0)
    d = run(session, w)
    got = d.out.cpu().numpy()
    for s in range(2):
        first, k, v = w.logical_kv(s)
        L = int(w.context_lens[s])
        qf = ref.to_f64(w.q[s], "bf16")
        want = np.zeros((8, 128))
        for g in range(2):
            K = ref.to_f64(k[:L - first, g], "bf16")
            V = ref.to_f64(v[:L - first, g], "bf16")
            o, _ = ref.attend(qf[4 * g:4 * g + 4], K, V, w.scale)
            want[4 * g:4 * g + 4] = o
        assert_close(got[s], want, "bf16", f"128K context seq {s} (L={L})")


# ------------------------------------------------- robustness re-run seeds

@pytest.mark.parametrize("seed", [101, 102, 103, 104, 105])
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_configs_robustness_seeds(lib, cfg, seed):
    """The five workloads redrawn with seeds 101..105 (lengths, K/V, Q and
    the physical-id permutation all change): both pools bit-exact after the
    step's write, and every output row and head (and lse) against the fp64
    oracle; the shortest and longest decode sequences also against the
    contiguous cache."""
    pkv, session = lib
    note(f"cfg{cfg} seed {seed}")
    w = wl.config(cfg, seed=seed)
    d = run(session, w)
    got = d.out.cpu().numpy()
    kp, vp = ref.build_pools(w, poison=True)
    pools_bit_exact(session, d, kp, vp, f"cfg{cfg} seed {seed}")
    del kp, vp
    kp, vp = ref.build_pools(w)
    if w.kind == "decode":
        out, lse = oracle_decode(w, kp, vp)
        assert_close(got, out, w.dtype, f"cfg{cfg} seed {seed}")
        check_lse(d, lse)
        order = np.argsort(w.context_lens)
        for s in sorted({int(order[0]), int(order[-1])}):
            first, k, v = w.logical_kv(s)
            o, _ = ref.contiguous_decode(w.q[s], k, v, first, int(w.context_lens[s]), num_kv_heads=w.num_kv_heads,
                                         window=w.window, scale=w.scale, dtype=w.dtype)
            assert_close(got[s], o, w.dtype, f"cfg{cfg} seed {seed} seq {s} vs contiguous")
    else:
        out, lse = oracle_prefill(w, kp, vp)
        assert_close(got, out, w.dtype, f"cfg{cfg} seed {seed}")
        check_lse(d, lse, TOL_LSE_PREFILL)


# ------------------------------------------------------ pools beyond 4 GiB

def test_decode_pool_beyond_4gib(lib):
    """Pools of 12.2 GiB each (400k blocks of 32 KB): the sequences' blocks
    are scattered over the whole pool, most of them at byte offsets above
    2^32, so every address computation of the write and of decode needs 64
    bits. Checked against attention over each sequence's logical rows (no
    host copy of the pool)."""
    pkv, session = lib
    note("decode, pools beyond 4 GiB")
    w = wl.make_decode(lens=[5000, 333, 17, 2048], num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                       dtype="bf16", seed=61, k_scale=3.0, spare_blocks=400000)
    blk_bytes = 16 * 8 * 128 * 2
    assert w.num_blocks * blk_bytes > 12 * 2 ** 30
    mapped = w.block_tables[w.block_tables >= 0]
    assert (mapped.astype(np.int64) * blk_bytes >= 2 ** 32).mean() > 0.5
    d = run(session, w)
    got = d.out.cpu().numpy()
    got_lse = d.lse.cpu().numpy()
    for s in range(w.num_seqs):
        first, k, v = w.logical_kv(s)
        o, l = ref.contiguous_decode(w.q[s], k, v, first, int(w.context_lens[s]), num_kv_heads=8, window=0,
                                     scale=w.scale, dtype="bf16")
        assert_close(got[s], o, "bf16", f"4GiB+ pool seq {s}")
        assert np.abs(got_lse[s] - l).max() <= TOL_LSE
    del d
    torch.cuda.empty_cache()


def test_prefill_pool_beyond_4gib(lib):
    """Chunked prefill over pools of 12.2 GiB each (400k blocks), the prefix
    and chunk blocks spread over the whole pool: sampled rows of every
    sequence against attention over its logical rows up to the row's
    position."""
    pkv, session = lib
    note("prefill, pools beyond 4 GiB")
    w = wl.make_prefill(prefix_len=512, chunk_lens=[300, 64, 1], num_heads=16, num_kv_heads=8, head_dim=128,
                        block_size=16, dtype="bf16", seed=62, spare_blocks=400000)
    blk_bytes = 16 * 8 * 128 * 2
    mapped = w.block_tables[w.block_tables >= 0]
    assert (mapped.astype(np.int64) * blk_bytes >= 2 ** 32).mean() > 0.5
    d = run(session, w)
    got = d.out.cpu().numpy()
    for s in range(w.num_seqs):
        first, k, v = w.logical_kv(s)
        assert first == 0
        L = int(w.context_lens[s])
        C = int(w.q_start[s + 1] - w.q_start[s])
        for i in sorted({0, C // 2, C - 1}):
            p = L - C + i
            row = int(w.q_start[s]) + i
            qf = ref.to_f64(w.q[row], "bf16")
            want = np.zeros((16, 128))
            for g in range(8):
                K = ref.to_f64(k[:p + 1, g], "bf16")
                V = ref.to_f64(v[:p + 1, g], "bf16")
                o, _ = ref.attend(qf[2 * g:2 * g + 2], K, V, w.scale)
                want[2 * g:2 * g + 2] = o
            assert_close(got[row], want, "bf16", f"4GiB+ prefill seq {s} row {i}")
    del d
    torch.cuda.empty_cache()
