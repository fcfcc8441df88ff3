"""Pins of the 8-bit KV encoding oracle (``oracle/quant.py``), CPU only.

The FP8 codec is checked against torch's float8_e4m3fn conversion (a library
routine, both directions); INT8 and FP8 rows against their round-trip error
bounds and exact cases; the quantized decode against the plain decode on data
the encoding represents exactly.  Planted mistakes (truncation, a wrong
scale, the other FP8 flavour) are each caught by one of these.
"""
import numpy as np
import pytest
import torch

import oracle.quant as oq
import oracle.ref as ref
import workloads as wl


def torch_e4m3(y):
    return torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = oq.e4m3_value(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(mine), np.isnan(theirs))
    ok = ~np.isnan(mine)
    assert np.array_equal(mine[ok], theirs[ok])
    assert np.nanmax(mine) == 448.0 and np.nanmin(np.abs(mine[mine != 0])) == 2.0 ** -9


def test_e4m3_encode_matches_torch_including_ties():
    rng = np.random.default_rng(7)
    v = oq._POS_VALUES
    mids = (v[1:] + v[:-1]) / 2  # exact in float32; ties go to the even code
    y = np.concatenate([rng.uniform(-448, 448, 50000), rng.uniform(-0.03, 0.03, 50000),
                        rng.standard_normal(50000), mids, -mids, v, -v,
                        [0.0, -0.0, 448.0, -448.0, 448.00003, 2.0 ** -10, -(2.0 ** -10)]]).astype(np.float32)
    assert np.array_equal(oq.e4m3_encode(y), torch_e4m3(y))


def rows(rng, n, D, scale=1.0):
    x = (rng.standard_normal((n, D)) * scale).astype(np.float32)
    x[0] = 0.0                       # an all-zero row
    x[1, 3] = 1e4 * scale            # one large element
    x[2] = x[2] * 1e-6               # tiny values
    return x


@pytest.mark.parametrize("fmt", ["i8", "fp8"])
def test_max_element_maps_to_qmax_and_zero_row(fmt):
    rng = np.random.default_rng(1)
    x = rows(rng, 64, 128)
    codes, scale = oq.quantize_rows(x, fmt)
    deq = oq.dequantize_rows(codes, scale, fmt)
    assert scale[0] == 0 and np.all(codes[0] == 0) and np.all(deq[0] == 0)
    qmax = oq.QMAX[fmt]
    vals = codes.view(np.int8).astype(np.float64) if fmt == "i8" else oq.e4m3_value(codes)
    imax = np.argmax(np.abs(x[1:]), axis=1)
    got = np.abs(vals[1:][np.arange(63), imax])
    assert np.all(got == qmax)
    assert np.allclose(scale[1:], np.abs(x[1:]).max(axis=1) / qmax, rtol=1e-7, atol=0)


def test_int8_round_trip_bound_and_exact_grid():
    rng = np.random.default_rng(2)
    x = rows(rng, 256, 128, scale=3.0)
    codes, scale = oq.quantize_rows(x, "i8")
    deq = oq.dequantize_rows(codes, scale, "i8")
    err = np.abs(deq - x.astype(np.float64))
    # half a code step, plus the float32 rounding of x * inv
    assert np.all(err <= scale[:, None].astype(np.float64) * (0.5 + 1e-5))
    # rows on the code grid with amax 127 (scale 1) come back exactly
    k = rng.integers(-127, 128, size=(32, 64)).astype(np.float32)
    k[:, 0] = 127
    c2, s2 = oq.quantize_rows(k, "i8")
    assert np.all(s2 == 1.0) and np.array_equal(c2.view(np.int8).astype(np.float32), k)


def test_fp8_round_trip_bound_and_exact_grid():
    rng = np.random.default_rng(3)
    x = rows(rng, 256, 128, scale=0.5)
    codes, scale = oq.quantize_rows(x, "fp8")
    deq = oq.dequantize_rows(codes, scale, "fp8")
    y = np.abs(x.astype(np.float64)) / np.where(scale > 0, scale, 1)[:, None]
    err = np.abs(deq - x.astype(np.float64))
    s64 = scale[:, None].astype(np.float64)
    normal = y >= 2.0 ** -6
    # 3 mantissa bits: half an ulp is 2^-4 relative; subnormal spacing 2^-9
    assert np.all(err[normal] <= np.abs(x.astype(np.float64))[normal] * 2.0 ** -4 * (1 + 1e-5))
    assert np.all(err[~normal] <= (s64 * np.ones_like(y))[~normal] * 2.0 ** -10 * (1 + 1e-5))
    g = oq._POS_VALUES[rng.integers(0, 127, size=(32, 64))].astype(np.float32)
    g *= np.where(rng.random(g.shape) < 0.5, -1, 1).astype(np.float32)
    g[:, 0] = 448.0
    c2, s2 = oq.quantize_rows(g, "fp8")
    assert np.all(s2 == 1.0) and np.array_equal(oq.e4m3_value(c2), g.astype(np.float64))


@pytest.mark.parametrize("fmt", ["i8", "fp8"])
def test_quantized_decode_equals_plain_decode_on_exact_data(fmt):
    """Pools whose rows are on the code grid with scale 1: the quantized
    decode must equal the plain decode of the same values."""
    w = wl.make_decode(seed=11, num_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                       dtype="f32", lens=[40, 1, 100], window=0)
    kp, vp = ref.build_pools(w)
    rng = np.random.default_rng(5)
    for pool in (kp, vp):
        live = np.isfinite(pool).all(axis=-1)
        if fmt == "i8":
            vals = rng.integers(-127, 128, size=pool.shape).astype(np.float32)
            vals[..., 0] = 127
        else:
            vals = oq._POS_VALUES[rng.integers(0, 127, size=pool.shape)].astype(np.float32)
            vals *= np.where(rng.random(pool.shape) < 0.5, -1, 1).astype(np.float32)
            vals[..., 0] = 448
        pool[live] = vals[live]
    kc, vc, ks, vs = oq.quantize_pools(kp, vp, "f32", fmt)
    assert np.all(ks[np.isfinite(ks)] == 1.0)
    got, glse = oq.decode(w.q, kc, vc, ks, vs, w.block_tables, w.context_lens, fmt=fmt, q_dtype="f32",
                          block_size=16, num_kv_heads=2, window=0, scale=w.scale)
    want, wlse = ref.decode(w.q, kp, vp, w.block_tables, w.context_lens, block_size=16, num_kv_heads=2,
                            window=0, scale=w.scale, dtype="f32")
    assert np.abs(got - want).max() <= 1e-12 and np.abs(glse - wlse).max() <= 1e-12


def _on_grid(pool, fmt, rng):
    """Replace every written row of ``pool`` by values on the code grid whose
    largest magnitude is QMAX, so that each row encodes exactly, scale 1."""
    live = np.isfinite(pool).all(axis=-1)
    if fmt == "i8":
        vals = rng.integers(-127, 128, size=pool.shape).astype(np.float32)
        vals[..., 0] = 127
    else:
        vals = oq._POS_VALUES[rng.integers(0, 127, size=pool.shape)].astype(np.float32)
        vals *= np.where(rng.random(pool.shape) < 0.5, -1, 1).astype(np.float32)
        vals[..., 0] = 448
    pool[live] = vals[live]


@pytest.mark.parametrize("fmt", ["i8", "fp8"])
def test_quantized_prefill_equals_plain_prefill_on_exact_data(fmt):
    """Chunked prefill over 8-bit pools whose rows encode exactly (scale 1)
    equals the plain prefill of the same values."""
    w = wl.make_prefill(prefix_len=32, chunk_lens=[20, 1, 0, 45], num_heads=8, num_kv_heads=2, head_dim=64,
                        block_size=16, dtype="f32", seed=13)
    kp, vp = ref.build_pools(w)
    rng = np.random.default_rng(6)
    _on_grid(kp, fmt, rng)
    _on_grid(vp, fmt, rng)
    kc, vc, ks, vs = oq.quantize_pools(kp, vp, "f32", fmt)
    assert np.all(ks[np.isfinite(ks)] == 1.0)
    got, glse = oq.prefill(w.q, w.q_start, kc, vc, ks, vs, w.block_tables, w.context_lens, fmt=fmt,
                           q_dtype="f32", block_size=16, num_kv_heads=2, window=0, scale=w.scale / 64)
    want, wlse = ref.prefill(w.q, w.q_start, kp, vp, w.block_tables, w.context_lens, block_size=16,
                             num_kv_heads=2, window=0, scale=w.scale / 64, dtype="f32")
    fin = np.isfinite(want)
    assert np.array_equal(fin, np.isfinite(got)) and fin.any()
    assert np.abs(got[fin] - want[fin]).max() <= 1e-9
    assert np.abs(glse[np.isfinite(wlse)] - wlse[np.isfinite(wlse)]).max() <= 1e-9


@pytest.mark.parametrize("fmt,window,sinks", [("i8", 0, 0), ("fp8", 0, 0), ("i8", 24, 0), ("fp8", 24, 3)])
def test_quantized_prefill_last_row_is_decode(fmt, window, sinks):
    """The last row of a chunk sits at position L - 1 and attends what a
    decode step of the same sequence attends: quantized prefill and
    quantized decode agree there (real-valued rows, row scales not 1)."""
    w = wl.make_prefill(prefix_len=48, chunk_lens=[30, 1, 17], num_heads=8, num_kv_heads=4, head_dim=64,
                        block_size=16, dtype="bf16", seed=14, window=window, sinks=sinks)
    kp, vp = ref.build_pools(w)
    kc, vc, ks, vs = oq.quantize_pools(kp, vp, "bf16", fmt)
    assert not np.all(ks[np.isfinite(ks)] == 1.0)
    out, lse = oq.prefill(w.q, w.q_start, kc, vc, ks, vs, w.block_tables, w.context_lens, fmt=fmt,
                          q_dtype="bf16", block_size=16, num_kv_heads=4, window=window, scale=w.scale, sinks=sinks)
    last = w.q_start[1:] - 1
    dout, dlse = oq.decode(w.q[last], kc, vc, ks, vs, w.block_tables, w.context_lens, fmt=fmt, q_dtype="bf16",
                           block_size=16, num_kv_heads=4, window=window, scale=w.scale, sinks=sinks)
    assert np.abs(out[last] - dout).max() <= 1e-12
    assert np.abs(lse[last] - dlse).max() <= 1e-12
    # and the encoding moves the result away from the 16-bit prefill (the
    # scales are applied, not dropped)
    o16, _ = ref.prefill(w.q, w.q_start, kp, vp, w.block_tables, w.context_lens, block_size=16, num_kv_heads=4,
                         window=window, scale=w.scale, dtype="bf16", sinks=sinks)
    d = np.abs(out - o16).max()
    assert 1e-6 < d < 0.2, d


def test_unwritten_rows_stay_nan():
    w = wl.make_decode(seed=12, num_heads=4, num_kv_heads=4, head_dim=64, block_size=16,
                       dtype="bf16", lens=[20, 3], window=0)
    kp, vp = ref.build_pools(w)
    kc, vc, ks, vs = oq.quantize_pools(kp, vp, "bf16", "i8")
    written = np.isfinite(ref.to_f64(kp, "bf16")).all(axis=-1)      # [NB, B, Hkv]
    assert np.all(np.isnan(ks.transpose(0, 2, 1)[~written]))
    assert np.all(kc[~written] == 0xFF)
    assert np.all(np.isfinite(ks.transpose(0, 2, 1)[written]))


@pytest.mark.parametrize("mistake", ["truncate", "scale128", "fnuz"])
def test_planted_mistakes_are_caught(mistake):
    rng = np.random.default_rng(9)
    x = rows(rng, 64, 128)
    amax = np.abs(x).max(1)
    good_scale = (amax / 127).astype(np.float32)
    if mistake == "truncate":
        inv = (127 / np.where(amax > 0, amax, 1)).astype(np.float32)
        codes = np.trunc(x * inv[:, None]).astype(np.int8).view(np.uint8)
        err = np.abs(oq.dequantize_rows(codes, good_scale, "i8") - x)
        assert not np.all(err <= good_scale[:, None] * (0.5 + 1e-5))
    elif mistake == "scale128":
        codes, _ = oq.quantize_rows(x, "i8")
        err = np.abs(oq.dequantize_rows(codes, (amax / 128).astype(np.float32), "i8") - x)
        assert not np.all(err <= good_scale[:, None] * (0.5 + 1e-5))
    else:  # FP8 with exponent bias 8 (the other 8-bit float flavour) decodes differently
        codes = np.arange(256, dtype=np.uint8)
        shifted = oq.e4m3_value(codes) / 2.0
        theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
        ok = ~np.isnan(shifted)
        assert not np.array_equal(shifted[ok], theirs[ok])
