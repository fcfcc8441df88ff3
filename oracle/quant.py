"""8-bit KV pages: the row encoding and attention over the decoded pools.
Test infrastructure only (see ``oracle/__init__.py``).

"Build a Memory-Compressed Attention Engine with KV Caching from Scratch",
section "Extending It: Your Roadmap to Senior-Level", item 2 (quantized KV
cache): cached keys and values are stored as INT8 or FP8 to cut the bytes a
decode step reads.  The page fixes nothing else; the encoding below is this
library's reading, written out as plain float32 steps so that the stored
bytes can be compared bit for bit:

* one row = the D values of one (block, slot, kv head); each row gets its own
  float32 scale (appending a token never touches another row's codes);
* amax = max_d |x_d|; scale = amax / QMAX; inv = QMAX / amax (0 when amax is
  0), both float32 divisions rounded to nearest;
* y_d = x_d * inv (float32 product, rounded to nearest);
* INT8 (QMAX 127): code = round-half-even(y_d), clamped to [-127, 127],
  stored as two's complement;
* FP8 (QMAX 448): code = y_d rounded to the nearest OCP E4M3 ("e4m3fn":
  bias 7, no infinities, 0x7F/0xFF NaN, largest finite 448), ties to the
  even code, magnitudes beyond 448 saturated to 448;
* decoded value = code * scale (exact in float64).

Scale pools are float32 ``[NB, Hkv, B]`` (one (block, kv head) has its B row
scales together); code pools are uint8 ``[NB, B, Hkv, D]`` like the 16-bit
pools.

Pinned by ``tests/test_oracle_quant.py`` (the FP8 codec against torch's
float8_e4m3fn conversion, round-trip bounds, exact cases; decode and prefill
over the decoded pools equal the plain attention on values that are on the
code grid, and a prefill chunk's last row equals the decode of its
sequence).
"""
from __future__ import annotations

import numpy as np

from . import ref

QMAX = {"i8": 127.0, "fp8": 448.0}


# ------------------------------------------------------------- FP8 E4M3

def e4m3_value(code) -> np.ndarray:
    """float64 value of each E4M3 code (0x7F and 0xFF are NaN).

    Fields: sign (bit 7), exponent e (bits 6..3, bias 7), mantissa m (bits
    2..0).  e = 0: m / 8 * 2^-6 (subnormal); otherwise (1 + m / 8) * 2^(e - 7).
    """
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


# Non-negative finite codes 0x00 .. 0x7E in increasing value order.
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALUES = e4m3_value(_POS_CODES)


def e4m3_encode(y) -> np.ndarray:
    """Nearest E4M3 code of each float value, ties to the even code, beyond
    448 saturated.  The sign of zero is kept (-0.0 -> 0x80)."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), _POS_VALUES[-1])
    hi = np.searchsorted(_POS_VALUES, a, side="left")  # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    neg = np.signbit(y)
    return np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)


# ------------------------------------------------------------ row encoding

def quantize_rows(x, fmt: str):
    """Encode rows (last axis = D) of float values: returns (codes uint8 with
    the shape of x, scale float32 with the shape of x minus its last axis)."""
    x = np.asarray(x, dtype=np.float32)
    qmax = np.float32(QMAX[fmt])
    amax = np.max(np.abs(x), axis=-1).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        scale = (amax / qmax).astype(np.float32)
        inv = np.where(amax > 0, qmax / amax, np.float32(0)).astype(np.float32)
    y = (x * inv[..., None]).astype(np.float32)
    if fmt == "i8":
        codes = np.clip(np.rint(y), -127, 127).astype(np.int8).view(np.uint8)
    elif fmt == "fp8":
        codes = e4m3_encode(y)
    else:
        raise ValueError(fmt)
    return codes, scale


def dequantize_rows(codes, scale, fmt: str) -> np.ndarray:
    """code * scale in float64 (exact: an 8-bit code times a float32)."""
    codes = np.asarray(codes, dtype=np.uint8)
    if fmt == "i8":
        v = codes.view(np.int8).astype(np.float64)
    elif fmt == "fp8":
        v = e4m3_value(codes)
    else:
        raise ValueError(fmt)
    return v * np.asarray(scale, dtype=np.float64)[..., None]


# ------------------------------------------------------------------ pools

def quantize_pools(k_pool, v_pool, dtype: str, fmt: str):
    """Encode every finite row of the [NB, B, Hkv, D] pools (storage dtype
    ``dtype``).  Rows that were never written (NaN) keep code 0xFF and scale
    NaN, so they decode to NaN.  Returns (k_codes, v_codes, k_scale, v_scale)
    with scales in the [NB, Hkv, B] layout."""
    out = []
    for pool in (k_pool, v_pool):
        x = ref.to_f64(pool, dtype).astype(np.float32)            # [NB, B, Hkv, D]
        codes, scale = quantize_rows(np.nan_to_num(x), fmt)
        written = np.isfinite(x).all(axis=-1)                     # [NB, B, Hkv]
        codes = np.where(written[..., None], codes, np.uint8(0xFF)).astype(np.uint8)
        scale = np.where(written, scale, np.float32(np.nan)).astype(np.float32)
        out.append((codes, np.ascontiguousarray(scale.transpose(0, 2, 1))))
    (kc, ks), (vc, vs) = out
    return kc, vc, ks, vs


def dequantize_pool(codes, scale_nhb, fmt: str) -> np.ndarray:
    """[NB, B, Hkv, D] float64 decoded pool from codes and [NB, Hkv, B] scales."""
    return dequantize_rows(codes, np.asarray(scale_nhb).transpose(0, 2, 1), fmt)


def decode(q, k_codes, v_codes, k_scale, v_scale, block_tables, context_lens, *, fmt, q_dtype,
           block_size, num_kv_heads, window, scale, seqs=None, heads=None, sinks=0):
    """Single-query decode over the decoded 8-bit pools: the attention of
    ``ref.decode`` with keys and values replaced by code * scale."""
    kp = dequantize_pool(k_codes, k_scale, fmt)
    vp = dequantize_pool(v_codes, v_scale, fmt)
    return ref.decode(q, kp, vp, block_tables, context_lens, block_size=block_size,
                      num_kv_heads=num_kv_heads, window=window, scale=scale, dtype=q_dtype,
                      kv_dtype="f64", seqs=seqs, heads=heads, sinks=sinks)


def prefill(q, q_start, k_codes, v_codes, k_scale, v_scale, block_tables, context_lens, *, fmt, q_dtype,
            block_size, num_kv_heads, window, scale, sinks=0, seqs=None, heads=None):
    """Causal chunked prefill over the decoded 8-bit pools: the attention of
    ``ref.prefill`` (the prefill of "Building a Streaming Sliding-Window
    Attention Engine in Pure Python", Step 3) with keys and values replaced
    by code * scale."""
    kp = dequantize_pool(k_codes, k_scale, fmt)
    vp = dequantize_pool(v_codes, v_scale, fmt)
    return ref.prefill(q, q_start, kp, vp, block_tables, context_lens, block_size=block_size,
                       num_kv_heads=num_kv_heads, window=window, scale=scale, dtype=q_dtype, kv_dtype="f64",
                       sinks=sinks, seqs=seqs, heads=heads)
