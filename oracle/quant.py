"""fp8 (E4M3) KV-cache quantisation with one scale per (token, kv head) row.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The gouthm page ("The KV cache is not your bottleneck", sections "The setup"
and "What the profile said") names quantising the KV cache as the way to buy
memory headroom at a small accuracy cost, and gives no scheme. Readings, the
plainest ones that keep every value of a row recoverable:

* format: OCP FP8 E4M3 ("E4M3FN"): 1 sign, 4 exponent (bias 7), 3 mantissa
  bits; normal values m/8 * 2^(e-7) for exponent field e in 1..15 (m in 8..15),
  subnormals k/8 * 2^-6 (k in 0..7); no infinities; S.1111.111 is NaN, so the
  largest finite magnitude is 448;
* one fp32 scale per row of head_dim values of one token and one kv head:
  scale = amax / 448 with amax = max |x| over the row; the stored codes are
  the values x * (448 / amax) rounded to the nearest E4M3 value, ties to the
  even code, magnitudes above 448 (reachable only by rounding) clamped to 448;
  a row whose amax is below 2^-100 (zeros, or values so small that 448 / amax
  would not stay finite in fp32) gets scale 0 and zero codes;
* both products and the quotients are single fp32 operations rounded to
  nearest even, in this order: inv = fl(448 / amax), y = fl(x * inv),
  scale = fl(amax / 448);
* a dequantised value is value(code) * scale, computed exactly (fp64).

Pins (tests/test_oracle_quant.py): every code's value against torch's
float8_e4m3fn conversion and hand-worked codes; encoding against torch's
conversion on random values, on every representable value and on every
midpoint between neighbours; saturation; the row rule (the largest magnitude
maps to 448, zero rows); the rounding error bound; planted mistakes.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
ZERO_ROW_AMAX = 2.0 ** -100    # rows with a smaller amax are stored as zeros


def e4m3_value(code: int) -> float:
    """Exact value of one code (NaN for S.1111.111)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_table() -> np.ndarray:
    """Values of all 256 codes, float64."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


_POS = e4m3_table()[:0x7F]          # codes 0x00 .. 0x7E: 0 .. 448, increasing


def encode_e4m3(y) -> np.ndarray:
    """Nearest E4M3 code of each finite value (ties to the even code, which is
    the even mantissa), magnitudes above 448 clamped to 448."""
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        raise ValueError("E4M3 encoding of a non-finite value")
    a = np.minimum(np.abs(y), E4M3_MAX)
    hi = np.searchsorted(_POS, a, side="left")          # first value >= a
    hi = np.minimum(hi, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(a == _POS[hi], hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    return np.where((y < 0) & (code != 0), code | 0x80, code).astype(np.uint8)


def quantize_rows(x):
    """Codes (uint8, x's shape) and per-row scales (float32, x.shape[:-1]) of
    the rows x[..., :] (float32 values; the last axis is head_dim)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    zero = amax < np.float32(ZERO_ROW_AMAX)
    safe = np.where(zero, np.float32(1.0), amax).astype(np.float32)
    inv = (np.float32(E4M3_MAX) / safe).astype(np.float32)
    y = (x * inv[..., None]).astype(np.float32)
    codes = encode_e4m3(y)
    codes[zero] = 0
    scales = np.where(zero, np.float32(0.0), (amax / np.float32(E4M3_MAX)).astype(np.float32))
    return codes, scales.astype(np.float32)


def dequantize_rows(codes, scales) -> np.ndarray:
    """value(code) * scale for every element, float64 (exact)."""
    vals = e4m3_table()[np.asarray(codes, dtype=np.uint8)]
    return vals * np.asarray(scales, dtype=np.float64)[..., None]
