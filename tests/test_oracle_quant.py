"""Pins for oracle.quant (fp8 E4M3 KV quantisation with per-row scales)."""
import numpy as np
import pytest
import torch

from oracle import quant as Q


def _torch_value(codes):
    t = torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy().astype(np.float64)


def _torch_encode(y):
    return torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def pin_values(q=Q):
    tab = np.array([q.e4m3_value(c) for c in range(256)])
    ref = _torch_value(np.arange(256))
    assert np.array_equal(np.isnan(tab), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(tab[ok], ref[ok])
    # hand-worked: zero, smallest subnormal, largest subnormal, smallest normal, one, max
    for code, val in ((0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
                      (0x38, 1.0), (0x3C, 1.5), (0x7E, 448.0), (0xB8, -1.0), (0xFE, -448.0)):
        assert q.e4m3_value(code) == val, hex(code)
    assert np.isnan(q.e4m3_value(0x7F)) and np.isnan(q.e4m3_value(0xFF))


def pin_encoding(q=Q):
    rng = np.random.default_rng(8)
    fin = np.array([q.e4m3_value(c) for c in range(0x7F)])          # 0 .. 448
    mids = (fin[:-1] + fin[1:]) / 2                                  # every tie
    ys = np.concatenate([
        rng.uniform(-448, 448, 200000), rng.standard_normal(200000) * 3,
        rng.standard_normal(100000) * 2.0 ** -8, fin, -fin, mids, -mids,
        np.nextafter(mids, 0), np.nextafter(mids, 1000)]).astype(np.float32)
    got = q.encode_e4m3(ys)
    want = _torch_encode(ys)
    assert np.array_equal(Q.e4m3_table()[got], _torch_value(want)), "value differs from torch"
    # ties go to the even code, e.g. 1 + 1/16 lies between 1 (0x38) and 1.125 (0x39)
    assert q.encode_e4m3(np.float32(1.0625))[()] == 0x38
    assert q.encode_e4m3(np.float32(1.1875))[()] == 0x3A
    assert q.encode_e4m3(np.float32(2.0 ** -10))[()] == 0x00      # half the smallest subnormal
    # above 448 only rounding can take a row value; it clamps to 448
    assert np.all(q.encode_e4m3(np.float32([448.5, 463.9, 464.0, 479.0, 1e6])) == 0x7E)
    assert np.all(q.encode_e4m3(np.float32([-460.0])) == 0xFE)


def pin_rows(q=Q):
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((40, 8, 128)) * rng.uniform(0.01, 30, (40, 8, 1))).astype(np.float32)
    x[3, 2] = 0.0
    x[4, 1] = np.float32(2.0 ** -101)              # below the zero-row limit
    x[4, 2, :3] = np.float32(2.0 ** -99)           # above it: an ordinary row
    x[4, 2, 3:] = 0.0
    codes, scales = q.quantize_rows(x)
    assert codes.shape == x.shape and scales.shape == x.shape[:2] and scales.dtype == np.float32
    assert scales[3, 2] == 0 and not codes[3, 2].any()
    assert scales[4, 1] == 0 and not codes[4, 1].any()
    assert np.all(codes[4, 2, :3] == 0x7E) and scales[4, 2] == np.float32(2.0 ** -99) / np.float32(448)
    amax = np.abs(x).max(-1)
    nz = amax >= 2.0 ** -100
    # the row's largest magnitude maps to +-448, the scale is amax / 448 in fp32
    assert np.all((codes & 0x7F).max(-1)[nz] == 0x7E)
    assert np.array_equal(scales[nz], (amax / np.float32(448)).astype(np.float32)[nz])
    # rounding error: half a step of E4M3 at the value (1/16 relative for normals,
    # 2^-10 absolute below 2^-6), on the scaled value, plus the fp32 roundings
    xh = q.dequantize_rows(codes, scales)
    err = np.abs(xh - x.astype(np.float64))
    s = scales.astype(np.float64)[..., None]
    bound = np.maximum(np.abs(x) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 2.0 ** -20) + \
        np.abs(x) * 2.0 ** -22
    assert np.all(err[nz] <= bound[nz])
    assert np.all(err[~nz] < 2.0 ** -100)           # rows stored as zeros
    # a row and its sign flip, a row times a power of two: same codes up to sign / same codes
    c2, s2 = q.quantize_rows(-x)
    assert np.array_equal(c2[nz] & 0x7F, codes[nz] & 0x7F) and np.array_equal(s2, scales)
    c3, s3 = q.quantize_rows(x * np.float32(4))
    assert np.array_equal(c3[nz], codes[nz]) and np.array_equal(s3[nz], scales[nz] * np.float32(4))


PINS = [pin_values, pin_encoding, pin_rows]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ---- planted mistakes ---------------------------------------------------------

class _Mut:
    """A copy of the module with one function replaced."""

    def __init__(self, **fns):
        self.__dict__.update({k: getattr(Q, k) for k in
                              ("e4m3_value", "encode_e4m3", "quantize_rows", "dequantize_rows",
                               "e4m3_table", "E4M3_MAX")})
        self.__dict__.update(fns)


def _truncating(y):
    """Rounds toward zero instead of to nearest."""
    y = np.asarray(y, np.float64)
    a = np.minimum(np.abs(y), 448.0)
    pos = Q.e4m3_table()[:0x7F]
    code = (np.searchsorted(pos, a, side="right") - 1).astype(np.uint8)
    return np.where((y < 0) & (code != 0), code | 0x80, code).astype(np.uint8)


def _ties_away(y):
    """Breaks ties away from zero."""
    y = np.asarray(y, np.float64)
    a = np.minimum(np.abs(y), 448.0)
    pos = Q.e4m3_table()[:0x7F]
    hi = np.minimum(np.searchsorted(pos, a, side="left"), len(pos) - 1)
    lo = np.maximum(hi - 1, 0)
    code = np.where(pos[hi] - a <= a - pos[lo], hi, lo).astype(np.uint8)
    return np.where((y < 0) & (code != 0), code | 0x80, code).astype(np.uint8)


def _fnuz_value(code):
    """Reads codes as the E4M3 FNUZ variant (bias 8)."""
    v = Q.e4m3_value(code)
    return v / 2 if v == v else v


def _fnuz_rows(x):
    """Scales to 240 (the FNUZ maximum) instead of 448."""
    x = np.asarray(x, np.float32)
    amax = np.abs(x).max(-1)
    safe = np.where(amax == 0, np.float32(1), amax).astype(np.float32)
    codes = Q.encode_e4m3((x * (np.float32(240) / safe)[..., None]).astype(np.float32))
    return codes, np.where(amax == 0, 0, amax / np.float32(240)).astype(np.float32)


def _block_scale_rows(x):
    """One scale per 16 rows instead of per row."""
    x = np.asarray(x, np.float32)
    codes, scales = Q.quantize_rows(x)
    sh = x.shape[:-1]
    flat = np.abs(x).reshape(-1, x.shape[-1]).max(-1)
    g = np.repeat(flat.reshape(-1, 16).max(-1) if flat.size % 16 == 0 else flat, 16)[:flat.size]
    g = g.reshape(sh).astype(np.float32)
    safe = np.where(g == 0, np.float32(1), g).astype(np.float32)
    codes = Q.encode_e4m3((x * (np.float32(448) / safe)[..., None]).astype(np.float32))
    return codes, (g / np.float32(448)).astype(np.float32)


@pytest.mark.parametrize("mut", [dict(encode_e4m3=_truncating), dict(encode_e4m3=_ties_away),
                                 dict(e4m3_value=_fnuz_value), dict(quantize_rows=_fnuz_rows),
                                 dict(quantize_rows=_block_scale_rows)],
                         ids=["truncate", "ties_away", "fnuz_values", "fnuz_scale", "block_scale"])
def test_mutant_fails_a_pin(mut):
    m = _Mut(**mut)
    failed = False
    for pin in PINS:
        try:
            pin(m)
        except AssertionError:
            failed = True
    assert failed
