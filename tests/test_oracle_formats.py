"""Pins for the oracle's number formats (CPU).

Each decoder is checked over every code against library reinterpretation or
a formula evaluated independently with exact rationals; each encoder against
a brute-force nearest-value search (tests/brute.py) and, where one exists, a
library conversion.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from brute import round_rne


def _same(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])


def test_bf16_decode_all_codes():
    codes = np.arange(65536, dtype=np.uint32)
    ref = (codes << 16).view(np.float32).astype(np.float64)
    assert _same(oracle.decode("bf16", codes.astype(np.uint16)), ref)


def test_f16_decode_all_codes():
    codes = np.arange(65536, dtype=np.uint16)
    assert _same(oracle.decode("f16", codes), codes.view(np.float16).astype(np.float64))


def _ocp_fp8(code, ebits, mbits, bias, fn):
    """OCP 8-bit float value from its fields (exact rational, None for NaN, 'inf' for inf)."""
    s = code >> 7
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    if fn and e == (1 << ebits) - 1 and m == (1 << mbits) - 1:
        return None
    if not fn and e == (1 << ebits) - 1:
        return None if m else ("-inf" if s else "inf")
    if e == 0:
        v = Fraction(m, 1 << mbits) * Fraction(2) ** (1 - bias)
    else:
        v = (1 + Fraction(m, 1 << mbits)) * Fraction(2) ** (e - bias)
    return -v if s else v


@pytest.mark.parametrize("fmt,ebits,mbits,bias,fn,tdt", [
    ("e4m3fn", 4, 3, 7, True, torch.float8_e4m3fn),
    ("e5m2", 5, 2, 15, False, torch.float8_e5m2),
])
def test_fp8_decode_all_codes(fmt, ebits, mbits, bias, fn, tdt):
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode(fmt, codes)
    lib = torch.from_numpy(codes.copy()).view(tdt).to(torch.float64).numpy()
    assert _same(got, lib)
    for c in range(256):
        v = _ocp_fp8(c, ebits, mbits, bias, fn)
        if v is None:
            assert np.isnan(got[c])
        elif isinstance(v, str):
            assert got[c] == (np.inf if v == "inf" else -np.inf)
        else:
            assert Fraction(float(got[c])) == v, c
    if fmt == "e4m3fn":
        assert np.nanmax(got) == 448.0 and np.nanmin(got[got > 0]) == 2.0 ** -9


def test_e8m0_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode("e8m0", codes)
    for b in range(255):
        assert Fraction(float(got[b])) == Fraction(2) ** (b - 127)
    assert np.isnan(got[255])
    if hasattr(torch, "float8_e8m0fnu"):
        lib = torch.from_numpy(codes.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
        assert _same(got, lib)


def _probe_values(fmt, n=3000, seed=0):
    """Random doubles over the format's range plus exact midpoints and their neighbours."""
    rng = np.random.default_rng(seed)
    lo, hi = (-133, 128) if fmt == "bf16" else (-25, 16)
    vals = list(rng.standard_normal(n) * np.exp2(rng.integers(lo, hi, n)))
    dec = (lambda c: float((np.uint32(c) << 16).view(np.float32))) if fmt == "bf16" else \
          (lambda c: float(np.uint16(c).view(np.float16)))
    top = 0x7F7F if fmt == "bf16" else 0x7BFF
    for c in list(rng.integers(0, top, 400)) + [0, 1, 2, top - 1]:
        a, b = dec(int(c)), dec(int(c) + 1)
        mid = (a + b) / 2  # exact in fp64: both have <= 11 significand bits
        vals += [mid, -mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf), a, b]
    big = dec(top)
    step = big - dec(top - 1)
    vals += [big + step / 2, np.nextafter(big + step / 2, 0), big * 4, 0.0, -0.0]
    return np.array(vals, dtype=np.float64)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_rne_encode_matches_brute_force(fmt):
    vals = _probe_values(fmt)
    got = oracle.encode(fmt, vals).view(np.uint16)
    ref = np.array([round_rne(float(v), fmt) for v in vals], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(vals[i], hex(got[i]), hex(ref[i])) for i in bad[:5]]


def test_f16_encode_matches_numpy():
    vals = _probe_values("f16", n=20000, seed=1)
    assert np.array_equal(oracle.encode("f16", vals).view(np.uint16),
                          vals.astype(np.float16).view(np.uint16))


def test_f32_encode_matches_numpy():
    rng = np.random.default_rng(2)
    vals = rng.standard_normal(10000) * np.exp2(rng.integers(-140, 120, 10000))
    assert np.array_equal(oracle.encode("f32", vals), vals.astype(np.float32))


def test_nan_encodes_to_nan():
    for fmt in ("bf16", "f16"):
        c = int(oracle.encode(fmt, np.array([np.nan]))[0].view(np.uint16))
        exp_mask = 0x7F80 if fmt == "bf16" else 0x7C00
        assert (c & exp_mask) == exp_mask and (c & ~exp_mask & 0x7FFF) != 0
