"""Brute-force references used to pin the oracle (test infrastructure).

Nothing here reuses the oracle's code: rounding is done by searching the
sorted table of every finite value of the format, with exact rational
comparisons, and values are decoded from the formats' bit layouts with
library reinterpretation (numpy views).
"""
from __future__ import annotations

import bisect
from fractions import Fraction
from functools import lru_cache

import numpy as np


@lru_cache(maxsize=None)
def _table(fmt: str):
    if fmt == "bf16":
        codes = np.arange(0, 0x7F80, dtype=np.uint32)  # +0 .. largest finite
        vals = (codes << 16).view(np.float32).astype(np.float64)
        inf_code = 0x7F80
    elif fmt == "f16":
        codes = np.arange(0, 0x7C00, dtype=np.uint16)
        vals = codes.view(np.float16).astype(np.float64)
        inf_code = 0x7C00
    else:
        raise KeyError(fmt)
    return [float(v) for v in vals], inf_code


def round_rne(x, fmt: str) -> int:
    """Code of the nearest `fmt` value to x (exact), ties to the even code; overflow -> inf."""
    vals, inf_code = _table(fmt)
    sign = 0x8000 if (x < 0 or (x == 0 and np.signbit(float(x)))) else 0
    a = abs(Fraction(x))
    top, below = Fraction(vals[-1]), Fraction(vals[-2])
    if a >= top + (top - below) / 2:
        return sign | inf_code
    i = bisect.bisect_left(vals, float(a))
    # bisect on floats may be off by one when a is not a double; fix with exact compares
    while i < len(vals) and Fraction(vals[i]) < a:
        i += 1
    while i > 0 and Fraction(vals[i - 1]) >= a:
        i -= 1
    if i == len(vals):  # between the largest finite value and the overflow threshold
        return sign | (len(vals) - 1)
    if Fraction(vals[i]) == a:
        return sign | i
    lo, hi = Fraction(vals[i - 1]), Fraction(vals[i])
    dlo, dhi = a - lo, hi - a
    if dlo < dhi:
        c = i - 1
    elif dhi < dlo:
        c = i
    else:
        c = i - 1 if (i - 1) % 2 == 0 else i
    return sign | c


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def f16_to_f64(bits) -> np.ndarray:
    return np.asarray(bits).view(np.float16).astype(np.float64)


def decode16(bits, dtype: str) -> np.ndarray:
    return bf16_to_f64(bits) if dtype == "bf16" else f16_to_f64(bits)


def exact_matmul(a: np.ndarray, b: np.ndarray):
    """Exact rational A @ B from float64 arrays (tiny shapes only)."""
    m, k = a.shape
    n = b.shape[1]
    af = [[Fraction(float(v)) for v in row] for row in a]
    bf = [[Fraction(float(b[p, j])) for p in range(k)] for j in range(n)]
    return [[sum(x * y for x, y in zip(af[i], bf[j])) for j in range(n)] for i in range(m)]


def near_tie(x: Fraction, fmt: str, rel: float = 1e-12) -> bool:
    """True if exact x lies within rel of a rounding midpoint of fmt."""
    c = round_rne(x, fmt) & 0x7FFF
    vals, _ = _table(fmt)
    if c >= len(vals):
        return False
    v = Fraction(vals[c])
    a = abs(Fraction(x))
    neighbours = []
    if c + 1 < len(vals):
        neighbours.append((v + Fraction(vals[c + 1])) / 2)
    if c > 0:
        neighbours.append((v + Fraction(vals[c - 1])) / 2)
    return any(abs(a - mid) <= rel * max(a, Fraction(1, 10 ** 30)) for mid in neighbours)
