"""Exact-arithmetic helpers for pinning the oracle.

Independent of the oracle: rounding here is a brute-force nearest-value search
over the exact values of every code of a format (decoded by numpy/torch bit
views), compared with Python ``Fraction`` arithmetic; ties go to the code with
an even bit pattern.  Transcendentals use ``decimal`` at 60 digits.
"""

from __future__ import annotations

import bisect
import decimal
from fractions import Fraction
from functools import lru_cache

import numpy as np
import torch

_CTX = decimal.Context(prec=60, Emax=decimal.MAX_EMAX, Emin=decimal.MIN_EMIN)


def bf16_value(bits: int) -> float:
    return float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0])


@lru_cache(maxsize=None)
def _bf16_grid():
    """Sorted exact values of all finite non-negative bf16 codes, with codes."""
    codes = np.arange(0x0000, 0x7F81, dtype=np.uint32)  # +0 .. +inf
    vals = (codes << 16).view(np.float32)
    items = [(Fraction(float(v)), int(c)) for v, c in zip(vals, codes) if np.isfinite(v)]
    items.sort()
    return [v for v, _ in items], [c for _, c in items]


@lru_cache(maxsize=None)
def _e4m3_grid():
    codes = torch.arange(0, 0x7F, dtype=torch.uint8)  # +0 .. 448 (0x7F is NaN)
    vals = codes.view(torch.float8_e4m3fn).float().tolist()
    items = sorted((Fraction(v), int(c)) for v, c in zip(vals, codes.tolist()))
    return [v for v, _ in items], [c for _, c in items]


def _nearest_even(x: Fraction, grid):
    vals, codes = grid
    a = abs(x)
    i = bisect.bisect_left(vals, a)
    if i < len(vals) and vals[i] == a:
        return codes[i]
    if i == len(vals):
        return None  # beyond the largest finite value
    lo, hi = i - 1, i
    dl, dh = a - vals[lo], vals[hi] - a
    if dl < dh:
        return codes[lo]
    if dh < dl:
        return codes[hi]
    return codes[lo] if codes[lo] % 2 == 0 else codes[hi]


def round_to_bf16(x: Fraction) -> int:
    """Exact x -> bf16 bits, nearest, ties to even; overflow -> infinity."""
    vals, codes = _bf16_grid()
    top = vals[-1]
    mid = top + (Fraction(2) ** 128 - top) / 2   # the largest finite code is odd
    a = abs(x)
    if a >= mid:
        c = 0x7F80
    elif a > top:
        c = codes[-1]
    else:
        c = _nearest_even(x, (vals, codes))
    return c | (0x8000 if x < 0 else 0)


def round_to_e4m3(x: Fraction) -> int:
    """Exact x (|x| <= 448) -> E4M3FN code, nearest, ties to even."""
    c = _nearest_even(x, _e4m3_grid())
    assert c is not None, "value beyond 448"
    return c | (0x80 if x < 0 else 0)


def round_to_f32(x: Fraction) -> float:
    """Exact x -> nearest binary32, ties to even (normal range only)."""
    f = np.float32(float(x))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = None
    for c in cands:
        d = abs(Fraction(float(c)) - x)
        even = (int(np.array([c], np.float32).view(np.uint32)[0]) & 1) == 0
        key = (d, not even)
        if best is None or key < best[0]:
            best = (key, c)
    return float(best[1])


def dec(x) -> decimal.Decimal:
    return _CTX.create_decimal_from_float(float(x)) if not isinstance(x, Fraction) else \
        _CTX.divide(decimal.Decimal(x.numerator), decimal.Decimal(x.denominator))


def silu_exact(g: float) -> Fraction:
    """silu(g) = g / (1 + e^-g) to 60 significant digits, as a Fraction."""
    d = _CTX.create_decimal_from_float(g)
    e = _CTX.exp(-d)
    s = _CTX.divide(d, _CTX.add(decimal.Decimal(1), e))
    return Fraction(s)


def rsqrt_exact(v: Fraction) -> Fraction:
    d = dec(v)
    return Fraction(_CTX.divide(decimal.Decimal(1), _CTX.sqrt(d)))
