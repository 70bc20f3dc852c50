"""Exact-rational quantiser for single groups.  TEST INFRASTRUCTURE ONLY.

These are independent re-derivations used to pin ``oracle.quant``: they use
Python ``fractions.Fraction`` (no floating point at all) and a search over
candidates instead of division, so a slip in the vectorised fp64 code (a wrong
rounding direction, an inexact quotient deciding a tie, a dropped clamp) shows
up as a mismatch.  Definitions: section 2.4 of "分块稀疏注意力与KV Cache量化：
长文本推理显存优化实践" (per-group scale and zero-point along channels) with the
rounding readings stated in ``oracle.quant``.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def fp16_values_sorted() -> np.ndarray:
    """Every finite non-negative fp16 value, ascending, as float64."""
    bits = np.arange(0, 0x7C00, dtype=np.uint16)
    return bits.view(np.float16).astype(np.float64)


_FP16 = None


def _fp16_table():
    global _FP16
    if _FP16 is None:
        _FP16 = [Fraction(float(v)) for v in fp16_values_sorted()]
    return _FP16


def least_fp16_at_least(r: Fraction) -> Fraction:
    """Smallest non-negative fp16 value >= r (binary search over the table)."""
    t = _fp16_table()
    lo, hi = 0, len(t) - 1
    if t[hi] < r:
        raise OverflowError("no finite fp16 >= r")
    while lo < hi:
        mid = (lo + hi) // 2
        if t[mid] >= r:
            hi = mid
        else:
            lo = mid + 1
    return t[lo]


def round_half_even(q: Fraction) -> int:
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def quantize_group_exact(x_f16, bits: int):
    """One group of fp16 values -> (codes list, scale Fraction, zero int)."""
    qmax = (1 << bits) - 1
    xs = [Fraction(float(v)) for v in np.asarray(x_f16, dtype=np.float16)]
    lo = min(min(xs), Fraction(0))
    hi = max(max(xs), Fraction(0))
    if hi == lo:
        return [0] * len(xs), Fraction(0), 0
    s = least_fp16_at_least((hi - lo) / qmax)
    z = round_half_even(-lo / s)
    codes = [min(max(round_half_even(x / s) + z, 0), qmax) for x in xs]
    return codes, s, z


def nearest_code_search(x: Fraction, s: Fraction, z: int, bits: int) -> int:
    """The code c in [0, qmax] minimising |x - (c - z) s|, ties to even (c - z).

    No division: every candidate's distance is compared directly, so this does
    not share the quotient step of either quantiser."""
    qmax = (1 << bits) - 1
    best, best_d = None, None
    for c in range(qmax + 1):
        d = abs(x - (c - z) * s)
        if best is None or d < best_d or (d == best_d and (c - z) % 2 == 0):
            best, best_d = c, d
    return best


def nearest_zero_search(lo: Fraction, s: Fraction, bits: int) -> int:
    """The integer z in [0, qmax] minimising |-lo - z s|, ties to even z."""
    qmax = (1 << bits) - 1
    best, best_d = None, None
    for z in range(qmax + 1):
        d = abs(-lo - z * s)
        if best is None or d < best_d or (d == best_d and z % 2 == 0):
            best, best_d = z, d
    return best
