"""Exact-rational recomputation of one group's scale search (pins the CPU oracle).

Independent of ``oracle/``: the element formats are derived here from their bit layouts, every
rounding to E2M1/E4M3 is "nearest value, ties to the even code" found by exact comparison
over the whole code set, and every candidate loss is summed exactly with ``fractions``.
The only binary32 operations kept are the ones the method defines as binary32 values:
the global-scale product eff = S * dec(c), its reciprocal, the normalised weight |w| * r and
the base ratio (amax / 6) / S (single IEEE operations done by numpy float32 scalars).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def e2m1_levels():
    """E2M1 magnitudes from the bit layout: 2 exponent bits (bias 1), 1 mantissa bit."""
    out = []
    for code in range(8):
        e, m = code >> 1, code & 1
        out.append(Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2)))
    return out


def e4m3_values():
    """E4M3 magnitudes for codes 0..126 (4 exponent bits, bias 7, 3 mantissa bits)."""
    out = []
    for code in range(127):
        e, m = code >> 3, code & 7
        out.append(Fraction(m, 8) * Fraction(1, 64) if e == 0
                   else Fraction(2) ** (e - 7) * (1 + Fraction(m, 8)))
    return out


E2M1 = e2m1_levels()
E4M3 = e4m3_values()


def nearest_even(value: Fraction, table) -> int:
    """Index of the table entry nearest to value; ties to the even index."""
    best_i, best_d = None, None
    for i, v in enumerate(table):
        d = abs(value - v)
        if best_d is None or d < best_d or (d == best_d and i % 2 == 0 and best_i % 2 == 1):
            best_i, best_d = i, d
    return best_i


def f32(x) -> np.float32:
    return np.float32(x)


def group_exact(w16, h16, S, lo=-9, hi=6, exhaustive=False):
    """Exact candidate losses of one group.

    Returns dict(base, codes, offsets, exact_losses, q_index) or base == 0 for a zero group.
    """
    w = [f32(v) for v in w16]
    a = [f32(abs(v)) for v in w]
    S = f32(S)
    amax = max(a)
    if amax == 0:
        return {"base": 0}
    s_star = f32(f32(amax / f32(6.0)) / S)
    b = nearest_even(Fraction(float(s_star)), E4M3)
    b = max(b, 1)
    if exhaustive:
        codes = list(range(1, 127))
    else:
        codes = [min(max(b + o, 1), 126) for o in range(lo, hi + 1)]
    losses, qidx = [], []
    for c in codes:
        eff = f32(S * f32(float(E4M3[c])))
        r = f32(f32(1.0) / eff)
        total = Fraction(0)
        idxs = []
        for j in range(16):
            x = f32(a[j] * r)
            k = nearest_even(Fraction(float(x)), E2M1)
            idxs.append(k)
            d = Fraction(float(a[j])) - E2M1[k] * Fraction(float(eff))
            weight = Fraction(1) if h16 is None else Fraction(float(f32(h16[j])))
            total += weight * d * d
        losses.append(total)
        qidx.append(idxs)
    return {"base": b, "codes": codes, "exact_losses": losses, "q_index": qidx}


def losses_at(w16, h16, S, codes):
    """Exact losses (and E2M1 indices) of one group at the given codes, in the given order."""
    a = [f32(abs(f32(v))) for v in w16]
    S = f32(S)
    losses, qidx = [], []
    for c in codes:
        eff = f32(S * f32(float(E4M3[c])))
        r = f32(f32(1.0) / eff)
        total = Fraction(0)
        idxs = []
        for j in range(16):
            x = f32(a[j] * r)
            k = nearest_even(Fraction(float(x)), E2M1)
            idxs.append(k)
            d = Fraction(float(a[j])) - E2M1[k] * Fraction(float(eff))
            weight = Fraction(1) if h16 is None else Fraction(float(f32(h16[j])))
            total += weight * d * d
        losses.append(total)
        qidx.append(idxs)
    return losses, qidx
