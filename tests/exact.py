"""Exact-rational brute force used to pin the oracle's quantizers.

Independent of the oracle's numpy code: every float operation is replaced by
exact rational arithmetic followed by an explicit nearest-representable
search (ties to even), and rint/clamp by a search over all candidate codes.
"""
from fractions import Fraction

import numpy as np

_F32_INF_EDGE = Fraction(2) ** 128 - Fraction(2) ** 103   # RNE overflow point


def _is_even_mantissa(v) -> bool:
    if isinstance(v, np.float16):
        return (int(np.array(v).view(np.uint16)) & 1) == 0
    return (int(np.array(v, dtype=np.float32).view(np.uint32)) & 1) == 0


def nearest(fr: Fraction, dtype=np.float32):
    """The dtype value nearest to the exact rational fr (ties to even)."""
    if dtype == np.float32 and abs(fr) >= _F32_INF_EDGE:
        return dtype(np.inf) if fr > 0 else dtype(-np.inf)
    if dtype == np.float16 and abs(fr) >= Fraction(65520):
        return dtype(np.inf) if fr > 0 else dtype(-np.inf)
    c = dtype(float(fr))
    cands = {c, np.nextafter(c, dtype(np.inf)), np.nextafter(c, dtype(-np.inf))}
    cands = [v for v in cands if np.isfinite(v)]
    return min(cands, key=lambda v: (abs(Fraction(float(v)) - fr),
                                     0 if _is_even_mantissa(dtype(v)) else 1))


def nearest_int(fr: Fraction, lo: int, hi: int) -> int:
    """Integer in [lo, hi] nearest to fr, ties to even, by search."""
    return min(range(lo, hi + 1), key=lambda c: (abs(fr - c), c % 2))


def quantize_row(xs):
    """Brute-force symmetric absmax int8 quantization of one fp32 row."""
    vals = [Fraction(float(v)) for v in xs]
    amax = max(abs(v) for v in vals)
    zero = ([0] * len(vals), np.float32(0))
    if amax == 0:
        return zero
    inv = nearest(Fraction(127) / amax)
    if not np.isfinite(inv):
        return zero
    scale = nearest(amax / 127)
    finv = Fraction(float(inv))
    codes = [nearest_int(Fraction(float(nearest(v * finv))), -127, 127) for v in vals]
    return codes, scale


def quantize_group_w4(ws):
    """Brute-force affine 4-bit quantization of one 64-weight group."""
    vals = [Fraction(float(v)) for v in ws]
    lo, hi = min(vals), max(vals)
    rng = Fraction(float(nearest(hi - lo)))
    gs = nearest(Fraction(float(nearest(rng / 15))), np.float16)
    gb = nearest(lo, np.float16)
    fgs, fgb = Fraction(float(gs)), Fraction(float(gb))
    if fgs == 0:
        return [0] * len(vals), gs, gb
    inv = Fraction(float(nearest(1 / fgs)))
    codes = []
    for v in vals:
        d = Fraction(float(nearest(v - fgb)))
        t = Fraction(float(nearest(d * inv)))
        codes.append(nearest_int(t, 0, 15))
    return codes, gs, gb
