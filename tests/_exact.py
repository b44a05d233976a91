"""Threshold-selection counts decided in exact rational arithmetic.

Test infrastructure (the exact-rational pin of the selection): every float32
value is a dyadic rational, an integer times 2^-149 at the finest, so a row's
masses scaled by 2^149 are Python integers and their prefix sums are exact.
The threshold, a binary64, is compared as the rational it encodes
(``fractions.Fraction``).  No rounding happens anywhere, so the count this
returns is the one the selection rule defines -- sort by descending mass,
keep the smallest prefix whose mass reaches tau, every block when tau >= 1
or when no prefix reaches it (ubos.tech blog, "How It Works in Practice",
Phase 2; mlsanity.com paper index, "Abstract (arXiv)").  The order of equal
masses does not change any prefix sum, so the count does not depend on the
tie-break.
"""

from fractions import Fraction

import numpy as np

SCALE_BITS = 149  # 2^-149 is the smallest positive float32


def scaled_ints(x):
    """float32 values (finite, >= 0) times 2^149, as exact Python integers
    (object array of the same shape)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.isfinite(x).all() or (np.signbit(x) & (x != 0)).any():
        raise ValueError("masses must be finite and >= 0")
    bits = x.view(np.uint32).astype(np.int64)
    exp = (bits >> 23) & 0xFF
    man = bits & 0x7FFFFF
    # normal: (2^23 + man) * 2^(exp - 150); denormal and zero: man * 2^-149
    sig = np.where(exp == 0, man, man | (1 << 23)).astype(object)
    shift = np.maximum(exp - 1, 0).astype(object)
    return np.left_shift(sig, shift)


def exact_counts(mass, tau, chunk=2048):
    """Count of kept blocks per row of ``mass`` (``[R, nb]`` float32) for the
    threshold ``tau`` (a Python float), in exact arithmetic."""
    mass = np.asarray(mass, dtype=np.float32)
    rows, nb = mass.shape
    out = np.full(rows, nb, dtype=np.int64)
    if tau >= 1.0:
        return out
    t = Fraction(tau)
    # S * 2^-149 >= num/den  <=>  S >= ceil(num * 2^149 / den) for integer S
    thr = -((-t.numerator << SCALE_BITS) // t.denominator)
    for a in range(0, rows, chunk):
        part = -np.sort(-mass[a:a + chunk], axis=1)
        sums = np.cumsum(scaled_ints(part), axis=1)
        hit = (sums >= thr).astype(bool)
        reached = hit.any(axis=1)
        out[a:a + chunk] = np.where(reached, hit.argmax(axis=1) + 1, nb)
    return out
