"""Pins for the oracle's bf16 codec against the binary32 format and exact rounding."""

import bisect
from fractions import Fraction

import numpy as np
import pytest

from oracle import bf16

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_decode_fixed_values():
    # values fixed by the binary32 format (bf16 = top half of a binary32 word)
    cases = {
        0x0000: 0.0,
        0x3F80: 1.0,
        0xBF80: -1.0,
        0x4000: 2.0,
        0x4049: 3.140625,
        0x3E80: 0.25,
        0x0080: 2.0 ** -126,            # smallest normal
        0x0001: 2.0 ** -133,            # smallest subnormal
        0x007F: 127 * 2.0 ** -133,      # largest subnormal
        0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127,  # largest finite
    }
    for bits, val in cases.items():
        assert bf16.decode(np.array([bits], np.uint16))[0] == val, hex(bits)
    assert np.isposinf(bf16.decode(np.array([0x7F80], np.uint16))[0])
    assert np.isneginf(bf16.decode(np.array([0xFF80], np.uint16))[0])
    assert np.isnan(bf16.decode(np.array([0x7FC0], np.uint16))[0])
    negz = bf16.decode(np.array([0x8000], np.uint16))[0]
    assert negz == 0.0 and np.signbit(negz)


def _finite_table():
    """All finite bf16 values (as exact Fractions) in ascending order with their patterns."""
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bf16.decode(pats)
    keep = np.isfinite(vals) & ~((pats == 0x8000))
    pairs = sorted((Fraction(float(v)), int(p)) for v, p in zip(vals[keep], pats[keep]))
    return [v for v, _ in pairs], [p for _, p in pairs]


_TABLE = None


def _nearest_even(x):
    """Brute force RNE: nearest finite bf16 by search over the sorted value table; ties to even pattern."""
    global _TABLE
    if _TABLE is None:
        _TABLE = _finite_table()
    vals, pats = _TABLE
    fx = Fraction(float(x))
    maxv = vals[-1]
    half_ulp_top = Fraction(2) ** 127 * Fraction(1, 2 ** 8)   # half the top binade's step (2**120)
    if fx >= maxv + half_ulp_top:
        return 0x7F80
    if fx <= -(maxv + half_ulp_top):
        return 0xFF80
    i = bisect.bisect_left(vals, fx)
    cands = [j for j in (i - 1, i) if 0 <= j < len(vals)]
    best = min(cands, key=lambda j: (abs(vals[j] - fx), pats[j] & 1))
    p = pats[best]
    if vals[best] == 0:
        return 0x8000 if np.signbit(x) else 0x0000
    return p


def test_encode_roundtrip_all_patterns():
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bf16.decode(pats)
    ok = ~np.isnan(vals)
    assert np.array_equal(bf16.encode(vals[ok]), pats[ok])
    assert np.all(bf16.encode(vals[~ok]) == 0x7FC0)


def test_encode_midpoints_tie_to_even():
    rng = np.random.default_rng(7)
    pats = rng.integers(0, 0x7F7F, size=4000).astype(np.uint16)   # positive finite, below max
    lo = bf16.decode(pats)
    hi = bf16.decode(pats + 1)
    mid = (lo + hi) / 2        # exact in float64
    got = bf16.encode(mid)
    want = np.where(pats % 2 == 0, pats, pats + 1).astype(np.uint16)
    assert np.array_equal(got, want)
    # just above / below a midpoint goes to the nearer neighbour
    assert np.array_equal(bf16.encode(np.nextafter(mid, np.inf)), (pats + 1).astype(np.uint16))
    assert np.array_equal(bf16.encode(np.nextafter(mid, -np.inf)), pats)
    # negative side mirrors
    assert np.array_equal(bf16.encode(-mid), want | np.uint16(0x8000))


def test_encode_against_brute_force_search():
    rng = np.random.default_rng(11)
    xs = np.concatenate([
        rng.standard_normal(600) * 10.0 ** rng.integers(-5, 6, 600),
        rng.standard_normal(100) * 2.0 ** -130,          # subnormal range
        rng.standard_normal(60) * 2.0 ** 127,             # near overflow
        np.array([2.0 ** -134, 2.0 ** -134 * 1.0000001, 3 * 2.0 ** -134, 2.0 ** -135,
                  (2 - 2.0 ** -8) * 2.0 ** 127, np.nextafter((2 - 2.0 ** -8) * 2.0 ** 127, 0),
                  2.0 ** -126 - 2.0 ** -134, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 0.0, -0.0]),
    ])
    got = bf16.encode(xs)
    want = np.array([_nearest_even(x) for x in xs], dtype=np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(xs[i], hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_overflow_and_subnormal_boundaries():
    top = (2 - 2.0 ** -8) * 2.0 ** 127          # midpoint between max finite and 2**128
    assert bf16.encode(np.array([top]))[0] == 0x7F80           # tie -> even -> overflow
    assert bf16.encode(np.array([np.nextafter(top, 0)]))[0] == 0x7F7F
    assert bf16.encode(np.array([2.0 ** -134]))[0] == 0x0000    # half the smallest subnormal: tie -> 0
    assert bf16.encode(np.array([np.nextafter(2.0 ** -134, 1)]))[0] == 0x0001
    assert bf16.encode(np.array([3 * 2.0 ** -134]))[0] == 0x0002  # tie between 1 and 2 -> even
    assert bf16.encode(np.array([np.inf, -np.inf]))[0] == 0x7F80


def test_ordinal_distance():
    pats = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x3F80, 0x3F81, 0xBF80], np.uint16)
    assert bf16.ordinal(pats).tolist() == [0, 0, 1, -1, 0x3F80, 0x3F81, -0x3F80]
