"""bfloat16 codec for the oracle (test infrastructure only).

Decode: a bf16 value is the upper half of an IEEE-754 binary32 word, as the
``qsa_select.rs`` page shows when it rebuilds f32 from ``u16 << 16`` in its
norm probes.

Encode: round-to-nearest, ties-to-even, *once*, from a float64 value, keeping
bf16 subnormals and overflowing to +/-inf.  The page set never states a rounding
mode (``predictor.rs`` takes bf16 from the ``half`` crate); RNE is the reading
taken.  This module computes it from the definition: pick the quantum
``q = 2**(max(e, -125) - 8)`` where ``x = m * 2**e`` with ``0.5 <= |m| < 1``
(8 significant bits for normal values; the fixed subnormal step ``2**-133``
below ``2**-126``), divide (exact: a power-of-two scale), round half-even with
``numpy.rint``, multiply back, and map ``|y| >= 2**128`` to infinity.

Pins (``tests/test_oracle_bf16.py``): decode against values fixed by the
binary32 format; encode against an exact ``fractions.Fraction`` rounding at
constructed midpoints, at the subnormal boundary and at the overflow threshold;
``encode(decode(b)) == b`` for every non-NaN pattern.
"""

import numpy as np

_POS_INF = np.uint16(0x7F80)
_QNAN = np.uint16(0x7FC0)


def decode(bits):
    """bf16 bit patterns (uint16 array) -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    w = b.astype(np.uint32) << np.uint32(16)
    return w.view(np.float32).astype(np.float64)


def round_to_bf16_grid(x):
    """Round float64 values to the nearest bf16 value (RNE), returned as float64.

    Overflow gives +/-inf; NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    finite = np.isfinite(x)
    xf = x[finite]
    _, e = np.frexp(xf)  # xf = m * 2**e, 0.5 <= |m| < 1 (e = 0 for xf == 0)
    qexp = np.maximum(e, -125) - 8
    y = np.ldexp(np.rint(np.ldexp(xf, -qexp)), qexp)
    y = np.where(np.abs(y) >= 2.0 ** 128, np.copysign(np.inf, xf), y)
    out[finite] = y
    out[~finite] = x[~finite]
    return out


def encode(x):
    """float64 values -> bf16 bit patterns (uint16), RNE from the float64 value."""
    x = np.asarray(x, dtype=np.float64)
    y = round_to_bf16_grid(x)
    nan = np.isnan(y)
    # y is exactly representable in binary32 with a zero low half (or is +/-inf),
    # so the float32 cast is exact and the top 16 bits are the bf16 pattern.
    w = np.where(nan, 0.0, y).astype(np.float32).view(np.uint32)
    bits = (w >> np.uint32(16)).astype(np.uint16)
    bits[nan] = _QNAN
    return bits


def ordinal(bits):
    """Signed ordinal of bf16 patterns: consecutive representable values differ by 1.

    +0 and -0 both map to 0.  Used to measure distances in ulps.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)
