"""Seeded projection generator for the oracle (test infrastructure only).

The ``predictor.rs`` page builds ``P [head_dim, r]`` once, in the constructor,
from ``projection_seed`` (module invariants; ``new_on_stream`` calls
``build_projection``), but the generator's body is not on the pages.  The
reading taken: ``P`` holds independent N(0, 1/r) draws rounded to bf16, produced
by a counter-based generator that any implementation can rebuild from this
definition:

* ``mix64`` is the SplitMix64 output function (Steele, Lea & Flood, OOPSLA 2014):
  xor-shift 30, multiply 0xBF58476D1CE4E5B9, xor-shift 27, multiply
  0x94D049BB133111EB, xor-shift 31, all mod 2**64.
* With ``GAMMA = 0x9E3779B97F4A7C15``, a stream's state is
  ``s = mix64(seed + (stream + 1) * GAMMA)`` and its i-th 64-bit draw is
  ``x_i = mix64(s + (i + 1) * GAMMA)``: the i-th SplitMix64 output from state s.
* A uniform on (0, 1] is ``((x >> 11) + 1) * 2**-53``.
* Normal number i uses the cosine branch of Box and Muller (1958) on draws 2i and
  2i+1: ``sqrt(-2 ln u0) * cos(2 pi u1)`` in float64 (``2 pi`` written as the
  double 6.283185307179586).
* ``P[d, j] = bf16(z_{d*r + j} / sqrt(r))`` from stream 0.

This module writes the steps out with Python integers and ``math`` (libm), one
value at a time; it is only ever asked for a few thousand values.

Pins (``tests/test_oracle_prng.py``): the published SplitMix64 outputs for
state 0; uniform range; normal moments and a Kolmogorov-Smirnov test; P's mean,
variance and determinism.
"""

import math

import numpy as np

from . import bf16

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
TWO_PI = 6.283185307179586
PROJECTION_STREAM = 0


def mix64(z):
    z &= MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def splitmix64(state, count):
    """The first ``count`` outputs of SplitMix64 started from ``state``."""
    out = []
    for i in range(count):
        out.append(mix64(state + (i + 1) * GAMMA))
    return out


def stream_state(seed, stream):
    return mix64(seed + (stream + 1) * GAMMA)


def draw(seed, stream, i):
    return mix64(stream_state(seed, stream) + (i + 1) * GAMMA)


def uniform_from_bits(x):
    return ((x >> 11) + 1) * 2.0 ** -53


def normals(seed, stream, count):
    """Standard normal numbers 0..count-1 of a stream, as Python floats."""
    return normals_from_state(stream_state(seed, stream), count)


def normals_from_state(s, count):
    """Normal number i from SplitMix64 outputs 2i and 2i+1 of state ``s``."""
    out = []
    for i in range(count):
        u0 = uniform_from_bits(mix64(s + (2 * i + 1) * GAMMA))
        u1 = uniform_from_bits(mix64(s + (2 * i + 2) * GAMMA))
        out.append(math.sqrt(-2.0 * math.log(u0)) * math.cos(TWO_PI * u1))
    return out


def projection_f64(head_dim, r, seed):
    """Unrounded P values z / sqrt(r), float64 [head_dim, r]."""
    z = normals(seed, PROJECTION_STREAM, head_dim * r)
    scale = math.sqrt(float(r))
    vals = [v / scale for v in z]
    return np.array(vals, dtype=np.float64).reshape(head_dim, r)


def projection(head_dim, r, seed):
    """P [head_dim, r] as bf16 bit patterns (uint16)."""
    return bf16.encode(projection_f64(head_dim, r, seed))
