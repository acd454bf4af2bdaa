"""Pins for the oracle's projection generator (SplitMix64 + Box-Muller, N(0, 1/r) in bf16)."""

import math

import numpy as np
import pytest
from scipy import stats

from oracle import bf16, prng


def test_splitmix64_published_vector():
    # SplitMix64 from state 0: the first outputs published with the generator's
    # reference implementation and reused as test vectors by later PRNG suites.
    assert prng.splitmix64(0, 3) == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_mix64_is_a_bijection_on_samples():
    xs = [prng.mix64(i * 0x1234567) for i in range(2000)]
    assert len(set(xs)) == len(xs)
    assert all(0 <= x < 2 ** 64 for x in xs)


def test_uniform_range():
    assert prng.uniform_from_bits(0) == 2.0 ** -53
    assert prng.uniform_from_bits((1 << 64) - 1) == 1.0
    us = [prng.uniform_from_bits(prng.draw(5, 1, i)) for i in range(5000)]
    assert min(us) > 0.0 and max(us) <= 1.0
    assert abs(np.mean(us) - 0.5) < 5 * math.sqrt(1 / 12 / len(us))


def test_normals_distribution():
    z = np.array(prng.normals(123, 0, 20000))
    n = z.size
    assert abs(z.mean()) < 5 / math.sqrt(n)
    assert abs(z.var() - 1.0) < 5 * math.sqrt(2.0 / n)
    assert stats.kstest(z, "norm").pvalue > 1e-4
    # the cosine branch of Box-Muller: odd and even draws are not interchangeable,
    # but a different stream must give different numbers
    assert prng.normals(123, 1, 8) != prng.normals(123, 0, 8)


def test_projection_moments_and_determinism():
    d, r = 128, 64
    p = prng.projection(d, r, 42)
    assert p.shape == (d, r) and p.dtype == np.uint16
    assert np.array_equal(p, prng.projection(d, r, 42))
    assert not np.array_equal(p, prng.projection(d, r, 43))
    v = bf16.decode(p)
    n = v.size
    sd = 1 / math.sqrt(r)
    assert abs(v.mean()) < 5 * sd / math.sqrt(n)
    assert abs(v.var() / (sd * sd) - 1.0) < 5 * math.sqrt(2.0 / n) + 2 ** -7
    # P is N(0, 1/r) rounded once to bf16: the rounding moves each value by <= 2**-8 relative
    raw = prng.projection_f64(d, r, 42)
    assert np.all(np.abs(v - raw) <= np.abs(raw) * 2.0 ** -8)


@pytest.mark.parametrize("d,r", [(64, 16), (128, 32)])
def test_projection_row_major_order(d, r):
    # element (d, j) is normal number d*r + j of stream 0
    p = prng.projection_f64(d, r, 9)
    z = prng.normals(9, 0, 3 * r + 2)
    assert p[3, 1] == z[3 * r + 1] / math.sqrt(r)
    assert p[0, 0] == z[0] / math.sqrt(r)


def test_normal_uses_consecutive_splitmix_outputs():
    # normal 0 from state 0 is built from the first two published SplitMix64 outputs
    x0, x1, x2 = 0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F
    u0 = ((x0 >> 11) + 1) / 2.0 ** 53
    u1 = ((x1 >> 11) + 1) / 2.0 ** 53
    z = prng.normals_from_state(0, 2)
    assert z[0] == math.sqrt(-2.0 * math.log(u0)) * math.cos(6.283185307179586 * u1)
    # and normal 1 starts at the third output
    u2 = ((x2 >> 11) + 1) / 2.0 ** 53
    assert abs(z[1]) <= math.sqrt(-2.0 * math.log(u2)) + 1e-15
