"""The library's float64 -> bf16 rounding (``f64_to_bf16_rne`` in ``csrc/common.h``, used by
every projection kernel and the host projection builder) against the oracle's encoder, which
rounds from the definition: a host program built from the header converts constructed ties and
near-ties at every bf16 exponent (normal and subnormal), the range edges, zeros, infinities,
NaN and random float64 bit patterns.  Round to nearest, ties to even, once from float64
(predictor.rs page, project_q / project_kv_block: bf16 results; the rounding mode is the
reading the oracle takes)."""

import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import bf16

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

PROGRAM = r"""
#include "common.h"
#include <cstdio>
#include <vector>
int main(int argc, char** argv) {
    FILE* f = fopen(argv[1], "rb");
    std::vector<double> x;
    double v;
    while (fread(&v, sizeof v, 1, f) == 1) x.push_back(v);
    fclose(f);
    std::vector<uint16_t> y(x.size());
    for (size_t i = 0; i < x.size(); ++i) y[i] = pred::f64_to_bf16_rne(x[i]);
    FILE* g = fopen(argv[2], "wb");
    fwrite(y.data(), sizeof(uint16_t), y.size(), g);
    fclose(g);
    return 0;
}
"""


def _inputs():
    rng = np.random.default_rng(7)
    xs = []
    # midpoints between neighbouring bf16 values, and the float64 values next to them, at every
    # exponent from the subnormal range to the top of the normal range
    for e in range(-134, 128):
        frac = np.arange(256, dtype=np.float64)
        if e < -126:   # subnormal grid: fixed step 2^-133
            base = (frac[: 2 ** max(0, e + 134)] + 0.5) * 2.0 ** -133
        else:
            base = (1.0 + (frac[:128] + 0.5) / 128.0) * 2.0 ** e
        bits = base.view(np.uint64)
        for d in (-2, -1, 0, 1, 2):
            xs.append((bits.astype(np.int64) + d).astype(np.uint64).view(np.float64))
    edges = [0.0, -0.0, np.inf, -np.inf, 2.0 ** -126, np.nextafter(2.0 ** -126, 0.0), 2.0 ** -133,
             2.0 ** -134, np.nextafter(2.0 ** -134, 1.0), 2.0 ** 128, np.nextafter(2.0 ** 128, 0.0),
             (2.0 - 2.0 ** -8) * 2.0 ** 127, (2.0 - 2.0 ** -7) * 2.0 ** 127, 1.7976931348623157e308,
             5e-324, -5e-324, 2.2250738585072014e-308]
    xs.append(np.array(edges))
    xs.append(-np.concatenate(xs))
    xs.append(rng.integers(0, 2 ** 63, 200000, dtype=np.uint64).view(np.float64))          # any pattern
    xs.append(rng.standard_normal(200000) * 2.0 ** rng.integers(-140, 130, 200000))
    x = np.concatenate(xs)
    return x[~np.isnan(x)]


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc not found")
def test_library_rounding_matches_oracle(tmp_path):
    src = tmp_path / "round.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "round"
    hipcc = HIPCC if os.path.exists(HIPCC) else shutil.which("hipcc")
    r = subprocess.run([hipcc, "-std=c++17", "-O2", "--offload-arch=gfx950", "-x", "hip",
                        "-I", os.path.join(ROOT, "rank_kv_block_amd", "csrc"), str(src), "-o", str(exe)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    x = _inputs()
    inp, out = tmp_path / "x.bin", tmp_path / "y.bin"
    x.astype("<f8").tofile(inp)
    r = subprocess.run([str(exe), str(inp), str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    got = np.fromfile(out, dtype="<u2")
    with np.errstate(over="ignore"):   # the oracle scales huge values past float64 before mapping them to inf
        want = bf16.encode(x)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (f"{bad.size} of {x.size} differ, first {x[bad[0]]!r}: "
                           f"library {got[bad[0]]:#06x}, oracle {want[bad[0]]:#06x}")
    # NaN goes to the quiet NaN pattern
    np.array([np.nan, -np.nan]).astype("<f8").tofile(inp)
    subprocess.run([str(exe), str(inp), str(out)], check=True, timeout=60)
    assert np.all(np.fromfile(out, dtype="<u2") == 0x7FC0)
