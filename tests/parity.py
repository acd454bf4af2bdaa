"""Comparison rules between the HIP path and the oracle (shared by the GPU tests and smoke()).

* bf16 tensors (q_proj, A_g): at most 1 bf16 ulp apart, element by element.
* scores: |gpu - oracle| <= max(1e-3 * |oracle|, 1e-3 * sqrt(r)), the oracle
  recomputing from the GPU's own q_proj and A_g.
* ranking: (i) bit-exact against the oracle's ranking of the GPU's own scores;
  (ii) against the oracle's float64 scores, at every cut where neighbouring
  oracle scores differ by more than the score tolerance, the first k victims
  form the same set.
"""

import numpy as np

from oracle import bf16, predictor


def max_ulp(a_bits, b_bits):
    a = bf16.ordinal(np.asarray(a_bits).view(np.uint16))
    b = bf16.ordinal(np.asarray(b_bits).view(np.uint16))
    return int(np.max(np.abs(a - b))) if a.size else 0


def assert_ulp(gpu_bits, want_bits, what, limit=1):
    g = np.asarray(gpu_bits).view(np.uint16)
    w = np.asarray(want_bits).view(np.uint16)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    d = np.abs(bf16.ordinal(g) - bf16.ordinal(w))
    if d.size and d.max() > limit:
        i = np.unravel_index(np.argmax(d), d.shape)
        raise AssertionError(f"{what}: {int(d.max())} ulp apart at {i} (gpu {hex(g[i])}, oracle {hex(w[i])}); "
                             f"{int((d > limit).sum())} elements over {limit} ulp")


def score_tol(oracle_scores, r):
    return np.maximum(1e-3 * np.abs(oracle_scores), 1e-3 * np.sqrt(r))


def assert_scores(gpu, want, r, what="scores"):
    gpu = np.asarray(gpu, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert gpu.shape == want.shape, (what, gpu.shape, want.shape)
    err = np.abs(gpu - want)
    tol = score_tol(want, r)
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} outside tolerance; worst at {i}: gpu {gpu[i]!r}, "
                             f"oracle {want[i]!r}, tol {tol[i]!r}")


def assert_ranking(victims, gpu_scores, oracle_scores, r, what="victims"):
    victims = np.asarray(victims)
    gpu_scores = np.atleast_2d(np.asarray(gpu_scores, dtype=np.float32))
    oracle_scores = np.atleast_2d(np.asarray(oracle_scores, dtype=np.float64))
    # (i) exact against the oracle's sort of the GPU's own scores
    want = predictor.rank_victims(gpu_scores)
    if not np.array_equal(victims, want):
        row, col = np.argwhere(victims != want)[0]
        raise AssertionError(f"{what} (i): row {row} differs first at position {col}: "
                             f"gpu {victims[row, col]}, oracle {want[row, col]}")
    # (ii) set equality at every well-separated cut of the oracle's own order
    n = victims.shape[1]
    for row in range(victims.shape[0]):
        o = oracle_scores[row]
        order = np.argsort(o, kind="stable")
        srt = o[order]
        pos_gpu = np.empty(n, np.int64)
        pos_gpu[victims[row]] = np.arange(n)
        prefix_max = np.maximum.accumulate(pos_gpu[order])
        gap = srt[1:] - srt[:-1]
        tol = np.maximum(1e-3 * np.maximum(np.abs(srt[1:]), np.abs(srt[:-1])), 1e-3 * np.sqrt(r))
        cuts = np.nonzero(gap > tol)[0] + 1          # first-k sets at these k
        bad = cuts[prefix_max[cuts - 1] != cuts - 1]
        if bad.size:
            raise AssertionError(f"{what} (ii): row {row}: first {bad[0]} victims differ from the oracle's "
                                 f"set across a gap of {gap[bad[0] - 1]!r}")
