"""Pins for the oracle's projections, scores and ranking.

Each check compares the oracle with something other than itself: hand-worked
values, exact rational arithmetic, special cases that reduce to a plain matrix
product, a brute-force q^T (P P^T) k with its rounding bound, invariants that
the definition implies, and Python's ``sorted``.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import bf16, predictor

U = 2.0 ** -8   # unit roundoff of bf16 (8 significant bits, round to nearest)


def _bits(x):
    return bf16.encode(np.asarray(x, dtype=np.float64))


def _rand_bits(rng, shape, scale=1.0):
    return _bits(rng.standard_normal(shape) * scale)


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ------------------------------------------------------------ hand-worked values

def test_hand_a1(golden_dir):
    g = _load(golden_dir, "hand_a1.json")
    P = _bits(g["P"])
    q = _bits(g["q"])
    qp = predictor.project_q(q, P)
    assert np.array_equal(bf16.decode(qp), np.array(g["q_proj"], float))
    k = _bits(g["k_blocks"])                          # [n, B, Hk, D]
    slots = predictor.project_kv_slots(k, P)          # [n, Hk, B, R]
    assert np.array_equal(bf16.decode(slots), np.array(g["a_slots"], float))
    a_g = np.zeros((1, 2, 1, 2, 2), np.uint16)
    predictor.project_kv_block(a_g, 0, k, [0, 1], P)
    s = predictor.score_blocks(qp[None, None, None], a_g, 0, None, 2)
    assert s[0, 0].tolist() == g["scores"]
    assert predictor.rank_victims(s[0].astype(np.float32))[0].tolist() == g["victims"]
    # same keys written through a swapped table: scores by logical index do not move
    a_sw = np.zeros_like(a_g)
    predictor.project_kv_block(a_sw, 0, k, g["swapped_table"]["table"], P)
    s_sw = predictor.score_blocks(qp[None, None, None], a_sw, 0, np.array([g["swapped_table"]["table"]]), 2)
    assert s_sw[0, 0].tolist() == g["swapped_table"]["scores"]
    # tie: block 1 with block 0's keys -> equal scores, lower index first
    k_tie = k.copy()
    k_tie[1] = k[0]
    a_t = np.zeros_like(a_g)
    predictor.project_kv_block(a_t, 0, k_tie, [0, 1], P)
    s_t = predictor.score_blocks(qp[None, None, None], a_t, 0, None, 2)
    assert s_t[0, 0].tolist() == g["tie_variant"]["scores"]
    assert predictor.rank_victims(s_t[0].astype(np.float32))[0].tolist() == g["tie_variant"]["victims"]
    # planted block
    kp = np.broadcast_to(_bits(g["planted"]["k"]), (1, 2, 1, 4)).copy()
    sp = predictor.project_kv_slots(kp, P)
    assert bf16.decode(sp[0, 0, 0]).tolist() == g["planted"]["a"]
    assert predictor.score_one(qp[None], sp).tolist() == [g["planted"]["score"]]
    # brute force q1^T (P P^T) k
    Pf = bf16.decode(P)
    q1 = bf16.decode(q[1])
    k10 = bf16.decode(k[1, 0, 0])
    assert q1 @ Pf @ Pf.T @ k10 == g["brute_force"]["value"]


def test_hand_a2_layout_and_gqa(golden_dir):
    g = _load(golden_dir, "hand_a2.json")
    P = _bits(g["P"])
    q = _bits(g["q"])
    qp = predictor.project_q(q, P)
    assert np.array_equal(bf16.decode(qp), np.array(g["q_proj"], float))
    k = _bits(g["k_block"])[None]                     # [1, B, Hk, D]
    a_g = np.zeros((1, 1, 2, 2, 2), np.uint16)
    predictor.project_kv_block(a_g, 0, k, [0], P)
    assert bf16.decode(a_g[0, 0]).ravel().tolist() == g["a_slot_flat"]
    s = predictor.score_blocks(qp[None, None, None], a_g, 0, None, 1)
    assert s[0, 0, 0] == g["score"]
    # the h mod nkv reading would give a different value on this example
    qm = qp[[0, 2, 1, 3]]                             # heads regrouped as h mod 2
    assert predictor.score_one(qm[None], a_g[0]).tolist() == [g["score_with_h_mod_nkv_mapping"]]


# --------------------------------------------------------------- projections

def _rne_fraction(fr):
    """Exact RNE of a Fraction to bf16 by searching the binade (normal range only)."""
    if fr == 0:
        return 0.0
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    assert e >= -126
    scaled = a * 128                      # 7 fraction bits
    lo = scaled.numerator // scaled.denominator
    rem = scaled - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * float(Fraction(lo, 128) * Fraction(2) ** e)


def test_projection_exact_rationals():
    rng = np.random.default_rng(3)
    for D, R in [(8, 4), (16, 8), (24, 8)]:
        x = _rand_bits(rng, (5, D))
        p = _rand_bits(rng, (D, R), 0.3)
        got = bf16.decode(predictor.project(x, p))
        xf, pf = bf16.decode(x), bf16.decode(p)
        for i in range(5):
            for j in range(R):
                exact = sum(Fraction(float(xf[i, d])) * Fraction(float(pf[d, j])) for d in range(D))
                assert got[i, j] == _rne_fraction(exact), (D, R, i, j)


def test_identity_projection_is_layout_pin():
    rng = np.random.default_rng(4)
    D = R = 16
    P = _bits(np.eye(D))
    q = _rand_bits(rng, (3, 4, D))
    assert np.array_equal(predictor.project_q(q, P), q)
    k = _rand_bits(rng, (5, 8, 2, D))                  # [n, B, Hk, D]
    slots = predictor.project_kv_slots(k, P)           # [n, Hk, B, R]
    assert np.array_equal(slots, k.transpose(0, 2, 1, 3))


def test_signed_permutation_projection_is_exact():
    rng = np.random.default_rng(5)
    D = R = 8
    perm = rng.permutation(D)
    signs = rng.choice([-1.0, 1.0], D)
    Pm = np.zeros((D, R))
    Pm[np.arange(D), perm] = signs * 0.5               # power-of-two scale stays exact
    x = _rand_bits(rng, (10, D))
    got = bf16.decode(predictor.project(x, _bits(Pm)))
    want = np.zeros((10, R))
    want[:, perm] = bf16.decode(x) * signs * 0.5
    assert np.array_equal(got, want)


# -------------------------------------------------------------------- scores

def _setup(rng, L=1, Hq=4, Hk=2, D=16, R=8, B=4, N=6, scale_k=1.0):
    P = _rand_bits(rng, (D, R), 1 / np.sqrt(R))
    a_g = np.zeros((L, N, Hk, B, R), np.uint16)
    for l in range(L):
        k = _rand_bits(rng, (N, B, Hk, D), scale_k)
        predictor.project_kv_block(a_g, l, k, np.arange(N), P)
    return P, a_g


def test_brute_force_through_projection():
    """score vs max q^T (P P^T) k in float64 without intermediate rounding, within the bf16 bound."""
    rng = np.random.default_rng(6)
    Hq, Hk, D, R, B, N = 4, 2, 16, 8, 4, 5
    g = Hq // Hk
    P = _rand_bits(rng, (D, R), 1 / np.sqrt(R))
    k = _rand_bits(rng, (N, B, Hk, D))
    q = _rand_bits(rng, (1, Hq, D))
    a_g = np.zeros((1, N, Hk, B, R), np.uint16)
    predictor.project_kv_block(a_g, 0, k, np.arange(N), P)
    qp = predictor.project_q(q, P)
    s = predictor.score_blocks(qp[None, None], a_g, 0, None, N)[0, 0]
    Pf = bf16.decode(P)
    M = Pf @ Pf.T
    qf, kf = bf16.decode(q), bf16.decode(k)
    for b in range(N):
        best, mag = -np.inf, 0.0
        for h in range(Hq):
            for t in range(B):
                v = qf[0, h] @ M @ kf[b, t, h // g]
                best = max(best, v)
                mag = max(mag, np.sum(np.abs((qf[0, h] @ Pf) * (kf[b, t, h // g] @ Pf))))
        assert abs(s[b] - best) <= (2 * U + U * U) * mag * (1 + 2.0 ** -40), (b, s[b], best)


def test_identity_projection_score_is_max_logit():
    """With P = I the score is the max raw (unscaled) q.k logit over heads, rows and tokens."""
    rng = np.random.default_rng(8)
    Hq, Hk, D, B, N, M = 8, 2, 8, 4, 7, 3
    g = Hq // Hk
    P = _bits(np.eye(D))
    k = _rand_bits(rng, (N, B, Hk, D))
    q = _rand_bits(rng, (M, Hq, D))
    a_g = np.zeros((1, N, Hk, B, D), np.uint16)
    predictor.project_kv_block(a_g, 0, k, np.arange(N), P)
    qp = predictor.project_q(q, P)
    s = predictor.score_blocks(qp[None, None], a_g, 0, None, N)[0, 0]
    qf, kf = bf16.decode(q), bf16.decode(k)
    for b in range(N):
        logits = [float(np.dot(qf[i, h], kf[b, t, h // g]))
                  for i in range(M) for h in range(Hq) for t in range(B)]
        assert s[b] == max(logits)


def test_invariants():
    rng = np.random.default_rng(9)
    Hq, Hk, D, R, B, N, M = 8, 2, 16, 8, 4, 9, 3
    g = Hq // Hk
    P, a_g = _setup(rng, Hq=Hq, Hk=Hk, D=D, R=R, B=B, N=N)
    qp = predictor.project_q(_rand_bits(rng, (M, Hq, D)), P)
    base = predictor.score_blocks(qp[None, None], a_g, 0, None, N)[0, 0]

    # physical placement: move the slots and route through a table
    perm = rng.permutation(N)
    moved = np.empty_like(a_g)
    moved[0, perm] = a_g[0]
    s = predictor.score_blocks(qp[None, None], moved, 0, perm[None], N)[0, 0]
    assert np.array_equal(s, base)

    # token order inside a block
    tok = rng.permutation(B)
    s = predictor.score_blocks(qp[None, None], a_g[:, :, :, tok], 0, None, N)[0, 0]
    assert np.array_equal(s, base)

    # query heads permuted inside a GQA group
    hp = np.concatenate([k * g + rng.permutation(g) for k in range(Hk)])
    s = predictor.score_blocks(qp[:, hp][None, None], a_g, 0, None, N)[0, 0]
    assert np.array_equal(s, base)

    # GQA expansion: nkv = nq with each kv head replicated g times
    a_exp = np.repeat(a_g, g, axis=2)
    s = predictor.score_blocks(qp[None, None], a_exp, 0, None, N)[0, 0]
    assert np.array_equal(s, base)

    # several query rows = max of single-row scores
    singles = [predictor.score_blocks(qp[i:i + 1][None, None], a_g, 0, None, N)[0, 0] for i in range(M)]
    assert np.array_equal(np.max(singles, axis=0), base)

    # batched sequences = per-sequence runs
    t2 = np.stack([rng.permutation(N), rng.permutation(N)])
    q2 = np.stack([qp, predictor.project_q(_rand_bits(rng, (M, Hq, D)), P)])
    both = predictor.score_blocks(q2[None], a_g, 0, t2, N)[0]
    for sidx in range(2):
        one = predictor.score_blocks(q2[sidx][None, None], a_g, 0, t2[sidx:sidx + 1], N)[0, 0]
        assert np.array_equal(both[sidx], one)

    # scaling the queries by 2**k scales every score by 2**k exactly
    q4 = _bits(bf16.decode(qp) * 4.0)
    s = predictor.score_blocks(q4[None, None], a_g, 0, None, N)[0, 0]
    assert np.array_equal(s, base * 4.0)
    assert np.array_equal(predictor.rank_victims(s[None].astype(np.float32)),
                          predictor.rank_victims(base[None].astype(np.float32)))


def test_planted_blocks_rank_last():
    """Blocks whose keys are 4x the first query head of their group score highest."""
    rng = np.random.default_rng(10)
    Hq, Hk, D, R, B, N = 8, 2, 32, 16, 4, 40
    g = Hq // Hk
    P = _rand_bits(rng, (D, R), 1 / np.sqrt(R))
    q = _rand_bits(rng, (1, Hq, D))
    k = _rand_bits(rng, (N, B, Hk, D))
    planted = rng.choice(N, 3, replace=False)
    for b in planted:
        for kk in range(Hk):
            k[b, :, kk, :] = _bits(bf16.decode(q[0, kk * g]) * 4.0)
    a_g = np.zeros((1, N, Hk, B, R), np.uint16)
    predictor.project_kv_block(a_g, 0, k, np.arange(N), P)
    qp = predictor.project_q(q, P)
    s = predictor.score_blocks(qp[None, None], a_g, 0, None, N)[0, 0]
    order = predictor.rank_victims(s[None].astype(np.float32))[0]
    assert sorted(order[-3:].tolist()) == sorted(planted.tolist())
    # identical planted scores keep index order among themselves
    assert order[-3:].tolist() == sorted(planted.tolist())


# -------------------------------------------------------------------- ranking

def _key_py(x):
    """Python-side reading of the ranking rule, on float values (NaN first, -0 == +0)."""
    if x != x:
        return (0, 0.0)
    return (1, x + 0.0)


def test_rank_matches_python_sorted():
    rng = np.random.default_rng(12)
    for n in [1, 2, 7, 64, 300]:
        s = rng.integers(-5, 6, size=(3, n)).astype(np.float32) * 0.5   # many ties
        s[0, :: max(1, n // 3)] = -0.0
        s[1, :: max(1, n // 4)] = np.nan
        s[2, 0] = -np.inf
        if n > 1:
            s[2, -1] = np.inf
        got = predictor.rank_victims(s)
        for row in range(3):
            vals = [float(v) for v in s[row]]
            want = sorted(range(n), key=lambda b: (_key_py(vals[b]), b))
            assert got[row].tolist() == want
            assert sorted(got[row].tolist()) == list(range(n))


def test_order_key_monotone():
    vals = np.array([-np.inf, -3.5, -1e-30, -0.0, 0.0, 1e-45, 2.0, np.inf], np.float32)
    keys = predictor.order_key(vals).astype(np.int64)
    assert keys[3] == keys[4]
    assert np.all(np.diff(np.delete(keys, 3)) > 0)
    assert predictor.order_key(np.array([np.nan], np.float32))[0] == 0
    assert keys.min() > 0


def test_select_is_the_sorted_prefix():
    """select_victims against Python's sorted() truncated to k, on rows with many ties, -0, NaN and inf."""
    rng = np.random.default_rng(13)
    for n in [1, 5, 64, 300]:
        s = rng.integers(-4, 5, size=(2, n)).astype(np.float32) * 0.25
        s[0, :: max(1, n // 5)] = -0.0
        s[1, :: max(1, n // 7)] = np.nan
        s[1, -1] = -np.inf
        for k in sorted({0, 1, n // 2, n - 1, n} - {-1}):
            got = predictor.select_victims(s, k)
            assert got.shape == (2, k)
            for row in range(2):
                vals = [float(v) for v in s[row]]
                want = sorted(range(n), key=lambda b: (_key_py(vals[b]), b))[:k]
                assert got[row].tolist() == want


# ------------------------------------------------- per-row causal keep sets

def _f(x):
    return np.array([[float(v) for v in row] for row in x])


def test_hand_keep(golden_dir):
    g = _load(golden_dir, "hand_keep.json")
    rc = g["rows_case"]
    s = predictor.score_rows(_bits(rc["q_proj"]), _bits(rc["slots"]), rc["first_pos"], rc["stride"])
    assert np.array_equal(s, _f(rc["scores"]))
    keep = predictor.keep_sets(s.astype(np.float32), rc["first_pos"], 2, 2)
    assert keep.tolist() == rc["keep_top2"]
    kc = g["keep_case"]
    s = _f(kc["scores"]).astype(np.float32)
    assert predictor.keep_sets(s, kc["first_pos"], kc["ratio"], 2).tolist() == kc["keep_top2"]
    assert predictor.keep_sets(s, kc["first_pos"], kc["ratio"], 3).tolist() == kc["keep_top3"]


def _keep_py(row, c, topk):
    """The page's comparator written out: larger score first, then lower index; NaN after numbers."""
    import functools

    def cmp(a, b):
        va, vb = float(row[a]), float(row[b])
        na, nb = va != va, vb != vb
        if na != nb:
            return 1 if na else -1
        if not na and va != vb:
            return -1 if va > vb else 1
        return -1 if a < b else (1 if a > b else 0)

    order = sorted(range(c), key=functools.cmp_to_key(cmp))[:topk]
    return order + [-1] * (topk - len(order))


def test_keep_sets_match_python_sorted():
    rng = np.random.default_rng(77)
    for trial in range(60):
        rows = int(rng.integers(1, 7))
        stride = int(rng.integers(1, 40))
        ratio = int(rng.integers(1, 9))
        first_pos = int(rng.integers(0, 3 * stride))
        topk = int(rng.integers(0, stride + 1))
        s = (rng.integers(-6, 6, size=(rows, stride)) * 0.5).astype(np.float32)   # many ties
        s[rng.random(s.shape) < 0.1] = -0.0
        s[rng.random(s.shape) < 0.05] = np.nan
        s[rng.random(s.shape) < 0.05] = -np.inf
        got = predictor.keep_sets(s, first_pos, ratio, topk)
        for i in range(rows):
            # complete blocks: every one of the block's ratio positions is at or before the row's
            c = sum(1 for b in range(stride) if (b + 1) * ratio - 1 <= first_pos + i)
            assert got[i].tolist() == _keep_py(s[i], c, topk), (trial, i)


def test_keep_sets_are_prefixes():
    rng = np.random.default_rng(5)
    s = rng.standard_normal((9, 50)).astype(np.float32)
    full = predictor.keep_sets(s, 40, 4, 50)
    for k in (0, 1, 7, 11, 50):
        assert np.array_equal(predictor.keep_sets(s, 40, 4, k), full[:, :k])


def test_score_rows_brute_force():
    rng = np.random.default_rng(12)
    rows, Hq, Hk, R, B, n = 5, 4, 2, 3, 3, 4
    q = _rand_bits(rng, (rows, Hq, R))
    a = _rand_bits(rng, (n, Hk, B, R))
    qd, ad = bf16.decode(q), bf16.decode(a)
    for first_pos in (0, 2, 6, 30):
        for stride in (3, 4, 6):
            got = predictor.score_rows(q, a, first_pos, stride)
            for i in range(rows):
                for b in range(stride):
                    visible = b < n and (b + 1) * B - 1 <= first_pos + i
                    if not visible:
                        assert got[i, b] == -np.inf
                        continue
                    best = max(sum(float(qd[i, h, j]) * float(ad[b, h // (Hq // Hk), t, j]) for j in range(R))
                               for h in range(Hq) for t in range(B))
                    assert abs(got[i, b] - best) <= 1e-12 * max(1.0, abs(best)), (first_pos, stride, i, b)


def test_score_rows_all_complete_reduces_to_score_blocks():
    """When every block is complete for every row, the max over rows is score_blocks' score."""
    rng = np.random.default_rng(3)
    q = _rand_bits(rng, (6, 8, 16))
    a = _rand_bits(rng, (10, 2, 4, 16))
    s = predictor.score_rows(q, a, 10 * 4, 10)
    assert np.isfinite(s).all()
    assert np.allclose(s.max(axis=0), predictor.score_one(q, a), rtol=1e-12, atol=1e-12)


# ------------------------------------------------- partial last blocks

def test_masked_score_brute_force():
    rng = np.random.default_rng(21)
    M, Hq, Hk, R, B, n = 2, 4, 2, 3, 4, 3
    q = _rand_bits(rng, (M, Hq, R))
    a = _rand_bits(rng, (n, Hk, B, R))
    qd, ad = bf16.decode(q), bf16.decode(a)
    for fill in range(0, B + 1):
        got = predictor.score_one(q, a, fill)
        for b in range(n):
            toks = range(fill) if b == n - 1 else range(B)
            vals = [sum(float(qd[i, h, j]) * float(ad[b, h // (Hq // Hk), t, j]) for j in range(R))
                    for i in range(M) for h in range(Hq) for t in toks]
            best = max(vals) if vals else -np.inf
            assert got[b] == best or abs(got[b] - best) <= 1e-12 * max(1.0, abs(best)), (fill, b)


def test_masked_score_equals_duplicated_tokens():
    """Masking tokens t >= fill equals overwriting them with copies of token 0 (a max ignores duplicates)."""
    rng = np.random.default_rng(8)
    q = _rand_bits(rng, (3, 8, 16))
    a = _rand_bits(rng, (6, 2, 8, 16))
    assert np.array_equal(predictor.score_one(q, a, 8), predictor.score_one(q, a))
    for fill in (1, 3, 7):
        dup = a.copy()
        dup[-1, :, fill:] = dup[-1, :, :1]
        assert np.allclose(predictor.score_one(q, a, fill), predictor.score_one(q, dup), rtol=1e-12, atol=1e-12)
    assert predictor.score_one(q, a, 0)[-1] == -np.inf
    assert np.array_equal(predictor.score_one(q, a, 0)[:-1], predictor.score_one(q, a)[:-1])
