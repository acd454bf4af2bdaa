"""GPU parity of the per-row causal scorer and the per-row keep sets (through the C ABI).

* pred_score_rows against oracle.score_rows, recomputed from the GPU's own A_g,
  within the score tolerance; -inf exactly where a block is not complete.
* pred_select_keep bit-exact against oracle.keep_sets of the same float32 scores
  (the GPU's own scores where they come from pred_score_rows); against the
  oracle's float64 scores the kept sets agree wherever the k-th and (k+1)-th
  oracle scores are further apart than the tolerance.
"""

import numpy as np
import pytest

import rank_kv_block_amd as rk
from oracle import bf16, predictor
from tests.devmem import a_g_layer
from tests.parity import assert_scores, score_tol

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print("[case]", *a, flush=True)


def _to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).cuda()


def _randn_bits(rng, shape, scale=1.0):
    return bf16.encode(rng.standard_normal(shape) * scale)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rk.lib()
    yield
    torch.cuda.synchronize()


def _workspace(stride, rows):
    b = rk.pred_rank_workspace_bytes(stride, rows)
    return torch.empty((b // 8 + 1,), dtype=torch.int64, device="cuda") if b else None


def _check_keep_sets(keep, gpu_scores, oracle_scores, first_pos, ratio, topk, r, what):
    """(i) exact against the oracle's keep sets of the GPU's scores; (ii) the same sets as the
    oracle's own float64 order wherever the cut at topk is well separated."""
    want = predictor.keep_sets(gpu_scores, first_pos, ratio, topk)
    if not np.array_equal(keep, want):
        row, col = np.argwhere(keep != want)[0]
        raise AssertionError(f"{what} (i): row {row} differs first at slot {col}: gpu {keep[row, col]}, "
                             f"oracle {want[row, col]}")
    if oracle_scores is None:
        return
    for i in range(keep.shape[0]):
        c = predictor.complete_blocks(first_pos, i, ratio, oracle_scores.shape[1])
        if c <= topk:
            assert set(keep[i, :c].tolist()) == set(range(c)), (what, i)
            continue
        o = oracle_scores[i, :c]
        srt = np.sort(o)[::-1]
        with np.errstate(invalid="ignore"):   # -inf columns past n: a NaN gap skips the check
            gap = srt[topk - 1] - srt[topk]
        if gap > 2 * score_tol(np.array([srt[topk - 1]]), r)[0]:
            assert set(keep[i].tolist()) == set(np.argsort(-o, kind="stable")[:topk].tolist()), (what, i)


# ------------------------------------------------------------- per-row scores

ROW_SHAPES = [
    # Hq, Hk, D, R, B, N, n, rows, first_pos, stride, table         path
    (32, 8, 64, 32, 16, 40, 40, 70, 500, 40, "perm"),             # mfma, r 32: three row parts, the last chunk partial
    (32, 8, 64, 32, 16, 40, 37, 45, 0, 43, "perm"),               # mfma, causal from position 0, ragged key group, tail columns
    (8, 2, 64, 64, 8, 96, 90, 100, 640, 90, "identity"),          # mfma, B 8: 4 blocks per key tile, 64 per group
    (4, 4, 32, 16, 32, 20, 20, 33, 37, 25, "identity"),           # mfma, r 16, B 32, one query head per kv head
    (8, 1, 64, 128, 16, 24, 24, 64, 200, 24, "perm"),             # mfma, r 128, g 8: four stages per chunk
    (16, 8, 64, 128, 16, 20, 20, 40, 300, 20, "perm"),            # mfma, r 128, g 2
    (24, 8, 64, 32, 8, 30, 30, 50, 120, 30, "identity"),          # mfma, g 3: stages of 3 of up to 8 heads
    (64, 8, 64, 64, 32, 12, 12, 40, 300, 12, "identity"),         # mfma, g 8: two stages per chunk
    (12, 2, 64, 64, 16, 30, 30, 70, 200, 30, "perm"),             # mfma, g 6: a full stage of 4 heads, then one of 2
    (6, 1, 64, 16, 8, 30, 30, 31, 100, 28, "perm"),               # mfma, g 6, r 16, B 8, stride < n
    (6, 3, 32, 16, 16, 20, 20, 40, 100, 22, "perm"),              # mfma, Hk 3
    (4, 2, 32, 24, 16, 20, 20, 40, 250, 20, "identity"),          # plain kernel (R 24)
]


@pytest.mark.parametrize("shape", ROW_SHAPES)
def test_score_rows_parity(shape):
    Hq, Hk, D, R, B, N, n, rows, first_pos, stride, table = shape
    _say("score_rows", shape)
    rng = np.random.default_rng(sum((i + 1) * v for i, v in enumerate(shape[:-1])))
    d = rk.dims(2, Hq, Hk, D, R, B, N)
    with rk.Predictor(d, 77 + R) as p:
        phys = rng.permutation(N)[:n].astype(np.int32) if table == "perm" else np.arange(n, dtype=np.int32)
        k = _randn_bits(rng, (1, n, B, Hk, D))
        rk.pred_project_kv_block(p.handle, 1, _to_dev(k).view(torch.bfloat16),
                                 torch.from_numpy(phys.reshape(1, n)).cuda())
        q = _randn_bits(rng, (rows, Hq, R))
        sc = torch.full((rows, stride), 12345.0, dtype=torch.float32, device="cuda")
        tab = None if table == "identity" else torch.from_numpy(phys).cuda()
        rk.pred_score_rows(p.handle, 1, _to_dev(q).view(torch.bfloat16), first_pos, tab, n, sc)
        got = sc.cpu().numpy()
        rk.pred_device_error(p.handle)
        slots = a_g_layer(p.handle, d, 1)[phys]
        want = predictor.score_rows(q, slots, first_pos, stride)
        masked = np.isneginf(want)
        assert np.array_equal(np.isneginf(got), masked), "-inf exactly where a block is not complete"
        assert_scores(got[~masked], want[~masked], R, "score_rows")
        # and the keep sets built on them
        for topk in sorted({1, min(5, stride), min(stride, 16)}):
            keep = torch.full((rows, topk), -7, dtype=torch.int32, device="cuda")
            rk.pred_select_keep(p.handle, sc, first_pos, B, topk, keep, _workspace(stride, rows))
            _check_keep_sets(keep.cpu().numpy(), got, want, first_pos, B, topk, R, f"keep {shape} k={topk}")


def _random_row_shapes(count=24, seed=2024):
    """Seeded small shapes across the MFMA scorer's parameters: any kv head count and group
    size, every r and block size it takes, ragged row counts and key groups, positions from
    the start of the context to past its end, strides below and above n, both table kinds."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        hk = int(rng.choice([1, 2, 3, 4, 5, 8]))
        g = int(rng.integers(1, 9))
        r = int(rng.choice([16, 32, 64, 128]))
        b = int(rng.choice([8, 16, 32]))
        d = int(rng.choice([32, 64]))
        n = int(rng.integers(1, 100))
        rows = int(rng.integers(1, 150))
        out.append((hk * g, hk, d, r, b, n + int(rng.integers(0, 40)), n, rows,
                    int(rng.integers(0, n * b + 64)), int(max(1, n + rng.integers(-5, 8))),
                    str(rng.choice(["perm", "identity"]))))
    return out


@pytest.mark.parametrize("shape", _random_row_shapes())
def test_score_rows_random_shapes(shape):
    test_score_rows_parity(shape)


# Shapes where every workgroup of the MFMA scorer (one kv head, one key group,
# one row part) runs dozens of 32-row chunks back to back, each chunk's maxima
# reaching the scores by atomics while the next chunk multiplies, with several
# row parts per key group and a shorter last part.  One table entry is invalid:
# its block scores NaN in every row that has it complete.
MANY_ITEM_SHAPES = [
    # Hq, Hk, D, R, B, N, n, rows, first_pos
    (8, 1, 64, 64, 16, 700, 640, 10000, 3000),     # one kv head, g 8 (two stages per chunk), 25 row parts
    (32, 8, 64, 32, 16, 1100, 1000, 6000, 0),      # most key groups past every row's complete count
    (16, 4, 64, 64, 16, 600, 520, 9000, 2000),     # four kv heads, 8 row parts of 36 chunks
]


@pytest.mark.parametrize("shape", MANY_ITEM_SHAPES)
def test_score_rows_many_items(shape):
    Hq, Hk, D, R, B, N, n, rows, first_pos = shape
    _say("score_rows many items", shape)
    rng = np.random.default_rng(sum((i + 3) * v for i, v in enumerate(shape)))
    d = rk.dims(1, Hq, Hk, D, R, B, N)
    with rk.Predictor(d, 11 + R) as p:
        phys = rng.permutation(N)[:n].astype(np.int32)
        k = _randn_bits(rng, (1, n, B, Hk, D))
        rk.pred_project_kv_block(p.handle, 0, _to_dev(k).view(torch.bfloat16),
                                 torch.from_numpy(phys.reshape(1, n)).cuda())
        bad = 5
        tab_host = phys.copy()
        tab_host[bad] = N + 3                       # outside [0, N)
        q = _randn_bits(rng, (rows, Hq, R))
        sc = torch.full((rows, n), 12345.0, dtype=torch.float32, device="cuda")
        rk.pred_score_rows(p.handle, 0, _to_dev(q).view(torch.bfloat16), first_pos,
                           torch.from_numpy(tab_host).cuda(), n, sc)
        got = sc.cpu().numpy()
        with pytest.raises(rk.PredError) as e:
            rk.pred_device_error(p.handle)
        assert e.value.code == rk.PRED_ERR_DEVICE
        # the causal mask on every row, the invalid block's NaN wherever it is complete
        cnt = np.minimum(n, (first_pos + np.arange(rows) + 1) // B)
        col = np.arange(n)[None, :]
        assert np.array_equal(np.isneginf(got), col >= cnt[:, None]), "-inf exactly past each row's count"
        has_bad = cnt > bad
        assert np.isnan(got[has_bad, bad]).all() and not np.isnan(np.delete(got, bad, axis=1)).any()
        # sampled rows against the oracle (the invalid block left out)
        slots = a_g_layer(p.handle, d, 0)[phys]
        sample = sorted(set(rng.choice(rows, 48, replace=False).tolist()) | {0, rows - 1, rows // 2})
        for i in sample:
            want = predictor.score_rows(q[i:i + 1], slots, first_pos + i, n)[0]
            m = np.isfinite(want)
            m[bad] = False
            assert_scores(got[i][m], want[m], R, f"many items, row {i}")


def test_score_rows_signs():
    """Scores of both signs: the kv heads of a cell meet through an integer max on the
    bit pattern for non-negative scores and an integer min for negative ones.  Every
    key of a block is close to +u or -u (u one projected key), every query close to
    +u, so every block's score has the block's sign in every row, and kv head k's
    keys are scaled by 1 + k / 4, so the heads disagree on each cell's value."""
    Hq, Hk, D, R, B, N, n, rows, first_pos, stride = 8, 4, 64, 32, 8, 80, 70, 100, 300, 72
    _say("score_rows signs", (Hq, Hk, D, R, B, N, n, rows, first_pos, stride))
    rng = np.random.default_rng(17)
    d = rk.dims(1, Hq, Hk, D, R, B, N)
    with rk.Predictor(d, 23) as p:
        phys = rng.permutation(N)[:n].astype(np.int32)
        v = rng.standard_normal(D)
        sign = np.where(np.arange(n) % 3 == 0, -1.0, 1.0)            # a third of the blocks negative
        scale = 1.0 + np.arange(Hk) / 4.0
        k = (sign[:, None, None, None] * scale[None, None, :, None] * v[None, None, None, :]
             + 0.01 * rng.standard_normal((n, B, Hk, D)))
        k_bits = bf16.encode(k.reshape(1, n, B, Hk, D))
        rk.pred_project_kv_block(p.handle, 0, _to_dev(k_bits).view(torch.bfloat16),
                                 torch.from_numpy(phys.reshape(1, n)).cuda())
        slots = a_g_layer(p.handle, d, 0)[phys]                      # [n, Hk, B, R] bits
        u = bf16.decode(slots[1, 0, 0])                              # block 1 is positive, kv head 0
        q = bf16.encode(u[None, None, :] * (1.0 + 0.05 * rng.standard_normal((rows, Hq, R))))
        sc = torch.full((rows, stride), 12345.0, dtype=torch.float32, device="cuda")
        rk.pred_score_rows(p.handle, 0, _to_dev(q).view(torch.bfloat16), first_pos,
                           torch.from_numpy(phys).cuda(), n, sc)
        got = sc.cpu().numpy()
        rk.pred_device_error(p.handle)
        want = predictor.score_rows(q, slots, first_pos, stride)
        masked = np.isneginf(want)
        assert np.array_equal(np.isneginf(got), masked), "-inf exactly where a block is not complete"
        fin = ~masked
        neg_cols = np.zeros(stride, dtype=bool)
        neg_cols[:n] = sign < 0
        neg = fin & neg_cols[None, :]
        assert (want[neg] < 0).all() and (want[fin & ~neg] > 0).all() and neg.sum() > 500
        assert_scores(got[fin], want[fin], R, "score_rows signs")


def test_score_rows_edge_cases():
    """No blocks, no complete block for any row, one row, and an invalid table entry (NaN + error)."""
    d = rk.dims(1, 8, 2, 32, 32, 16, 16)
    rng = np.random.default_rng(4)
    with rk.Predictor(d, 5, flags=rk.PRED_FLAG_ZERO_AG) as p:
        q = _to_dev(_randn_bits(rng, (40, 8, 32))).view(torch.bfloat16)
        _say("score_rows n=0")
        sc = torch.zeros((40, 9), dtype=torch.float32, device="cuda")
        rk.pred_score_rows(p.handle, 0, q, 10, None, 0, sc)
        assert np.isneginf(sc.cpu().numpy()).all()
        _say("score_rows nothing complete")
        sc = torch.zeros((40, 16), dtype=torch.float32, device="cuda")
        rk.pred_score_rows(p.handle, 0, q[:10], 0, None, 16, sc[:10])   # positions 0..9 < block_size
        assert np.isneginf(sc[:10].cpu().numpy()).all()
        _say("score_rows one row")
        sc1 = torch.zeros((1, 16), dtype=torch.float32, device="cuda")
        rk.pred_score_rows(p.handle, 0, q[:1], 16 * 5 - 1, None, 16, sc1)
        got = sc1.cpu().numpy()
        assert np.isfinite(got[0, :5]).all() and np.isneginf(got[0, 5:]).all()
        assert np.all(got[0, :5] == 0.0)   # A_g zeroed
        _say("score_rows into an output that is not 16-byte aligned")
        k = _to_dev(_randn_bits(rng, (1, 9, 16, 2, 32))).view(torch.bfloat16)
        rk.pred_project_kv_block(p.handle, 0, k, torch.arange(9, dtype=torch.int32, device="cuda").view(1, 9))
        aligned = torch.zeros((40, 9), dtype=torch.float32, device="cuda")
        rk.pred_score_rows(p.handle, 0, q, 100, None, 9, aligned)
        big = torch.full((41, 9), 7.0, dtype=torch.float32, device="cuda")
        view = big[1:]                                   # starts 36 bytes into the allocation
        assert view.data_ptr() % 16 != 0
        rk.pred_score_rows(p.handle, 0, q, 100, None, 9, view)
        assert torch.equal(view.cpu(), aligned.cpu()) and torch.all(big[0] == 7.0)
        got = aligned.cpu().numpy()
        cnt = np.minimum(9, (100 + np.arange(40) + 1) // 16)
        assert np.array_equal(np.isneginf(got), np.arange(9)[None, :] >= cnt[:, None])
        _say("score_rows invalid table entry")
        tab = torch.tensor([0, 1, 99, 3], dtype=torch.int32, device="cuda")
        sc = torch.zeros((4, 4), dtype=torch.float32, device="cuda")
        rk.pred_score_rows(p.handle, 0, q[:4], 100, tab, 4, sc)
        got = sc.cpu().numpy()
        assert np.isnan(got[:, 2]).all() and np.isfinite(got[:, [0, 1, 3]]).all()
        with pytest.raises(rk.PredError) as e:
            rk.pred_device_error(p.handle)
        assert e.value.code == rk.PRED_ERR_DEVICE
        with pytest.raises(rk.PredError) as e:
            rk.pred_score_rows(p.handle, 1, q[:4], 0, None, 4, sc)   # layer 1 of 1
        assert e.value.code == rk.PRED_ERR_OUT_OF_RANGE


# ------------------------------------------------------------- keep sets alone

KEEP_SHAPES = [
    # rows, stride, first_pos, ratio, topks                        path
    (9, 7, 0, 1, (0, 1, 3, 7)),                                    # one workgroup (256)
    (33, 300, 0, 2, (1, 64, 300)),                                 # one workgroup (1024); rows without blocks
    (16, 2048, 30000, 16, (1, 64, 2048)),                          # one workgroup (2048)
    (5, 2049, 1500, 1, (1, 64, 2049)),                             # chunked, one merge level
    (4, 5000, 1 << 20, 1, (1, 64, 5000)),                          # chunked, every block complete
    (7, 9000, 4000, 1, (1, 100, 9000)),                            # two merge levels
    (3, 40000, 39990, 1, (1, 1000, 40000)),                        # pairwise merges
    (600, 2048, 30000, 16, (1, 64, 256, 257)),                     # >= 512 rows, top <= 256: radix select
    (520, 700, 0, 1, (1, 37, 256, 699)),                           # radix select, rows shorter than top-k
]


@pytest.mark.parametrize("rows,stride,first_pos,ratio,topks", KEEP_SHAPES)
def test_select_keep_exact(rows, stride, first_pos, ratio, topks):
    rng = np.random.default_rng(rows * 7 + stride)
    s = (rng.integers(-300, 300, size=(rows, stride)) * 0.25).astype(np.float32)   # many ties
    s[:, ::41] = -0.0
    s[:, 3::97] = np.nan
    s[:, 5::89] = np.inf
    s[-1, :] = 1.0                                                                  # one row all equal
    d = rk.dims(1, 1, 1, 8, 8, 1, 1)
    with rk.Predictor(d, 1) as p:
        sc = torch.from_numpy(s).cuda()
        ws = _workspace(stride, rows)
        for topk in topks:
            _say("select_keep", rows, stride, first_pos, ratio, topk)
            keep = torch.full((rows, topk), -7, dtype=torch.int32, device="cuda")
            rk.pred_select_keep(p.handle, sc, first_pos, ratio, topk, keep, ws)
            got = keep.cpu().numpy()
            want = predictor.keep_sets(s, first_pos, ratio, topk)
            assert np.array_equal(got, want), (rows, stride, topk)


def test_select_keep_errors():
    d = rk.dims(1, 1, 1, 8, 8, 1, 1)
    with rk.Predictor(d, 1) as p:
        sc = torch.zeros((4, 3000), dtype=torch.float32, device="cuda")
        keep = torch.empty((4, 8), dtype=torch.int32, device="cuda")
        with pytest.raises(rk.PredError) as e:
            rk.pred_select_keep(p.handle, sc, 0, 1, 8, keep, None)
        assert e.value.code == rk.PRED_ERR_WORKSPACE
        ws = _workspace(3000, 4)
        for first_pos, ratio in ((0, 0), (-1, 4)):
            with pytest.raises(rk.PredError) as e:
                rk.pred_select_keep(p.handle, sc, first_pos, ratio, 8, keep, ws)
            assert e.value.code == rk.PRED_ERR_OUT_OF_RANGE
        with pytest.raises(rk.PredError) as e:
            rk.pred_select_keep(p.handle, sc, 0, 1, 3001, torch.empty((4, 3001), dtype=torch.int32, device="cuda"), ws)
        assert e.value.code == rk.PRED_ERR_OUT_OF_RANGE
        rk.pred_select_keep(p.handle, sc, 0, 1, 0, torch.empty((4, 0), dtype=torch.int32, device="cuda"), ws)
