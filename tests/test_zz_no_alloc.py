"""The no-allocation ranking entry point (pred_rank_victims_noalloc) against pred_rank_victims.

Two calls in a row on one device, the second smaller than the first, each equal bit for bit to
the workspace entry point's ranking of the same scores (and so to the oracle's sort); a shape
above the static scratch is refused before anything runs."""

import numpy as np
import pytest

import rank_kv_block_amd as rk
from oracle import predictor

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rk.lib()
    yield
    torch.cuda.synchronize()


def _scores(rng, segs, n):
    s = (rng.integers(-400, 400, size=(segs, n)) * 0.25).astype(np.float32)   # many ties
    s[:, ::61] = -0.0
    s[0, 1] = np.nan
    return s


def _rank_with_workspace(h, sc):
    segs, n = sc.shape
    vic = torch.full((segs, n), -5, dtype=torch.int32, device="cuda")
    ws_b = rk.pred_rank_workspace_bytes(n, segs)
    ws = torch.empty((ws_b // 8 + 1,), dtype=torch.int64, device="cuda") if ws_b else None
    rk.pred_rank_victims(h, sc, vic, ws)
    return vic


def test_noalloc_rank_matches_workspace_entry_point():
    rng = np.random.default_rng(77)
    d = rk.dims(1, 1, 1, 8, 8, 1, 1)
    # the 8B decode step's 32 rows of 8192 keys (2 MiB of scratch), then smaller calls that reuse
    # the same scratch: one row of 20000 (two buffers), 3 rows of 3000, 5 rows of 700 (no scratch)
    shapes = [(32, 8192), (1, 20000), (3, 3000), (5, 700)]
    with rk.Predictor(d, 1) as p:
        for segs, n in shapes:
            _say("noalloc rank", segs, n)
            s = _scores(rng, segs, n)
            sc = torch.from_numpy(s).cuda()
            vic = torch.full((segs, n), -7, dtype=torch.int32, device="cuda")
            rk.pred_rank_victims_noalloc(p.handle, sc, vic)
            want = _rank_with_workspace(p.handle, sc)
            torch.cuda.synchronize()
            got = vic.cpu().numpy()
            assert np.array_equal(got, want.cpu().numpy()), (segs, n)
            assert np.array_equal(got, predictor.rank_victims(s)), (segs, n)


def test_noalloc_rank_refuses_shapes_above_its_scratch():
    d = rk.dims(1, 1, 1, 8, 8, 1, 1)
    with rk.Predictor(d, 1) as p:
        n, segs = 8192, 129                    # 129 * 8192 * 8 bytes > 8 MiB
        assert rk.pred_rank_workspace_bytes(n, segs) > rk.PRED_NOALLOC_SCRATCH_BYTES
        sc = torch.zeros((segs, n), dtype=torch.float32, device="cuda")
        vic = torch.full((segs, n), -3, dtype=torch.int32, device="cuda")
        with pytest.raises(rk.PredError) as e:
            rk.pred_rank_victims_noalloc(p.handle, sc, vic)
        assert e.value.code == rk.PRED_ERR_WORKSPACE
        torch.cuda.synchronize()
        assert (vic.cpu().numpy() == -3).all()  # nothing ran
        # the largest shape that fits still works
        n2, segs2 = 8192, 128
        assert rk.pred_rank_workspace_bytes(n2, segs2) == rk.PRED_NOALLOC_SCRATCH_BYTES
        s = _scores(np.random.default_rng(5), segs2, n2)
        sc2 = torch.from_numpy(s).cuda()
        vic2 = torch.empty((segs2, n2), dtype=torch.int32, device="cuda")
        rk.pred_rank_victims_noalloc(p.handle, sc2, vic2)
        torch.cuda.synchronize()
        assert np.array_equal(vic2.cpu().numpy(), predictor.rank_victims(s))
