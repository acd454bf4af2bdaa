"""GPU parity of pred_score_blocks_masked (a partly filled last block per sequence) on every score path."""

import numpy as np
import pytest

import rank_kv_block_amd as rk
from oracle import bf16, predictor
from tests.devmem import a_g_layer
from tests.parity import assert_scores

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print("[case]", *a, flush=True)


def _to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).cuda()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rk.lib()
    yield
    torch.cuda.synchronize()


MASK_SHAPES = [
    # Hq, Hk, D, R, B, N, n, S, M, L    path
    (32, 8, 64, 32, 16, 200, 60, 3, 1, 2),     # decode stream, one wave-load per kv region
    (8, 2, 64, 16, 8, 100, 45, 2, 1, 1),       # decode stream, several blocks per wave-load
    (8, 1, 64, 128, 32, 40, 13, 2, 1, 1),      # decode stream, 16 load slots
    (64, 8, 64, 64, 32, 160, 21, 7, 1, 1),     # decode matrix-core variant: 8 queries, two tiles per block
    (16, 2, 64, 32, 16, 160, 22, 7, 1, 1),     # decode matrix-core variant: four blocks per wave
    (32, 8, 64, 64, 16, 80, 37, 2, 8, 1),      # many-row MFMA scorer
    (4, 2, 32, 24, 16, 40, 19, 2, 1, 1),       # plain kernel
]


@pytest.mark.parametrize("shape", MASK_SHAPES)
def test_score_blocks_masked(shape):
    Hq, Hk, D, R, B, N, n, S, M, L = shape
    _say("masked", shape)
    rng = np.random.default_rng(sum((i + 3) * v for i, v in enumerate(shape)))
    d = rk.dims(L, Hq, Hk, D, R, B, N)
    with rk.Predictor(d, 500 + R) as p:
        perm = rng.permutation(N)[: S * n].reshape(S, n).astype(np.int32)
        for l in range(L):
            k = bf16.encode(rng.standard_normal((1, S * n, B, Hk, D)))
            rk.pred_project_kv_block(p.handle, l, _to_dev(k).view(torch.bfloat16),
                                     torch.from_numpy(perm.reshape(1, S * n)).cuda())
        q = bf16.encode(rng.standard_normal((L, S, M, Hq, R)))
        fills = [0, B, 1, B - 1, 3][:S] + [int(rng.integers(0, B + 1)) for _ in range(max(0, S - 5))]
        fill_t = torch.tensor(fills, dtype=torch.int32, device="cuda")
        sc = torch.full((L, S, n), 7.0, dtype=torch.float32, device="cuda")
        rk.pred_score_blocks_masked(p.handle, 0, _to_dev(q).view(torch.bfloat16), torch.from_numpy(perm).cuda(),
                                    fill_t, sc)
        got = sc.cpu().numpy()
        rk.pred_device_error(p.handle)
        a_g = np.stack([a_g_layer(p.handle, d, l) for l in range(L)])
        want = predictor.score_blocks(q, a_g, 0, perm, n, last_fill=fills)
        inf = np.isneginf(want)
        assert np.array_equal(np.isneginf(got), inf)
        assert_scores(got[~inf], want[~inf], R, f"masked {shape}")
        # no fill array: every block full, identical to pred_score_blocks
        sc2 = torch.empty_like(sc)
        rk.pred_score_blocks_masked(p.handle, 0, _to_dev(q).view(torch.bfloat16), torch.from_numpy(perm).cuda(),
                                    None, sc2)
        sc3 = torch.empty_like(sc)
        rk.pred_score_blocks(p.handle, 0, _to_dev(q).view(torch.bfloat16), torch.from_numpy(perm).cuda(), sc3)
        assert torch.equal(sc2, sc3)


def test_fill_out_of_range_is_clamped_and_reported():
    d = rk.dims(1, 8, 2, 64, 32, 16, 20)
    rng = np.random.default_rng(9)
    with rk.Predictor(d, 3) as p:
        k = bf16.encode(rng.standard_normal((1, 20, 16, 2, 64)))
        rk.pred_project_kv_block(p.handle, 0, _to_dev(k).view(torch.bfloat16))
        q = _to_dev(bf16.encode(rng.standard_normal((1, 2, 1, 8, 32)))).view(torch.bfloat16)
        tab = torch.arange(20, dtype=torch.int32, device="cuda").view(2, 10)
        sc = torch.empty((1, 2, 10), dtype=torch.float32, device="cuda")
        rk.pred_score_blocks_masked(p.handle, 0, q, tab, torch.tensor([17, -2], dtype=torch.int32, device="cuda"), sc)
        got = sc.cpu().numpy()
        with pytest.raises(rk.PredError) as e:
            rk.pred_device_error(p.handle)
        assert e.value.code == rk.PRED_ERR_DEVICE
        ref = torch.empty_like(sc)
        rk.pred_score_blocks_masked(p.handle, 0, q, tab, torch.tensor([16, 0], dtype=torch.int32, device="cuda"), ref)
        rk.pred_device_error(p.handle)
        assert np.array_equal(got, ref.cpu().numpy())
        assert np.isneginf(got[0, 1, -1])
