"""GPU parity of every kernel against the oracle on small and ragged shapes (through the C ABI)."""

import json
import os

import numpy as np
import pytest

import rank_kv_block_amd as rk
from oracle import bf16, predictor, prng
from tests.parity import assert_ranking, assert_scores, assert_ulp

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print("[case]", *a, flush=True)


def _bits_np(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _to_dev(bits):
    """bf16 bit patterns (uint16) -> device int16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).cuda()


def _tab_dev(ids):
    """Block ids -> device int32 tensor."""
    return torch.from_numpy(np.array(ids, dtype=np.int32, order="C")).cuda()   # a writable contiguous copy


def _read_slots(h, d, pairs):
    """A_g [L, N, Hk, B, R] with the listed (layer, slot) pairs read from the device, zeros elsewhere."""
    a = np.zeros((d.num_layers, d.max_blocks, d.num_kv_heads, d.block_size, d.r), np.uint16)
    for l, b in pairs:
        a[l, b] = rk.pred_read_slot(h, l, b)
    return a


def _randn_bits(rng, shape, scale=1.0):
    return bf16.encode(rng.standard_normal(shape) * scale)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rk.lib()
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------- projection P

@pytest.mark.parametrize("D,R,seed", [(64, 16, 1001), (128, 32, 1002), (128, 64, 1005)])
def test_projection_on_device_matches_oracle(D, R, seed):
    _say("P", D, R, seed)
    d = rk.dims(1, 8, 8, D, R, 16, 4)
    with rk.Predictor(d, seed) as p:
        assert np.array_equal(rk.pred_copy_projection(p.handle), prng.projection(D, R, seed))


@pytest.mark.parametrize("D,R,n_vec", [(32, 32, 20000), (64, 16, 17000), (128, 64, 16400), (256, 32, 9000),
                                       (128, 32, 37), (256, 48, 300), (96, 24, 5000)])
def test_project_q_sizes(D, R, n_vec):
    """project_q alone, at sizes that take the streaming MFMA kernel (>= 1024 16x16 tiles), the
    head_dim-split kernel (small calls) and the plain kernel (r not a multiple of 16 / other head_dim)."""
    _say("project_q", D, R, n_vec)
    rng = np.random.default_rng(D * 1000 + R + n_vec)
    d = rk.dims(1, 1, 1, D, R, 16, 4)
    seed = 4242 + D + R
    with rk.Predictor(d, seed) as p:
        P = prng.projection(D, R, seed)
        q = _randn_bits(rng, (n_vec, 1, D))
        qp = torch.empty((n_vec, 1, R), dtype=torch.bfloat16, device="cuda")
        rk.pred_project_q(p.handle, _to_dev(q), qp)
        torch.cuda.synchronize()
        assert_ulp(_bits_np(qp), predictor.project_q(q, P), "q_proj")


# ---------------------------------------------------------------- hand examples

def _pad(a, shape):
    out = np.zeros(shape, dtype=np.float64)
    out[tuple(slice(0, s) for s in np.shape(a))] = a
    return out


def test_hand_examples_on_gpu(golden_dir):
    """Hand-worked values, zero-padded to head_dim = r = 8 (padding adds exact zeros)."""
    for name in ["hand_a1.json", "hand_a2.json"]:
        _say("hand", name)
        g = json.load(open(os.path.join(golden_dir, name)))
        dm = g["dims"]
        Hq, Hk, B, N = dm["num_q_heads"], dm["num_kv_heads"], dm["block_size"], dm["max_blocks"]
        d = rk.dims(1, Hq, Hk, 8, 8, B, N)
        P = bf16.encode(_pad(g["P"], (8, 8)))
        with rk.Predictor(d, projection=P, flags=rk.PRED_FLAG_ZERO_AG) as p:
            q = _to_dev(bf16.encode(_pad(g["q"], (Hq, 8))))
            qp = torch.empty((1, 1, 1, Hq, 8), dtype=torch.bfloat16, device="cuda")
            rk.pred_project_q(p.handle, q, qp)
            kb = np.array(g["k_blocks"] if "k_blocks" in g else [g["k_block"]], dtype=np.float64)
            k = _to_dev(bf16.encode(_pad(kb, kb.shape[:-1] + (8,))))
            rk.pred_project_kv_block(p.handle, 0, k.view(1, *k.shape))
            scores = torch.empty((1, 1, N), dtype=torch.float32, device="cuda")
            rk.pred_score_blocks(p.handle, 0, qp, None, scores)
            vic = torch.empty((1, N), dtype=torch.int32, device="cuda")
            rk.pred_rank_victims(p.handle, scores.view(1, N), vic)
            torch.cuda.synchronize()
            qpf = bf16.decode(_bits_np(qp)).reshape(Hq, 8)
            assert np.array_equal(qpf[:, :2], np.array(g["q_proj"], float)) and not qpf[:, 2:].any()
            slot0 = bf16.decode(rk.pred_read_slot(p.handle, 0, 0))[:, :, :2]
            s = scores.cpu().numpy().reshape(N)
            if name == "hand_a1.json":
                assert np.array_equal(slot0, np.array(g["a_slots"][0], float))
                assert s.tolist() == g["scores"]
                assert vic.cpu().numpy()[0].tolist() == g["victims"]
            else:
                assert slot0.ravel().tolist() == g["a_slot_flat"]
                assert s.tolist() == [g["score"]]


# ---------------------------------------------------------------- random shapes

SHAPES = [
    # L, Hq, Hk, D, R, B, N, n, S, M, table
    (2, 4, 1, 64, 16, 16, 70, 67, 1, 1, "perm"),          # C1-like, ragged
    (3, 32, 8, 128, 32, 16, 300, 150, 2, 1, "perm"),       # C2-like, two sequences
    (1, 64, 8, 128, 64, 32, 100, 97, 1, 1, "identity"),    # C5-like
    (1, 32, 8, 128, 64, 16, 90, 90, 1, 1, "perm"),         # C4 dims at one row
    (2, 8, 8, 64, 32, 16, 64, 41, 1, 2, "perm"),           # g = 1, two rows
    (1, 16, 2, 64, 128, 8, 120, 33, 3, 1, "perm"),         # r = 128, short blocks
    (1, 16, 4, 128, 32, 16, 64, 37, 1, 3, "identity"),     # 3 rows x g=4 -> 12 heads, padded to 16
    (1, 32, 8, 128, 64, 16, 64, 23, 1, 17, "perm"),        # 17 rows: many-row path
    (1, 12, 4, 64, 24, 16, 30, 30, 1, 1, "perm"),          # r = 24: plain per-block kernel
    (1, 8, 2, 32, 16, 12, 60, 29, 2, 1, "identity"),       # block_size 12: plain per-block kernel
    (1, 16, 2, 64, 128, 32, 40, 37, 1, 1, "perm"),         # 1 KiB-wide kv regions: 16 load slots per wave
    # 5..16 queries per kv head: the decode scorer's matrix-core variant
    (2, 16, 2, 64, 32, 16, 100, 45, 2, 1, "perm"),         # r = 32: one 16-token tile, four blocks per wave
    (1, 16, 1, 64, 64, 64, 30, 19, 1, 1, "perm"),          # block_size 64: four tiles, 16 load slots
    (1, 16, 2, 128, 128, 16, 40, 21, 1, 2, "identity"),    # r = 128: four k-steps; 2 rows x g = 8 = 16 queries
    (1, 24, 4, 64, 64, 32, 80, 33, 2, 1, "perm"),          # g = 6: columns 6..15 repeat a query
    (1, 8, 8, 64, 32, 32, 40, 27, 1, 5, "perm"),           # g = 1, 5 rows
    (1, 16, 2, 64, 16, 16, 70, 31, 2, 1, "perm"),          # 8 queries at r = 16: vector-ALU decode kernel
    (1, 8, 1, 64, 32, 8, 40, 23, 1, 1, "perm"),            # 8 queries, 512-byte kv regions: vector-ALU kernel
    # largest shapes the limits allow
    (1, 8, 2, 64, 256, 16, 30, 13, 1, 1, "perm"),          # r = 256: plain per-block kernel
    (1, 16, 2, 64, 128, 64, 24, 9, 1, 1, "perm"),          # r = 128, block_size 64: 16 KiB kv regions (U = 1024)
    (1, 4, 1, 64, 128, 64, 24, 11, 2, 1, "identity"),      # the same with 4 queries: vector-ALU kernel, 16 slots
    (2, 32, 8, 128, 32, 16, 9000, 8200, 1, 1, "perm"),     # larger ragged case, two layers
    (1, 8, 2, 256, 32, 16, 40, 21, 1, 1, "identity"),      # head_dim 256: widest MFMA projection tiles
    (1, 8, 2, 96, 16, 16, 40, 20, 2, 1, "perm"),           # head_dim 96: plain projection kernel
    # many query rows: the MFMA scorer
    (1, 32, 8, 128, 64, 16, 300, 260, 1, 64, "perm"),      # prefill-chunk dims, ragged key tiles
    (2, 16, 4, 64, 32, 32, 150, 70, 2, 40, "perm"),        # block_size 32, two layers, two sequences
    (1, 8, 1, 64, 16, 8, 50, 45, 1, 33, "identity"),       # block_size 8, r = 16, one kv head
    (1, 16, 2, 128, 128, 16, 40, 33, 1, 9, "perm"),        # r = 128, 72 queries per kv head
    (1, 8, 2, 64, 24, 16, 30, 20, 1, 6, "perm"),           # 24 queries per kv head at r = 24: plain kernel
    (1, 8, 2, 64, 32, 12, 48, 20, 2, 5, "identity"),       # 20 queries per kv head, block_size 12: plain kernel
]


def test_parity_shapes_reach_every_score_kernel():
    """The shapes below exercise each kernel pred_score_blocks can launch."""
    seen = {}
    for L, Hq, Hk, D, R, B, N, n, S, M, table in SHAPES:
        with rk.Predictor(rk.dims(L, Hq, Hk, D, R, B, N), 1) as p:
            seen.setdefault(rk.pred_score_kernel_name(p.handle, M), []).append((Hq, Hk, R, B, M))
    assert set(seen) == {"score_prefill_kernel", "score_decode_mfma_kernel", "score_decode_kernel",
                         "score_generic_kernel"}, seen
    with rk.Predictor(rk.dims(1, 64, 8, 128, 64, 32, 16), 1) as p:       # 70B-shaped decode
        assert rk.pred_score_kernel_name(p.handle, 1) == "score_decode_mfma_kernel"
        assert rk.pred_score_kernel_name(p.handle, 3) == "score_prefill_kernel"
    with rk.Predictor(rk.dims(1, 32, 8, 128, 32, 16, 16), 1) as p:       # 8B-shaped decode
        assert rk.pred_score_kernel_name(p.handle, 1) == "score_decode_kernel"
        assert rk.pred_score_kernel_name(p.handle, 2) == "score_decode_mfma_kernel"
        with pytest.raises(rk.PredError):
            rk.pred_score_kernel_name(p.handle, 0)


@pytest.mark.parametrize("shape", SHAPES, ids=[f"L{s[0]}-q{s[1]}-kv{s[2]}-d{s[3]}-r{s[4]}-b{s[5]}-n{s[7]}"
                                              f"-S{s[8]}-M{s[9]}" for s in SHAPES])
def test_random_shape_parity(shape):
    L, Hq, Hk, D, R, B, N, n, S, M, table = shape
    _say("shape", shape)
    rng = np.random.default_rng([x for x in shape if isinstance(x, int)])
    d = rk.dims(L, Hq, Hk, D, R, B, N)
    seed = int(rng.integers(0, 2 ** 63))
    with rk.Predictor(d, seed, flags=rk.PRED_FLAG_ZERO_AG) as p:
        P = prng.projection(D, R, seed)
        # tables: S disjoint slices of one permutation (or the identity)
        if table == "perm":
            perm = rng.permutation(N)[: S * n].reshape(S, n).astype(np.int32)
        else:
            assert S * n <= N
            perm = np.arange(S * n, dtype=np.int32).reshape(S, n) if S > 1 else None
        phys = perm if perm is not None else np.arange(n, dtype=np.int32)[None]
        k = _randn_bits(rng, (L, S * n, B, Hk, D))
        ktab = np.broadcast_to(phys.reshape(1, S * n), (L, S * n)).copy()
        rk.pred_project_kv_block(p.handle, 0, _to_dev(k), _tab_dev(ktab))
        q = _randn_bits(rng, (L, S, M, Hq, D))
        qp = torch.empty((L, S, M, Hq, R), dtype=torch.bfloat16, device="cuda")
        rk.pred_project_q(p.handle, _to_dev(q), qp)
        scores = torch.empty((L, S, n), dtype=torch.float32, device="cuda")
        tab_dev = _tab_dev(perm) if perm is not None else None
        rk.pred_score_blocks(p.handle, 0, qp, tab_dev, scores)
        vic = torch.empty((L * S, n), dtype=torch.int32, device="cuda")
        ws_b = rk.pred_rank_workspace_bytes(n, L * S)
        ws = torch.empty((ws_b // 8 + 1,), dtype=torch.int64, device="cuda") if ws_b else None
        rk.pred_rank_victims(p.handle, scores.view(L * S, n), vic, ws)
        rk.pred_device_error(p.handle)

        # projections
        assert_ulp(_bits_np(qp), predictor.project_q(q, P), "q_proj")
        a_g = _read_slots(p.handle, d, [(l, int(b)) for l in range(L) for b in phys.reshape(-1)])
        want_slots = predictor.project_kv_slots(k.reshape(L * S * n, B, Hk, D), P).reshape(L, S * n, Hk, B, R)
        got_slots = np.stack([a_g[l][phys.reshape(-1)] for l in range(L)])
        assert_ulp(got_slots, want_slots, "A_g")
        # scores from the GPU's own q_proj and A_g
        want = predictor.score_blocks(_bits_np(qp), a_g, 0, phys if perm is not None else None, n)
        got = scores.cpu().numpy()
        assert_scores(got, want, R)
        assert_ranking(vic.cpu().numpy(), got.reshape(L * S, n), want.reshape(L * S, n), R)


# ---------------------------------------------------------------- ranking

@pytest.mark.parametrize("n,segs", [(1, 1), (5, 3), (64, 1), (256, 2), (257, 2), (513, 2), (1024, 3), (1025, 2), (2048, 4), (2049, 3),
                                    (3000, 5), (4095, 2),
                                    (8191, 1), (8192, 2), (8193, 1),
                                    (16384, 1), (16385, 1), (24576, 3), (32768, 2), (32769, 1), (40000, 2), (65536, 1), (100000, 1)])
def test_rank_exact(n, segs):
    _say("rank", n, segs)
    rng = np.random.default_rng(n * 7 + segs)
    s = (rng.integers(-300, 300, size=(segs, n)) * 0.25).astype(np.float32)   # many ties
    s[:, :: 97] = -0.0
    s[:, 1:: 89] = 0.0
    if n > 10:
        s[0, 3] = np.nan
        s[0, 5] = -np.inf
        s[-1, -1] = np.inf
    d = rk.dims(1, 1, 1, 8, 8, 1, 1)
    with rk.Predictor(d, 1) as p:
        sc = torch.from_numpy(s).cuda()
        vic = torch.empty((segs, n), dtype=torch.int32, device="cuda")
        ws_b = rk.pred_rank_workspace_bytes(n, segs)
        ws = torch.empty((ws_b // 8 + 1,), dtype=torch.int64, device="cuda") if ws_b else None
        rk.pred_rank_victims(p.handle, sc, vic, ws)
        got = vic.cpu().numpy()
    assert np.array_equal(got, predictor.rank_victims(s))


@pytest.mark.parametrize("kind", ["all_equal", "low_bits", "two_values", "descending"])
def test_rank_special_orders(kind):
    _say("rank special", kind)
    n = 3000
    if kind == "all_equal":
        s = np.full((2, n), 7.25, np.float32)
    elif kind == "low_bits":     # keys that differ only in the last mantissa bits
        s = (np.float32(1.0) + np.random.default_rng(1).integers(0, 16, (2, n)).astype(np.float32) * np.float32(2 ** -23))
    elif kind == "two_values":
        s = np.where(np.random.default_rng(2).random((2, n)) < 0.5, -1.5, 2.5).astype(np.float32)
    else:
        s = np.linspace(1000, -1000, 2 * n, dtype=np.float32).reshape(2, n)
    d = rk.dims(1, 1, 1, 8, 8, 1, 1)
    with rk.Predictor(d, 1) as p:
        vic = torch.empty((2, n), dtype=torch.int32, device="cuda")
        ws = torch.empty((rk.pred_rank_workspace_bytes(n, 2) // 8,), dtype=torch.int64, device="cuda")
        rk.pred_rank_victims(p.handle, torch.from_numpy(s).cuda(), vic, ws)
        got = vic.cpu().numpy()
    assert np.array_equal(got, predictor.rank_victims(s))


@pytest.mark.parametrize("n,segs,ks", [(200, 3, (1, 7, 199, 200)), (1000, 2, (1, 64, 999)), (2048, 2, (1, 1024, 2047)),
                                       (5000, 3, (1, 64, 1023, 1024, 1025, 4999)), (8192, 2, (1, 100, 8192)),
                                       (20000, 1, (1, 64, 1024, 8191, 8192, 8193, 19999)),
                                       (40000, 1, (1, 777, 32768, 39999)),
                                       (1500, 520, (1, 64, 256, 257)), (600, 512, (1, 255))])   # radix select
def test_select_exact(n, segs, ks):
    """pred_select_victims: exactly the first k of the full ranking, on every path (one workgroup,
    chunked with one or two counting-merge levels, pairwise merges, radix select for many rows)."""
    rng = np.random.default_rng(n + 31 * segs)
    s = (rng.integers(-200, 200, size=(segs, n)) * 0.5).astype(np.float32)   # many ties
    s[:, :: 53] = -0.0
    s[0, 2] = np.nan
    s[-1, -1] = -np.inf
    want_all = predictor.rank_victims(s)
    d = rk.dims(1, 1, 1, 8, 8, 1, 1)
    with rk.Predictor(d, 1) as p:
        sc = torch.from_numpy(s).cuda()
        ws_b = rk.pred_rank_workspace_bytes(n, segs)
        ws = torch.empty((ws_b // 8 + 1,), dtype=torch.int64, device="cuda") if ws_b else None
        for k in ks:
            _say("select", n, segs, k)
            vic = torch.full((segs, k), -7, dtype=torch.int32, device="cuda")
            rk.pred_select_victims(p.handle, sc, k, vic, ws)
            got = vic.cpu().numpy()
            assert np.array_equal(got, want_all[:, :k]), (n, segs, k)
        with pytest.raises(rk.PredError) as e:
            rk.pred_select_victims(p.handle, sc, n + 1, torch.empty((segs, n + 1), dtype=torch.int32, device="cuda"), ws)
        assert e.value.code == rk.PRED_ERR_OUT_OF_RANGE
        rk.pred_select_victims(p.handle, sc, 0, torch.empty((segs, 0), dtype=torch.int32, device="cuda"), ws)


def test_rank_requires_workspace():
    d = rk.dims(1, 1, 1, 8, 8, 1, 1)
    with rk.Predictor(d, 1) as p:
        for n in (2049, 20000):
            sc = torch.zeros((1, n), dtype=torch.float32, device="cuda")
            vic = torch.empty((1, n), dtype=torch.int32, device="cuda")
            with pytest.raises(rk.PredError) as e:
                rk.pred_rank_victims(p.handle, sc, vic, None)
            assert e.value.code == rk.PRED_ERR_WORKSPACE


# ---------------------------------------------------------------- error paths

def test_invalid_table_entries_are_reported():
    _say("invalid table")
    d = rk.dims(1, 4, 2, 64, 16, 16, 8)
    with rk.Predictor(d, 3, flags=rk.PRED_FLAG_ZERO_AG) as p:
        rng = np.random.default_rng(0)
        k = _to_dev(_randn_bits(rng, (1, 3, 16, 2, 64)))
        bad = torch.tensor([[0, 9, 2]], dtype=torch.int32, device="cuda")
        rk.pred_project_kv_block(p.handle, 0, k, bad)
        with pytest.raises(rk.PredError) as e:
            rk.pred_device_error(p.handle)
        assert e.value.code == rk.PRED_ERR_DEVICE
        rk.pred_device_error(p.handle)          # cleared
        qp = torch.zeros((1, 1, 1, 4, 16), dtype=torch.bfloat16, device="cuda")
        scores = torch.empty((1, 1, 3), dtype=torch.float32, device="cuda")
        rk.pred_score_blocks(p.handle, 0, qp, torch.tensor([[0, -1, 2]], dtype=torch.int32, device="cuda"), scores)
        with pytest.raises(rk.PredError):
            rk.pred_device_error(p.handle)
        s = scores.cpu().numpy().ravel()
        assert np.isnan(s[1]) and s[0] == 0.0 and s[2] == 0.0
        # the many-row scorer reports it the same way
        qm = torch.zeros((1, 1, 9, 4, 16), dtype=torch.bfloat16, device="cuda")
        rk.pred_score_blocks(p.handle, 0, qm, torch.tensor([[0, 8, 2]], dtype=torch.int32, device="cuda"), scores)
        with pytest.raises(rk.PredError):
            rk.pred_device_error(p.handle)
        s = scores.cpu().numpy().ravel()
        assert np.isnan(s[1]) and s[0] == 0.0 and s[2] == 0.0


@pytest.mark.parametrize("R,B,n", [(32, 16, 9), (64, 32, 5), (128, 16, 6)])
def test_invalid_table_entries_matrix_core_decode(R, B, n):
    """The decode scorer's matrix-core variant (8 queries per kv head): an out-of-range entry gives NaN
    and raises the error word; its neighbours (in the same wave) keep their scores."""
    _say("invalid table, decode mfma", R, B, n)
    N = 12
    d = rk.dims(1, 16, 2, 64, R, B, N)
    with rk.Predictor(d, 5, flags=rk.PRED_FLAG_ZERO_AG) as p:
        assert rk.pred_score_kernel_name(p.handle, 1) == "score_decode_mfma_kernel"
        rng = np.random.default_rng(R + B)
        k = _randn_bits(rng, (1, N, B, 2, 64))
        rk.pred_project_kv_block(p.handle, 0, _to_dev(k))
        q = _randn_bits(rng, (1, 1, 1, 16, R))
        tab = rng.permutation(N)[:n].astype(np.int32)
        bad = tab.copy()
        bad[1], bad[n - 2] = N, -3
        scores = torch.full((1, 1, n), 7.0, dtype=torch.float32, device="cuda")
        rk.pred_score_blocks(p.handle, 0, _to_dev(q), _tab_dev(bad[None]), scores)
        with pytest.raises(rk.PredError) as e:
            rk.pred_device_error(p.handle)
        assert e.value.code == rk.PRED_ERR_DEVICE
        got = scores.cpu().numpy().ravel()
        a_g = _read_slots(p.handle, d, [(0, b) for b in range(N)])
        want = predictor.score_blocks(q, a_g, 0, tab[None], n).ravel()
        ok = np.ones(n, bool)
        ok[[1, n - 2]] = False
        assert np.isnan(got[~ok]).all()
        assert_scores(got[ok], want[ok], R, "valid neighbours")


def test_zero_sized_calls_are_noops():
    """Every entry point accepts a zero count as a no-op: no error, no write."""
    d = rk.dims(2, 4, 2, 64, 16, 16, 8)
    with rk.Predictor(d, 3, flags=rk.PRED_FLAG_ZERO_AG) as p:
        h = p.handle
        lib = rk.lib()
        st = None
        assert lib.pred_project_q(h, None, 0, None, st) == 0
        assert lib.pred_project_kv_block(h, 0, 2, None, None, 0, st) == 0
        assert lib.pred_project_kv_block(h, 0, 0, None, None, 5, st) == 0
        assert lib.pred_project_step(h, 0, 2, None, None, 0, None, 0, None, st) == 0
        assert lib.pred_score_blocks(h, 0, 2, None, 1, None, 0, 1, None, st) == 0      # no blocks
        assert lib.pred_score_blocks(h, 0, 2, None, 1, None, 4, 0, None, st) == 0      # no sequences
        assert lib.pred_score_blocks(h, 0, 0, None, 1, None, 4, 1, None, st) == 0      # no layers
        assert lib.pred_rank_victims(h, None, 0, 3, None, None, 0, st) == 0
        assert lib.pred_rank_victims(h, None, 5, 0, None, None, 0, st) == 0
        assert lib.pred_select_victims(h, None, 5, 2, 0, None, None, 0, st) == 0
        assert lib.pred_score_rows(h, 0, None, 0, 0, None, 4, None, 4, st) == 0
        assert lib.pred_select_keep(h, None, 0, 4, 0, 16, 2, None, None, 0, st) == 0
        # n_rows = 0 with work to do is an error, not a no-op
        assert lib.pred_score_blocks(h, 0, 1, None, 0, None, 4, 1, None, st) == rk.PRED_ERR_OUT_OF_RANGE
        torch.cuda.synchronize()
        rk.pred_device_error(h)
        assert not rk.pred_read_slot(h, 0, 0).any()


def test_host_side_range_errors():
    d = rk.dims(2, 4, 2, 64, 16, 16, 8)
    with rk.Predictor(d, 3) as p:
        k = torch.zeros((1, 1, 16, 2, 64), dtype=torch.bfloat16, device="cuda")
        with pytest.raises(rk.PredError) as e:
            rk.pred_project_kv_block(p.handle, 2, k)
        assert e.value.code == rk.PRED_ERR_OUT_OF_RANGE
        qp = torch.zeros((2, 1, 1, 4, 16), dtype=torch.bfloat16, device="cuda")
        sc = torch.empty((2, 1, 9), dtype=torch.float32, device="cuda")
        with pytest.raises(rk.PredError) as e:
            rk.pred_score_blocks(p.handle, 0, qp, None, sc)        # 9 blocks > max_blocks without a table
        assert e.value.code == rk.PRED_ERR_OUT_OF_RANGE
        with pytest.raises(rk.PredError) as e:
            rk.pred_score_blocks(p.handle, 1, qp, None, sc[:, :, :4].contiguous())   # layers 1..2 of 2
        assert e.value.code == rk.PRED_ERR_OUT_OF_RANGE


def test_oom_is_reported_before_allocation():
    free, _ = torch.cuda.mem_get_info()
    # A_g sized at the whole free memory: above the 95% budget
    per_block = 8 * 16 * 64 * 2
    d = rk.dims(1, 8, 8, 128, 64, 16, free // per_block)
    with pytest.raises(rk.PredError) as e:
        rk.pred_create(d, 1)
    assert e.value.code == rk.PRED_ERR_OOM
    assert "halves A_g" in str(e.value)


# ------------------------------------------------- decode scorer variants at their limits

# (dims L, Hq, Hk, D, R, B, N), rows, sequences, blocks, slot ids ("high": most ids above the
# first 4 GiB of the layer slab), expected kernel variant
VARIANT_CASES = [
    # one layer's A_g slab is 4.6 GB: 64-bit slab offsets (4 queries per kv head)
    ((1, 32, 8, 128, 64, 32, 140000), 1, 1, 600, "high",
     "score_decode_kernel<lanes_per_row=8,queries=4,slots=4,q_in_lds=1,offset=u64,uniform_slots=0>"),
    # the same slab with 8 queries per kv head: the matrix-core variant needs 32-bit offsets, so the
    # vector-ALU kernel takes it
    ((1, 32, 8, 128, 64, 32, 140000), 2, 1, 300, "high",
     "score_decode_kernel<lanes_per_row=8,queries=8,slots=4,q_in_lds=1,offset=u64,uniform_slots=0>"),
    # a (layer, sequence) q_proj slab of 64 KiB (4 rows x 64 heads x r = 128) does not fit the
    # 32 KiB LDS stage: queries come from global memory
    ((1, 64, 64, 64, 128, 16, 300), 4, 2, 133, "perm",
     "score_decode_kernel<lanes_per_row=16,queries=4,slots=4,q_in_lds=0,offset=u64,uniform_slots=0>"),
    # r = 32, block_size 64, 8 queries per kv head: matrix-core decode with each block's four
    # wave-loads per kv region split over a pair of waves
    ((1, 16, 2, 64, 32, 64, 40), 1, 1, 27, "perm",
     "score_decode_mfma_kernel<r=32,slots=2,waves_per_block=2>"),
]


@pytest.mark.parametrize("case", VARIANT_CASES, ids=[c[5].split("<")[0] + f"-N{c[0][6]}-M{c[1]}-S{c[2]}"
                                                     for c in VARIANT_CASES])
def test_decode_variant_parity(case):
    """Kernel variants that only unusual shapes reach (a layer slab of 4 GiB or more, a q_proj slab
    above the LDS stage, a block split over two waves): the call takes the intended variant, and A_g,
    scores and ranking match the oracle.  Only the scored slots are written and read back."""
    (L, Hq, Hk, D, R, B, N), M, S, n, ids, want_variant = case
    _say("variant", case)
    rng = np.random.default_rng([N, M, S, n, R])
    d = rk.dims(L, Hq, Hk, D, R, B, N)
    seed = int(rng.integers(0, 2 ** 63))
    with rk.Predictor(d, seed) as p:
        assert rk.pred_score_kernel_variant(p.handle, M, n) == want_variant
        if ids == "high":
            slab = N * Hk * B * R * 2
            first_high = -(-(1 << 32) // (Hk * B * R * 2))           # first slot past 4 GiB
            assert slab > (1 << 32) and first_high < N
            hi = rng.choice(np.arange(first_high, N), (2 * S * n) // 3, replace=False)
            lo = rng.choice(first_high, S * n - hi.size, replace=False)
            phys = rng.permutation(np.concatenate([hi, lo])).astype(np.int32).reshape(S, n)
        else:
            phys = rng.permutation(N)[: S * n].astype(np.int32).reshape(S, n)
        P = prng.projection(D, R, seed)
        k = _randn_bits(rng, (1, S * n, B, Hk, D))
        rk.pred_project_kv_block(p.handle, 0, _to_dev(k), _tab_dev(phys.reshape(1, -1)))
        q = _randn_bits(rng, (1, S, M, Hq, D))
        qp = torch.empty((1, S, M, Hq, R), dtype=torch.bfloat16, device="cuda")
        rk.pred_project_q(p.handle, _to_dev(q), qp)
        scores = torch.empty((1, S, n), dtype=torch.float32, device="cuda")
        rk.pred_score_blocks(p.handle, 0, qp, _tab_dev(phys), scores)
        vic = torch.empty((S, n), dtype=torch.int32, device="cuda")
        ws_b = rk.pred_rank_workspace_bytes(n, S)
        ws = torch.empty((ws_b // 8 + 1,), dtype=torch.int64, device="cuda") if ws_b else None
        rk.pred_rank_victims(p.handle, scores.view(S, n), vic, ws)
        rk.pred_device_error(p.handle)
        qp_bits = _bits_np(qp)
        assert_ulp(qp_bits, predictor.project_q(q, P), "q_proj")
        slots = np.stack([rk.pred_read_slot(p.handle, 0, int(b)) for b in phys.reshape(-1)])
        assert_ulp(slots, predictor.project_kv_slots(k[0], P), "A_g")
        slots = slots.reshape(S, n, Hk, B, R)
        got = scores.cpu().numpy()[0]
        want = np.stack([predictor.score_one(qp_bits[0, s], slots[s]) for s in range(S)])
        assert_scores(got, want, R)
        assert_ranking(vic.cpu().numpy(), got, want, R)


# ------------------------------------------------- run-time score path override

OVERRIDE_SHAPES = [
    # L, Hq, Hk, D, R, B, N, n, S, M: each auto choice in turn
    (1, 32, 8, 128, 64, 16, 300, 260, 1, 64),    # many-row MFMA scorer
    (1, 64, 8, 128, 64, 32, 100, 97, 1, 1),      # matrix-core decode
    (2, 32, 8, 128, 32, 16, 300, 150, 2, 1),     # vector-ALU decode
]


@pytest.mark.parametrize("shape", OVERRIDE_SHAPES, ids=[f"q{s[1]}-kv{s[2]}-r{s[4]}-b{s[5]}-M{s[9]}"
                                                       for s in OVERRIDE_SHAPES])
def test_forced_score_paths_agree(shape):
    """pred_set_score_path routes the same call through the vector-ALU decode kernel or the plain
    kernel; each forced path's scores match the default path's and the oracle's within the score
    tolerance, and the kernel name follows the setting."""
    L, Hq, Hk, D, R, B, N, n, S, M = shape
    _say("forced paths", shape)
    rng = np.random.default_rng(list(shape))
    d = rk.dims(L, Hq, Hk, D, R, B, N)
    with rk.Predictor(d, 99, flags=rk.PRED_FLAG_ZERO_AG) as p:
        phys = rng.permutation(N)[: S * n].astype(np.int32).reshape(S, n)
        k = _randn_bits(rng, (L, S * n, B, Hk, D))
        rk.pred_project_kv_block(p.handle, 0, _to_dev(k), _tab_dev(np.broadcast_to(phys.reshape(1, -1), (L, S * n))))
        q = _randn_bits(rng, (L, S, M, Hq, D))
        qp = torch.empty((L, S, M, Hq, R), dtype=torch.bfloat16, device="cuda")
        rk.pred_project_q(p.handle, _to_dev(q), qp)
        tab = _tab_dev(phys)
        got = {}
        names = {}
        assert rk.pred_get_score_path() == rk.PRED_SCORE_PATH_AUTO
        try:
            for path in (rk.PRED_SCORE_PATH_AUTO, rk.PRED_SCORE_PATH_DECODE, rk.PRED_SCORE_PATH_GENERIC):
                rk.pred_set_score_path(path)
                names[path] = rk.pred_score_kernel_name(p.handle, M)
                sc = torch.empty((L, S, n), dtype=torch.float32, device="cuda")
                rk.pred_score_blocks(p.handle, 0, qp, tab, sc)
                torch.cuda.synchronize()
                got[path] = sc.cpu().numpy()
        finally:
            rk.pred_set_score_path(rk.PRED_SCORE_PATH_AUTO)
        rk.pred_device_error(p.handle)
        assert names[rk.PRED_SCORE_PATH_DECODE] == "score_decode_kernel"
        assert names[rk.PRED_SCORE_PATH_GENERIC] == "score_generic_kernel"
        with pytest.raises(rk.PredError):
            rk.pred_set_score_path(7)
        a_g = _read_slots(p.handle, d, [(l, int(b)) for l in range(L) for b in phys.reshape(-1)])
        want = predictor.score_blocks(_bits_np(qp), a_g, 0, phys, n)
        for path, s in got.items():
            assert_scores(s, want, R, f"scores on path {path} ({names[path]})")
            assert_scores(s, got[rk.PRED_SCORE_PATH_AUTO], R, f"path {path} against the default path")


def test_forced_generic_row_scores():
    """The override also routes pred_score_rows through its plain per-cell kernel; both agree."""
    _say("forced rows")
    Hq, Hk, D, R, B, n, rows = 16, 4, 64, 32, 16, 40, 70
    rng = np.random.default_rng(3)
    d = rk.dims(1, Hq, Hk, D, R, B, n)
    with rk.Predictor(d, 5, flags=rk.PRED_FLAG_ZERO_AG) as p:
        k = _randn_bits(rng, (1, n, B, Hk, D))
        rk.pred_project_kv_block(p.handle, 0, _to_dev(k))
        qp = _to_dev(_randn_bits(rng, (rows, Hq, R), 0.5))
        first_pos = n * B - rows
        out = {}
        try:
            for path in (rk.PRED_SCORE_PATH_AUTO, rk.PRED_SCORE_PATH_GENERIC):
                rk.pred_set_score_path(path)
                sc = torch.empty((rows, n + 3), dtype=torch.float32, device="cuda")
                rk.pred_score_rows(p.handle, 0, qp, first_pos, None, n, sc)
                torch.cuda.synchronize()
                out[path] = sc.cpu().numpy()
        finally:
            rk.pred_set_score_path(rk.PRED_SCORE_PATH_AUTO)
        a, g = out[rk.PRED_SCORE_PATH_AUTO], out[rk.PRED_SCORE_PATH_GENERIC]
        assert np.array_equal(np.isneginf(a), np.isneginf(g))
        m = ~np.isneginf(a)
        assert_scores(g[m], a[m], R, "generic row scores against the MFMA row scorer")


# ------------------------------------------------- projections: correctly rounded at scale

def _surely_rounded(q, P):
    """Outputs where the oracle's float64 dot product, whatever its rounding error (at most
    D * 2^-52 * sum|products|), is farther from both bf16 rounding midpoints around it than that
    error: there the oracle's bf16 is the correctly rounded one, so the GPU must equal it bit for
    bit.  The midpoints are halfway to the neighbouring bf16 values (ordinals +-1)."""
    x = bf16.decode(q).reshape(-1, q.shape[-1])
    p = bf16.decode(P)
    y = x @ p
    err = x.shape[1] * 2.0 ** -52 * (np.abs(x) @ np.abs(p))
    o = bf16.ordinal(bf16.encode(y))

    def from_ordinal(k):
        k = np.clip(k, -0x7F80, 0x7F80)
        return bf16.decode(np.where(k >= 0, k, 0x8000 | (-k)).astype(np.uint16))

    v = from_ordinal(o)
    lo_mid = (from_ordinal(o - 1) + v) / 2
    hi_mid = (from_ordinal(o + 1) + v) / 2
    with np.errstate(invalid="ignore"):
        dist = np.minimum(np.abs(y - lo_mid), np.abs(hi_mid - y))
    return np.isfinite(dist) & (dist > err)


def _tie_projection(D, R, rng):
    """P with P[j, j] = 1 and P[D/2 + j, j] = 2^-8 (0 elsewhere), and queries whose two
    terms land every output exactly on a bf16 rounding midpoint or one ulp of float32 beside
    it: ties to even and near-ties the bound cannot decide."""
    P = np.zeros((D, R))
    for j in range(R):
        P[j, j] = 1.0
        P[D // 2 + j, j] = 2.0 ** -8
    return bf16.encode(P)


@pytest.mark.parametrize("D,R,n_vec,kind", [(128, 64, 20000, "normal"), (128, 32, 40000, "normal"),
                                            (64, 64, 17000, "cancel"), (128, 64, 16400, "ties"),
                                            (256, 32, 33000, "normal"), (32, 64, 16500, "small"),
                                            (128, 64, 16390, "nonfinite")])
def test_project_q_large_calls_exact(D, R, n_vec, kind):
    """Large project_q calls (>= 4096 16x16 output tiles: the streaming float64 MFMA kernel)
    return the correctly rounded bf16 of the exact dot products bit for bit: on random data, on
    cancelling pairs (outputs near zero with large sums of |products|), on exact rounding
    midpoints and float32-near midpoints (ties to even), on values near the float32 subnormal
    range, and with infinities and NaNs in the input."""
    assert (n_vec + 15) // 16 * (R // 16) >= 4096
    _say("project_q large call", D, R, n_vec, kind)
    rng = np.random.default_rng(D * 7 + R + n_vec)
    d = rk.dims(1, 1, 1, D, R, 16, 4)
    if kind == "ties":
        P = _tie_projection(D, R, rng)
        qf = np.zeros((n_vec, D))
        qf[:, :R] = rng.integers(1, 255, size=(n_vec, R)) * 2.0 ** -7 + 1.0     # 1 + k 2^-7: bf16-exact
        qf[:, D // 2:D // 2 + R] = rng.choice([1.0, 3.0, 5.0, -1.0, 1.0 + 2 ** -7, 1.0 - 2 ** -8], size=(n_vec, R))
        q = bf16.encode(qf).reshape(n_vec, 1, D)
    else:
        P = prng.projection(D, R, 777 + D + R)
        if kind == "cancel":
            # pairs of equal P rows and opposite query values: the sums cancel to small residuals
            P = P.copy()
            P[1::2] = P[0::2]
            x = rng.standard_normal((n_vec, D // 2))
            qf = np.empty((n_vec, D))
            qf[:, 0::2] = x
            qf[:, 1::2] = -x * (1.0 + rng.integers(-2, 3, size=x.shape) * 2.0 ** -7)
            q = bf16.encode(qf).reshape(n_vec, 1, D)
        elif kind == "small":
            q = _randn_bits(rng, (n_vec, 1, D), 2.0 ** -60)        # products near 2^-120
        else:
            q = _randn_bits(rng, (n_vec, 1, D))
            if kind == "nonfinite":
                q = q.copy()
                q[3, 0, 5] = 0x7F80      # +inf
                q[700, 0, 9] = 0xFF80    # -inf
                q[900, 0, 1] = 0x7FC0    # NaN
                q[1500, 0, 7] = 0x7F7F   # largest finite: some sums overflow float32
                q[1500, 0, 8] = 0x7F7F
    with rk.Predictor(d, projection=P) as p:
        qp = torch.empty((n_vec, 1, R), dtype=torch.bfloat16, device="cuda")
        rk.pred_project_q(p.handle, _to_dev(q), qp)
        torch.cuda.synchronize()
        got = _bits_np(qp)
    want = predictor.project_q(q, P)
    if kind == "nonfinite":
        # NaN outputs may carry any NaN payload; everything else exactly
        gnan = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
        wnan = ((want & 0x7F80) == 0x7F80) & ((want & 0x7F) != 0)
        assert np.array_equal(gnan, wnan)
        assert np.array_equal(got[~gnan], want[~wnan])
    elif kind == "ties":
        # every term is a multiple of 2^-15 below 2^9: the oracle's float64 sums are exact
        bad = got != want
        assert not bad.any(), f"{int(bad.sum())} outputs differ; first at {np.argwhere(bad)[0]}"
    else:
        sure = _surely_rounded(q, P).reshape(got.shape)
        assert sure.mean() > 0.99, sure.mean()
        bad = (got != want) & sure
        assert not bad.any(), f"{int(bad.sum())} outputs differ; first at {np.argwhere(bad)[0]}"
        assert_ulp(got, want, "q_proj")   # and everywhere within the 1-ulp bar


@pytest.mark.parametrize("R,B,Hk,n_blocks", [(64, 16, 8, 128), (32, 16, 8, 300), (64, 32, 4, 130)])
def test_project_kv_block_large_calls_exact(R, B, Hk, n_blocks):
    """Large project_kv_block calls (the prefill chunk's 128 new blocks) through the paged output
    map: every slot equals the correctly rounded projection, slots go through the block table,
    and an invalid entry is skipped and reported."""
    D = 128
    n_vec = n_blocks * B * Hk
    assert (n_vec + 15) // 16 * (R // 16) >= 4096
    _say("project_kv_block large call", R, B, Hk, n_blocks)
    rng = np.random.default_rng(R + B + Hk + n_blocks)
    N = n_blocks + 20
    d = rk.dims(1, Hk, Hk, D, R, B, N)
    with rk.Predictor(d, 4321 + R, flags=rk.PRED_FLAG_ZERO_AG) as p:
        P = prng.projection(D, R, 4321 + R)
        k = _randn_bits(rng, (1, n_blocks, B, Hk, D))
        tab = rng.permutation(N)[:n_blocks].astype(np.int32)
        bad = tab.copy()
        bad[7] = N + 3
        rk.pred_project_kv_block(p.handle, 0, _to_dev(k), _tab_dev(bad[None]))
        with pytest.raises(rk.PredError) as e:
            rk.pred_device_error(p.handle)
        assert e.value.code == rk.PRED_ERR_DEVICE
        want = predictor.project_kv_slots(k[0], P)
        got = np.stack([rk.pred_read_slot(p.handle, 0, int(b)) for b in tab])
        ok = np.ones(n_blocks, bool)
        ok[7] = False
        sure = _surely_rounded(k[0], P).reshape(n_blocks, B, Hk, R).transpose(0, 2, 1, 3)
        assert ((got != want) & sure)[ok].sum() == 0
        assert_ulp(got[ok], want[ok], "A_g")
        assert not got[7].any()            # slot tab[7] was never written (A_g zeroed)
