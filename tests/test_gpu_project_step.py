"""GPU tests of pred_project_step: project_kv_block then project_q in one call (one launch when both are small)."""

import numpy as np
import pytest

import rank_kv_block_amd as rk
from oracle import bf16, predictor, prng
from tests.parity import assert_ulp

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print("[case]", *a, flush=True)


def _bits_np(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).cuda()


def _read_layer_slots(h, layers, slots):
    return np.stack([np.stack([rk.pred_read_slot(h, l, b) for b in slots[i]]) for i, l in enumerate(layers)])


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rk.lib()
    yield
    torch.cuda.synchronize()


# (layers, new blocks per layer, query vectors): one shared launch (decode: 1 new
# block per layer), a ragged shared launch, and calls large enough for two launches
CASES = [
    (dict(L=32, Hq=32, Hk=8, D=128, R=32, B=16), 32, 1, 32),      # 8B-shaped decode step
    (dict(L=4, Hq=8, Hk=2, D=64, R=32, B=16), 3, 5, 7),           # ragged tiles
    (dict(L=2, Hq=4, Hk=1, D=256, R=48, B=8), 2, 3, 11),          # head_dim 256, r = 3 column tiles
    (dict(L=1, Hq=32, Hk=8, D=128, R=64, B=16), 1, 128, 2048),    # prefill chunk: two launches
    (dict(L=2, Hq=8, Hk=2, D=96, R=24, B=16), 2, 3, 5),           # plain kernels (no MFMA path)
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_project_step_matches_separate_calls_and_oracle(case):
    dm, nl, n_new, n_vec = CASES[case]
    _say("project_step", dm, nl, n_new, n_vec)
    rng = np.random.default_rng(7100 + case)
    N = 3 * n_new + 5
    d = rk.dims(dm["L"], dm["Hq"], dm["Hk"], dm["D"], dm["R"], dm["B"], N)
    seed = 5150 + case
    P = prng.projection(dm["D"], dm["R"], seed)
    k = bf16.encode(rng.standard_normal((nl, n_new, dm["B"], dm["Hk"], dm["D"])))
    q = bf16.encode(rng.standard_normal((n_vec, dm["Hq"], dm["D"])))
    table = np.stack([rng.permutation(N)[:n_new] for _ in range(nl)]).astype(np.int32)
    layer0 = dm["L"] - nl
    layers = list(range(layer0, dm["L"]))
    outs = []
    for fused in (True, False):
        with rk.Predictor(d, seed, flags=rk.PRED_FLAG_ZERO_AG) as p:
            qp = torch.full((n_vec, dm["Hq"], dm["R"]), 7.0, dtype=torch.bfloat16, device="cuda")
            kd, qd, td = _to_dev(k).view(torch.bfloat16), _to_dev(q).view(torch.bfloat16), torch.from_numpy(table).cuda()
            if fused:
                rk.pred_project_step(p.handle, layer0, kd, td, qd, qp)
            else:
                rk.pred_project_kv_block(p.handle, layer0, kd, td)
                rk.pred_project_q(p.handle, qd, qp)
            torch.cuda.synchronize()
            rk.pred_device_error(p.handle)
            outs.append((_bits_np(qp), _read_layer_slots(p.handle, layers, table)))
    (q_f, a_f), (q_s, a_s) = outs
    assert np.array_equal(q_f, q_s), "q_proj differs from pred_project_q"
    assert np.array_equal(a_f, a_s), "A_g slots differ from pred_project_kv_block"
    assert_ulp(q_f, predictor.project_q(q, P), "q_proj")
    want = np.stack([predictor.project_kv_slots(k[i], P) for i in range(nl)])
    assert_ulp(a_f, want, "A_g")


def test_project_step_one_part_empty():
    """n_new = 0 projects only the queries; n_vec = 0 only the blocks."""
    rng = np.random.default_rng(7200)
    d = rk.dims(2, 8, 2, 64, 32, 16, 6)
    seed = 77
    P = prng.projection(64, 32, seed)
    with rk.Predictor(d, seed, flags=rk.PRED_FLAG_ZERO_AG) as p:
        q = bf16.encode(rng.standard_normal((3, 8, 64)))
        qp = torch.zeros((3, 8, 32), dtype=torch.bfloat16, device="cuda")
        k0 = torch.zeros((2, 0, 16, 2, 64), dtype=torch.bfloat16, device="cuda")
        rk.pred_project_step(p.handle, 0, k0, None, _to_dev(q).view(torch.bfloat16), qp)
        torch.cuda.synchronize()
        assert_ulp(_bits_np(qp), predictor.project_q(q, P), "q_proj")
        assert not rk.pred_read_slot(p.handle, 0, 0).any()
        k = bf16.encode(rng.standard_normal((2, 2, 16, 2, 64)))
        q0 = torch.zeros((0, 8, 64), dtype=torch.bfloat16, device="cuda")
        qp0 = torch.zeros((0, 8, 32), dtype=torch.bfloat16, device="cuda")
        rk.pred_project_step(p.handle, 0, _to_dev(k).view(torch.bfloat16), None, q0, qp0)
        torch.cuda.synchronize()
        rk.pred_device_error(p.handle)
        got = _read_layer_slots(p.handle, [0, 1], [[0, 1], [0, 1]])
        want = np.stack([predictor.project_kv_slots(k[i], P) for i in range(2)])
        assert_ulp(got, want, "A_g")


def test_project_step_invalid_table_entry():
    """An out-of-range table entry is skipped and raises the device error word; the rest is written."""
    rng = np.random.default_rng(7300)
    d = rk.dims(1, 8, 2, 64, 32, 16, 4)
    seed = 78
    P = prng.projection(64, 32, seed)
    with rk.Predictor(d, seed, flags=rk.PRED_FLAG_ZERO_AG) as p:
        k = bf16.encode(rng.standard_normal((1, 2, 16, 2, 64)))
        q = bf16.encode(rng.standard_normal((2, 8, 64)))
        qp = torch.zeros((2, 8, 32), dtype=torch.bfloat16, device="cuda")
        table = torch.tensor([[3, 4]], dtype=torch.int32, device="cuda")   # 4 == max_blocks: invalid
        rk.pred_project_step(p.handle, 0, _to_dev(k).view(torch.bfloat16), table, _to_dev(q).view(torch.bfloat16), qp)
        with pytest.raises(rk.PredError) as e:
            rk.pred_device_error(p.handle)
        assert e.value.code == rk.PRED_ERR_DEVICE
        assert_ulp(rk.pred_read_slot(p.handle, 0, 3)[None], predictor.project_kv_slots(k[0, :1], P), "A_g")
        assert_ulp(_bits_np(qp), predictor.project_q(q, P), "q_proj")


def test_project_step_checks_both_parts_first():
    """A bad query argument fails the call before the block projection is enqueued."""
    rng = np.random.default_rng(7400)
    d = rk.dims(1, 8, 2, 64, 32, 16, 4)
    with rk.Predictor(d, 79, flags=rk.PRED_FLAG_ZERO_AG) as p:
        k = _to_dev(bf16.encode(rng.standard_normal((1, 1, 16, 2, 64)))).view(torch.bfloat16)
        q = _to_dev(bf16.encode(rng.standard_normal((2, 8, 64)))).view(torch.bfloat16)
        buf = torch.zeros(2 * 8 * 32 + 1, dtype=torch.bfloat16, device="cuda")
        qp = buf[1:].view(2, 8, 32)                      # 2-byte offset: not 16-byte aligned
        with pytest.raises(rk.PredError) as e:
            rk.pred_project_step(p.handle, 0, k, None, q, qp)
        assert e.value.code == rk.PRED_ERR_UNSUPPORTED
        torch.cuda.synchronize()
        assert not rk.pred_read_slot(p.handle, 0, 0).any()
        assert not buf.view(torch.int16).any()
