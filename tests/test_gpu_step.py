"""GPU tests of pred_decode_step, the whole decode step in one call (and captured in a HIP graph)."""

import numpy as np
import pytest

import rank_kv_block_amd as rk
from oracle import predictor
from tests.devmem import a_g_layer
from tests.parity import assert_ranking, assert_scores

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print("[case]", *a, flush=True)


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rk.lib()
    yield
    torch.cuda.synchronize()


def _workload(n=150, N=600, L=4, S=3, M=1, table="slices"):
    from rank_kv_block_amd.workloads import Config, Workload
    c = Config("step_test", 9, L=L, Hq=8, Hk=2, D=64, R=32, B=16, N=N, n=n, S=S, M=M, step_layers=L,
               keys="normal", table=table, planted=0, new_blocks=1,
               description=f"{L} layers x {S} sequences x {n} blocks, nq=8, nkv=2, head_dim=64, r=32")
    return Workload(c)


def _separate_calls(wl):
    """The step as the four single-purpose entry points, into the workload's own outputs."""
    c = wl.cfg
    nl = c.step_layers
    rk.pred_project_kv_block(wl.h, 0, wl.k_new[:nl], wl.table_new[:nl])
    rk.pred_project_q(wl.h, wl.q[:nl], wl.q_proj)
    rk.pred_score_blocks(wl.h, 0, wl.q_proj, wl.tables, wl.scores)
    rk.pred_rank_victims(wl.h, wl.scores.view(nl * c.S, c.n), wl.victims, wl.workspace)


def _step(wl, k, q_proj, scores, victims, fill=None, stream=None):
    c = wl.cfg
    nl = c.step_layers
    rk.pred_decode_step(wl.h, 0, wl.k_new[:nl], wl.table_new[:nl], wl.q[:nl], q_proj, wl.tables, fill, scores, k,
                        victims, wl.workspace, stream=stream)


@pytest.mark.parametrize("n,M", [(150, 1), (2500, 1), (300, 8), (400, 2)])
def test_decode_step_equals_separate_calls(n, M):
    _say("decode_step", n, M)
    wl = _workload(n=n, N=max(600, 3 * n), M=M)
    try:
        c = wl.cfg
        nl, S = c.step_layers, c.S
        _separate_calls(wl)
        torch.cuda.synchronize()
        qp = torch.empty_like(wl.q_proj)
        sc = torch.full_like(wl.scores, 3.0)
        vic = torch.full_like(wl.victims, -5)
        _step(wl, n, qp, sc, vic)
        torch.cuda.synchronize()
        rk.pred_device_error(wl.h)
        assert torch.equal(qp.view(torch.int16), wl.q_proj.view(torch.int16))
        assert torch.equal(sc, wl.scores)
        assert torch.equal(vic, wl.victims)
        # the k lowest only
        vk = torch.full((nl * S, 16), -5, dtype=torch.int32, device="cuda")
        _step(wl, 16, qp, sc, vk)
        assert torch.equal(vk, wl.victims[:, :16])
        # and against the oracle, recomputed from the GPU's own q_proj and A_g
        a_g = np.stack([a_g_layer(wl.h, wl.d, l) for l in range(nl)])
        tables = wl.phys.numpy()
        want = predictor.score_blocks(_bits(qp), a_g, 0, tables, n)
        got = sc.cpu().numpy()
        assert_scores(got, want, c.R, "decode_step scores")
        assert_ranking(vic.cpu().numpy(), got.reshape(nl * S, n), want.reshape(nl * S, n), c.R, "decode_step")
    finally:
        wl.close()


def test_decode_step_masked_last_block():
    wl = _workload()
    try:
        c = wl.cfg
        fill = torch.tensor([1, c.B, 7], dtype=torch.int32, device="cuda")
        qp = torch.empty_like(wl.q_proj)
        sc = torch.empty_like(wl.scores)
        vic = torch.empty_like(wl.victims)
        _step(wl, c.n, qp, sc, vic, fill=fill)
        ref = torch.empty_like(sc)
        rk.pred_score_blocks_masked(wl.h, 0, qp, wl.tables, fill, ref)
        torch.cuda.synchronize()
        assert torch.equal(sc, ref)
    finally:
        wl.close()


def test_decode_step_checks_everything_first():
    """A bad argument of a later part (k > n_blocks) fails before the first part is enqueued."""
    wl = _workload()
    try:
        c = wl.cfg
        qp = torch.zeros_like(wl.q_proj)
        sc = torch.zeros_like(wl.scores)
        vic = torch.zeros((c.step_layers * c.S, c.n + 1), dtype=torch.int32, device="cuda")
        with pytest.raises(rk.PredError) as e:
            _step(wl, c.n + 1, qp, sc, vic)
        assert e.value.code == rk.PRED_ERR_OUT_OF_RANGE
        torch.cuda.synchronize()
        assert not qp.view(torch.int16).any() and not sc.any() and not vic.any()
    finally:
        wl.close()


def test_decode_step_graph_replays():
    """The step captured into a graph: every replay (with eager work in between) equals the eager step."""
    wl = _workload(n=2500, N=7500)
    try:
        c = wl.cfg
        qp = torch.empty_like(wl.q_proj)
        sc = torch.empty_like(wl.scores)
        vic = torch.empty_like(wl.victims)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            _step(wl, c.n, qp, sc, vic)              # eager, on the capture stream's kind of stream
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        want = (qp.clone(), sc.clone(), vic.clone())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            _step(wl, c.n, qp, sc, vic)
        for rep in range(4):
            _say("graph replay", rep)
            qp.zero_()
            sc.fill_(-1.0)
            vic.fill_(-9)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(qp.view(torch.int16), want[0].view(torch.int16)), rep
            assert torch.equal(sc, want[1]), rep
            assert torch.equal(vic, want[2]), rep
            wl.step(0)                                # eager work of the program between replays
            torch.cuda.synchronize()
        rk.pred_device_error(wl.h)
        del g
    finally:
        wl.close()
