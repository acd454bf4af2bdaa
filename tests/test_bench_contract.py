"""bench.py keeps its output contract: one JSON line with the metric, the roofline of the dominant kernel
and the oracle's CPU baseline; more than one GPU is refused before any GPU work."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, timeout):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                          text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"], 120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.gpu
def test_bench_json_line():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("[case] bench.py --config tiny --configs batched_decode", flush=True)
    r = _run(["--config", "tiny", "--steps", "3", "--warmup", "1", "--cpu-budget", "0.5", "--configs",
              "batched_decode", "--config-steps", "2"], 300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ["metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"]:
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"] == "tiny" and d["vs_baseline"] is None
    rl = d["roofline"]
    for key in ["bound", "achieved", "peak", "unit", "frac", "traffic"]:
        assert key in rl, key
    assert rl["bound"] == "hbm" and rl["peak"] == 8000.0 and rl["achieved"] > 0
    assert abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    assert rl["kernel"] == "score_decode_kernel"
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    # the other workloads, timed after the headline one in the same process
    cfg = d["configs"]["batched_decode"]
    assert cfg["ms_per_step"] > 0 and cfg["score_kernel_us"]["median"] > 0
    assert cfg["roofline"]["bound"] == "hbm" and cfg["roofline"]["kernel"] == "score_decode_kernel"
    assert cfg["score_kernel_variant"].startswith("score_decode_kernel<")
    assert d["child_processes_at_exit"] == 0
