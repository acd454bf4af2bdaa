"""Throughput of the block predictor's hot path on one MI355X.

One step = one pass of the whole path over one batch of the workload:
project_kv_block (the step's new blocks) and project_q (one pred_project_step
call), score_blocks and rank_victims (see rank_kv_block_amd/workloads.py).  The default workload is the
Llama-3-8B-shaped decode step: 32 layers x 8192 blocks, 2 GiB of A_g per step.

Prints one JSON line.  `value` is the A_g bytes the step's scoring reads per
second of whole-step time, in GB/s; the score kernel alone is timed with HIP
events on the stream it runs on and reported in `roofline`.  The oracle's time
on a bounded sample of the same work, on this host's cores, is `cpu_baseline`.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E peak, 8 TB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix peak, 2.5 PFLOP/s


# sources of each score kernel family (the recorded counters hold only while these are unchanged)
_KERNEL_SOURCES = {"score_decode": ["score_decode.hip", "common.h", "kernels.h"],
                   "score_prefill": ["score_prefill.hip", "common.h", "kernels.h"],
                   "score_rows": ["score_rows.hip", "common.h", "kernels.h"]}


def _score_kernel_source_hash(family="score_decode"):
    h = hashlib.sha256()
    for f in _KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, "rank_kv_block_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(workload, family="score_decode"):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match the current kernel."""
    path = os.path.join(ROOT, "profiles", f"{family}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256_16") != _score_kernel_source_hash(family):
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(wl, budget_s=12.0):
    """The oracle as it stands, timed on this host's cores on the GPU's own q_proj and
    A_g: project_q + score + rank of the step's (layer, sequence) rows, repeated or
    cut so that about budget_s seconds of host time are measured."""
    import numpy as np
    import torch
    from oracle import predictor
    from tests.devmem import a_g_layer
    import rank_kv_block_amd as rk

    c = wl.cfg
    qp_all = wl.q_proj.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    q_all = wl.q.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    P = rk.pred_copy_projection(wl.h)
    phys = wl.phys.numpy()
    l0 = wl.layer0_for_step(0)
    rows = []
    for li in range(c.step_layers):
        a_layer = a_g_layer(wl.h, wl.d, l0 + li)
        for s in range(c.S):
            rows.append((li, s, np.ascontiguousarray(a_layer[phys[s]])))
            if len(rows) * c.n * c.slot_bytes > (4 << 30):   # bound host memory
                break
        del a_layer
        if len(rows) * c.n * c.slot_bytes > (4 << 30):
            break
    done = 0
    blocks = 0
    elapsed = 0.0
    parts = {"project_q": 0.0, "score_blocks": 0.0, "rank_victims": 0.0}
    while elapsed < budget_s:
        li, s, slots = rows[done % len(rows)]
        t0 = time.perf_counter()
        predictor.project_q(q_all[l0 + li, s], P)
        t1 = time.perf_counter()
        sc = predictor.score_one(qp_all[li, s], slots)
        t2 = time.perf_counter()
        predictor.rank_victims(sc.astype(np.float32)[None])
        t3 = time.perf_counter()
        parts["project_q"] += t1 - t0
        parts["score_blocks"] += t2 - t1
        parts["rank_victims"] += t3 - t2
        elapsed += t3 - t0
        done += 1
        blocks += c.n
    threads = 1
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        pass
    gbs = blocks * c.slot_bytes / elapsed / 1e9
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "blocks_per_s": round(blocks / elapsed, 1), "seconds": round(elapsed, 2),
            "seconds_per_part": {k: round(v, 3) for k, v in parts.items()},
            "rank_keys_per_s": round(blocks / parts["rank_victims"], 1) if parts["rank_victims"] > 0 else None,
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model,
            "sample": f"{done} (layer, sequence) score rows of {c.n} blocks each (project_q + score_blocks + "
                      f"rank_victims, float64 NumPy on the GPU's own q_proj and A_g), cycling over "
                      f"{len(rows)} distinct rows of the same workload"}


def roofline_of(c, kernel, score_ms):
    """Roofline of one score launch of workload c from its mean duration: HBM for the decode
    kernels (algorithmic A_g bytes), bf16 MFMA for the many-row kernel (algorithmic flops)."""
    nl = c.step_layers
    a_g_bytes = c.blocks_per_step * c.slot_bytes
    aux_bytes = c.blocks_per_step * 8 + nl * c.S * c.M * c.Hq * c.R * 2   # table entry + score per block, q_proj
    if kernel == "score_prefill_kernel":
        # a contraction: every (query row, head) against every key of every block
        flops = 2.0 * nl * c.S * c.M * c.Hq * c.R * c.n * c.B
        achieved = flops / (score_ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFS, 4),
                "traffic": _traffic(c.name, "score_prefill"),
                "kernel": kernel, "algorithmic_flops_per_launch": flops,
                "algorithmic_bytes_per_launch": a_g_bytes + aux_bytes}
    achieved = a_g_bytes / (score_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": _traffic(c.name),
            "kernel": kernel, "algorithmic_bytes_per_launch": a_g_bytes, "aux_bytes_per_launch": aux_bytes}


def time_steps(wl, steps, warmup):
    """Warm up, then time `steps` whole steps (project_step + score_blocks + rank_victims) on
    torch's current stream: host wall time per step, the HIP-event time (ms) of the score launch
    of every `stride`-th step (every 4th from 32 steps, every 2nd from 16), and the stride.  A
    timed event pair costs its step ~6 us of GPU idle (measured on the 8B step: 339-343 us with a pair
    on every step, 335.5 with one on every 4th, 333.5 with none; the score kernel's own time
    is the same either way), so bracketing every step would put the measurement into the
    step time it measures."""
    import torch
    import rank_kv_block_amd as rk
    c = wl.cfg
    nl = c.step_layers
    for i in range(warmup):
        wl.step(wl.layer0_for_step(i))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    stride = 4 if steps >= 32 else (2 if steps >= 16 else 1)
    ev = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for i in range(0, steps, stride)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        l0 = wl.layer0_for_step(i)
        rk.pred_project_step(wl.h, l0, wl.k_new[l0:l0 + nl], wl.table_new[l0:l0 + nl], wl.q[l0:l0 + nl], wl.q_proj)
        pair = ev.get(i)
        if pair is not None:
            pair[0].record(stream)
        rk.pred_score_blocks(wl.h, l0, wl.q_proj, wl.tables, wl.scores)
        if pair is not None:
            pair[1].record(stream)
        rk.pred_rank_victims(wl.h, wl.scores.view(nl * c.S, c.n), wl.victims, wl.workspace)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    rk.pred_device_error(wl.h)
    return (t1 - t0) / steps, sorted(a.elapsed_time(b) for a, b in ev.values()), stride


def keep_set_timing(wl, stream):
    """Per-row causal scores and keep sets of the first layer and sequence of a many-row
    workload: each query row against the blocks complete at its position, then every row's
    top-k; each entry point timed with HIP events on `stream`, median of 20."""
    import torch
    import rank_kv_block_amd as rk
    c = wl.cfg
    wl.keep_setup(64)
    evr, evs_k = [], []
    for i in range(20):
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        tab = None if wl.tables is None else wl.tables[0]
        e0.record(stream)
        rk.pred_score_rows(wl.h, 0, wl.q_proj[0, 0], c.first_pos, tab, c.n, wl.row_scores)
        e1.record(stream)
        rk.pred_select_keep(wl.h, wl.row_scores, c.first_pos, c.B, wl.topk, wl.keep, wl.keep_ws)
        e2.record(stream)
        evr.append((e0, e1))
        evs_k.append((e1, e2))
    torch.cuda.synchronize()
    rk.pred_device_error(wl.h)
    tr = sorted(a.elapsed_time(b) for a, b in evr)
    ts = sorted(a.elapsed_time(b) for a, b in evs_k)
    # algorithmic work: every complete (row, block) pair, all heads and tokens
    pairs = sum(c.complete_blocks(i) for i in range(c.M))
    rflops = 2.0 * pairs * c.B * c.Hq * c.R
    r_med = tr[len(tr) // 2]
    r_ach = rflops / (r_med * 1e-3) / 1e12
    return {"rows": c.M, "blocks": c.n, "first_pos": c.first_pos, "topk": wl.topk,
            "score_rows_us": {"median": round(r_med * 1e3, 2), "min": round(tr[0] * 1e3, 2),
                              "max": round(tr[-1] * 1e3, 2)},
            "select_keep_us": {"median": round(ts[len(ts) // 2] * 1e3, 2), "min": round(ts[0] * 1e3, 2),
                               "max": round(ts[-1] * 1e3, 2)},
            "roofline": {"bound": "mfma", "achieved": round(r_ach, 2), "peak": MFMA_BF16_PEAK_TFS,
                         "unit": "TFLOP/s", "frac": round(r_ach / MFMA_BF16_PEAK_TFS, 4),
                         "traffic": _traffic(c.name, "score_rows"),
                         "kernel": "score_rows_kernel", "algorithmic_flops_per_launch": rflops}}


def other_configs(names, steps, warmup, keep_alive):
    """Each other workload in turn, set up and timed as the headline one (whole step and score
    kernel): one entry per workload with its score kernel's roofline.  Workloads are freed only
    after all are timed (appended to keep_alive): after a large free, a memory-bound kernel timed
    within the next seconds runs measurably slower (the batched decode step by ~3%; 25 s of idle
    restores it), most likely the driver clearing the freed memory in the background."""
    import torch
    import rank_kv_block_amd as rk
    from rank_kv_block_amd.workloads import CONFIGS, Workload
    out = {}
    for name in names:
        c = CONFIGS[name]
        print(f"[bench] config {name}: {c.description}", file=sys.stderr, flush=True)
        t_setup = time.perf_counter()
        wl = Workload(c)
        keep_alive.append(wl)
        setup_s = time.perf_counter() - t_setup
        step_s, each, stride = time_steps(wl, steps, warmup)
        kernel = rk.pred_score_kernel_name(wl.h, c.M)
        score_ms = sum(each) / len(each)
        a_g_bytes = c.blocks_per_step * c.slot_bytes
        out[name] = {
            "description": c.description,
            "a_g_bytes_per_step": a_g_bytes,
            "ms_per_step": round(step_s * 1e3, 4),
            "step_a_g_gbs": round(a_g_bytes / step_s / 1e9, 2),
            "blocks_per_s": round(c.blocks_per_step / step_s, 1),
            "score_kernel_us": {"mean": round(score_ms * 1e3, 2), "median": round(each[len(each) // 2] * 1e3, 2),
                                "min": round(each[0] * 1e3, 2), "max": round(each[-1] * 1e3, 2),
                                "launches_timed": len(each), "of_every_nth_step": stride},
            "score_kernel_variant": rk.pred_score_kernel_variant(wl.h, c.M, c.n),
            "roofline": roofline_of(c, kernel, score_ms),
            "setup_s": round(setup_s, 2),
        }
        if a_g_bytes < (1 << 20) and kernel != "score_prefill_kernel":
            # a few KiB per call: launch latency, not a bandwidth or matrix roofline
            out[name]["roofline"] = {"bound": "launch latency", "score_call_us": round(score_ms * 1e3, 2),
                                     "kernel": kernel, "algorithmic_bytes_per_launch": a_g_bytes}
        if c.M > 1:
            out[name]["keep_sets"] = keep_set_timing(wl, torch.cuda.current_stream())
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="llama3_8b_decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--per-layer-calls", action="store_true",
                    help="also time the step's layers scored one layer per call (multi-layer workloads)")
    ap.add_argument("--configs", default="tiny,batched_decode,long_context_70b,prefill_chunk",
                    help="other workloads timed after the headline one, in the same process (comma list, or "
                         "'none')")
    ap.add_argument("--config-steps", type=int, default=40, help="timed steps of each other workload")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run one plain device copy of MIB MiB (a known-size reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the predictor's path has no multi-GPU part here); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import rank_kv_block_amd as rk
    from rank_kv_block_amd.workloads import CONFIGS, Workload

    rk.lib()   # fails loudly when the HIP library is missing
    c = CONFIGS[args.config]
    torch.cuda.set_device(0)
    print(f"[bench] setting up {c.name}: {c.description}", file=sys.stderr, flush=True)
    wl = Workload(c)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    stream = torch.cuda.current_stream()
    nl = c.step_layers
    print(f"[bench] warmup {args.warmup}, timing {args.steps} steps", file=sys.stderr, flush=True)
    step_s, score_each, ev_stride = time_steps(wl, args.steps, args.warmup)
    score_ms = sum(score_each) / len(score_each)

    # per-call breakdown of a step, in a separate loop so the timed steps above
    # carry no extra events: median of 20 steps per entry point
    names = ["project_kv_block", "project_q", "project_step", "score_blocks", "rank_victims", "score_blocks_masked"]
    evs = {k: [] for k in names}
    # the decode case of a partly filled last block: half of block_size + 1 tokens in every sequence
    fill = torch.full((c.S,), c.B // 2 + 1, dtype=torch.int32, device="cuda")
    for i in range(20):
        l0 = wl.layer0_for_step(i)
        calls = [
            lambda: rk.pred_project_kv_block(wl.h, l0, wl.k_new[l0:l0 + nl], wl.table_new[l0:l0 + nl]),
            lambda: rk.pred_project_q(wl.h, wl.q[l0:l0 + nl], wl.q_proj),
            lambda: rk.pred_project_step(wl.h, l0, wl.k_new[l0:l0 + nl], wl.table_new[l0:l0 + nl], wl.q[l0:l0 + nl],
                                         wl.q_proj),
            lambda: rk.pred_score_blocks(wl.h, l0, wl.q_proj, wl.tables, wl.scores),
            lambda: rk.pred_rank_victims(wl.h, wl.scores.view(nl * c.S, c.n), wl.victims, wl.workspace),
            lambda: rk.pred_score_blocks_masked(wl.h, l0, wl.q_proj, wl.tables, fill, wl.scores),
        ]
        for name, call in zip(names, calls):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            evs[name].append((e0, e1))
    torch.cuda.synchronize()
    breakdown = {}
    for name in names:
        t = sorted(a.elapsed_time(b) for a, b in evs[name])
        breakdown[name] = round(t[len(t) // 2] * 1e3, 2)
    # the k lowest only (the eviction batch), k = 64: the same scores, the same workspace
    k_sel = min(64, c.n)
    sel_out = torch.empty((nl * c.S, k_sel), dtype=torch.int32, device="cuda")
    evk = []
    for i in range(20):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        rk.pred_select_victims(wl.h, wl.scores.view(nl * c.S, c.n), k_sel, sel_out, wl.workspace)
        e1.record(stream)
        evk.append((e0, e1))
    torch.cuda.synchronize()
    tk = sorted(a.elapsed_time(b) for a, b in evk)
    breakdown[f"select_victims_k{k_sel}"] = round(tk[len(tk) // 2] * 1e3, 2)

    # the whole step as one call (pred_decode_step) and as a replayed HIP graph of
    # that call, against the four separate calls: host wall time per step over 30
    # steps of the same layers (launch overhead shows where the GPU work is short)
    l0f = wl.layer0_for_step(0)
    qp_f, sc_f, vic_f = torch.empty_like(wl.q_proj), torch.empty_like(wl.scores), torch.empty_like(wl.victims)

    def fused():
        rk.pred_decode_step(wl.h, l0f, wl.k_new[l0f:l0f + nl], wl.table_new[l0f:l0f + nl], wl.q[l0f:l0f + nl],
                            qp_f, wl.tables, None, sc_f, c.n, vic_f, wl.workspace)

    def separate():
        rk.pred_project_kv_block(wl.h, l0f, wl.k_new[l0f:l0f + nl], wl.table_new[l0f:l0f + nl])
        rk.pred_project_q(wl.h, wl.q[l0f:l0f + nl], qp_f)
        rk.pred_score_blocks(wl.h, l0f, qp_f, wl.tables, sc_f)
        rk.pred_rank_victims(wl.h, sc_f.view(nl * c.S, c.n), vic_f, wl.workspace)

    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        fused()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fused()
    fused_us = {}
    for name, fn in (("separate_calls", separate), ("decode_step", fused), ("graph_replay", graph.replay)):
        fn()
        torch.cuda.synchronize()
        t_a = time.perf_counter()
        for _ in range(30):
            fn()
        torch.cuda.synchronize()
        fused_us[name] = round((time.perf_counter() - t_a) / 30 * 1e6, 2)
    del graph
    rk.pred_device_error(wl.h)

    # per-row causal scores and keep sets of the first layer and sequence (many-row workloads)
    keep_sets = keep_set_timing(wl, stream) if c.M > 1 else None

    # the same layers scored one per call (a per-layer decode loop), each layer in turn
    per_layer = None
    if nl > 1 and args.per_layer_calls:
        l0 = wl.layer0_for_step(0)
        evl = []
        for rep in range(3):
            for li in range(nl):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                rk.pred_score_blocks(wl.h, l0 + li, wl.q_proj[li:li + 1], wl.tables, wl.scores[li:li + 1])
                e1.record(stream)
                evl.append((e0, e1))
        torch.cuda.synchronize()
        rk.pred_device_error(wl.h)
        lt = sorted(a.elapsed_time(b) for a, b in evl)
        med = lt[len(lt) // 2]
        layer_bytes = c.S * c.n * c.slot_bytes
        per_layer = {"calls": len(lt), "median_us": round(med * 1e3, 2), "min_us": round(lt[0] * 1e3, 2),
                     "max_us": round(lt[-1] * 1e3, 2), "a_g_gbs_at_median": round(layer_bytes / (med * 1e-3) / 1e9, 1)}
    blocks = c.blocks_per_step
    a_g_bytes = blocks * c.slot_bytes
    kernel = rk.pred_score_kernel_name(wl.h, c.M)
    roofline = roofline_of(c, kernel, score_ms)
    out = {
        "metric": "score_blocks A_g GB/s (% of HBM peak) and blocks scored/s, 1 GPU",
        "value": round(a_g_bytes / step_s / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; no model weights or datasets)",
        "config": {"workload": c.name, "description": c.description, "layers_per_step": nl, "sequences": c.S,
                   "blocks_per_sequence": c.n, "query_rows": c.M, "num_q_heads": c.Hq, "num_kv_heads": c.Hk,
                   "head_dim": c.D, "r": c.R, "block_size": c.B, "a_g_bytes_per_step": a_g_bytes},
        "blocks_per_s": round(blocks / step_s, 1),
        "pct_hbm_peak_step": round(100.0 * a_g_bytes / step_s / 1e9 / HBM_PEAK_GBS, 2),
        "score_kernel_ms": round(score_ms, 4),
        "score_kernel_us": {"median": round(score_each[len(score_each) // 2] * 1e3, 2),
                            "min": round(score_each[0] * 1e3, 2), "max": round(score_each[-1] * 1e3, 2),
                            "launches_timed": len(score_each), "of_every_nth_step": ev_stride},
        "score_kernel_path": kernel,
        "score_kernel_variant": rk.pred_score_kernel_variant(wl.h, c.M, c.n),
        "roofline": roofline,
    }
    out["step_breakdown_median_us"] = breakdown
    # ranking: keys ordered per second (every (layer, sequence) row of n blocks)
    out["rank_keys_per_s"] = round(nl * c.S * c.n / (breakdown["rank_victims"] * 1e-6), 1)
    if per_layer is not None:
        out["score_per_layer_call"] = per_layer
    out["step_wall_us"] = fused_us
    if keep_sets is not None:
        out["keep_sets"] = keep_sets
    if not args.no_cpu_baseline:
        print("[bench] oracle cpu baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    others = [n for n in args.configs.split(",") if n and n != "none" and n != c.name]
    alive = [wl]
    if others:
        out["configs"] = other_configs(others, args.config_steps, min(args.warmup, 3), alive)
    for w in alive:
        w.close()
    del side
    torch.cuda.synchronize()
    # this process starts no other process; say so from the process table at the end
    try:
        import psutil
        out["child_processes_at_exit"] = len(psutil.Process().children(recursive=True))
    except ImportError:
        pass
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
