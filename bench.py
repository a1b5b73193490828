"""Benchmark: one selection pass (window score, head sum + stats, both top-k
budgets, K/V/hidden gathers) on a 128K-token GQA layer, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--eager] [--calibrate-copy MIB]
                    [--score-sweep N1,N2,...]

Prints one JSON line.  `value` is context tokens per second of the whole pass
with every input already resident in HBM, timed over K replays of the pass
captured as a HIP graph (one per input copy; `--eager` times eager calls
instead).  `breakdown_us` comes from K eager passes with HIP events recorded
between the calls on the stream the kernels run on; `roofline` times the
window-score call (the dominant kernels) as replays of a graph of
back-to-back calls, and prices it against
MI355X's 8 TB/s HBM peak using its algorithmic bytes (K read once + window
queries + score written), and against a measured 1 GiB device copy
(`copy_ceiling_gbs`); `chain_hbm` does the same for steps 1-3 and for the
whole pass.  `cpu_baseline` is the CPU oracle timed on the host cores over
whole passes of the same workload.

`--score-sweep` instead times the score call alone (two passes, and one pass
with given normalisers) on one sequence of each length N, GQA 32/8, d=128,
w=32, with random bf16 inputs drawn on the GPU, and prints one JSON line per
length.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
CALLS_PER_GRAPH = 10   # single calls are timed as graphs of this many back-to-back calls
METRIC = "scored+selected context tokens/sec at N=128K (GQA 32/8, d=128); % HBM peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "score_pass_traffic.json")
SCORE_SRC = os.path.join(ROOT, "token_selection_tsp_amd", "csrc", "score.hip")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def score_bytes(wl, T: int, B: int) -> int:
    """Algorithmic bytes of the window-score pass: K read once, the window
    queries read once, the fp32 score written once."""
    k = T * wl.h_kv * wl.d * 2
    q = B * wl.w * wl.h_q * wl.d * 2
    s = wl.h_kv * T * 4
    return k + q + s


def chain_bytes(wl, T: int, B: int, l_kv, l_tsp) -> dict:
    """Algorithmic bytes of the other steps: the head sum and stats read the
    score and write the token row and the stats; both top-k budgets read
    their rows and write the indices; the gathers read and write every kept
    K, V and hidden row once."""
    stats = wl.h_kv * T * 4 + T * 4 + B * 3 * 4
    topk = wl.h_kv * T * 4 + T * 4 + (wl.h_kv * sum(l_kv) + sum(l_tsp)) * 4
    gather = 2 * (2 * sum(l_kv) * wl.h_kv * wl.d * 2 + sum(l_tsp) * wl.hidden * 2)
    return {"stats": stats, "topk_both": topk, "gather_kvh": gather}


def copy_ceiling(dev, mib: int = 1024, reps: int = 5) -> float:
    """Read + write GB/s of a plain device-to-device copy of mib MiB (HIP
    events around each copy, best of reps)."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e-3)
    del src, dst
    return 2 * n / best / 1e9


def measured_traffic():
    """HBM bytes per score pass from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        src = hashlib.sha256(open(SCORE_SRC, "rb").read()).hexdigest()
        if rec.get("score_hip_sha256") != src:
            return None
        return rec.get("bytes_per_pass")
    except (OSError, ValueError):
        return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, x, scale, min_seconds=10.0, max_runs=15):
    """The oracle, as it is, on whole passes of the workload: repeated until
    about min_seconds of CPU work (at most max_runs), median reported; then
    one more pass limited to a single BLAS thread."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threadpool_limits = None
        threads = os.cpu_count() or 1
    cu = x["cu_seqlens"]
    k_kv, k_tsp = wl.kv_tokens(), wl.tsp_tokens()
    lens = np.diff(cu)
    l_kv = [oracle.budget_length(int(n), wl.w, int(k)) for n, k in zip(lens, k_kv)]
    l_tsp = [oracle.budget_length(int(n), wl.w, int(k)) for n, k in zip(lens, k_tsp)]
    hid = x["hidden"].reshape(x["hidden"].shape[0], 1, -1)

    def one_pass():
        t0 = time.perf_counter()
        q = oracle.bf16_to_f64(x["q"])
        k = oracle.bf16_to_f64(x["k"])
        s, _ = oracle.window_score(q, k, cu, wl.h_q, wl.h_kv, wl.w, scale)
        tok = oracle.head_sum(s)
        oracle.layer_stats(s, cu, wl.w, wl.group)
        ikv = oracle.select_rows(s, cu, wl.w, k_kv)
        its = oracle.select_rows(tok[None, :], cu, wl.w, k_tsp)
        oracle.gather(x["k"], cu, ikv, l_kv)
        oracle.gather(x["v"], cu, ikv, l_kv)
        oracle.gather(hid, cu, its, l_tsp)
        return time.perf_counter() - t0

    times = []
    while len(times) < max_runs and (len(times) < 3 or sum(times) < min_seconds):
        times.append(one_pass())
    t = statistics.median(times)
    T = int(cu[-1])
    out = {"value": T / t, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{len(times)} whole passes of {wl.name} (score, stats, both top-k, K/V/hidden "
                     f"gathers), {sum(times):.1f} s in all; median {t:.2f} s per pass",
           "seconds_per_pass": t, "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            t1 = one_pass()
        out["one_thread_seconds_per_pass"] = t1
        out["one_thread_value"] = T / t1
    return out


def score_sweep(dev, lengths, reps: int, warmup: int) -> int:
    """The score call alone at several sequence lengths: median over reps
    replays of a graph of CALLS_PER_GRAPH back-to-back calls, three input
    copies rotated.  Inputs are N(0, 1/4) bf16 drawn on the GPU (timing
    only; the parity tests cover correctness)."""
    import torch
    import token_selection_tsp_amd as kv
    h_q, h_kv, d, w, copies = 32, 8, 128, 32, 3
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    stream = torch.cuda.current_stream(dev)

    def timed(call):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(CALLS_PER_GRAPH):
                call(i % copies)
        for _ in range(max(warmup, 1)):
            g.replay()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in ev:
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return statistics.median(e0.elapsed_time(e1) * 1e3 / CALLS_PER_GRAPH for e0, e1 in ev)

    for n in lengths:
        cu = [0, n]
        qs = [(torch.randn(1, w, h_q, d, generator=gen, device=dev) * 0.5).to(torch.bfloat16)
              for _ in range(copies)]
        ks = [(torch.randn(n, h_kv, d, generator=gen, device=dev) * 0.5).to(torch.bfloat16)
              for _ in range(copies)]
        lses = [kv.window_score(qs[c], ks[c], cu, return_lse=True)[1] for c in range(copies)]
        torch.cuda.synchronize()
        nbytes = n * h_kv * d * 2 + w * h_q * d * 2 + h_kv * n * 4
        t2 = timed(lambda c: kv.window_score(qs[c], ks[c], cu))
        t1 = timed(lambda c: kv.window_score(qs[c], ks[c], cu, lse_in=lses[c]))
        print(json.dumps({"tokens": n, "h_q": h_q, "h_kv": h_kv, "d": d, "w": w, "algorithmic_bytes": nbytes,
                          "score_us": t2, "score_frac": nbytes / (t2 * 1e-6) / 1e9 / HBM_PEAK_GBS,
                          "given_lse_us": t1, "given_lse_frac": nbytes / (t1 * 1e-6) / 1e9 / HBM_PEAK_GBS}),
              flush=True)
        del qs, ks, lses
        torch.cuda.empty_cache()
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="n128k_gqa32x8_d128")
    ap.add_argument("--copies", type=int, default=3,
                    help="input copies rotated so K is never resident in the 256 MB last-level cache")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="time eager calls instead of replaying the pass as a HIP graph")
    ap.add_argument("--score-sweep", default="", metavar="N1,N2,...",
                    help="instead of the pass, time the score call alone at these sequence lengths")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the pass, run a plain device copy of MIB MiB a few times (the "
                         "known-size reference for the memory byte counters)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the path is measured on "
              f"one GPU's share and its sharding is a design note", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import token_selection_tsp_amd as kv
    from token_selection_tsp_amd import synth

    if not os.path.exists(kv.kvsel.LIB_PATH):
        from token_selection_tsp_amd import build as _b
        _b.build()
    kv.library()
    assert torch.cuda.is_available(), "no GPU"
    dev = torch.device("cuda:0")

    if a.calibrate_copy:
        n = a.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 3}), flush=True)
        return 0

    if a.score_sweep:
        return score_sweep(dev, [int(v) for v in a.score_sweep.split(",")], a.steps, a.warmup)

    wl = synth.WORKLOADS[a.workload]
    log(f"generating {wl.name}")
    x = synth.layer_inputs(wl, parts=("q", "k", "v", "hidden"))
    cu = x["cu_seqlens"]
    T = int(cu[-1])
    B = len(cu) - 1
    k_kv, k_tsp = wl.kv_tokens(), wl.tsp_tokens()
    scale = float(np.float32(1.0 / math.sqrt(wl.d)))

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    copies = []
    for c in range(a.copies):
        copies.append(tuple(to_dev(x[p]) for p in ("q", "k", "v", "hidden")))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    names = ["score", "stats", "topk_both", "gather_kvh"]

    def step(i, ev=None):
        # ev: len(names) + 1 events, recorded between the calls
        q, k, v, h = copies[i % len(copies)]
        mark = (lambda j: ev[j].record(stream)) if ev is not None else (lambda j: None)
        mark(0)
        score = kv.window_score(q, k, cu, scale=scale)
        mark(1)
        _, tok, _ = kv.accumulate_stats(score, cu, wl.w, wl.group)
        mark(2)
        ikv, its = kv.topk2(score, tok, cu, wl.w, k_kv, k_tsp)
        mark(3)
        kv.gather_multi(cu, wl.w, [(k, ikv, k_kv), (v, ikv, k_kv), (h, its, k_tsp)])
        mark(4)

    log(f"warmup {a.warmup}")
    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()

    # per-call breakdown: K eager passes with events between the calls
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(a.steps)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(a.steps):
        step(i, evs[i])
    e1.record(stream)
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / a.steps
    per = {n: [evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(a.steps)] for j, n in enumerate(names)}
    avg = {n: sum(v) / len(v) for n, v in per.items()}
    steps13_ms = avg["score"] + avg["stats"] + avg["topk_both"]

    # Single calls are timed as graphs of CALLS_PER_GRAPH back-to-back calls
    # on the rotating input copies, with HIP events around each replay on
    # the kernels' stream: the events then bracket the kernels and the gaps
    # between them only (an event pair around every eager call adds several
    # microseconds of its own, and a short call can wait on the Python host).
    def time_calls(call, reps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(CALLS_PER_GRAPH):
                call(i % len(copies))
        for _ in range(max(a.warmup, 1)):
            g.replay()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in ev:
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) / CALLS_PER_GRAPH for e0, e1 in ev]   # ms per call, per replay

    # the score call alone
    score_alone = time_calls(lambda c: kv.window_score(copies[c][0], copies[c][1], cu, scale=scale), a.steps)

    # the one-pass score (normalisers given, as the layer's own attention
    # would supply them)
    lse_of = [kv.window_score(c[0], c[1], cu, scale=scale, return_lse=True)[1] for c in copies]
    lse_in_us = statistics.mean(time_calls(
        lambda c: kv.window_score(copies[c][0], copies[c][1], cu, scale=scale, lse_in=lse_of[c]),
        max(a.steps // 2, 1))) * 1e3

    # the score call with every window row's entropy (StructKV's row-level variant)
    ent_us = statistics.mean(time_calls(
        lambda c: kv.window_score_entropy(copies[c][0], copies[c][1], cu, scale=scale),
        max(a.steps // 2, 1))) * 1e3

    # K and V written straight into paged caches (16-token blocks, a
    # shuffled block table) with the selection of copy 0: K back-to-back calls
    q0, k0, v0, h0 = copies[0]
    s0 = kv.window_score(q0, k0, cu, scale=scale)
    _, tok0, _ = kv.accumulate_stats(s0, cu, wl.w, wl.group)
    ikv0, _ = kv.topk2(s0, tok0, cu, wl.w, k_kv, k_tsp)
    bs = 16
    lkv = [min(n, int(kk) + wl.w) for n, kk in zip(np.diff(cu), k_kv)]
    need = [-(-L // bs) for L in lkv]
    nblocks = sum(need)
    perm = np.random.default_rng(0).permutation(nblocks)
    table = np.zeros((B, max(need)), dtype=np.int32)
    at = 0
    for b, nb in enumerate(need):
        table[b, :nb] = perm[at:at + nb]
        at += nb
    table_d = torch.from_numpy(table).to(dev)
    kc = torch.empty((nblocks, bs) + tuple(k0.shape[1:]), dtype=k0.dtype, device=dev)
    vc = torch.empty_like(kc)
    paged_jobs = [[(copies[c][1], ikv0, k_kv, kc, table_d), (copies[c][2], ikv0, k_kv, vc, table_d)]
                  for c in range(len(copies))]
    kv.gather_paged(cu, wl.w, paged_jobs[0])
    torch.cuda.synchronize()
    paged_us = statistics.mean(time_calls(lambda c: kv.gather_paged(cu, wl.w, paged_jobs[c]), a.steps)) * 1e3
    paged_bytes = 2 * 2 * sum(lkv) * int(np.prod(k0.shape[1:])) * k0.element_size()

    if a.eager:
        ms, launch = eager_ms, "eager"
    else:
        # the pass as a HIP graph per input copy (captured once, replayed):
        # the kernels run back to back without host launch overhead
        graphs = []
        for c in range(len(copies)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(c)
            graphs.append(g)
        for i in range(a.warmup):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        t_start.record(stream)
        for i in range(a.steps):
            graphs[i % len(graphs)].replay()
        t_end.record(stream)
        torch.cuda.synchronize()
        ms, launch = t_start.elapsed_time(t_end) / a.steps, "hip graph replay"

    sb = score_bytes(wl, T, B)
    ltsp = [min(n, int(kk) + wl.w) for n, kk in zip(np.diff(cu), k_tsp)]
    cb = chain_bytes(wl, T, B, lkv, ltsp)
    copy_gbs = copy_ceiling(dev)
    steps13_bytes = sb + cb["stats"] + cb["topk_both"]
    full_bytes = steps13_bytes + cb["gather_kvh"]
    score_ms = sum(score_alone) / len(score_alone)
    score_s = score_ms * 1e-3
    achieved = sb / score_s / 1e9
    traffic = measured_traffic()
    out = {
        "metric": METRIC,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "tokens": T, "h_q": wl.h_q, "h_kv": wl.h_kv,
                   "d": wl.d, "w": wl.w, "hidden": wl.hidden,
                   "kv_budget": wl.kv_budget.describe(), "tsp_budget": wl.tsp_budget.describe()},
        "roofline": {"bound": "hbm", "kernel": "window score pass (kvsel_window_score)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes": sb, "avg_us": score_ms * 1e3,
                     "frac_of_copy_ceiling": achieved / copy_gbs,
                     "p10_p50_p90_us": [round(float(v) * 1e3, 2) for v in
                                        np.percentile(score_alone, [10, 50, 90])],
                     "timing": f"HIP events around each of K replays of a graph of {CALLS_PER_GRAPH} "
                               "back-to-back score calls on the rotating input copies"},
        "launch": launch,
        "score_given_lse": {"avg_us": lse_in_us, "achieved_gbs": sb / (lse_in_us * 1e-6) / 1e9,
                            "frac": sb / (lse_in_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                            "note": "kvsel_window_score_lse: one pass over K, normalisers from the "
                                    "layer's own attention (not part of value)"},
        "score_row_entropy": {"avg_us": ent_us, "achieved_gbs": sb / (ent_us * 1e-6) / 1e9,
                              "frac": sb / (ent_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                              "note": "kvsel_window_score_entropy: the score call plus every window "
                                      "row's attention entropy (not part of value)"},
        "kv_paged_gather": {"avg_us": paged_us, "achieved_gbs": paged_bytes / (paged_us * 1e-6) / 1e9,
                            "bytes": paged_bytes,
                            "note": "kvsel_gather_paged: K and V of the KV budget into 16-token blocks "
                                    "through a shuffled block table (not part of value)"},
        "eager_ms_per_step": eager_ms,
        "steps_1_3_tokens_per_s": T / (steps13_ms * 1e-3),
        "chain_hbm": {
            "steps_1_3": {"algorithmic_bytes": steps13_bytes, "us": steps13_ms * 1e3,
                          "frac": steps13_bytes / (steps13_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
            "full": {"algorithmic_bytes": full_bytes, "us": ms * 1e3,
                     "frac": full_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
            "note": "algorithmic bytes of each chain over its time (steps 1-3 from the eager "
                    "per-call events, the full chain from `ms_per_step`) against 8 TB/s"},
        "copy_ceiling_gbs": copy_gbs,
        "breakdown_us": {n: round(v * 1e3, 2) for n, v in avg.items()},
    }
    if not a.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(wl, x, scale)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
