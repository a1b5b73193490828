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


def _counter_means(d):
    """Mean counter value per kernel name over the dispatches of one
    rocprofv3 --pmc run (its *_counter_collection.csv under d)."""
    import csv
    import glob
    paths = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if len(paths) != 1:
        raise SystemExit(f"expected one counter_collection.csv under {d}, found {len(paths)}")
    vals = {}
    with open(paths[0]) as f:
        for r in csv.DictReader(f):
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: statistics.mean(v) for k, v in vals.items()}


def write_traffic(root: str) -> int:
    """The score call's HBM bytes from FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for a plain copy of
    1 GiB; recorded with the SHA-256 of the kernel source it was taken on."""
    f = _counter_means(os.path.join(root, "pmc_FETCH_SIZE"))
    w = _counter_means(os.path.join(root, "pmc_WRITE_SIZE"))
    cf = _counter_means(os.path.join(root, "pmccopy_FETCH_SIZE"))
    cw = _counter_means(os.path.join(root, "pmccopy_WRITE_SIZE"))
    copy = [k for k in cf if "copyBuffer" in k]   # dst.copy_(src): a device-to-device memcpy
    if len(copy) != 1:
        raise SystemExit(f"expected one copy kernel in the calibration runs, found {copy}")
    kib = float(1 << 20)   # 1 GiB in KiB
    ff, wf = kib / cf[copy[0]], kib / cw[copy[0]]

    def one(name_part):
        ks = [k for k in f if name_part in k]
        if len(ks) != 1:
            raise SystemExit(f"expected one kernel matching {name_part}, found {ks}")
        k = ks[0]
        return k, {"fetch_kib_raw": round(f[k], 1), "write_kib_raw": round(w.get(k, 0.0), 1),
                   "bytes_scaled": int(round(f[k] * 1024 * ff + w.get(k, 0.0) * 1024 * wf))}

    # the plain score call at d=128 with 128 rows: two waves per key stream, two row blocks each
    ka, pa = one("k_score_pass_aILi128ELi2ELi2ELb0E")
    kb, pb = one("k_score_pass_bILi128ELi2ELi2ELb0E")
    others = {k: {"fetch_bytes": int(round(f[k] * 1024 * ff)), "write_bytes": int(round(w.get(k, 0.0) * 1024 * wf))}
              for k in f if k not in (ka, kb) and k != copy[0]}
    from token_selection_tsp_amd import synth
    wl = synth.WORKLOADS["n128k_gqa32x8_d128"]
    rec = {
        "kernel": "kvsel_window_score (k_score_pass_a + k_score_pass_b)",
        "workload": wl.name,
        "score_hip_sha256": hashlib.sha256(open(SCORE_SRC, "rb").read()).hexdigest(),
        "bytes_per_pass": pa["bytes_scaled"] + pb["bytes_scaled"],
        "algorithmic_bytes": score_bytes(wl, 131072, 1),
        "per_kernel": {"pass_a": pa, "pass_b": pb},
        "other_kernels_per_launch": others,
        "calibration": {"copy_bytes": 1 << 30, "copy_kernel": copy[0], "fetch_kib_raw": cf[copy[0]],
                        "write_kib_raw": cw[copy[0]], "fetch_factor": ff, "write_factor": wf},
        "commands": ["cd /tmp && export TMPDIR=/tmp   # then, with REPO the repository root:",
                     "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $REPO/gpurun_out/pmc_FETCH_SIZE -o b -- "
                     "python3 $REPO/bench.py --steps 3 --warmup 1 --no-cpu-baseline",
                     "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $REPO/gpurun_out/pmc_WRITE_SIZE -o b -- "
                     "python3 $REPO/bench.py --steps 3 --warmup 1 --no-cpu-baseline",
                     "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $REPO/gpurun_out/pmccopy_FETCH_SIZE -o c -- "
                     "python3 $REPO/bench.py --calibrate-copy 1024",
                     "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $REPO/gpurun_out/pmccopy_WRITE_SIZE -o c -- "
                     "python3 $REPO/bench.py --calibrate-copy 1024",
                     "python3 $REPO/bench.py --traffic-from $REPO/gpurun_out"]}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps({"bytes_per_pass": rec["bytes_per_pass"], "fetch_factor": ff, "write_factor": wf}))
    return 0


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


def cpu_baseline_structkv(wl, xs, scale):
    """The oracle on one whole pass of the multi-layer chain: every layer's
    window score, running sum and statistics, the pivot, both budgets'
    selections and the pivot layer's gathers (its V and hidden rows are drawn
    outside the timed parts)."""
    import numpy as np
    import oracle
    from token_selection_tsp_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    cu = xs[0]["cu_seqlens"]
    k_kv, k_tsp = wl.kv_tokens(), wl.tsp_tokens()
    lens = np.diff(cu)
    t0 = time.perf_counter()
    acc, ent = None, []
    accs = []
    for x in xs:
        s, _ = oracle.window_score(oracle.bf16_to_f64(x["q"]), oracle.bf16_to_f64(x["k"]), cu, wl.h_q, wl.h_kv,
                                   wl.w, scale)
        acc = oracle.accumulate(s, acc)
        accs.append(acc)
        oracle.head_sum(acc)
        ent.append(oracle.layer_stats(s, cu, wl.w, wl.group)[0, 0])
    p = oracle.pivot_layer(ent)
    t_layers = time.perf_counter() - t0
    xp = synth.layer_inputs(wl, layer=p, parts=("k", "v", "hidden"))
    t1 = time.perf_counter()
    ikv = oracle.select_rows(accs[p], cu, wl.w, k_kv)
    its = oracle.select_rows(oracle.head_sum(accs[p])[None, :], cu, wl.w, k_tsp)
    l_kv = [oracle.budget_length(int(n), wl.w, int(k)) for n, k in zip(lens, k_kv)]
    l_tsp = [oracle.budget_length(int(n), wl.w, int(k)) for n, k in zip(lens, k_tsp)]
    oracle.gather(xp["k"], cu, ikv, l_kv)
    oracle.gather(xp["v"], cu, ikv, l_kv)
    oracle.gather(xp["hidden"].reshape(xp["hidden"].shape[0], 1, -1), cu, its, l_tsp)
    t = t_layers + time.perf_counter() - t1
    T = int(cu[-1])
    return {"value": len(xs) * T / t, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"1 whole pass of {wl.name} ({len(xs)} layers scored, pivot, both selections, gathers), "
                      f"{t:.1f} s", "seconds_per_pass": t, "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


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


def ceilings(dev, reps: int, warmup: int) -> int:
    """Reference rates of the memory system, from the library's own probe
    (kvsel_probe_read) and score call, one JSON line each:

    * plain_read: 1 GiB read as 2 KB rows (larger than the 256 MB
      last-level cache, so every replay streams from HBM);
    * k_layout_read: the N=128K key cache [T, 8, 128] bf16 (268 MB) read one
      KV head at a time, the score kernels' access pattern, with 32 and 128
      work-groups per head; three copies rotated;
    * llc_reread: a 128 MB buffer read by back-to-back calls (each call
      re-reads what the last one read) against four such buffers rotated
      (512 MB: nothing left in the cache);
    * score_llc: the score call on a 57344-key sequence (117 MB of K) with
      given normalisers (one visit of K) and in two passes, on one input
      copy back to back against four copies rotated.

    Each figure is the median over reps replays of a graph of
    CALLS_PER_GRAPH back-to-back calls, HIP events around each replay."""
    import torch
    import token_selection_tsp_amd as kv
    stream = torch.cuda.current_stream(dev)

    def timed(call):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(CALLS_PER_GRAPH):
                call(i)
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

    def emit(rec):
        print(json.dumps(rec), flush=True)

    out = torch.empty(1 << 16, dtype=torch.int32, device=dev)
    # plain read, 1 GiB
    nb = 1 << 30
    buf = torch.empty(nb // 4, dtype=torch.int32, device=dev).fill_(1)
    for wgs in (1024, 2048, 4096):
        us = timed(lambda i: kv.probe_read(buf, nb // 2048, 1, 2048, 2048, wgs, out))
        emit({"probe": "plain_read", "bytes": nb, "work_groups": wgs, "us": us, "gbs": nb / us / 1e3})
    del buf
    # the key cache's layout at N=128K, one KV head per work-group
    T, h_kv, d, copies = 131072, 8, 128, 3
    ks = [torch.empty(T * h_kv * d // 2, dtype=torch.int32, device=dev).fill_(c) for c in range(copies)]
    kb = T * h_kv * d * 2
    for wph in (32, 128):
        us = timed(lambda i: kv.probe_read(ks[i % copies], T, h_kv, 2 * d, h_kv * 2 * d, wph, out))
        emit({"probe": "k_layout_read", "tokens": T, "h_kv": h_kv, "d": d, "bytes": kb,
              "work_groups_per_head": wph, "us": us, "gbs": kb / us / 1e3})
    del ks
    # last-level cache: 128 MB re-read back to back vs four buffers rotated
    nb = 128 << 20
    bufs = [torch.empty(nb // 4, dtype=torch.int32, device=dev).fill_(c) for c in range(4)]
    for mode, pick in (("same", lambda i: 0), ("rotated", lambda i: i % 4)):
        us = timed(lambda i: kv.probe_read(bufs[pick(i)], nb // 2048, 1, 2048, 2048, 2048, out))
        emit({"probe": "llc_reread", "bytes": nb, "mode": mode, "us": us, "gbs": nb / us / 1e3})
    del bufs
    # the score call on 117 MB of K: same copy back to back vs four rotated
    n, h_q, w = 57344, 32, 32
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    qs = [(torch.randn(1, w, h_q, d, generator=gen, device=dev) * 0.5).to(torch.bfloat16) for _ in range(4)]
    ks = [(torch.randn(n, h_kv, d, generator=gen, device=dev) * 0.5).to(torch.bfloat16) for _ in range(4)]
    cu = [0, n]
    lses = [kv.window_score(qs[c], ks[c], cu, return_lse=True)[1] for c in range(4)]
    sc = torch.empty((h_kv, n), dtype=torch.float32, device=dev)
    nbytes = n * h_kv * d * 2 + w * h_q * d * 2 + h_kv * n * 4
    for mode, pick in (("same", lambda i: 0), ("rotated", lambda i: i % 4)):
        u1 = timed(lambda i: kv.window_score(qs[pick(i)], ks[pick(i)], cu, lse_in=lses[pick(i)], out=sc))
        u2 = timed(lambda i: kv.window_score(qs[pick(i)], ks[pick(i)], cu, out=sc))
        emit({"probe": "score_llc", "tokens": n, "k_bytes": n * h_kv * d * 2, "mode": mode,
              "given_lse_us": u1, "given_lse_gbs": nbytes / u1 / 1e3,
              "two_pass_us": u2, "two_pass_gbs": nbytes / u2 / 1e3})
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
    ap.add_argument("--all-configs", action="store_true",
                    help="one JSON line per workload (the five configurations) instead of the 128K line")
    ap.add_argument("--configs", default="", metavar="NAME,NAME",
                    help="with --all-configs: only these workloads")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="about how long the oracle baseline runs per workload")
    ap.add_argument("--eager", action="store_true",
                    help="time eager calls instead of replaying the pass as a HIP graph")
    ap.add_argument("--score-sweep", default="", metavar="N1,N2,...",
                    help="instead of the pass, time the score call alone at these sequence lengths")
    ap.add_argument("--ceilings", action="store_true",
                    help="instead of the pass, measure the reference read rates (plain, key-cache layout, "
                         "last-level-cache re-read) with the library's probe and score call")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the pass, run a plain device copy of MIB MiB a few times (the "
                         "known-size reference for the memory byte counters)")
    ap.add_argument("--traffic-from", default="", metavar="DIR",
                    help="no GPU: write the score pass's HBM traffic record (profiles/score_pass_traffic.json) "
                         "from the rocprofv3 FETCH_SIZE / WRITE_SIZE outputs under DIR (pmc_FETCH_SIZE, "
                         "pmc_WRITE_SIZE of this bench; pmccopy_FETCH_SIZE, pmccopy_WRITE_SIZE of "
                         "--calibrate-copy 1024)")
    a = ap.parse_args()
    if a.traffic_from:
        return write_traffic(a.traffic_from)
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

    if a.ceilings:
        return ceilings(dev, a.steps, a.warmup)

    if a.score_sweep:
        return score_sweep(dev, [int(v) for v in a.score_sweep.split(",")], a.steps, a.warmup)

    if a.all_configs:
        only = [v for v in a.configs.split(",") if v]
        for name in synth.WORKLOAD_ORDER:
            if only and name not in only:
                continue
            wl = synth.WORKLOADS[name]
            if wl.layers > 1:
                out = measure_structkv(wl, a, dev)
            else:
                out = measure_layer(wl, a, dev, extras=False)
            print(json.dumps(out), flush=True)
            torch.cuda.empty_cache()
        return 0
    print(json.dumps(measure_layer(synth.WORKLOADS[a.workload], a, dev, extras=True)), flush=True)
    return 0


def _time_graphs(graphs, reps, warmup, stream):
    """ms per replay: warm-up replays, then HIP events around each of reps
    replays (rotating over the graphs)."""
    import torch
    for i in range(max(warmup, 1)):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i, (e0, e1) in enumerate(ev):
        e0.record(stream)
        graphs[i % len(graphs)].replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in ev]


def _capture(fn, n):
    import torch
    gs = []
    for c in range(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn(c)
        gs.append(g)
    return gs


def _line(wl, T, B, ms, steps, warmup, tokens, extra_config=None):
    cfg = {"workload": wl.name, "batch": B, "tokens": T, "h_q": wl.h_q, "h_kv": wl.h_kv, "d": wl.d, "w": wl.w,
           "hidden": wl.hidden, "kv_budget": wl.kv_budget.describe(), "tsp_budget": wl.tsp_budget.describe()}
    if extra_config:
        cfg.update(extra_config)
    return {"metric": METRIC, "value": tokens / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
            "warmup": warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": cfg}


def measure_layer(wl, a, dev, extras: bool) -> dict:
    """One selection pass on a single-layer workload: the score call with
    the head sum and statistics, both budgets' top-k, the K/V/hidden
    gathers.  With ``extras`` also the variant calls, the copy ceiling and
    the chain fractions (the default 128K line)."""
    import numpy as np
    import torch

    import token_selection_tsp_amd as kv
    from token_selection_tsp_amd import synth

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

    names = ["score_stats", "topk_both", "gather_kvh"]

    def step(i, ev=None):
        # ev: len(names) + 1 events, recorded between the calls.  The score
        # call also does the head sum and the statistics (in its second pass).
        q, k, v, h = copies[i % len(copies)]
        mark = (lambda j: ev[j].record(stream)) if ev is not None else (lambda j: None)
        mark(0)
        score, _, tok, _ = kv.window_score_stats(q, k, cu, scale=scale)
        mark(1)
        ikv, its = kv.topk2(score, tok, cu, wl.w, k_kv, k_tsp)
        mark(2)
        kv.gather_multi(cu, wl.w, [(k, ikv, k_kv), (v, ikv, k_kv), (h, its, k_tsp)])
        mark(3)

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
    steps13_ms = avg["score_stats"] + avg["topk_both"]

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
        return [v / CALLS_PER_GRAPH for v in _time_graphs([g], reps, a.warmup, stream)]

    # the score call alone (the roofline's kernel pair)
    score_alone = time_calls(lambda c: kv.window_score(copies[c][0], copies[c][1], cu, scale=scale), a.steps)

    if a.eager:
        ms, launch = eager_ms, "eager"
    else:
        # the pass as a HIP graph per input copy (captured once, replayed):
        # the kernels run back to back without host launch overhead
        graphs = _capture(step, len(copies))
        ms, launch = sum(_time_graphs(graphs, a.steps, a.warmup, stream)) / a.steps, "hip graph replay"

    sb = score_bytes(wl, T, B)
    lkv = [min(n, int(kk) + wl.w) for n, kk in zip(np.diff(cu), k_kv)]
    ltsp = [min(n, int(kk) + wl.w) for n, kk in zip(np.diff(cu), k_tsp)]
    cb = chain_bytes(wl, T, B, lkv, ltsp)
    steps13_bytes = sb + cb["stats"] + cb["topk_both"]
    full_bytes = steps13_bytes + cb["gather_kvh"]
    score_ms = sum(score_alone) / len(score_alone)
    achieved = sb / (score_ms * 1e-3) / 1e9
    out = _line(wl, T, B, ms, a.steps, a.warmup, T)
    out["roofline"] = {"bound": "hbm", "kernel": "window score pass (kvsel_window_score)",
                       "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": achieved / HBM_PEAK_GBS,
                       "traffic": measured_traffic() if extras else None,
                       "algorithmic_bytes": sb, "avg_us": score_ms * 1e3,
                       "p10_p50_p90_us": [round(float(v) * 1e3, 2) for v in np.percentile(score_alone, [10, 50, 90])],
                       "timing": f"HIP events around each of K replays of a graph of {CALLS_PER_GRAPH} "
                                 "back-to-back score calls on the rotating input copies"}
    out["launch"] = launch
    out["eager_ms_per_step"] = eager_ms
    out["steps_1_3_tokens_per_s"] = T / (steps13_ms * 1e-3)
    out["chain_hbm"] = {
        "steps_1_3": {"algorithmic_bytes": steps13_bytes, "us": steps13_ms * 1e3,
                      "frac": steps13_bytes / (steps13_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "full": {"algorithmic_bytes": full_bytes, "us": ms * 1e3,
                 "frac": full_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "note": "algorithmic bytes of each chain over its time (steps 1-3 from the eager per-call events, "
                "the full chain from `ms_per_step`) against 8 TB/s; steps 1-3 count one read of the score "
                "rows for the statistics although the fused call does not re-read them"}
    out["breakdown_us"] = {n: round(v * 1e3, 2) for n, v in avg.items()}

    if extras:
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
        # the score call with the head sum and statistics (the pass's first call)
        stats_us = statistics.mean(time_calls(
            lambda c: kv.window_score_stats(copies[c][0], copies[c][1], cu, scale=scale),
            max(a.steps // 2, 1))) * 1e3
        # K and V written straight into paged caches (16-token blocks, a
        # shuffled block table) with the selection of copy 0
        q0, k0, v0, h0 = copies[0]
        s0, _, tok0, _ = kv.window_score_stats(q0, k0, cu, scale=scale)
        ikv0, _ = kv.topk2(s0, tok0, cu, wl.w, k_kv, k_tsp)
        bs = 16
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
        copy_gbs = copy_ceiling(dev)
        out["roofline"]["frac_of_copy_ceiling"] = achieved / copy_gbs
        out["score_given_lse"] = {"avg_us": lse_in_us, "achieved_gbs": sb / (lse_in_us * 1e-6) / 1e9,
                                  "frac": sb / (lse_in_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                  "note": "kvsel_window_score_lse: one pass over K, normalisers from the "
                                          "layer's own attention (not part of value)"}
        out["score_row_entropy"] = {"avg_us": ent_us, "achieved_gbs": sb / (ent_us * 1e-6) / 1e9,
                                    "frac": sb / (ent_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                    "note": "kvsel_window_score_entropy: the score call plus every window "
                                            "row's attention entropy (not part of value)"}
        out["score_with_stats"] = {"avg_us": stats_us,
                                   "note": "kvsel_window_score_stats: the score call with the head sum and "
                                           "the statistics in its second pass (the pass's first call)"}
        out["kv_paged_gather"] = {"avg_us": paged_us, "achieved_gbs": paged_bytes / (paged_us * 1e-6) / 1e9,
                                  "bytes": paged_bytes,
                                  "note": "kvsel_gather_paged: K and V of the KV budget into 16-token blocks "
                                          "through a shuffled block table (not part of value)"}
        out["copy_ceiling_gbs"] = copy_gbs
    if not a.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(wl, x, scale, min_seconds=a.cpu_seconds)
    del copies
    return out


def measure_structkv(wl, a, dev) -> dict:
    """The 16-layer StructKV chain: per layer the score call with the
    running accumulation and the statistics; one device-to-host read of the
    per-layer entropies; the pivot on the host; both budgets' top-k on the
    pivot layer's accumulated score; the pivot layer's K/V/hidden gathers.
    The layers run as one HIP graph per input copy; after the host pivot,
    the selection replays a graph captured for that pivot layer (captured
    the first time the layer comes up, as a serving loop would cache one per
    pivot); the timed step spans all of it."""
    import numpy as np
    import torch

    import token_selection_tsp_amd as kv
    from token_selection_tsp_amd import synth

    L = wl.layers
    log(f"generating {wl.name} ({L} layers)")
    xs = [synth.layer_inputs(wl, layer=l, parts=("q", "k")) for l in range(L)]
    cu = xs[0]["cu_seqlens"]
    T = int(cu[-1])
    B = len(cu) - 1
    k_kv, k_tsp = wl.kv_tokens(), wl.tsp_tokens()
    scale = float(np.float32(1.0 / math.sqrt(wl.d)))

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    ncp = max(1, min(a.copies, 2))   # 16 layers' keys per copy: 2.1 GB; two copies exceed the cache
    layers = [[(to_dev(x["q"]), to_dev(x["k"])) for x in xs] for _ in range(ncp)]
    acc = [torch.empty((wl.h_kv, T), dtype=torch.float32, device=dev) for _ in range(L)]
    tok = [torch.empty(T, dtype=torch.float32, device=dev) for _ in range(L)]
    stats = [torch.empty((B, 3), dtype=torch.float32, device=dev) for _ in range(L)]   # one aligned slot per layer
    score = torch.empty((wl.h_kv, T), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    # every layer's outputs go straight into preallocated slots
    def run_layers(c):
        for l in range(L):
            q, k = layers[c][l]
            kv.window_score_stats(q, k, cu, scale=scale, out=score, c_in=acc[l - 1] if l else None,
                                  c_out=acc[l], tok_out=tok[l], stats_out=stats[l])

    run_layers(0)
    torch.cuda.synchronize()
    pivot = kv.pivot_layer(torch.stack([st[0, 0] for st in stats]).cpu().numpy())
    log(f"{wl.name}: pivot layer {pivot}; generating its V and hidden rows")
    xp = synth.layer_inputs(wl, layer=pivot, parts=("k", "v", "hidden"))
    kvh = [(to_dev(xp["k"]), to_dev(xp["v"]), to_dev(xp["hidden"])) for _ in range(ncp)]
    del xp

    def select(c, p):
        k, v, h = kvh[c]
        ikv, its = kv.topk2(acc[p], tok[p], cu, wl.w, k_kv, k_tsp)
        kv.gather_multi(cu, wl.w, [(k, ikv, k_kv), (v, ikv, k_kv), (h, its, k_tsp)])

    graphs = _capture(run_layers, ncp)
    sel_graphs = {}

    def select_graph(c, p):
        if (c, p) not in sel_graphs:
            select(c, p)                    # eager once: buffers and launch plans exist before capture
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                select(c, p)
            sel_graphs[(c, p)] = g
        return sel_graphs[(c, p)]

    for c in range(ncp):
        select_graph(c, pivot)

    def step(i):
        graphs[i % ncp].replay()
        p = kv.pivot_layer(torch.stack([st[0, 0] for st in stats]).cpu().numpy())   # one device-to-host read
        assert p == pivot, (p, pivot)
        select_graph(i % ncp, p).replay()

    for i in range(max(a.warmup, 1)):
        step(i)
    torch.cuda.synchronize()
    times = []
    for i in range(a.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = sum(times) / len(times)
    layers_ms = sum(_time_graphs(graphs, a.steps, a.warmup, stream)) / a.steps
    # the score call of one layer (graph of back-to-back calls, layers rotated)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(CALLS_PER_GRAPH):
            q, k = layers[0][i % L]
            kv.window_score(q, k, cu, scale=scale, out=score)
    score_ms = sum(_time_graphs([g], a.steps, a.warmup, stream)) / a.steps / CALLS_PER_GRAPH
    sb = score_bytes(wl, T, B)
    achieved = sb / (score_ms * 1e-3) / 1e9
    out = _line(wl, T, B, ms, a.steps, a.warmup, L * T, {"layers": L, "pivot_layer": int(pivot)})
    out["roofline"] = {"bound": "hbm", "kernel": "window score pass of one layer (kvsel_window_score)",
                       "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": achieved / HBM_PEAK_GBS, "traffic": None, "algorithmic_bytes": sb,
                       "avg_us": score_ms * 1e3,
                       "timing": f"HIP events around K replays of a graph of {CALLS_PER_GRAPH} back-to-back "
                                 "score calls over the layers"}
    out["launch"] = "hip graph replay of the layers; pivot on the host; the pivot layer's selection from its graph"
    out["breakdown_us"] = {"layers_score_stats": round(layers_ms * 1e3, 2),
                           "pivot_select_gather": round((ms - layers_ms) * 1e3, 2)}
    out["note"] = ("value counts every scored token of every layer (layers x N); the step includes the "
                   "device-to-host read of the per-layer statistics and the host pivot")
    if not a.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline_structkv(wl, xs, scale)
    del layers, kvh, acc, tok, graphs, sel_graphs
    return out


if __name__ == "__main__":
    sys.exit(main())
