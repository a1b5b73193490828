"""Whole selection passes at once, on three streams of the same GPU.

The library keeps no state between calls (every buffer, counters included,
comes from the caller), so passes on different streams with their own
inputs and workspaces must not disturb each other: each stream's outputs
equal, bit for bit, those of the same pass run alone."""
import numpy as np
import pytest

import token_selection_tsp_amd as kv
from token_selection_tsp_amd import synth
from gpu_util import dev_bf16, host, log, scale_of

pytestmark = pytest.mark.gpu


def _inputs(seed, lens):
    wl = synth.small("streams", seed, lens, 32, 8, 128, 32, hidden=512, hubs=20, alpha=2.0)
    x = synth.layer_inputs(wl, parts=("q", "k", "v", "hidden"))
    dev = {p: dev_bf16(x[p]) for p in ("q", "k", "v")}
    dev["hidden"] = dev_bf16(x["hidden"].reshape(x["hidden"].shape[0], -1))
    return wl, x["cu_seqlens"], dev


def _pass(wl, cu, d):
    """Score with row entropies, head sum and stats, both budgets, the three
    gathers: every output, in call order."""
    scale = scale_of(wl.d)
    score, ent, mean = kv.window_score_entropy(d["q"], d["k"], cu, scale=scale)
    _, tok, stats = kv.accumulate_stats(score, cu, wl.w, wl.group)
    k_kv, k_tsp = wl.kv_tokens(), wl.tsp_tokens()
    ikv, its = kv.topk2(score, tok, cu, wl.w, k_kv, k_tsp)
    kc, vc, hc = kv.gather_multi(cu, wl.w, [(d["k"], ikv, k_kv), (d["v"], ikv, k_kv),
                                            (d["hidden"], its, k_tsp)])
    return [score, ent, mean, tok, stats, ikv, its, kc, vc, hc]


def test_streams_match_one_at_a_time():
    import torch
    a = _inputs(71, (40000, 9000))
    b = _inputs(72, (23000, 31000, 5000))
    c = _inputs(73, (3000, 700, 12000))     # short rows: the one-launch top-k
    log("streams: one at a time")
    want_a = [host(t) for t in _pass(*a)]
    want_b = [host(t) for t in _pass(*b)]
    want_c = [host(t) for t in _pass(*c)]
    torch.cuda.synchronize()
    s1, s2, s3 = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    for rep in range(3):
        log(f"streams: concurrent, repeat {rep}")
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            got_a = _pass(*a)
        with torch.cuda.stream(s2):
            got_b = _pass(*b)
        with torch.cuda.stream(s3):
            got_c = _pass(*c)
        s1.synchronize()
        s2.synchronize()
        s3.synchronize()
        for name, got, want in (("a", got_a, want_a), ("b", got_b, want_b), ("c", got_c, want_c)):
            for i, (g, w) in enumerate(zip(got, want)):
                assert np.array_equal(host(g), w), f"stream {name}, output {i}, repeat {rep}"
