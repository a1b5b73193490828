"""kvsel_window_score_stats against kvsel_window_score followed by
kvsel_accumulate_stats: score, normalisers, accumulated score and head sum
bit for bit; the statistics within the fp32 rounding bound of the oracle fed
the same score (and end to end against the oracle on small cases).  Shapes
cover several row groups (rows > 128), several launch groups (> 64
sequences), ragged tails, d = 64 and 128, with and without a running sum,
c_out aliasing c_in, absent outputs, and HIP-graph replays."""
import numpy as np
import pytest

import oracle
import token_selection_tsp_amd as kv
from token_selection_tsp_amd import synth
from gpu_util import check_stats, dev_bf16, dev_f32, host, log, scale_of, score_oracle

pytestmark = pytest.mark.gpu

CASES = [
    # name, lengths, h_q, h_kv, d, w
    ("c2", (32768,), 32, 8, 128, 32),
    ("ragged", (5000, 40, 3100, 777), 32, 8, 128, 32),
    ("rowgroups", (3000, 900), 32, 1, 128, 32),            # 1024 rows: eight row groups
    ("d64", (4000, 1234), 16, 4, 64, 16),
    ("tiny", (9, 40, 33), 8, 2, 64, 8),
]


def _ids(c):
    return c[0]


def _inputs(name, lens, h_q, h_kv, d, w, seed):
    wl = synth.small(name, seed, lens, h_q, h_kv, d, w, hubs=max(0, min(5, min(lens) - w)), alpha=2.0)
    return wl, synth.layer_inputs(wl, parts=("q", "k"))


@pytest.mark.parametrize("case", CASES, ids=_ids)
@pytest.mark.parametrize("with_cin", [False, True])
def test_score_stats_equals_two_calls(case, with_cin):
    name, lens, h_q, h_kv, d, w = case
    wl, x = _inputs(name, lens, h_q, h_kv, d, w, 600 + len(name))
    cu = x["cu_seqlens"]
    T = int(cu[-1])
    scale = scale_of(d)
    q, k = dev_bf16(x["q"]), dev_bf16(x["k"])
    c_in = dev_f32(synth.random_f32_rows(7, h_kv, T)) if with_cin else None
    log(f"score_stats {name} c_in={with_cin}")
    score, lse, c_out, tok, stats = kv.window_score_stats(q, k, cu, scale=scale, return_lse=True, c_in=c_in)
    ref_s, ref_l = kv.window_score(q, k, cu, scale=scale, return_lse=True)
    ref_c, ref_t, ref_st = kv.accumulate_stats(ref_s, cu, w, wl.group, c_in=c_in)
    assert np.array_equal(host(score), host(ref_s)), "score"
    assert np.array_equal(host(lse), host(ref_l)), "lse"
    assert np.array_equal(host(tok), host(ref_t)), "tok"
    if with_cin:
        assert np.array_equal(host(c_out), host(ref_c)), "c_out"
    else:
        assert c_out is None
    s64 = host(score).astype(np.float64)
    ora = score_oracle(x, wl, scale)[0] if T <= 40000 else None
    check_stats(stats, s64, cu, w, wl.group, ora_score=ora, what=f"{name} fused stats")
    check_stats(ref_st, s64, cu, w, wl.group, what=f"{name} two-call stats")


def test_score_stats_many_sequences_and_options():
    """70 sequences (two launch groups), c_out aliasing c_in, and each
    output left out in turn."""
    import torch
    rng = np.random.default_rng(70)
    lens = [int(v) for v in rng.integers(8, 500, size=70)]
    wl, x = _inputs("many", tuple(lens), 8, 2, 64, 8, 77)
    cu = x["cu_seqlens"]
    T = int(cu[-1])
    scale = scale_of(64)
    q, k = dev_bf16(x["q"]), dev_bf16(x["k"])
    base = synth.random_f32_rows(9, 2, T)
    ref_s = kv.window_score(q, k, cu, scale=scale)
    ref_c, ref_t, ref_st = kv.accumulate_stats(ref_s, cu, 8, wl.group, c_in=dev_f32(base))
    log("score_stats: 70 sequences, c_out aliasing c_in")
    acc = dev_f32(base)
    score, c_out, tok, stats = kv.window_score_stats(q, k, cu, scale=scale, c_in=acc, c_out=acc)
    assert c_out.data_ptr() == acc.data_ptr()
    assert np.array_equal(host(acc), host(ref_c))
    assert np.array_equal(host(tok), host(ref_t))
    s64 = host(score).astype(np.float64)
    check_stats(stats, s64, cu, 8, wl.group, ora_score=score_oracle(x, wl, scale)[0], what="70 sequences")
    log("score_stats: outputs left out")
    _, c2, t2, st2 = kv.window_score_stats(q, k, cu, scale=scale, want_tok=False)
    assert c2 is None and t2 is None
    assert np.allclose(host(st2), host(stats), rtol=0, atol=0)
    _, _, t3, st3 = kv.window_score_stats(q, k, cu, scale=scale, want_stats=False)
    assert st3 is None and np.array_equal(host(t3), host(kv.accumulate_stats(ref_s, cu, 8, wl.group)[1]))
    c4 = torch.empty_like(ref_s)
    s4, c4o, t4, st4 = kv.window_score_stats(q, k, cu, scale=scale, c_out=c4, want_tok=False, want_stats=False)
    assert c4o is c4 and np.array_equal(host(c4), host(ref_s)) and np.array_equal(host(s4), host(ref_s))


def test_score_stats_graph_replays():
    """Captured once and replayed with other work between the replays: the
    epilogue's counters are cleared inside every call, so every replay gives
    the eager results."""
    import torch
    wl, x = _inputs("graph", (20000, 9000), 32, 8, 128, 32, 88)
    cu = x["cu_seqlens"]
    scale = scale_of(128)
    q, k = dev_bf16(x["q"]), dev_bf16(x["k"])
    c_in = dev_f32(synth.random_f32_rows(3, 8, int(cu[-1])))
    eager = kv.window_score_stats(q, k, cu, scale=scale, c_in=c_in)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = kv.window_score_stats(q, k, cu, scale=scale, c_in=c_in)
    other = (q.flip(0).contiguous(), k.flip(0).contiguous())
    for rep in range(3):
        log(f"score_stats graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(eager, cap)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs"
        kv.window_score_stats(*other, cu, scale=scale, c_in=c_in)
        torch.cuda.synchronize()
