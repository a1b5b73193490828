"""Seeded random shapes through the whole pass, GPU against the oracle.
Small: lengths 1..300 per sequence (at least the window), up to 5
sequences, d in {64, 128}, GQA groups 1..8, windows 1..33.  Medium: up to
4 sequences of 1000..20000 keys (several work units, ragged tails, every
path of the planner and both top-k paths), windows 1..64 (up to 512 rows
per KV head, several row groups), 1..8 KV heads; these also go through the
call with the statistics in its second pass, the one-pass call fed the
oracle's normalisers and the call with row entropies.  Scores within the
score tolerance; the GPU's own scores selected bit for bit like the oracle's
selection of them; gathers bit-exact."""
import numpy as np
import pytest

import oracle
import token_selection_tsp_amd as kv
from token_selection_tsp_amd import synth
from gpu_util import assert_close, check_rows, check_stats, dev_bf16, dev_f32, host, log, scale_of, score_oracle

pytestmark = pytest.mark.gpu


def _case(seed):
    rng = np.random.default_rng(np.random.SeedSequence([seed, 4242]))
    w = int(rng.integers(1, 34))
    B = int(rng.integers(1, 6))
    lens = [int(rng.integers(w, max(w, 300) + 1)) for _ in range(B)]
    d = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8]))
    h_kv = int(rng.choice([1, 2, 4]))
    k_kv = [int(rng.integers(0, n + 3)) for n in lens]
    k_ts = [int(rng.integers(0, n + 3)) for n in lens]
    return lens, G * h_kv, h_kv, d, w, k_kv, k_ts


def _case_medium(seed):
    rng = np.random.default_rng(np.random.SeedSequence([seed, 7777]))
    w = int(rng.integers(1, 65))
    B = int(rng.integers(1, 5))
    lens = [int(rng.integers(max(w, 1000), 20001)) for _ in range(B)]
    d = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8]))
    h_kv = int(rng.choice([1, 2, 4, 8]))
    k_kv = [int(rng.integers(0, n - w + 3)) for n in lens]
    k_ts = [int(rng.integers(0, n - w + 3)) for n in lens]
    return lens, G * h_kv, h_kv, d, w, k_kv, k_ts


@pytest.mark.parametrize("seed", range(16))
def test_random_small_pass(seed):
    lens, h_q, h_kv, d, w, k_kv, k_ts = _case(seed)
    log(f"random pass seed={seed} lens={lens} h={h_q}/{h_kv} d={d} w={w}")
    wl = synth.small("rand", 500 + seed, lens, h_q, h_kv, d, w, hidden=40,
                     hubs=max(0, min(3, min(lens) - w)))
    _whole_pass(wl, lens, h_q, h_kv, d, w, k_kv, k_ts)


@pytest.mark.parametrize("seed", range(16))
def test_random_medium_pass(seed):
    lens, h_q, h_kv, d, w, k_kv, k_ts = _case_medium(seed)
    log(f"random medium pass seed={seed} lens={lens} h={h_q}/{h_kv} d={d} w={w}")
    wl = synth.small("randm", 900 + seed, lens, h_q, h_kv, d, w, hidden=40, hubs=3)
    _whole_pass(wl, lens, h_q, h_kv, d, w, k_kv, k_ts, variants=True)


def _whole_pass(wl, lens, h_q, h_kv, d, w, k_kv, k_ts, variants=False):
    x = synth.layer_inputs(wl, parts=("q", "k", "v", "hidden"))
    cu = x["cu_seqlens"]
    scale = scale_of(d)
    q, k, v, h = (dev_bf16(x[p]) for p in ("q", "k", "v", "hidden"))
    score, lse = kv.window_score(q, k, cu, scale=scale, return_lse=True)
    ora_s, ora_l = score_oracle(x, wl, scale)
    assert_close(host(score), ora_s, what="score")
    check_rows(x, wl, scale, lse=lse, ora_lse=ora_l, what="lse")
    _, tok, stats = kv.accumulate_stats(score, cu, w, h_q // h_kv)
    s64 = host(score).astype(np.float64)
    assert_close(host(tok), oracle.head_sum(s64), rtol=1e-6, atol=0, what="tok")
    check_stats(stats, s64, cu, w, h_q // h_kv, ora_score=ora_s)
    idx_kv, idx_ts = kv.topk2(score, tok, cu, w, k_kv, k_ts)
    want_kv = oracle.select_rows(s64, cu, w, k_kv)
    want_ts = oracle.select_rows(host(tok).astype(np.float64)[None, :], cu, w, k_ts)
    assert np.array_equal(host(idx_kv), want_kv.astype(np.int32))
    assert np.array_equal(host(idx_ts).reshape(want_ts.shape), want_ts.astype(np.int32))
    lk = [oracle.budget_length(n, w, kk) for n, kk in zip(lens, k_kv)]
    lt = [oracle.budget_length(n, w, kk) for n, kk in zip(lens, k_ts)]
    k_c, v_c, h_c = kv.gather_multi(cu, w, [(k, idx_kv, k_kv), (v, idx_kv, k_kv), (h, idx_ts, k_ts)])
    assert np.array_equal(host(k_c).view(np.uint16), oracle.gather(x["k"], cu, want_kv, lk))
    assert np.array_equal(host(v_c).view(np.uint16), oracle.gather(x["v"], cu, want_kv, lk))
    hid = x["hidden"].reshape(x["hidden"].shape[0], 1, -1)
    assert np.array_equal(host(h_c).view(np.uint16).reshape(-1, 1, hid.shape[2]),
                          oracle.gather(hid, cu, want_ts, lt))
    if not variants:
        return
    # the same shapes through the other score calls: the statistics in the
    # second pass (score, normalisers and head sum bit for bit, statistics
    # within their bound), the one-pass call fed the oracle's normalisers,
    # and the call with row entropies (score and normalisers bit for bit)
    s2, l2, _, t2, st2 = kv.window_score_stats(q, k, cu, scale=scale, return_lse=True)
    assert np.array_equal(host(s2), host(score)) and np.array_equal(host(l2), host(lse))
    assert np.array_equal(host(t2), host(tok))
    check_stats(st2, s64, cu, w, h_q // h_kv, ora_score=ora_s, what="fused stats")
    one = kv.window_score(q, k, cu, scale=scale, lse_in=dev_f32(ora_l))
    assert_close(host(one), ora_s, what="score from given lse")
    s3, l3, ent, mean = kv.window_score_entropy(q, k, cu, scale=scale, return_lse=True)
    assert np.array_equal(host(s3), host(score)) and np.array_equal(host(l3), host(lse))
    ora_e = oracle.window_row_entropy(oracle.bf16_to_f64(x["q"]), oracle.bf16_to_f64(x["k"]), cu, h_q, h_kv, w,
                                      scale)
    check_rows(x, wl, scale, ent=ent, mean=mean, ora_ent=ora_e, what="row entropy")
