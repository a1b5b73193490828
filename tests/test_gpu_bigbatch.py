"""A batch of 150 sequences: more than one launch's worth (64 sequences per
launch), so every call splits its work over launch groups.  The whole pass,
the row entropies and the paged gather against the oracle."""
import numpy as np
import pytest

import oracle
import token_selection_tsp_amd as kv
from token_selection_tsp_amd import synth
from gpu_util import assert_close, check_rows, check_stats, dev_bf16, host, log, scale_of, score_oracle

pytestmark = pytest.mark.gpu


def test_batch_of_150_sequences():
    import torch
    rng = np.random.default_rng(150)
    w, h_q, h_kv, d = 8, 8, 2, 64
    lens = [int(x) for x in rng.integers(w, 400, size=150)]
    lens[70] = w                                   # a sequence that is all window
    wl = synth.small("big_batch", 150, lens, h_q, h_kv, d, w, hidden=64, hubs=0, sink=True)
    x = synth.layer_inputs(wl, parts=("q", "k", "v", "hidden"))
    cu = x["cu_seqlens"]
    scale = scale_of(d)
    q, k, v, h = (dev_bf16(x[p]) for p in ("q", "k", "v", "hidden"))
    log("150 sequences: score")
    score, lse = kv.window_score(q, k, cu, scale=scale, return_lse=True)
    ora_s, ora_l = score_oracle(x, wl, scale)
    assert_close(host(score), ora_s, what="score")
    check_rows(x, wl, scale, lse=lse, ora_lse=ora_l, what="lse")
    log("150 sequences: stats")
    _, tok, stats = kv.accumulate_stats(score, cu, w, h_q // h_kv)
    s64 = host(score).astype(np.float64)
    assert_close(host(tok), oracle.head_sum(s64), rtol=1e-6, atol=0, what="tok")
    check_stats(stats, s64, cu, w, h_q // h_kv, ora_score=ora_s)
    log("150 sequences: top-k and gathers")
    k_kv = [int(rng.integers(0, n + 2)) for n in lens]
    k_ts = [int(rng.integers(0, n + 2)) for n in lens]
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
    log("150 sequences: row entropy")
    score2, ent, mean = kv.window_score_entropy(q, k, cu, scale=scale)
    assert np.array_equal(host(score2), host(score))
    want_e = oracle.window_row_entropy(oracle.bf16_to_f64(x["q"]), oracle.bf16_to_f64(x["k"]), cu,
                                       h_q, h_kv, w, scale)
    check_rows(x, wl, scale, ent=ent, mean=mean, ora_ent=want_e, what="150 sequences")
    log("150 sequences: paged gather")
    bs = 4
    need = [-(-L // bs) for L in lk]
    nb = sum(need)
    perm = rng.permutation(nb)
    table = np.full((len(lens), max(need)), -1, dtype=np.int32)
    at = 0
    for b, n_b in enumerate(need):
        table[b, :n_b] = perm[at:at + n_b]
        at += n_b
    init = rng.integers(0, 2 ** 16, size=(nb, bs, h_kv, d), dtype=np.uint16)
    cache = dev_bf16(init)
    kv.gather_paged(cu, w, [(k, idx_kv, k_kv, cache, torch.from_numpy(table).cuda())])
    want_c = oracle.gather_paged(x["k"], cu, want_kv, lk, table, bs, init)
    assert np.array_equal(host(cache).view(np.uint16), want_c)
