"""Pins for the CPU oracle: closed forms, library routines, invariants,
hand-worked examples and brute force.  No GPU involved."""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
from token_selection_tsp_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_examples.json")


def _val(s):
    """Evaluate a golden entry: a number, a fraction 'a/b', 'ln(x)' or an
    arithmetic expression over those."""
    if isinstance(s, (int, float)):
        return float(s)
    expr = s.replace("ln(", "math.log(")
    return float(eval(expr, {"math": math, "__builtins__": {}}))


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


def _rand(seed, shape, scale=1.0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape) * scale


# ------------------------------------------------------------ hand-worked examples

@pytest.mark.parametrize("ex", [e for e in _golden() if "q" in e], ids=lambda e: e["name"])
def test_hand_worked_window_score(ex):
    q = np.array([[[[_val(x) for x in h] for h in row] for row in b] for b in ex["q"]])
    k = np.array([[[_val(x) for x in h] for h in t] for t in ex["k"]])
    score, lse = oracle.window_score(q, k, ex["cu_seqlens"], ex["h_q"], ex["h_kv"], ex["w"], ex["scale"])
    want = np.array([[_val(x) for x in r] for r in ex["score"]])
    np.testing.assert_allclose(score, want, rtol=1e-14, atol=1e-15)
    want_lse = np.array([[[_val(x) for x in r] for r in h] for h in ex["lse"]])
    np.testing.assert_allclose(lse, want_lse, rtol=1e-14)
    st = oracle.layer_stats(want, ex["cu_seqlens"], ex["w"], ex["h_q"] // ex["h_kv"])
    want_st = np.array([[_val(x) for x in r] for r in ex["stats"]])
    np.testing.assert_allclose(st, want_st, rtol=1e-13, atol=1e-16)


@pytest.mark.parametrize("ex", _golden(), ids=lambda e: e["name"])
def test_hand_worked_selection(ex):
    for case in ex["select"]:
        w = case.get("w", ex.get("w"))
        keys = np.array(case["keys"], dtype=np.float64)
        got = oracle.select_with_window(keys, len(keys), w, case["k"])
        assert got.tolist() == case["idx"]


# ------------------------------------------------------------ closed forms

def _uniform_closed_form(n, w, G):
    """q = 0: every window row i (position n-w+i) spreads its mass uniformly
    over its n-w+i+1 visible keys."""
    out = np.zeros(n)
    for i in range(w):
        p = n - w + i
        out[: p + 1] += G / (p + 1)
    return out


@pytest.mark.parametrize("lens,w,h_q,h_kv", [((17,), 1, 1, 1), ((40, 9), 5, 4, 2), ((64, 33, 7), 7, 8, 2)])
def test_uniform_attention_closed_form(lens, w, h_q, h_kv):
    d = 8
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = np.zeros((len(lens), w, h_q, d))
    k = _rand(1, (cu[-1], h_kv, d), 3.0)
    score, lse = oracle.window_score(q, k, cu, h_q, h_kv, w, 0.3)
    G = h_q // h_kv
    for b, n in enumerate(lens):
        want = _uniform_closed_form(n, w, G)
        for g in range(h_kv):
            np.testing.assert_allclose(score[g, cu[b]:cu[b + 1]], want, rtol=1e-13)
        np.testing.assert_allclose(lse[b], np.log(n - w + np.arange(w) + 1.0)[None, :].repeat(h_q, 0), rtol=1e-13)


def test_single_row_is_library_softmax():
    n, d = 300, 16
    q = _rand(2, (1, 1, 1, d))
    k = _rand(3, (n, 1, d))
    scale = 1.0 / math.sqrt(d)
    score, lse = oracle.window_score(q, k, [0, n], 1, 1, 1, scale)
    logits = scale * (k[:, 0, :] @ q[0, 0, 0])
    np.testing.assert_allclose(score[0], scipy.special.softmax(logits), rtol=1e-12)
    np.testing.assert_allclose(lse[0, 0, 0], scipy.special.logsumexp(logits), rtol=1e-13)


def test_softmax_rows_normalise_and_total_mass():
    lens = (50, 23)
    w, h_q, h_kv, d = 6, 6, 3, 8
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = _rand(4, (2, w, h_q, d), 2.0)
    k = _rand(5, (cu[-1], h_kv, d), 2.0)
    scale = 0.4
    score, lse = oracle.window_score(q, k, cu, h_q, h_kv, w, scale)
    G = h_q // h_kv
    for b, n in enumerate(lens):
        off = cu[b]
        for g in range(h_kv):
            assert abs(score[g, off:off + n].sum() - w * G) < 1e-12
        # each row, renormalised by the returned lse, sums to one over its visible keys
        for h in range(h_q):
            g = h // G
            for i in range(w):
                p = n - w + i
                s = scale * (k[off:off + p + 1, g, :] @ q[b, i, h])
                assert abs(np.exp(s - lse[b, h, i]).sum() - 1.0) < 1e-12
    assert np.all(score >= 0)


def test_dominant_key_takes_all_mass():
    n, w, h_q, h_kv, d = 80, 4, 4, 2, 8
    q = np.zeros((1, w, h_q, d)); q[..., 0] = 1.0
    k = _rand(6, (n, h_kv, d), 0.1); k[..., 0] = 0.0
    jstar = 11
    k[jstar, 1, 0] = 200.0          # only in KV head 1, logit gap 100 >> 40
    score, _ = oracle.window_score(q, k, [0, n], h_q, h_kv, w, 0.5)
    G = h_q // h_kv
    assert abs(score[1, jstar] - w * G) < 1e-9 * w * G
    # KV head 0 holds no planted key and its logits are all zero: uniform rows
    np.testing.assert_allclose(score[0], _uniform_closed_form(n, w, G), rtol=1e-12)


@pytest.mark.parametrize("t", [0, 3, 6])
def test_causal_window_key(t):
    """A dominant key inside the window at position n-w+t is visible only to
    rows i >= t, which put all their mass on it; rows i < t spread theirs
    uniformly (q constant, other keys equal)."""
    n, w, G, d = 30, 7, 2, 4
    q = np.ones((1, w, G, d))
    k = np.zeros((n, 1, d))
    k[n - w + t] = 100.0
    score, _ = oracle.window_score(q, k, [0, n], G, 1, w, 1.0)
    assert abs(score[0, n - w + t] - G * (w - t)) < 1e-9
    want_prefix = sum(G / (n - w + i + 1) for i in range(t))   # rows that do not see it
    np.testing.assert_allclose(score[0, 0], want_prefix, rtol=1e-9, atol=1e-12)


def test_group_mapping_uses_shared_kv_head():
    """Heads 0,1 use KV head 0; heads 2,3 use KV head 1.  Zero queries on the
    second group give exactly the uniform closed form on KV head 1."""
    n, w, d = 20, 3, 4
    q = _rand(7, (1, w, 4, d)); q[:, :, 2:, :] = 0.0
    k = _rand(8, (n, 2, d))
    score, _ = oracle.window_score(q, k, [0, n], 4, 2, w, 1.0)
    np.testing.assert_allclose(score[1], _uniform_closed_form(n, w, 2), rtol=1e-13)
    assert np.abs(score[0] - _uniform_closed_form(n, w, 2)).max() > 1e-3


# ------------------------------------------------------------ stats and pivot

def test_stats_closed_forms():
    n, w, G = 64, 4, 2
    mass = w * G
    uni = np.full((1, n), mass / n)
    st = oracle.layer_stats(uni, [0, n], w, G)[0]
    np.testing.assert_allclose(st, [math.log(n), 0.0, 0.0], atol=1e-15, rtol=1e-14)
    onehot = np.zeros((1, n)); onehot[0, 5] = mass
    st = oracle.layer_stats(onehot, [0, n], w, G)[0]
    np.testing.assert_allclose(st, [0.0, (n - 1) / n, (n - 1) / n ** 2], atol=1e-15, rtol=1e-14)
    # two KV heads average: uniform and one-hot
    both = np.concatenate([uni, onehot])
    st = oracle.layer_stats(both, [0, n], w, G)[0]
    np.testing.assert_allclose(st, [math.log(n) / 2, (n - 1) / n / 2, (n - 1) / n ** 2 / 2], rtol=1e-14)
    # half the mass on m positions: entropy ln m exactly
    m = 8
    half = np.zeros((1, n)); half[0, :m] = mass / m
    st = oracle.layer_stats(half, [0, n], w, G)[0]
    np.testing.assert_allclose(st[0], math.log(m), rtol=1e-14)
    np.testing.assert_allclose(st[1], (n - m) / n, rtol=1e-14)


def test_stats_ragged_segments():
    lens = (10, 30)
    cu = [0, 10, 40]
    w, G = 2, 1
    x = np.zeros((1, 40))
    x[0, :10] = 2 / 10                    # sequence 0 uniform
    x[0, 10 + 3] = 2                      # sequence 1 one-hot
    st = oracle.layer_stats(x, cu, w, G)
    np.testing.assert_allclose(st[0], [math.log(10), 0, 0], atol=1e-15, rtol=1e-14)
    np.testing.assert_allclose(st[1], [0, 29 / 30, 29 / 900], atol=1e-15, rtol=1e-14)


def test_pivot_planted():
    assert oracle.pivot_layer([5.0, 4.9, 3.0, 2.9]) == 2
    assert oracle.pivot_layer([5.0, 4.0, 3.0, 2.0]) == 1      # equal drops: smallest layer
    assert oracle.pivot_layer([1.0, 2.0, 3.0]) == 1           # no drop: largest (least negative)
    assert oracle.pivot_layer([7.0]) == 0
    e = np.linspace(9, 8, 16); e[9:] -= 2.5                     # sharp drop into layer 9
    assert oracle.pivot_layer(e) == 9


def test_pivot_with_sparsity_rise_planted():
    # layer 2 has the largest drop but sparsity falls there; layer 4 is the
    # largest drop among the layers whose sparsity rose
    e = [5.0, 4.8, 2.0, 1.9, 1.0, 0.95]
    sp = [0.10, 0.20, 0.15, 0.16, 0.30, 0.31]
    assert oracle.pivot_layer(e) == 2
    assert oracle.pivot_layer_sparsity(e, sp) == 4
    # equal drops among rising layers: the smallest layer
    assert oracle.pivot_layer_sparsity([4.0, 3.0, 2.0, 1.0], [0.1, 0.2, 0.3, 0.4]) == 1
    assert oracle.pivot_layer_sparsity([4.0, 3.0, 3.5, 2.5], [0.3, 0.2, 0.4, 0.5]) == 3
    # sparsity never rises: the plain largest-drop rule
    assert oracle.pivot_layer_sparsity([5.0, 4.9, 3.0], [0.3, 0.3, 0.2]) == 2
    # equal sparsity is not a rise
    assert oracle.pivot_layer_sparsity([5.0, 1.0, 0.9], [0.2, 0.2, 0.25]) == 2
    assert oracle.pivot_layer_sparsity([3.0], [0.5]) == 0
    with pytest.raises(ValueError):
        oracle.pivot_layer_sparsity([1.0, 2.0], [0.1])


# ------------------------------------------------------------ row entropy

@pytest.mark.parametrize("lens,w,h_q,h_kv", [((17,), 1, 1, 1), ((40, 9), 5, 4, 2), ((64, 33, 7), 7, 8, 2)])
def test_row_entropy_uniform_closed_form(lens, w, h_q, h_kv):
    """q = 0: row i is uniform over its n-w+i+1 visible keys, entropy ln(n-w+i+1)."""
    d = 8
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = np.zeros((len(lens), w, h_q, d))
    k = _rand(11, (cu[-1], h_kv, d), 3.0)
    ent = oracle.window_row_entropy(q, k, cu, h_q, h_kv, w, 0.3)
    for b, n in enumerate(lens):
        want = np.log(n - w + np.arange(w) + 1.0)
        np.testing.assert_allclose(ent[b], np.broadcast_to(want, (h_q, w)), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(oracle.mean_row_entropy(ent),
                               [np.log(n - w + np.arange(w) + 1.0).mean() for n in lens], rtol=1e-13)


def test_row_entropy_single_row_is_library_entropy():
    import scipy.stats
    n, d = 300, 16
    q = _rand(12, (1, 1, 1, d), 2.0)
    k = _rand(13, (n, 1, d), 2.0)
    scale = 1.0 / math.sqrt(d)
    ent = oracle.window_row_entropy(q, k, [0, n], 1, 1, 1, scale)
    logits = scale * (k[:, 0, :] @ q[0, 0, 0])
    assert abs(ent[0, 0, 0] - scipy.stats.entropy(scipy.special.softmax(logits))) < 1e-12


def test_row_entropy_two_level_closed_form():
    """m keys at logit a, the other n - m at logit 0: with Z = m e^a + n - m,
    P = e^a / Z on the m keys and 1 / Z elsewhere, so
    H = ln Z - m a e^a / Z."""
    n, m, d = 97, 5, 4
    a = 2.5
    q = np.zeros((1, 1, 1, d)); q[0, 0, 0, 0] = 1.0
    k = np.zeros((n, 1, d))
    hot = [0, 13, 40, 77, 96]
    k[hot, 0, 0] = a                      # scale 1: logit a on the hot keys
    ent = oracle.window_row_entropy(q, k, [0, n], 1, 1, 1, 1.0)
    z = m * math.exp(a) + (n - m)
    assert abs(ent[0, 0, 0] - (math.log(z) - m * a * math.exp(a) / z)) < 1e-13


def test_row_entropy_dominant_key_is_zero_and_bounds():
    n, w, h_q, h_kv, d = 80, 4, 4, 2, 8
    q = np.zeros((1, w, h_q, d)); q[..., 0] = 1.0
    k = _rand(14, (n, h_kv, d), 0.1); k[..., 0] = 0.0
    k[11, 1, 0] = 200.0                   # logit gap 100 in KV head 1
    ent = oracle.window_row_entropy(q, k, [0, n], h_q, h_kv, w, 0.5)
    assert np.all(ent[0, 2:] < 1e-30)     # query heads 2, 3 read KV head 1
    # random rows: 0 <= H <= ln(visible keys)
    lens = (50, 23)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = _rand(15, (2, 6, 6, 8), 2.0)
    k = _rand(16, (cu[-1], 3, 8), 2.0)
    ent = oracle.window_row_entropy(q, k, cu, 6, 3, 6, 0.4)
    for b, n in enumerate(lens):
        cap = np.log(n - 6 + np.arange(6) + 1.0)
        assert np.all(ent[b] >= 0) and np.all(ent[b] <= cap[None, :] + 1e-12)
        assert np.all(ent[b] < cap[None, :] - 1e-3)   # non-uniform rows stay below the cap


def test_accumulate_and_head_sum():
    s = np.array([[1.0, 2.0, 3.0], [10.0, 20.0, 30.0]])
    c = oracle.accumulate(s)
    assert c.tolist() == s.tolist()
    c2 = oracle.accumulate(s, c)
    assert c2.tolist() == [[2, 4, 6], [20, 40, 60]]
    assert oracle.head_sum(c2).tolist() == [22, 44, 66]
    layers = [np.full((2, 3), float(l + 1)) for l in range(4)]
    acc = None
    for l, x in enumerate(layers):
        acc = oracle.accumulate(x, acc)
        assert np.all(acc == (l + 1) * (l + 2) / 2)


# ------------------------------------------------------------ selection

def _brute_select(x, n, w, k):
    nc = n - w
    order = sorted(range(nc), key=lambda j: (-x[j], j))      # library sort
    kept = sorted(order[: min(k, nc)])
    return kept + list(range(nc, n))


@pytest.mark.parametrize("seed", range(6))
def test_select_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    for n in list(range(1, 20)) + [31, 64]:
        for w in sorted({1, 2, min(n, 5), n}):
            if w > n:
                continue
            x = rng.integers(0, 3, size=n).astype(np.float64)     # 3-value set: many ties
            for k in range(0, n - w + 3):
                got = oracle.select_with_window(x, n, w, k)
                want = _brute_select(list(x), n, w, k)
                assert got.tolist() == want
                assert len(got) == oracle.budget_length(n, w, k) == min(n, k + w)
                assert np.all(np.diff(got[: len(got) - w]) > 0)
                assert got[len(got) - w:].tolist() == list(range(n - w, n))


def test_select_signed_zero_ties_by_position():
    x = np.array([0.0, -0.0, 0.0, -1.0, 5.0])
    assert oracle.select_with_window(x, 5, 1, 2).tolist() == [0, 1, 4]


def test_select_rows_ragged():
    cu = [0, 6, 10]
    keys = np.array([[3, 1, 3, 2, 3, 0, 9, 8, 7, 6], [0, 0, 0, 0, 0, 0, 1, 2, 3, 4]], dtype=float)
    out = oracle.select_rows(keys, cu, 2, [2, 1])
    assert out.tolist() == [[0, 2, 4, 5, 0, 2, 3], [0, 1, 4, 5, 1, 2, 3]]


def test_select_rejects_nonfinite():
    with pytest.raises(ValueError):
        oracle.select_with_window(np.array([1.0, np.nan, 2.0]), 3, 1, 1)


# ------------------------------------------------------------ gather

def test_gather_brute_force():
    rng = np.random.default_rng(3)
    cu = [0, 7, 12]
    heads, row = 3, 5
    src = rng.integers(0, 65535, size=(12, heads, row)).astype(np.uint16)
    lengths = [4, 3]
    idx = np.array([[0, 2, 5, 6, 1, 3, 4], [1, 2, 3, 6, 0, 1, 4], [6, 5, 4, 3, 4, 3, 2]])
    got = oracle.gather(src, cu, idx, lengths)
    for h in range(heads):
        for s in range(7):
            b = 0 if s < 4 else 1
            off = cu[b]
            assert got[s, h].tolist() == src[off + idx[h, s], h].tolist()
    shared = oracle.gather(src, cu, idx[:1], lengths)
    for h in range(heads):
        for s in range(7):
            off = 0 if s < 4 else 7
            assert shared[s, h].tolist() == src[off + idx[0, s], h].tolist()


def test_gather_paged_brute_force():
    """Every selected row lands in block block_table[b][s // bs], slot s % bs,
    by a plain loop over (b, s, h); every other slot keeps its contents;
    block numbers outside [0, num_blocks) write nothing."""
    rng = np.random.default_rng(9)
    cu = [0, 40, 47, 90]
    heads, row = 2, 3
    src = rng.integers(0, 65535, size=(90, heads, row)).astype(np.uint16)
    lengths = [13, 7, 20]
    L = sum(lengths)
    idx = np.stack([np.concatenate([rng.choice(n, size=Lb, replace=False)
                                    for n, Lb in zip((40, 7, 43), lengths)]) for _ in range(heads)])
    bs, max_blocks, num_blocks = 4, 6, 20
    bt = rng.permutation(num_blocks)[:3 * max_blocks].reshape(3, max_blocks).astype(np.int32)
    bt[2, 1] = -1                      # an unmapped block: slots 4..7 of sequence 2 are dropped
    bt[0, 3] = num_blocks + 5          # out of range: slot 12 of sequence 0 is dropped
    cache = np.full((num_blocks, bs, heads, row), 0xBEEF, dtype=np.uint16)
    got = oracle.gather_paged(src, cu, idx, lengths, bt, bs, cache)
    assert np.all(cache == 0xBEEF)     # the input is not modified
    want = cache.copy()
    start = 0
    written = np.zeros((num_blocks, bs), dtype=bool)
    for b, Lb in enumerate(lengths):
        for s in range(Lb):
            blk = bt[b, s // bs]
            if not 0 <= blk < num_blocks:
                continue
            for h in range(heads):
                want[blk, s % bs, h] = src[cu[b] + idx[h, start + s], h]
            written[blk, s % bs] = True
        start += Lb
    assert np.array_equal(got, want)
    assert written.sum() == L - 4 - 1
    assert np.all(got[~written] == 0xBEEF)


def test_gather_paged_identity_table_is_flat_gather():
    """Consecutive blocks per sequence: the cache read in block order is the
    flat gather of each sequence, padded to whole blocks."""
    rng = np.random.default_rng(10)
    cu = [0, 30, 55]
    src = rng.integers(0, 65535, size=(55, 1, 8)).astype(np.uint16)
    lengths = [9, 16]
    idx = np.concatenate([rng.choice(30, 9, replace=False), rng.choice(25, 16, replace=False)])[None, :]
    bs, max_blocks = 4, 4
    bt = np.arange(2 * max_blocks, dtype=np.int32).reshape(2, max_blocks)
    cache = np.zeros((2 * max_blocks, bs, 1, 8), dtype=np.uint16)
    got = oracle.gather_paged(src, cu, idx, lengths, bt, bs, cache).reshape(2, max_blocks * bs, 1, 8)
    flat = oracle.gather(src, cu, idx, lengths)
    assert np.array_equal(got[0, :9], flat[:9]) and np.all(got[0, 9:] == 0)
    assert np.array_equal(got[1, :16], flat[9:])


# ------------------------------------------------------------ input marshalling

def test_bf16_promotion_exact():
    vals = np.array([1.0, -2.5, 3.140625, 65280.0, 1e-3], dtype=np.float32)
    bits = synth.bf16_bits(vals)
    f = oracle.bf16_to_f64(bits)
    assert f[0] == 1.0 and f[1] == -2.5 and f[2] == 3.140625 and f[3] == 65280.0
    assert abs(f[4] - 1e-3) < 1e-3 * 2 ** -8
    # round-to-nearest-even on an exact tie: 1 + 2^-8 sits between 1 and 1 + 2^-7
    tie = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], dtype=np.float32)
    assert oracle.bf16_to_f64(synth.bf16_bits(tie)).tolist() == [1.0, 1.0 + 2 ** -6]


def test_workloads_have_stated_shapes():
    wl = synth.WORKLOADS["n128k_gqa32x8_d128"]
    assert wl.seq_lengths() == [131072] and wl.kv_tokens().tolist() == [4096]
    assert wl.tsp_tokens().tolist() == [13107]
    rag = synth.WORKLOADS["ragged8_4k_32k"]
    ls = rag.seq_lengths()
    assert len(ls) == 8 and all(4096 <= x <= 32768 for x in ls)
    assert rag.kv_tokens().tolist() == [x // 10 for x in ls]
    c1 = synth.WORKLOADS["n1k_gqa8x2_d64"]
    assert c1.kv_tokens().tolist() == [256] and c1.tsp_tokens().tolist() == [512]
    h = c1.hub_positions(0, 0, 1024)
    assert h[0] == 0 and len(h) == 17
    s5 = synth.WORKLOADS["structkv16_n64k"]
    assert s5.alpha_at(0) == 0.5 and s5.alpha_at(15) == 3.0
    assert (s5.hub_positions(0, 0, 65536) == s5.hub_positions(7, 0, 65536)).all()


def test_small_workload_oracle_end_to_end():
    wl = synth.small("e2e", 11, (90, 40), h_q=4, h_kv=2, d=16, w=5)
    x = synth.layer_inputs(wl, parts=("q", "k", "v", "hidden"))
    q = oracle.bf16_to_f64(x["q"])
    k = oracle.bf16_to_f64(x["k"])
    cu = x["cu_seqlens"]
    score, lse = oracle.window_score(q, k, cu, wl.h_q, wl.h_kv, wl.w, 1 / 4)
    # the planted sink (position 0) carries a large share of every head's mass
    for g in range(2):
        seg = score[g, :90]
        assert seg[0] > 3 * np.median(seg)
    kv_idx = oracle.select_rows(score, cu, wl.w, wl.kv_tokens())
    lens = [oracle.budget_length(n, wl.w, k) for n, k in zip(wl.seq_lengths(), wl.kv_tokens())]
    kc = oracle.gather(x["k"], cu, kv_idx, lens)
    assert kc.shape == (sum(lens), 2, 16)
