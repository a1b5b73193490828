"""Accumulate/stats, top-k and gather on the GPU against the oracle, fed the
same arrays (bit-exact where the result is integer or a copy)."""
import math

import numpy as np
import pytest

import oracle
import token_selection_tsp_amd as kv
from token_selection_tsp_amd import synth
from gpu_util import assert_close, check_stats, dev_bf16, dev_f32, host, log
from tolerances import stats_kernel

pytestmark = pytest.mark.gpu


def _scores(seed, h_kv, cu, mass, distinct=None):
    """Positive score-like rows whose per-sequence totals are `mass`."""
    T = int(cu[-1])
    x = synth.random_f32_rows(seed, h_kv, T, distinct=distinct).astype(np.float64) + 1e-3
    for b in range(len(cu) - 1):
        seg = x[:, cu[b]:cu[b + 1]]
        seg *= mass / seg.sum(axis=1, keepdims=True)
    return x.astype(np.float32)


# ------------------------------------------------------------ accumulate / stats

@pytest.mark.parametrize("lens,h_kv", [((1000,), 2), ((4096, 17, 3000), 8), ((131072,), 8), ((5,), 1)])
def test_accumulate_stats_matches_oracle(lens, h_kv):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    w, G = 4, 4
    s = _scores(1, h_kv, cu, w * G)
    c_in = _scores(2, h_kv, cu, 3.0)
    log(f"accumulate_stats {lens} h_kv={h_kv}")
    c_out, tok, stats = kv.accumulate_stats(dev_f32(s), cu, w, G, c_in=dev_f32(c_in))
    want_c = oracle.accumulate(s.astype(np.float64), c_in.astype(np.float64))
    assert np.array_equal(host(c_out), want_c.astype(np.float32))      # one fp32 add: exact
    assert_close(host(tok), oracle.head_sum(want_c), rtol=1e-6, atol=0, what="tok")
    check_stats(stats, s.astype(np.float64), cu, w, G)
    # no c_in: c_out is a copy, tok the plain head sum
    c2, tok2, _ = kv.accumulate_stats(dev_f32(s), cu, w, G, c_out=dev_f32(np.zeros_like(s)), want_stats=False)
    assert np.array_equal(host(c2), s)
    assert_close(host(tok2), oracle.head_sum(s.astype(np.float64)), rtol=1e-6, atol=0, what="tok")


def test_stats_closed_forms_on_gpu():
    # 8 / 1024 is exact in fp32, so the uniform case sits exactly on the
    # below-uniform threshold and is not counted
    n, w, G = 1024, 4, 2
    mass = w * G
    uni = np.full((2, n), mass / n, dtype=np.float32)
    onehot = np.zeros((2, n), dtype=np.float32); onehot[:, 7] = mass
    for x, want in ((uni, [math.log(n), 0.0, 0.0]), (onehot, [0.0, (n - 1) / n, (n - 1) / n ** 2])):
        _, _, st = kv.accumulate_stats(dev_f32(x), [0, n], w, G, want_tok=False)
        got = host(st)[0].astype(np.float64)
        assert_close(got, want, rtol=0.0, atol=stats_kernel(x.astype(np.float64), [0, n], w, G)[0])


# ------------------------------------------------------------ top-k

def _topk_case(keys, cu, w, ks):
    got = host(kv.topk(dev_f32(keys), cu, w, ks))
    want = oracle.select_rows(keys.astype(np.float64), cu, w, ks)
    assert got.shape == want.shape
    assert np.array_equal(got, want.astype(np.int32))


# One launch picks one of two paths from the longest row and the number of
# sequences.  Single rows up to about 18.8K candidates take the
# one-work-group path (every key listed up to 16384, the sampled bracket
# above); longer single rows take the two-launch path (every key listed up
# to 16384 per chunk set, the bracket above).  Heavy ties overflow the
# candidate list and exercise each path's full-row fallback.
@pytest.mark.parametrize("distinct", [None, 3, 1, 2000])
@pytest.mark.parametrize("n", [9, 100, 1025, 8192 + 77, 40000])
def test_topk_bit_exact(n, distinct):
    w = 4
    keys = synth.random_f32_rows(n + (distinct or 0), 3, n, distinct=distinct)
    for k in sorted({0, 1, 2, n // 3, n - w - 1, n - w, n - w + 5}):
        if k < 0:
            continue
        log(f"topk n={n} distinct={distinct} k={k}")
        _topk_case(keys, [0, n], w, [k])


def test_topk_one_workgroup_path_bracketed():
    # a single row of 17968 candidates: the one-work-group path with the
    # sampled bracket (longer than 16384), random keys and heavy ties
    n, w = 18000, 32
    for distinct in (None, 3, 200):
        keys = synth.random_f32_rows(31 + (distinct or 0), 3, n, distinct=distinct)
        for k in (1, 1797, 4096, n - w - 1):
            log(f"topk one-wg bracketed distinct={distinct} k={k}")
            _topk_case(keys, [0, n], w, [k])


def test_topk_many_sequences_both_paths():
    # eight sequences up to 32K (one work-group per row and sequence), then
    # three of 50K (two launches); ragged tails, ties, both budgets
    w = 32
    rng = np.random.default_rng(7)
    for lens in ([int(x) for x in rng.integers(4096, 32768, size=8)], [50000, 49001, 50103]):
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        for distinct in (None, 3):
            keys = synth.random_f32_rows(11 + (distinct or 0), 4, int(cu[-1]), distinct=distinct)
            ks = [max(0, (n - w) // 10) for n in lens]
            ks[1] = 0                      # none kept: the window alone
            ks[-1] = lens[-1] - w          # every candidate kept
            log(f"topk many sequences {lens} distinct={distinct}")
            _topk_case(keys, cu, w, ks)
            _topk2_case(keys[:3], keys[3:], cu, w, [max(1, n // 20) for n in lens], [max(1, n // 5) for n in lens])


def test_topk_one_workgroup_path_list_overflow():
    # twelve sequences of 40000 take the one-work-group path; with one or two
    # distinct values the bracket holds more keys than the LDS list, so the
    # threshold comes from the whole-row select
    w = 32
    lens = [40000] * 12
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    for distinct in (1, 2):
        keys = synth.random_f32_rows(41 + distinct, 2, int(cu[-1]), distinct=distinct)
        log(f"topk list overflow distinct={distinct}")
        _topk_case(keys, cu, w, [(n - w) // 3 for n in lens])


def test_topk_ragged_batch_and_rows():
    lens = [50, 4096, 17, 1, 3000]
    w = 1
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    keys = synth.random_f32_rows(5, 9, int(cu[-1]), distinct=50)
    _topk_case(keys, cu, w, [10, 409, 0, 0, 2999])


def test_topk_special_values():
    n, w = 600, 8
    rng = np.random.default_rng(0)
    keys = rng.choice(np.array([0.0, -0.0, 1e-30, 3.5, -2.0, 1e30, -1e30, 5e-45], dtype=np.float32),
                      size=(2, n))
    for k in (1, 7, 100, 591):
        _topk_case(keys, [0, n], w, [k])


def test_topk_long_row():
    n, w = 131072, 32
    keys = _scores(3, 9, np.array([0, n]), 128.0)
    log("topk long row")
    _topk_case(keys, [0, n], w, [4096])
    _topk_case(keys[:1], [0, n], w, [13107])


@pytest.mark.parametrize("nc", [64 * 4096, 64 * 4096 + 1, 300_000])
def test_topk_chunk_scan_paths(nc):
    # The two-launch path scans its per-chunk counts in one wave for rows of
    # up to 64 chunks of 4096 candidates and over the whole work-group for
    # longer rows: both sides of that boundary, random keys (bracketed) and
    # heavy ties (the candidate list overflows: whole-row select), through
    # topk and topk2
    w = 32
    n = nc + w
    keys = _scores(21, 2, np.array([0, n]), 64.0)
    for k in (1, 5000, nc // 10):
        log(f"topk chunk scans nc={nc} k={k}")
        _topk_case(keys, [0, n], w, [k])
    ties = synth.random_f32_rows(22, 1, n, distinct=7)
    log(f"topk chunk scans nc={nc} ties")
    _topk_case(ties, [0, n], w, [nc // 3])
    log(f"topk2 chunk scans nc={nc}")
    _topk2_case(keys, ties, [0, n], w, [4096], [nc // 3])


def _topk2_case(keys_a, keys_b, cu, w, ka, kb):
    ga, gb = kv.topk2(dev_f32(keys_a), dev_f32(keys_b), cu, w, ka, kb)
    for got, keys, ks in ((ga, keys_a, ka), (gb, keys_b, kb)):
        want = oracle.select_rows(keys.astype(np.float64), cu, w, ks)
        got = host(got).reshape(want.shape)
        assert np.array_equal(got, want.astype(np.int32))


def test_topk2_both_budgets():
    # per-head rows with one budget and a head-sum row with another, as in a
    # selection pass: equal to the oracle's two independent selections
    n, w = 131072, 32
    keys = _scores(5, 8, np.array([0, n]), 128.0)
    tok = keys.sum(axis=0, dtype=np.float32)[None, :]
    log("topk2 128K")
    _topk2_case(keys, tok, [0, n], w, [4096], [13107])
    lens = [50, 4096, 17, 32, 30000]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ka = synth.random_f32_rows(11, 3, int(cu[-1]), distinct=40)
    kb = synth.random_f32_rows(12, 1, int(cu[-1]))
    log("topk2 ragged")
    _topk2_case(ka, kb, cu, 1, [10, 409, 0, 31, 2999], [49, 0, 3, 5, 26000])


def test_topk2_matches_two_calls():
    lens = [9000, 700, 30001]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ka = synth.random_f32_rows(13, 4, int(cu[-1]), distinct=500)
    kb = synth.random_f32_rows(14, 2, int(cu[-1]))
    w, k1, k2 = 8, [900, 70, 3000], [4500, 0, 25000]
    a1 = host(kv.topk(dev_f32(ka), cu, w, k1))
    b1 = host(kv.topk(dev_f32(kb), cu, w, k2))
    a2, b2 = kv.topk2(dev_f32(ka), dev_f32(kb), cu, w, k1, k2)
    assert np.array_equal(a1, host(a2)) and np.array_equal(b1, host(b2))


# ------------------------------------------------------------ gather

@pytest.mark.parametrize("row_bytes,heads", [(256, 8), (128, 2), (16, 3), (8192, 1), (48, 1)])
def test_gather_bit_exact(row_bytes, heads):
    lens = [300, 1000, 40]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    rng = np.random.default_rng(row_bytes + heads)
    src = rng.integers(0, 2 ** 16, size=(T, heads, row_bytes // 2), dtype=np.uint16)
    w = 4
    ks = [30, 0, 100]
    keys = synth.random_f32_rows(7, heads, T)
    idx = oracle.select_rows(keys.astype(np.float64), cu, w, ks).astype(np.int32)
    lengths = [oracle.budget_length(n, w, k) for n, k in zip(lens, ks)]
    dsrc = dev_bf16(src)
    per = host(kv.gather(dsrc, cu, _i32(idx), w, ks))
    assert np.array_equal(per.view(np.uint16), oracle.gather(src, cu, idx, lengths))
    shared = host(kv.gather(dsrc, cu, _i32(idx[:1]), w, ks))
    assert np.array_equal(shared.view(np.uint16), oracle.gather(src, cu, idx[:1], lengths))


def _i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def test_gather_multi_matches_oracle():
    # K and V (per-head indices) and hidden rows (shared indices, another
    # budget) in one launch, on a ragged batch; odd row sizes
    lens = [300, 17, 4096, 1000]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, heads, w = int(cu[-1]), 4, 8
    rng = np.random.default_rng(21)
    kbits = rng.integers(0, 2**16, size=(T, heads, 64), dtype=np.uint16)
    vbits = rng.integers(0, 2**16, size=(T, heads, 24), dtype=np.uint16)
    hbits = rng.integers(0, 2**16, size=(T, 1, 2056), dtype=np.uint16)
    k_kv, k_ts = [40, 3, 1000, 999], [100, 0, 2048, 5]
    lk = [oracle.budget_length(n, w, k) for n, k in zip(lens, k_kv)]
    lt = [oracle.budget_length(n, w, k) for n, k in zip(lens, k_ts)]
    ik = np.concatenate([rng.integers(0, n, size=(heads, l)) for n, l in zip(lens, lk)], axis=1)
    it = np.concatenate([rng.integers(0, n, size=(1, l)) for n, l in zip(lens, lt)], axis=1)
    log("gather_multi")
    outs = kv.gather_multi(cu, w, [(dev_bf16(kbits), _i32(ik), k_kv), (dev_bf16(vbits), _i32(ik), k_kv),
                                   (dev_bf16(hbits[:, 0]), _i32(it[0]), k_ts)])
    for got, src, idx, ln in ((outs[0], kbits, ik, lk), (outs[1], vbits, ik, lk), (outs[2], hbits, it, lt)):
        want = oracle.gather(src, cu, idx, ln)
        assert np.array_equal(host(got).view(np.uint16).reshape(want.shape), want)


def test_gather_out_of_range_rows_are_zero():
    cu = np.array([0, 10], dtype=np.int32)
    src = np.arange(10 * 8, dtype=np.uint16).reshape(10, 1, 8) + 1
    idx = np.array([[-1, 3, 10, 2, 9]], dtype=np.int32)      # k=4, w=1 -> 5 entries
    got = host(kv.gather(dev_bf16(src), cu, _i32(idx), 1, [4])).view(np.uint16)
    assert not got[0].any() and not got[2].any()
    assert np.array_equal(got[1], src[3]) and np.array_equal(got[3], src[2]) and np.array_equal(got[4], src[9])


def _miss_row(n, w, sampled_value, hidden_value, rest_value, seed):
    """Keys laid out against the top-k sample (1024 points spaced
    (n - w) // 1024 apart, four adjacent keys at each): every sampled key
    gets sampled_value, 4096 keys between the sample points get
    hidden_value, the rest rest_value; small distinct noise on all."""
    nc = n - w
    stride = nc // 1024
    j = np.arange(n)
    sampled = (j % stride < 4) & (j < 1024 * stride)
    hidden = (j % stride >= stride // 2) & (j % stride < stride // 2 + 4) & (j < 1024 * stride)
    assert sampled.sum() == 4096 and hidden.sum() == 4096 and not (sampled & hidden).any()
    rng = np.random.default_rng(seed)
    x = np.full(n, rest_value, dtype=np.float64) + rng.random(n) * 1e-3
    x[sampled] = sampled_value + rng.random(4096) * 1e-3
    x[hidden] = hidden_value + rng.random(4096) * 1e-3
    return x.astype(np.float32)[None, :]


@pytest.mark.parametrize("n", [131072, 18000])
def test_topk_bracket_miss_both_ways(n):
    # the sampled bracket misses the k-th key on purpose; the selection must
    # still be exact (whole-row select).  131072: the two-launch path;
    # 18000: the one-work-group path.
    w = 32
    cu = [0, n]
    log(f"topk bracket miss n={n}: k-th key above the bracket")
    high_hidden = _miss_row(n, w, sampled_value=1.0, hidden_value=2.0, rest_value=0.5, seed=1)
    _topk_case(high_hidden, cu, w, [4096])
    log(f"topk bracket miss n={n}: k-th key below the bracket")
    high_sampled = _miss_row(n, w, sampled_value=3.0, hidden_value=2.0, rest_value=0.5, seed=2)
    _topk_case(high_sampled, cu, w, [8192])
    # both budgets in one call, one row each way
    a = np.concatenate([high_hidden, high_sampled])
    _topk2_case(a, high_hidden, cu, w, [4096], [4096])
