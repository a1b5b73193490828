"""Window-row attention entropy on the GPU against the oracle.

Tolerance: |gpu - oracle| <= 1e-4 + 1e-3 * |oracle| (nats).  The kernels
form each row's entropy as -ln2 * sum_j P_j x_j from fp32 logits x (log2
units) whose rounding is a few 1e-6 at the magnitudes here, so a row's
absolute error stays far below 1e-4; the relative part is the score's."""

import numpy as np
import pytest

import oracle
import token_selection_tsp_amd as kv
from token_selection_tsp_amd import synth
from gpu_util import assert_close, dev_bf16, host, log, scale_of, score_oracle

pytestmark = pytest.mark.gpu

E_RTOL, E_ATOL = 1e-3, 1e-4

# (lengths, h_q, h_kv, d, w): the score tests' mix of chunks, ragged tails,
# GQA groups, windows and row groups above 128
SHAPES = [
    ((1000,), 8, 2, 64, 8),
    ((37,), 4, 4, 128, 1),
    ((300, 33, 129), 16, 2, 128, 5),
    ((2500,), 32, 8, 128, 32),
    ((700, 64), 8, 1, 64, 33),
    ((2065,), 12, 4, 64, 7),
    ((5000, 1), 32, 8, 128, 1),
    ((33,), 2, 2, 64, 33),
    ((1, 2, 3, 4, 5, 1030), 4, 2, 128, 1),
    ((9, 8, 40), 8, 2, 64, 8),
    ((5000,), 32, 1, 128, 32),            # one KV head: 1024 rows in eight row groups
]


def _ids(s):
    return f"n{sum(s[0])}_b{len(s[0])}_h{s[1]}x{s[2]}_d{s[3]}_w{s[4]}"


def _ent_oracle(x, wl, scale):
    q = oracle.bf16_to_f64(x["q"])
    k = oracle.bf16_to_f64(x["k"])
    return oracle.window_row_entropy(q, k, x["cu_seqlens"], wl.h_q, wl.h_kv, wl.w, scale)


def _ent_oracle_row(x, wl, scale, b, h, i):
    """One row by the oracle: row i of sequence b sees keys 0 .. n-w+i, the
    same softmax as the single window row of that prefix."""
    cu = x["cu_seqlens"]
    off, n = int(cu[b]), int(cu[b + 1] - cu[b])
    p = n - wl.w + i
    g = h // wl.group
    q = oracle.bf16_to_f64(x["q"][b:b + 1, i:i + 1, h:h + 1])
    k = oracle.bf16_to_f64(x["k"][off:off + p + 1, g:g + 1])
    return oracle.window_row_entropy(q, k, [0, p + 1], 1, 1, 1, scale)[0, 0, 0]


def _run(x, scale):
    q, k = dev_bf16(x["q"]), dev_bf16(x["k"])
    return kv.window_score_entropy(q, k, x["cu_seqlens"], scale=scale, return_lse=True)


@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
def test_row_entropy_matches_oracle(shape):
    lens, h_q, h_kv, d, w = shape
    wl = synth.small("ent", 300 + sum(lens), lens, h_q, h_kv, d, w, hubs=min(3, min(lens) - w))
    x = synth.layer_inputs(wl, parts=("q", "k"))
    scale = scale_of(d)
    log(f"window_score_entropy {shape}")
    score, lse, ent, mean = _run(x, scale)
    want = _ent_oracle(x, wl, scale)
    assert_close(host(ent), want, rtol=E_RTOL, atol=E_ATOL, what="row entropy")
    assert_close(host(mean), oracle.mean_row_entropy(want), rtol=E_RTOL, atol=E_ATOL, what="mean entropy")
    # the score and normalisers are those of the plain call
    ora_s, ora_l = score_oracle(x, wl, scale)
    assert_close(host(score), ora_s, what="score")
    plain, plain_lse = kv.window_score(dev_bf16(x["q"]), dev_bf16(x["k"]), x["cu_seqlens"], scale=scale,
                                       return_lse=True)
    assert_close(host(score), host(plain), rtol=1e-6, atol=1e-9, what="score vs plain call")
    assert np.array_equal(host(lse), host(plain_lse))
    # bit-identical on a second run
    _, _, ent2, mean2 = _run(x, scale)
    assert np.array_equal(host(ent2), host(ent)) and np.array_equal(host(mean2), host(mean))


def test_row_entropy_uniform_rows_closed_form():
    """Zero queries: row i is uniform over its n-w+i+1 visible keys, so its
    entropy is ln(n-w+i+1)."""
    lens, h_q, h_kv, d, w = (1500, 700), 8, 2, 128, 16
    wl = synth.small("ent0", 77, lens, h_q, h_kv, d, w, hubs=3)
    x = synth.layer_inputs(wl, parts=("q", "k"))
    x["q"] = np.zeros_like(x["q"])
    log("window_score_entropy zero queries")
    _, _, ent, mean = _run(x, scale_of(d))
    for b, n in enumerate(lens):
        want = np.log(n - w + np.arange(w) + 1.0)
        assert_close(host(ent)[b], np.broadcast_to(want, (h_q, w)), rtol=E_RTOL, atol=E_ATOL, what="uniform")
        assert_close(host(mean)[b], want.mean(), rtol=E_RTOL, atol=E_ATOL, what="uniform mean")


def test_row_entropy_large_logits():
    """Strong hubs (scale 1, hub strength 30): rows concentrate on a few keys
    and some entropies are near zero, where only the absolute bound holds.
    Logits here reach ~1e3 in log2 units, whose fp32 spacing is ~1e-4, and
    the two passes round their dot products in different orders, so the
    absolute bound is 2e-3 (a few ulps of the largest logit, times ln2)."""
    lens, h_q, h_kv, d, w = (3000,), 8, 2, 128, 8
    wl = synth.small("entbig", 9, lens, h_q, h_kv, d, w, hubs=5, alpha=30.0)
    x = synth.layer_inputs(wl, parts=("q", "k"))
    _, _, ent, _ = _run(x, 1.0)
    want = _ent_oracle(x, wl, 1.0)
    log(f"smallest oracle row entropy {want.min():.3g}")
    assert_close(host(ent), want, rtol=E_RTOL, atol=2e-3, what="row entropy, large logits")


@pytest.mark.parametrize("name", ["n32k_gqa32x8_d128", "n128k_gqa32x8_d128", "ragged8_4k_32k",
                                  "structkv16_n64k"])
def test_row_entropy_workloads_sampled(name):
    """Full-size workloads in the launch configuration of the benchmark:
    sampled rows against the oracle one by one; every row within
    [0, ln(visible keys)]; the mean is the mean of the rows."""
    wl = synth.WORKLOADS[name]
    x = synth.layer_inputs(wl, layer=wl.layers - 1, parts=("q", "k"))
    scale = scale_of(wl.d)
    log(f"window_score_entropy workload {name}")
    _, _, ent, mean = _run(x, scale)
    e = host(ent).astype(np.float64)
    m = host(mean).astype(np.float64)
    cu = x["cu_seqlens"]
    rng = np.random.default_rng(5)
    for b in range(len(cu) - 1):
        n = int(cu[b + 1] - cu[b])
        cap = np.log(n - wl.w + np.arange(wl.w) + 1.0)
        assert np.all(e[b] >= -E_ATOL) and np.all(e[b] <= cap[None, :] + E_ATOL)
        np.testing.assert_allclose(m[b], e[b].mean(), rtol=1e-6)
    picks = [(int(rng.integers(len(cu) - 1)), int(rng.integers(wl.h_q)), int(rng.integers(wl.w)))
             for _ in range(6)]
    picks += [(0, 0, wl.w - 1), (len(cu) - 2, wl.h_q - 1, 0)]
    for b, h, i in picks:
        want = _ent_oracle_row(x, wl, scale, b, h, i)
        got = e[b, h, i]
        assert abs(got - want) <= E_ATOL + E_RTOL * abs(want), (name, b, h, i, got, want)
