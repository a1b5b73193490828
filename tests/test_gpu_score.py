"""Window score on the GPU against the oracle (element by element)."""
import numpy as np
import pytest

import oracle
import token_selection_tsp_amd as kv
from token_selection_tsp_amd import synth
from gpu_util import assert_close, check_rows, dev_bf16, host, log, scale_of, score_oracle

pytestmark = pytest.mark.gpu

# (lengths, h_q, h_kv, d, w): several 1024-key chunks and 32-key tiles,
# ragged tails, GQA groups 1..32 (3 included), windows 1..33, row groups > 128.
SHAPES = [
    ((1000,), 8, 2, 64, 8),
    ((37,), 4, 4, 128, 1),
    ((300, 33, 129), 16, 2, 128, 5),
    ((2500,), 32, 8, 128, 32),
    ((700, 64), 8, 1, 64, 33),
    ((2065,), 12, 4, 64, 7),
    ((33,), 2, 2, 64, 33),
    ((5000, 1), 32, 8, 128, 1),
    ((1, 2, 3, 4, 5, 1030), 4, 2, 128, 1),
    ((5000,), 32, 1, 128, 32),            # one KV head: 1024 rows, eight row groups
    ((3000, 777), 16, 1, 64, 20),         # G = 16: 320 rows, a ragged last row group
]


def _run(wl, x, scale):
    q = dev_bf16(x["q"])
    k = dev_bf16(x["k"])
    return kv.window_score(q, k, x["cu_seqlens"], scale=scale, return_lse=True)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"n{sum(s[0])}_b{len(s[0])}_h{s[1]}x{s[2]}_d{s[3]}_w{s[4]}")
def test_window_score_matches_oracle(shape):
    lens, h_q, h_kv, d, w = shape
    wl = synth.small("score", 100 + sum(lens), lens, h_q, h_kv, d, w, hubs=min(3, min(lens) - w))
    x = synth.layer_inputs(wl, parts=("q", "k"))
    scale = scale_of(d)
    log(f"window_score {shape}")
    score, lse = _run(wl, x, scale)
    ora_s, ora_l = score_oracle(x, wl, scale)
    assert_close(host(score), ora_s, what="score")
    check_rows(x, wl, scale, lse=lse, ora_lse=ora_l, what="lse")
    # total attention mass per (sequence, KV head) is w * G
    cu = x["cu_seqlens"]
    s = host(score).astype(np.float64)
    for b in range(len(lens)):
        tot = s[:, cu[b]:cu[b + 1]].sum(axis=1)
        np.testing.assert_allclose(tot, w * (h_q // h_kv), rtol=1e-5)
    # bit-identical on a second run
    score2, lse2 = _run(wl, x, scale)
    assert np.array_equal(host(score2), host(score)) and np.array_equal(host(lse2), host(lse))


def test_window_score_large_logits():
    """Logits far from zero (scale 1, keys and queries with norm ~ 40) still
    give a normalised distribution: the online max keeps 2^x finite."""
    lens, h_q, h_kv, d, w = (3000,), 8, 2, 128, 8
    wl = synth.small("big", 9, lens, h_q, h_kv, d, w, hubs=5, alpha=30.0)
    x = synth.layer_inputs(wl, parts=("q", "k"))
    score, lse = _run(wl, x, 1.0)
    ora_s, ora_l = score_oracle(x, wl, 1.0)
    assert np.all(np.isfinite(host(score)))
    assert_close(host(score), ora_s, what="score")
    check_rows(x, wl, 1.0, lse=lse, ora_lse=ora_l, what="lse, large logits")


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_window_score_workloads(name):
    wl = synth.WORKLOADS[name]
    layers = [0, wl.layers // 2, wl.layers - 1] if wl.layers > 1 else [0]
    for layer in layers:
        log(f"window_score workload {name} layer {layer}")
        x = synth.layer_inputs(wl, layer=layer, parts=("q", "k"))
        scale = scale_of(wl.d)
        score, lse = _run(wl, x, scale)
        ora_s, ora_l = score_oracle(x, wl, scale)
        assert_close(host(score), ora_s, what=f"{name} score")
        check_rows(x, wl, scale, lse=lse, ora_lse=ora_l, what=f"{name} layer {layer}")


def _dev_f32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


@pytest.mark.parametrize("shape", [SHAPES[0], SHAPES[2], SHAPES[3], SHAPES[4], SHAPES[8]],
                         ids=lambda s: f"n{sum(s[0])}_b{len(s[0])}_h{s[1]}x{s[2]}_d{s[3]}_w{s[4]}")
def test_window_score_with_given_normalisers(shape):
    # with the oracle's normalisers (as the layer's own attention would give
    # them) the one-pass score matches the oracle's score
    lens, h_q, h_kv, d, w = shape
    wl = synth.small("score", 100 + sum(lens), lens, h_q, h_kv, d, w, hubs=min(3, min(lens) - w))
    x = synth.layer_inputs(wl, parts=("q", "k"))
    scale = scale_of(d)
    ora_s, ora_l = score_oracle(x, wl, scale)
    log(f"window_score lse_in {shape}")
    got = kv.window_score(dev_bf16(x["q"]), dev_bf16(x["k"]), x["cu_seqlens"], scale=scale,
                          lse_in=_dev_f32(ora_l))
    assert_close(host(got), ora_s, what="score from given lse")


@pytest.mark.parametrize("name", ["n32k_gqa32x8_d128", "n128k_gqa32x8_d128", "ragged8_4k_32k"])
def test_window_score_with_own_normalisers(name):
    # fed the normalisers the two-pass call returns, the one-pass call gives
    # the two-pass scores within the score tolerance, and the oracle's
    wl = synth.WORKLOADS[name]
    x = synth.layer_inputs(wl, parts=("q", "k"))
    scale = scale_of(wl.d)
    q, k = dev_bf16(x["q"]), dev_bf16(x["k"])
    log(f"window_score lse_in workload {name}")
    score, lse = kv.window_score(q, k, x["cu_seqlens"], scale=scale, return_lse=True)
    one = kv.window_score(q, k, x["cu_seqlens"], scale=scale, lse_in=lse)
    assert_close(host(one), host(score), what=f"{name} one-pass vs two-pass")
    ora_s, _ = score_oracle(x, wl, scale)
    assert_close(host(one), ora_s, what=f"{name} one-pass vs oracle")


def test_window_score_long_d64():
    """Head dim 64 at 64K keys (4 KB tiles, the d=64 load plan, full-size
    chunks), two sequences, whole oracle comparison of scores, normalisers
    and row entropies."""
    lens, h_q, h_kv, d, w = (65536, 3000), 16, 4, 64, 16
    wl = synth.small("d64long", 64, lens, h_q, h_kv, d, w, hubs=40, alpha=2.0)
    x = synth.layer_inputs(wl, parts=("q", "k"))
    scale = scale_of(d)
    log("window_score d=64 at 64K")
    score, lse = _run(wl, x, scale)
    ora_s, ora_l = score_oracle(x, wl, scale)
    assert_close(host(score), ora_s, what="d64 score")
    _, ent, mean = kv.window_score_entropy(dev_bf16(x["q"]), dev_bf16(x["k"]), x["cu_seqlens"], scale=scale)
    want = oracle.window_row_entropy(oracle.bf16_to_f64(x["q"]), oracle.bf16_to_f64(x["k"]), x["cu_seqlens"],
                                     h_q, h_kv, w, scale)
    check_rows(x, wl, scale, lse=lse, ora_lse=ora_l, ent=ent, mean=mean, ora_ent=want, what="d64")
