"""Window-row attention entropy on the GPU against the oracle.

Tolerance, per row: tolerances.row_entropy_bound, derived from the kernel's
arithmetic -- the fp32 logits' error (2 (d + 2) u scale sum_t |q_t k_t| per
key) propagated through dH/dx_k = -P_k (x_k - xbar), plus the fp32
accumulation of the row's sums (512 u (1 + 2H)).  The per-sequence mean is
held to the mean of its rows' bounds."""

import numpy as np
import pytest

import oracle
import token_selection_tsp_amd as kv
from token_selection_tsp_amd import synth
from gpu_util import assert_close, check_rows, dev_bf16, host, log, scale_of, score_oracle

pytestmark = pytest.mark.gpu

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
    check_rows(x, wl, scale, ent=ent, mean=mean, ora_ent=want, what="row entropy")
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
    want = np.stack([np.broadcast_to(np.log(n - w + np.arange(w) + 1.0), (h_q, w)) for n in lens])
    # the logits are exactly 0, so only the arithmetic part of the bound applies
    check_rows(x, wl, scale_of(d), ent=ent, mean=mean, ora_ent=want, what="uniform rows")


def test_row_entropy_large_logits():
    """Strong hubs (scale 1, hub strength 30): rows concentrate on a few keys
    and some entropies are near zero.  Logits reach ~1e3, so the fp32
    logits' own error dominates the per-row bound there."""
    lens, h_q, h_kv, d, w = (3000,), 8, 2, 128, 8
    wl = synth.small("entbig", 9, lens, h_q, h_kv, d, w, hubs=5, alpha=30.0)
    x = synth.layer_inputs(wl, parts=("q", "k"))
    _, _, ent, mean = _run(x, 1.0)
    want = _ent_oracle(x, wl, 1.0)
    eb, _ = check_rows(x, wl, 1.0, ent=ent, mean=mean, ora_ent=want, what="row entropy, large logits")
    log(f"smallest oracle row entropy {want.min():.3g}; bounds {eb.min():.2e} .. {eb.max():.2e}")


@pytest.mark.parametrize("name", ["n32k_gqa32x8_d128", "n128k_gqa32x8_d128", "ragged8_4k_32k",
                                  "structkv16_n64k"])
def test_row_entropy_workloads_every_row(name):
    """Full-size workloads in the launch configuration of the benchmark
    (the 16-layer workload at its last layer; its pivot layer is compared
    in the StructKV pipeline test): every window row against the oracle,
    within its bound."""
    wl = synth.WORKLOADS[name]
    x = synth.layer_inputs(wl, layer=wl.layers - 1, parts=("q", "k"))
    scale = scale_of(wl.d)
    log(f"window_score_entropy workload {name}")
    _, _, ent, mean = _run(x, scale)
    log(f"window_score_entropy workload {name}: oracle")
    want = _ent_oracle(x, wl, scale)
    log(f"{name}: worst |err| {np.max(np.abs(host(ent) - want)):.2e}")
    eb, _ = check_rows(x, wl, scale, ent=ent, mean=mean, ora_ent=want, what=f"row entropy {name}")
    log(f"{name}: bounds {eb.min():.2e} .. {eb.max():.2e}")
