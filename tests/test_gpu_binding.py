"""The binding's checks of caller-supplied buffers: a wrong shape, dtype or
device raises before anything is launched (the sentinel contents of the
buffer are untouched and the stream stays usable), and a right one works."""
import numpy as np
import pytest

import token_selection_tsp_amd as kv
from token_selection_tsp_amd import synth
from gpu_util import dev_bf16, host, log, scale_of

pytestmark = pytest.mark.gpu


def _inputs():
    wl = synth.small("bind", 12, (700, 300), 8, 2, 64, 8, hidden=64, hubs=3)
    x = synth.layer_inputs(wl, parts=("q", "k", "v", "hidden"))
    return wl, x, [dev_bf16(x[p]) for p in ("q", "k", "v", "hidden")]


def _untouched(t, fill):
    import torch
    torch.cuda.synchronize()
    assert bool((t == fill).all()), "a rejected buffer was written"


def test_wrong_buffers_raise_before_launch():
    import torch
    wl, x, (q, k, v, h) = _inputs()
    cu = x["cu_seqlens"]
    T = int(cu[-1])
    scale = scale_of(wl.d)
    log("binding: score out")
    small = torch.full((wl.h_kv, T - 1), 7.0, device="cuda")
    with pytest.raises(ValueError):
        kv.window_score(q, k, cu, scale=scale, out=small)
    _untouched(small, 7.0)
    with pytest.raises(TypeError):
        kv.window_score(q, k, cu, scale=scale, out=torch.empty((wl.h_kv, T)))          # host tensor
    with pytest.raises(ValueError):
        kv.window_score(q, k, cu, scale=scale, lse_in=torch.zeros((2, wl.h_q, wl.w - 1), device="cuda"))
    score = kv.window_score(q, k, cu, scale=scale, out=torch.empty((wl.h_kv, T), device="cuda"))
    log("binding: accumulate buffers")
    bad = torch.full((wl.h_kv, T // 2), 5.0, device="cuda")
    with pytest.raises(ValueError):
        kv.accumulate_stats(score, cu, wl.w, wl.group, c_out=bad)
    with pytest.raises(ValueError):
        kv.accumulate_stats(score, cu, wl.w, wl.group, c_in=bad)
    _untouched(bad, 5.0)
    _, tok, _ = kv.accumulate_stats(score, cu, wl.w, wl.group)
    log("binding: top-k outputs")
    k_kv, k_ts = [100, 50], [200, 20]
    L = kv.selected_length(cu, k_kv, wl.w)
    short = torch.full((wl.h_kv, L - 1), -3, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        kv.topk(score, cu, wl.w, k_kv, out=short)
    with pytest.raises(ValueError):
        kv.topk2(score, tok, cu, wl.w, k_kv, k_ts, out_b=short)
    with pytest.raises(TypeError):
        kv.topk(score, cu, wl.w, k_kv, out=torch.empty((wl.h_kv, L), dtype=torch.int64, device="cuda"))
    _untouched(short, -3)
    ikv, its = kv.topk2(score, tok, cu, wl.w, k_kv, k_ts)
    log("binding: gather outputs")
    dst = torch.full((L - 1, wl.h_kv, wl.d), 1.5, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        kv.gather(k, cu, ikv, wl.w, k_kv, out=dst)
    with pytest.raises(ValueError):
        kv.gather_multi(cu, wl.w, [(k, ikv, k_kv), (v, ikv, k_kv)], outs=[dst, dst])
    with pytest.raises(ValueError):
        kv.gather_multi(cu, wl.w, [(k, ikv, k_kv), (v, ikv, k_kv)], outs=[dst])
    with pytest.raises(TypeError):
        kv.gather(k, cu, ikv, wl.w, k_kv, out=torch.empty((L, wl.h_kv, wl.d), dtype=torch.float16, device="cuda"))
    _untouched(dst, 1.5)
    good = torch.empty((L, wl.h_kv, wl.d), dtype=torch.bfloat16, device="cuda")
    got = kv.gather(k, cu, ikv, wl.w, k_kv, out=good)
    assert got.data_ptr() == good.data_ptr()
    assert np.array_equal(host(got), host(kv.gather(k, cu, ikv, wl.w, k_kv)))
