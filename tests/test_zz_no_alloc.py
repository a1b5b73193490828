"""kvsel_window_score_noalloc through the C ABI against kvsel_window_score:
the same scores and normalisers bit for bit, on two calls in a row (the
second on a smaller input, so it runs over the first call's leftovers in
the shared scratch), then again after a call that the fixed scratch
cannot hold has been refused.  Both are also within the score acceptance
rule of the oracle."""
import ctypes

import numpy as np
import pytest

import token_selection_tsp_amd as kv
from token_selection_tsp_amd import kvsel, synth
from gpu_util import assert_close, check_rows, dev_bf16, host, log, scale_of, score_oracle

pytestmark = pytest.mark.gpu


def _abi_noalloc(q, k, cu, scale, score, lse):
    """Direct C-ABI call (no binding logic, no allocation)."""
    import torch
    lib = kvsel.library()
    arr = np.ascontiguousarray(np.asarray(cu, dtype=np.int32))
    v = kvsel.Varlen(len(arr) - 1, arr.ctypes.data)
    B, w, h_q, d = q.shape
    h_kv = k.shape[1]
    st = lib.kvsel_window_score_noalloc(ctypes.byref(v), q.data_ptr(), k.data_ptr(), h_q, h_kv, d, w,
                                        float(np.float32(scale)), score.data_ptr(),
                                        None if lse is None else lse.data_ptr(),
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def _case(name, lens, h_q, h_kv, d, w, seed):
    wl = synth.small(name, seed, lens, h_q, h_kv, d, w, hubs=min(5, min(lens) - w), alpha=2.0)
    return wl, synth.layer_inputs(wl, parts=("q", "k"))


def test_noalloc_matches_window_score_twice():
    import torch
    cases = [_case("noalloc_big", (40000, 9000, 20000), 32, 8, 128, 32, 71),     # first call: larger
             _case("noalloc_small", (3000, 517), 8, 2, 64, 8, 72)]               # second call: smaller
    for wl, x in cases:
        cu = x["cu_seqlens"]
        T, B = int(cu[-1]), len(cu) - 1
        scale = scale_of(wl.d)
        q, k = dev_bf16(x["q"]), dev_bf16(x["k"])
        log(f"noalloc {wl.name}: T={T}")
        score = torch.full((wl.h_kv, T), -1.0, device="cuda")
        lse = torch.full((B, wl.h_q, wl.w), -1.0, device="cuda")
        assert _abi_noalloc(q, k, cu, scale, score, lse) == kvsel.KVSEL_OK
        ref, ref_lse = kv.window_score(q, k, cu, scale=scale, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(score, ref), f"{wl.name}: score differs from kvsel_window_score"
        assert torch.equal(lse, ref_lse), f"{wl.name}: lse differs from kvsel_window_score"
        ora_s, ora_l = score_oracle(x, wl, scale)
        assert_close(host(score), ora_s, what=f"{wl.name} score vs oracle")
        check_rows(x, wl, scale, lse=lse, ora_lse=ora_l, what=f"{wl.name}")
        # the binding's form of the same call, without lse
        out = torch.empty((wl.h_kv, T), device="cuda")
        assert kv.window_score_noalloc(q, k, cu, out, scale=scale) is out
        torch.cuda.synchronize()
        assert torch.equal(out, ref)


def test_noalloc_refuses_oversize_then_still_works():
    import torch
    # 600000 keys at 64 KV heads: 5 MiB of partials (the scratch holds 4);
    # real buffers of the full size, so nothing could be read out of bounds
    n, h = 600000, 64
    q = torch.zeros((1, 1, h, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((n, h, 64), dtype=torch.bfloat16, device="cuda")
    out = torch.full((h, n), 3.0, device="cuda")
    log("noalloc oversize: refused")
    assert _abi_noalloc(q, k, [0, n], 0.125, out, None) == kvsel.KVSEL_EWORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
    del q, k, out
    wl, x = _case("noalloc_after", (5000,), 16, 4, 128, 16, 73)
    cu = x["cu_seqlens"]
    q, k = dev_bf16(x["q"]), dev_bf16(x["k"])
    out = torch.empty((wl.h_kv, int(cu[-1])), device="cuda")
    assert _abi_noalloc(q, k, cu, scale_of(wl.d), out, None) == kvsel.KVSEL_OK
    ref = kv.window_score(q, k, cu, scale=scale_of(wl.d))
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
