"""The two-stage TSP prefill driver at a small Llama-like shape: the
normalisers the layer's flash attention returns for the window rows agree
with the library's own two-pass normalisers; the one-pass score built on
them matches the oracle; the propagated set is the oracle's selection up to
near-ties; the second stage runs on the propagated rows at their original
positions."""
import types

import numpy as np
import pytest

import oracle
import token_selection_tsp_amd as kv
from token_selection_tsp_amd import prefill
from gpu_util import assert_close, check_rows, host, log, selection_agrees

pytestmark = pytest.mark.gpu


def test_prefill_tsp_small():
    import torch
    s = prefill.Shape(layers=4, hidden=512, heads=8, kv_heads=2, head_dim=64, mlp=1024)
    cfg = prefill.TspConfig(tsp_layer=1, window=16, kv_budget=256, tsp_rate=0.1)
    n = 4096
    m = prefill.Model(s, seed=3)
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(4)
    x = (torch.randn(n, s.hidden, generator=gen, device="cuda:0") * 0.5).to(torch.bfloat16)
    pos = torch.arange(n, device="cuda:0")
    cu = np.array([0, n], dtype=np.int32)
    w = cfg.window
    with torch.no_grad():
        h = x
        for li in range(cfg.tsp_layer + 1):
            L = m.layers[li]
            q, k, v = m.qkv(L, h, pos)
            attn, lse = m.attention(q, k, v, want_lse=True)
            if li == cfg.tsp_layer:
                break
            h = m.finish(L, h, attn)
        q_win = q[n - w:].unsqueeze(0).contiguous()
        lse_win = lse[:, n - w:].unsqueeze(0).contiguous()
        log("prefill: flash normalisers against the two-pass ones")
        score2, lse2 = kv.window_score(q_win, k, cu, return_lse=True)
        score1 = kv.window_score(q_win, k, cu, lse_in=lse_win)
        scale = float(np.float32(1.0 / np.sqrt(s.head_dim)))
        qb = host(q_win).view(np.uint16)
        kb = host(k).view(np.uint16)
        ora_s, ora_l = oracle.window_score(oracle.bf16_to_f64(qb), oracle.bf16_to_f64(kb), cu, s.heads,
                                           s.kv_heads, w, scale)
        # both normalisers come from bf16 products accumulated in fp32: each
        # within the derived bound of the oracle's, so within twice of each other
        xs = {"q": qb, "k": kb, "cu_seqlens": cu}
        shape = types.SimpleNamespace(h_q=s.heads, h_kv=s.kv_heads, w=w)
        check_rows(xs, shape, scale, lse=lse_win, ora_lse=ora_l, what="flash lse vs oracle")
        check_rows(xs, shape, scale, lse=lse2, ora_lse=ora_l, what="two-pass lse vs oracle")
        check_rows(xs, shape, scale, lse=lse_win, ora_lse=host(lse2), what="flash lse vs two-pass", factor=2.0)
        assert_close(host(score1), ora_s, what="one-pass score vs oracle")
        # the driver's own pass gives the same propagated set as the oracle's
        # selection on the oracle's scores, up to near-ties at the cut
        out, p, caches = prefill.forward_tsp(m, x, cfg)
        k_tsp = int(n * cfg.tsp_rate)
        want = oracle.select_rows(oracle.head_sum(ora_s)[None, :], cu, w, [k_tsp])[0]
        selection_agrees(host(p).astype(np.int64), want, oracle.head_sum(ora_s), n, w, k_tsp)
        assert out.shape == (k_tsp + w, s.hidden)
        assert bool(torch.isfinite(out.float()).all())
        assert len(caches) == cfg.tsp_layer + 1
        for kc, vc in caches:
            assert kc.shape == (cfg.kv_budget + w, s.kv_heads, s.head_dim) and vc.shape == kc.shape
        full = prefill.forward_full(m, x)
        assert full.shape == (n, s.hidden) and bool(torch.isfinite(full.float()).all())
