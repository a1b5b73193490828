"""Two-stage Token-Selective Propagation prefill on a random-weight
Llama-3-8B-shaped stack: timing context for the selection path.

FastKV summary page, sections 2A-2B: the layers up to the TSP layer see the
whole context; at the TSP layer the window's attention scores the tokens,
and only the selected subset (with the window) goes on through the later
layers, while every layer keeps its own compressed KV cache.  The pages
quote the end-to-end effect as a time-to-first-token gain (FastKV
abstract: 2.00x over HeadKV; summary page section 4: up to 1.82x over the
full context); this driver measures the same kind of ratio on one MI355X.

What runs where:
  * the model's own work (RMSNorm, projections, rotary embedding, causal
    attention, SwiGLU MLP) is plain PyTorch on the GPU (hipBLASLt GEMMs,
    the ROCm flash-attention kernel), with random weights: the numbers are
    timings only, nothing is evaluated for accuracy;
  * every selection step is libkvsel: the window score takes the
    normalisers the layer's flash attention already computed
    (kvsel_window_score_lse, one pass over K), then the head sum, both
    budgets' top-k and the gathers.

Stage 1 runs layers 0 .. tsp_layer on all N tokens; each layer's K/V cache
is compressed to its own KV budget.  At tsp_layer the propagated set (TSP
budget plus window) is selected, and its hidden rows continue through the
remaining layers with their original positions for the rotary embedding.
"""
from __future__ import annotations

import argparse
import json
import math
import sys
import time
from dataclasses import dataclass
from typing import List, Optional

from . import kvsel


@dataclass
class Shape:
    layers: int = 32
    hidden: int = 4096
    heads: int = 32
    kv_heads: int = 8
    head_dim: int = 128
    mlp: int = 14336
    rope_theta: float = 500000.0
    eps: float = 1e-5


def llama3_8b() -> Shape:
    return Shape()


class Layer:
    """One decoder layer's random bf16 weights."""

    def __init__(self, s: Shape, gen, device):
        import torch
        q_out = s.heads * s.head_dim
        kv_out = s.kv_heads * s.head_dim

        def w(rows, cols):
            return (torch.randn(rows, cols, generator=gen, device=device, dtype=torch.float32)
                    * (1.0 / math.sqrt(rows))).to(torch.bfloat16)

        self.ln1 = torch.ones(s.hidden, device=device, dtype=torch.bfloat16)
        self.ln2 = torch.ones(s.hidden, device=device, dtype=torch.bfloat16)
        self.wqkv = w(s.hidden, q_out + 2 * kv_out)
        self.wo = w(q_out, s.hidden)
        self.wgu = w(s.hidden, 2 * s.mlp)
        self.wd = w(s.mlp, s.hidden)


def _rms(x, wgt, eps):
    import torch
    xf = x.float()
    return (xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + eps)).to(x.dtype) * wgt


def _rope(x, pos, theta):
    """Rotary embedding of x [N, heads, d] at integer positions pos [N]."""
    import torch
    d = x.shape[-1]
    inv = 1.0 / (theta ** (torch.arange(0, d, 2, device=x.device, dtype=torch.float32) / d))
    ang = pos.float()[:, None] * inv[None, :]
    cos, sin = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]
    x1, x2 = x[..., : d // 2].float(), x[..., d // 2:].float()
    return torch.cat([x1 * cos - x2 * sin, x1 * sin + x2 * cos], dim=-1).to(x.dtype)


class Model:
    def __init__(self, s: Shape, seed: int = 0, device: str = "cuda:0"):
        import torch
        self.s = s
        gen = torch.Generator(device=device)
        gen.manual_seed(seed)
        self.layers = [Layer(s, gen, device) for _ in range(s.layers)]

    def qkv(self, L: Layer, x, pos):
        """Normalised input -> rotated q [N, h, d], k [N, h_kv, d], v [N, h_kv, d]."""
        s = self.s
        h = _rms(x, L.ln1, s.eps)
        qkv = h @ L.wqkv
        q_out, kv_out = s.heads * s.head_dim, s.kv_heads * s.head_dim
        q = qkv[:, :q_out].view(-1, s.heads, s.head_dim)
        k = qkv[:, q_out:q_out + kv_out].view(-1, s.kv_heads, s.head_dim)
        v = qkv[:, q_out + kv_out:].view(-1, s.kv_heads, s.head_dim).contiguous()
        return _rope(q, pos, s.rope_theta), _rope(k, pos, s.rope_theta).contiguous(), v

    def attention(self, q, k, v, want_lse: bool):
        """Causal attention over one sequence; with want_lse also each row's
        natural-log normaliser [h, N].  Every layer of both prefill paths
        (full context, and both TSP stages) runs this same flash kernel, K
        and V expanded to the query heads, so that the two paths' times
        compare like with like; the normalisers are the kernel's own."""
        import torch
        s = self.s
        g = s.heads // s.kv_heads
        qt = q.transpose(0, 1).unsqueeze(0)                      # [1, h, N, d]
        ke = k.transpose(0, 1).unsqueeze(0).repeat_interleave(g, 1)
        ve = v.transpose(0, 1).unsqueeze(0).repeat_interleave(g, 1)
        scale = float(1.0 / math.sqrt(s.head_dim))
        out, lse = torch.ops.aten._scaled_dot_product_flash_attention(qt, ke, ve, 0.0, True, False,
                                                                      scale=scale)[:2]
        return out[0].transpose(0, 1).reshape(q.shape[0], -1), (lse[0] if want_lse else None)

    def finish(self, L: Layer, x, attn):
        import torch
        s = self.s
        x = x + attn @ L.wo
        h = _rms(x, L.ln2, s.eps)
        gu = h @ L.wgu
        act = torch.nn.functional.silu(gu[:, :s.mlp]) * gu[:, s.mlp:]
        return x + act @ L.wd


@dataclass
class TspConfig:
    tsp_layer: int = 15
    window: int = 32
    kv_budget: int = 4096        # tokens kept per KV head in every stage-1 layer's cache
    tsp_rate: float = 0.10       # share of the tokens propagated past tsp_layer


def forward_full(m: Model, x):
    """All layers on all tokens (the baseline); returns the final hidden rows."""
    import torch
    pos = torch.arange(x.shape[0], device=x.device)
    for L in m.layers:
        q, k, v = m.qkv(L, x, pos)
        attn, _ = m.attention(q, k, v, want_lse=False)
        x = m.finish(L, x, attn)
    return x


def forward_tsp(m: Model, x, cfg: TspConfig, timings: Optional[dict] = None):
    """Two-stage TSP prefill of one sequence.  Returns (hidden rows of the
    propagated tokens after the last layer, their positions, the compressed
    (K, V) cache of every stage-1 layer).  With ``timings``, the time spent
    in libkvsel calls is added to timings["select_s"] (synchronising around
    them, so only for the overhead measurement)."""
    import torch
    n = x.shape[0]
    w = cfg.window
    cu = [0, n]
    pos = torch.arange(n, device=x.device)
    caches: List[tuple] = []
    k_kv = [min(cfg.kv_budget, n - w)]
    k_tsp = [int(n * cfg.tsp_rate)]

    def timed(fn):
        if timings is None:
            return fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        r = fn()
        torch.cuda.synchronize()
        timings["select_s"] = timings.get("select_s", 0.0) + time.perf_counter() - t0
        return r

    for li in range(cfg.tsp_layer + 1):
        L = m.layers[li]
        q, k, v = m.qkv(L, x, pos)
        attn, lse = m.attention(q, k, v, want_lse=True)
        q_win = q[n - w:].unsqueeze(0).contiguous()                       # [1, w, h, d]
        lse_win = lse[:, n - w:].unsqueeze(0).contiguous()                # [1, h, w]
        x_next = m.finish(L, x, attn)

        def select(li=li, q_win=q_win, k=k, v=v, lse_win=lse_win, x_next=x_next):
            score = kvsel.window_score(q_win, k, cu, lse_in=lse_win)
            if li < cfg.tsp_layer:
                idx_kv = kvsel.topk(score, cu, w, k_kv)
                return kvsel.gather_multi(cu, w, [(k, idx_kv, k_kv), (v, idx_kv, k_kv)]), None, None
            group = m.s.heads // m.s.kv_heads
            _, tok, _ = kvsel.accumulate_stats(score, cu, w, group, want_stats=False)
            idx_kv, idx_tsp = kvsel.topk2(score, tok, cu, w, k_kv, k_tsp)
            kc, vc, hc = kvsel.gather_multi(cu, w, [(k, idx_kv, k_kv), (v, idx_kv, k_kv),
                                                    (x_next, idx_tsp, k_tsp)])
            return (kc, vc), idx_tsp, hc

        (kc_vc, idx_tsp, hc) = timed(select)
        caches.append(kc_vc)
        x = x_next
    # stage 2: the propagated rows at their original positions
    x = hc
    pos = idx_tsp.long()
    for L in m.layers[cfg.tsp_layer + 1:]:
        q, k, v = m.qkv(L, x, pos)
        attn, _ = m.attention(q, k, v, want_lse=False)
        x = m.finish(L, x, attn)
    return x, pos, caches


def _time(fn, reps: int) -> float:
    import torch
    ts = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        ts.append(time.perf_counter() - t0)
    ts.sort()
    return ts[len(ts) // 2]


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--tokens", type=int, default=131072)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--tsp-layer", type=int, default=15)
    ap.add_argument("--window", type=int, default=32)
    ap.add_argument("--kv-budget", type=int, default=4096)
    ap.add_argument("--tsp-rate", type=float, default=0.10)
    ap.add_argument("--reps", type=int, default=3)
    a = ap.parse_args(argv)
    import torch
    assert torch.cuda.is_available(), "the prefill driver needs a GPU"
    kvsel.library()
    s = Shape(layers=a.layers)
    cfg = TspConfig(tsp_layer=a.tsp_layer, window=a.window, kv_budget=a.kv_budget, tsp_rate=a.tsp_rate)
    m = Model(s, seed=0)
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(1)
    x = (torch.randn(a.tokens, s.hidden, generator=gen, device="cuda:0") * 0.5).to(torch.bfloat16)
    with torch.no_grad():
        forward_tsp(m, x, cfg)                                  # warm-up
        forward_full(m, x)
        t_full = _time(lambda: forward_full(m, x), a.reps)
        t_tsp = _time(lambda: forward_tsp(m, x, cfg), a.reps)
        tm = {}
        forward_tsp(m, x, cfg, timings=tm)
    out = {"workload": "llama3_8b_shape_random_weights", "tokens": a.tokens, "layers": a.layers,
           "tsp_layer": a.tsp_layer, "window": a.window, "kv_budget": a.kv_budget, "tsp_rate": a.tsp_rate,
           "propagated_tokens": int(a.tokens * a.tsp_rate) + a.window,
           "ttft_full_ms": t_full * 1e3, "ttft_tsp_ms": t_tsp * 1e3, "speedup": t_full / t_tsp,
           "selection_ms": tm.get("select_s", 0.0) * 1e3,
           "selection_share": tm.get("select_s", 0.0) / t_tsp,
           "attention": "one flash kernel (aten _scaled_dot_product_flash_attention, K/V expanded to the "
                        "query heads) in every layer of both paths"}
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
