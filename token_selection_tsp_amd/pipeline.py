"""The whole selection pass of one layer, chained from the four library calls.

FastKV (summary page, sections 2A-2B): at the TSP layer the window's
attention scores the tokens; each KV head keeps its own top tokens for the
cache (KV retention budget) and the head-summed score picks the tokens that
propagate (TSP budget); both keep the window.  StructKV (summary page,
sections 2A-2C): the same with the score accumulated over layers up to a
pivot layer found from per-layer entropy, and decoupled budgets R_KV and
R_struct.

Only argument plumbing lives here; every step runs in libkvsel's kernels.
"""
from __future__ import annotations

from typing import List, NamedTuple, Sequence

from . import kvsel


class Selection(NamedTuple):
    score: object      # fp32 [h_kv, T] this layer's window score
    acc: object        # fp32 [h_kv, T] accumulated score the budgets select on
    tok: object        # fp32 [T] head sum of `acc`
    stats: object      # fp32 [B, 3] entropy, sparsity, variance of this layer
    idx_kv: object     # int32 [h_kv, L_kv] kept positions per KV head (cache)
    idx_tsp: object    # int32 [L_tsp] propagated positions per sequence
    k_c: object        # [L_kv, h_kv, d] compressed keys
    v_c: object        # [L_kv, h_kv, d] compressed values
    h_c: object        # [L_tsp, D] shortened hidden sequence


def score_layer(q_win, k, cu_seqlens, scale=None, c_in=None, c_out=None, lse_in=None):
    """Window score of one layer, the running accumulation, its head sum and
    the layer's stats.  Returns (score, acc, tok, stats).  ``lse_in``: the
    window rows' normalisers from the layer's own attention, if available
    (one pass over K instead of two)."""
    w = q_win.shape[1]
    group = q_win.shape[2] // k.shape[1]
    if lse_in is None:   # one call: the accumulation and statistics ride on the score's second pass
        score, acc, tok, stats = kvsel.window_score_stats(q_win, k, cu_seqlens, scale=scale, c_in=c_in,
                                                          c_out=c_out)
    else:
        score = kvsel.window_score(q_win, k, cu_seqlens, scale=scale, lse_in=lse_in)
        acc, tok, stats = kvsel.accumulate_stats(score, cu_seqlens, w, group, c_in=c_in, c_out=c_out)
    return score, (acc if acc is not None else score), tok, stats


def select_and_gather(acc, tok, k, v, hidden, cu_seqlens, w: int, k_kv: Sequence[int],
                      k_tsp: Sequence[int]):
    """Both budgets' top-k plus window and the three gathers."""
    idx_kv, idx_tsp = kvsel.topk2(acc, tok, cu_seqlens, w, k_kv, k_tsp)
    jobs = [(t, i, kk) for t, i, kk in ((k, idx_kv, k_kv), (v, idx_kv, k_kv), (hidden, idx_tsp, k_tsp))
            if t is not None]
    outs = iter(kvsel.gather_multi(cu_seqlens, w, jobs)) if jobs else iter(())
    k_c = next(outs) if k is not None else None
    v_c = next(outs) if v is not None else None
    h_c = next(outs) if hidden is not None else None
    return idx_kv, idx_tsp, k_c, v_c, h_c


def fastkv_layer(q_win, k, v, hidden, cu_seqlens, k_kv, k_tsp, scale=None, lse_in=None) -> Selection:
    """Token-Selective Propagation at one layer (FastKV)."""
    score, acc, tok, stats = score_layer(q_win, k, cu_seqlens, scale=scale, lse_in=lse_in)
    w = q_win.shape[1]
    sel = select_and_gather(acc, tok, k, v, hidden, cu_seqlens, w, k_kv, k_tsp)
    return Selection(score, acc, tok, stats, *sel)


class StructKVState:
    """Layer-by-layer StructKV accumulation: keeps the accumulated score and
    its head sum after every layer so the budgets can select at the pivot.

    With ``row_entropy`` each layer also records the mean attention entropy
    of its window rows (kvsel_window_score_entropy), the row-level reading
    of the entropy the pivot search watches (StructKV summary page, section
    2B)."""

    def __init__(self, row_entropy: bool = False):
        self.row_entropy = row_entropy
        self.acc: List[object] = []
        self.tok: List[object] = []
        self.stats: List[object] = []
        self.mean_row_ent: List[object] = []

    def add_layer(self, q_win, k, cu_seqlens, scale=None):
        c_in = self.acc[-1] if self.acc else None
        w = q_win.shape[1]
        group = q_win.shape[2] // k.shape[1]
        if self.row_entropy:
            score, _, mean = kvsel.window_score_entropy(q_win, k, cu_seqlens, scale=scale)
            self.mean_row_ent.append(mean)
            acc, tok, stats = kvsel.accumulate_stats(score, cu_seqlens, w, group, c_in=c_in)
        else:
            score, acc, tok, stats = kvsel.window_score_stats(q_win, k, cu_seqlens, scale=scale, c_in=c_in)
        if c_in is None:            # first layer: keep its own copy as the running sum
            acc = score
        self.acc.append(acc)
        self.tok.append(tok)
        self.stats.append(stats)
        return score

    def pivot(self, sequence: int = 0, entropy: str = "distribution", sparsity_rise: bool = False) -> int:
        """Pivot layer of one sequence (one device-to-host read).

        ``entropy``: "distribution" uses the entropy of the window's per-head
        attention distribution (the stats of kvsel_accumulate_stats); "row"
        the mean entropy of the window rows (needs ``row_entropy``).
        ``sparsity_rise``: take the largest entropy drop among the layers
        whose sparsity rose (kvsel_pivot_layer_sparsity)."""
        import torch
        if entropy == "row":
            if not self.row_entropy:
                raise ValueError("row entropies were not recorded (StructKVState(row_entropy=True))")
            ent = torch.stack([m[sequence] for m in self.mean_row_ent]).cpu().numpy()
        elif entropy == "distribution":
            ent = torch.stack([s[sequence, 0] for s in self.stats]).cpu().numpy()
        else:
            raise ValueError(f"unknown entropy {entropy!r}")
        if not sparsity_rise:
            return kvsel.pivot_layer(ent)
        spar = torch.stack([s[sequence, 1] for s in self.stats]).cpu().numpy()
        return kvsel.pivot_layer_sparsity(ent, spar)

    def compress_caches(self, kv_layers, cu_seqlens, w: int, idx_kv, k_kv, paged=None):
        """R_KV compression of every layer's cache with the pivot's per-head
        selection (StructKV summary page, section 2C: the memory budget is
        applied to the cache kept for decoding, independently of R_struct).

        ``kv_layers``: [(k_l, v_l), ...] bf16 [T, h_kv, d] per layer;
        ``idx_kv``: int32 [h_kv, L] from the pivot.  Without ``paged`` returns
        [(k_c, v_c), ...] flat [L, h_kv, d]; with ``paged`` = [(k_cache,
        v_cache, block_table), ...] per layer writes into those caches and
        returns None.  Two layers' K and V go per launch (four gathers)."""
        jobs = []
        for l, (k_l, v_l) in enumerate(kv_layers):
            if paged is None:
                jobs += [(k_l, idx_kv, k_kv), (v_l, idx_kv, k_kv)]
            else:
                kc, vc, table = paged[l]
                jobs += [(k_l, idx_kv, k_kv, kc, table), (v_l, idx_kv, k_kv, vc, table)]
        outs = []
        for j0 in range(0, len(jobs), kvsel.GATHER_MAX_JOBS):
            batch = jobs[j0:j0 + kvsel.GATHER_MAX_JOBS]
            if paged is None:
                outs += kvsel.gather_multi(cu_seqlens, w, batch)
            else:
                kvsel.gather_paged(cu_seqlens, w, batch)
        if paged is not None:
            return None
        return [(outs[2 * l], outs[2 * l + 1]) for l in range(len(kv_layers))]