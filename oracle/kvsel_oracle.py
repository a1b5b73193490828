"""CPU oracle for attention-score token selection.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or call this module; the library
path (``token_selection_tsp_amd``) never does, and it shares no code with it.

Plain NumPy, float64 throughout, one obviously-correct step after another.
Each function cites the passage it follows.  Pages:

* FastKV summary page (gist.science, paper 2502.01068), section 2A "Token-
  Selective Propagation": at the TSP layer the importance of the tokens is
  judged from the attention of a window of recent tokens, and only the
  selected subset *together with the window tokens* goes on to later layers.
  Section 2B: two independent knobs, the TSP rate (tokens propagated) and
  the KV retention rate (cache entries kept per layer).
* FastKV abstract (chatpaper.ai page, English abstract): the KV compression
  is GQA-aware.
* StructKV summary page (gist.science, paper 2604.06746), section 2A: a
  global in-degree score summed over layers from the input layer to a pivot
  layer; section 2B: the pivot is where attention entropy drops sharply
  (sparsity and variance are monitored too); section 2C: a structural budget
  R_struct (tokens propagated) decoupled from the memory budget R_KV.

The pages give no formula for these steps.  The readings taken here (causal
window softmax with scale 1/sqrt(d), plain sums, ties to the lowest index,
ascending output with the window appended, stats of the window's per-head
attention mass normalised by its exact total w*G) are listed with their
reasons in the design notes of the repository.

Parity pins: every function here is pinned by the ``-m "not gpu"`` tests
against closed forms, library routines (scipy softmax, Python's sort),
invariants and brute force; no page prints a worked numeric example, so no
pin comes from the pages' own numbers.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np


# ---------------------------------------------------------------- inputs

def bf16_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly.  A bfloat16 value
    is the upper half of the float32 with the same bits."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _segments(cu_seqlens) -> List[Tuple[int, int]]:
    cu = [int(x) for x in np.asarray(cu_seqlens).reshape(-1)]
    return [(cu[b], cu[b + 1] - cu[b]) for b in range(len(cu) - 1)]


# ---------------------------------------------------------------- step 1+2

def window_score(q: np.ndarray, k: np.ndarray, cu_seqlens, h_q: int, h_kv: int, w: int,
                 scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Window attention and its GQA-grouped column sums.

    FastKV page, section 2A: the tokens' importance comes from the attention
    of the window of the last ``w`` tokens.  For sequence b (packed rows
    ``off .. off+n-1``), query head h and window row i (position
    ``p_i = n - w + i``), the logits over keys j <= p_i (causal) are
    ``scale * <q[b,i,h], k[off+j, g(h)]>`` with ``g(h) = h // (h_q // h_kv)``
    (GQA: the query heads of a group share one KV head, FastKV abstract),
    and P is their softmax.  The score of key j for KV head g sums P over
    the window rows and the query heads of the group.

    Arguments: ``q`` float [B, w, h_q, d]; ``k`` float [T, h_kv, d];
    ``cu_seqlens`` [B+1].
    Returns ``score`` float64 [h_kv, T] and ``lse`` float64 [B, h_q, w], the
    natural-log normaliser of each softmax row.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    T = k.shape[0]
    G = h_q // h_kv
    B = q.shape[0]
    score = np.zeros((h_kv, T), dtype=np.float64)
    lse = np.zeros((B, h_q, w), dtype=np.float64)
    for b, (off, n) in enumerate(_segments(cu_seqlens)):
        if n < w:
            raise ValueError("sequence shorter than the window")
        pos = n - w + np.arange(w)                        # window positions
        hidden_from_row = np.arange(n)[None, :] > pos[:, None]   # causal mask
        for g in range(h_kv):
            kb = k[off:off + n, g, :]                     # [n, d]
            for hh in range(G):
                h = g * G + hh
                s = scale * (q[b, :, h, :] @ kb.T)        # [w, n] logits
                s[hidden_from_row] = -np.inf
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                z = e.sum(axis=1, keepdims=True)
                p = e / z                                 # softmax per row
                lse[b, h, :] = (m + np.log(z))[:, 0]
                score[g, off:off + n] += p.sum(axis=0)    # sum over window rows
    return score, lse


def window_row_entropy(q: np.ndarray, k: np.ndarray, cu_seqlens, h_q: int, h_kv: int, w: int,
                       scale: float) -> np.ndarray:
    """Attention entropy of every window row (StructKV page, section 2B: the
    pivot search watches the attention entropy, read here at the level of
    the softmax rows themselves).

    Same rows as ``window_score``: sequence b, query head h, window row i at
    position ``p_i = n - w + i``, causal softmax P over keys ``j <= p_i``.
    The row's entropy is ``-sum_j P_j ln P_j`` in nats, with ``0 ln 0 = 0``
    (keys whose probability underflows to zero add nothing).
    Returns float64 [B, h_q, w].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    G = h_q // h_kv
    B = q.shape[0]
    ent = np.zeros((B, h_q, w), dtype=np.float64)
    for b, (off, n) in enumerate(_segments(cu_seqlens)):
        if n < w:
            raise ValueError("sequence shorter than the window")
        for h in range(h_q):
            kb = k[off:off + n, h // G, :]
            for i in range(w):
                s = scale * (kb[:n - w + i + 1] @ q[b, i, h, :])   # visible keys only
                e = np.exp(s - s.max())
                p = e / e.sum()
                nz = p > 0
                ent[b, h, i] = -np.sum(p[nz] * np.log(p[nz]))
    return ent


def mean_row_entropy(row_entropy: np.ndarray) -> np.ndarray:
    """One entropy per sequence and layer: the mean of the window rows'
    entropies over all query heads and rows.  Returns float64 [B]."""
    e = np.asarray(row_entropy, dtype=np.float64)
    return e.reshape(e.shape[0], -1).mean(axis=1)


# ---------------------------------------------------------------- step 2 (StructKV part)

def accumulate(score: np.ndarray, c_in: Optional[np.ndarray] = None) -> np.ndarray:
    """Running global in-degree score (StructKV page, section 2A: attention
    contributions summed from the input layer up to the pivot):
    ``C_l = C_{l-1} + score_l``, with ``C_{-1} = 0``."""
    s = np.asarray(score, dtype=np.float64)
    return s.copy() if c_in is None else np.asarray(c_in, dtype=np.float64) + s


def head_sum(x: np.ndarray) -> np.ndarray:
    """One score per token for the propagated sequence: the sum over KV heads.
    The hidden row of a token is shared by all heads, so the propagated set
    (FastKV section 2A, StructKV R_struct) is one set per sequence."""
    return np.asarray(x, dtype=np.float64).sum(axis=0)


def layer_stats(score: np.ndarray, cu_seqlens, w: int, group: int) -> np.ndarray:
    """Per-sequence attention entropy, sparsity and variance of one layer
    (StructKV page, section 2B monitors these three to find the pivot).

    For sequence b of length n and KV head g, the window's attention mass
    ``score[g, off:off+n]`` totals exactly ``w * group`` (every softmax row
    sums to one), so ``p = score / (w * group)`` is a distribution over the
    n positions.  Then
      entropy  = -sum_j p_j ln p_j            (0 ln 0 = 0, nats)
      sparsity = #{j : p_j < 1/n} / n         (below-uniform share)
      variance = mean_j (p_j - 1/n)^2
    each averaged over the KV heads.  Returns float64 [B, 3].
    """
    s = np.asarray(score, dtype=np.float64)
    h_kv = s.shape[0]
    mass = float(w * group)
    segs = _segments(cu_seqlens)
    out = np.zeros((len(segs), 3), dtype=np.float64)
    for b, (off, n) in enumerate(segs):
        ent = spar = var = 0.0
        for g in range(h_kv):
            x = s[g, off:off + n]
            p = x / mass
            pos = p > 0
            ent += -np.sum(p[pos] * np.log(p[pos]))
            # p < 1/n  <=>  x * n < mass  (both sides times the positive n*mass)
            spar += np.count_nonzero(x * n < mass) / n
            var += np.mean((p - 1.0 / n) ** 2)
        out[b] = (ent / h_kv, spar / h_kv, var / h_kv)
    return out


def pivot_layer(entropy: Sequence[float]) -> int:
    """Pivot layer L* (StructKV page, section 2B: the layer where attention
    entropy drops sharply): the layer l >= 1 with the largest drop
    ``E[l-1] - E[l]``, the smallest such l on ties; 0 for a single layer."""
    e = np.asarray(entropy, dtype=np.float64).reshape(-1)
    if e.size < 2:
        return 0
    drops = e[:-1] - e[1:]
    return int(np.argmax(drops)) + 1   # argmax returns the first maximum


def pivot_layer_sparsity(entropy: Sequence[float], sparsity: Sequence[float]) -> int:
    """Pivot layer L* with both signs of the phase transition (StructKV page,
    section 2B: entropy falls sharply *and* sparsity rises there).

    Among the layers l >= 1 whose sparsity rose (``S[l] > S[l-1]``), the one
    with the largest entropy drop ``E[l-1] - E[l]``, the smallest such l on
    ties.  If no layer's sparsity rose, the rule falls back to the largest
    entropy drop alone (``pivot_layer``); 0 for a single layer."""
    e = np.asarray(entropy, dtype=np.float64).reshape(-1)
    sp = np.asarray(sparsity, dtype=np.float64).reshape(-1)
    if e.shape != sp.shape:
        raise ValueError("entropy and sparsity differ in length")
    if e.size < 2:
        return 0
    best, best_drop = -1, None
    for l in range(1, e.size):
        if sp[l] > sp[l - 1]:
            drop = e[l - 1] - e[l]
            if best_drop is None or drop > best_drop:
                best, best_drop = l, drop
    return best if best >= 0 else pivot_layer(e)


# ---------------------------------------------------------------- step 3

def budget_length(n: int, w: int, k: int) -> int:
    """Length of one selection: the kept candidates plus the window,
    ``min(n, k + w)``."""
    return min(n, max(k, 0) + w)


def select_with_window(x: np.ndarray, n: int, w: int, k: int) -> np.ndarray:
    """Top-k of one sequence's scores plus the window (FastKV section 2A:
    the selected subset travels together with the window tokens).

    Candidates are positions ``0 .. n-w-1`` (the window is always kept, so it
    does not compete).  The ``min(k, n-w)`` largest values are kept, ties
    going to the lower position; the kept positions are returned in
    ascending order followed by the window ``n-w .. n-1``.
    """
    x = np.asarray(x, dtype=np.float64)[:n]
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite score")
    nc = n - w
    ke = min(max(int(k), 0), nc)
    j = np.arange(nc)
    order = np.lexsort((j, -x[:nc]))      # value descending, then position ascending
    kept = np.sort(order[:ke])
    return np.concatenate([kept, np.arange(nc, n)]).astype(np.int64)


def select_rows(keys: np.ndarray, cu_seqlens, w: int, k_per_seq: Sequence[int]) -> np.ndarray:
    """``select_with_window`` for every row of ``keys`` [rows, T] and every
    sequence; each row's result is the per-sequence selections concatenated
    in sequence order (sequence-local positions).  Returns int64 [rows, L]."""
    keys = np.asarray(keys, dtype=np.float64)
    if keys.ndim == 1:
        keys = keys[None, :]
    segs = _segments(cu_seqlens)
    parts = []
    for r in range(keys.shape[0]):
        row = [select_with_window(keys[r, off:off + n], n, w, int(k_per_seq[b]))
               for b, (off, n) in enumerate(segs)]
        parts.append(np.concatenate(row) if row else np.zeros(0, np.int64))
    return np.stack(parts)


# ---------------------------------------------------------------- step 4

def gather(src: np.ndarray, cu_seqlens, idx: np.ndarray, lengths: Sequence[int]) -> np.ndarray:
    """Compact rows by the selected positions (FastKV section 2A/2B: the
    propagated tokens' hidden rows; the retained K/V entries per KV head).

    ``src`` [T, heads, ...] (any dtype, copied bit for bit); ``idx``
    [idx_rows, L] with ``idx_rows`` = heads (one index set per head) or 1
    (shared); ``lengths`` the per-sequence selection lengths (sum L).
    Output row ``s`` of sequence b, head h takes
    ``src[off_b + idx[h or 0, s], h]``.  Returns [L, heads, ...].
    """
    src = np.asarray(src)
    idx = np.asarray(idx)
    heads = src.shape[1]
    per_head = idx.shape[0] == heads and heads > 1
    L = int(sum(lengths))
    dst = np.zeros((L,) + src.shape[1:], dtype=src.dtype)
    start = 0
    for b, (off, n) in enumerate(_segments(cu_seqlens)):
        Lb = int(lengths[b])
        for h in range(heads):
            r = idx[h if per_head else 0, start:start + Lb].astype(np.int64)
            dst[start:start + Lb, h] = src[off + r, h]
        start += Lb
    return dst


def gather_paged(src: np.ndarray, cu_seqlens, idx: np.ndarray, lengths: Sequence[int], block_table,
                 block_size: int, cache: np.ndarray) -> np.ndarray:
    """The compacted rows of ``gather`` written into a paged cache instead of
    a flat array (the consumer side of the FastKV KV-retention budget: the
    kept K/V entries become the decode cache, held in fixed-size blocks).

    Selected row ``s`` (sequence-local, ``0 <= s < lengths[b]``) of sequence
    b goes to block ``block_table[b][s // block_size]``, slot
    ``s % block_size``: ``cache[blk, s % block_size, h] = row``.  Rows whose
    block number is outside ``[0, num_blocks)`` are not written.  ``cache``
    [num_blocks, block_size, heads, ...] is not modified; the result is a
    copy with the rows written."""
    out = np.array(cache, copy=True)
    rows = gather(src, cu_seqlens, idx, lengths)
    bt = np.asarray(block_table)
    start = 0
    for b, Lb in enumerate(lengths):
        for s in range(int(Lb)):
            blk = int(bt[b, s // block_size])
            if 0 <= blk < out.shape[0]:
                out[blk, s % block_size] = rows[start + s]
        start += int(Lb)
    return out
