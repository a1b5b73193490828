"""Acceptance bounds derived from the arithmetic (test infrastructure).

Each function returns the largest difference a correct implementation may
show for one quantity, computed per case from float64 values; the
derivations are written next to each function and pinned on the CPU by
tests/test_tolerances.py, which perturbs the inputs within the stated
per-element errors and checks that the float64 result moves by no more than
the bound.

u = 2^-24 is the unit roundoff of fp32 (round to nearest).
"""
from __future__ import annotations

import math

import numpy as np

U32 = 2.0 ** -24

# Score acceptance (fixed by the method's correctness criterion):
# |gpu - oracle| <= SCORE_ATOL + SCORE_RTOL * |oracle| elementwise.
SCORE_RTOL = 1e-3
SCORE_ATOL = 1e-6


def _f(t):
    """-t ln t with 0 ln 0 = 0 (float64, elementwise)."""
    t = np.asarray(t, dtype=np.float64)
    out = np.zeros_like(t)
    pos = t > 0
    out[pos] = -t[pos] * np.log(t[pos])
    return out


def _segs(cu):
    cu = [int(x) for x in np.asarray(cu).reshape(-1)]
    return [(cu[b], cu[b + 1] - cu[b]) for b in range(len(cu) - 1)]


def stats_propagated(score, cu, w: int, group: int, rtol: float = SCORE_RTOL, atol: float = SCORE_ATOL,
                     dev=None):
    """How far the per-sequence statistics (entropy, sparsity, variance of
    p = score / (w*group), averaged over KV heads) can move when every score
    moves by at most atol + rtol*|score| (the score acceptance rule), or by
    at most ``dev`` (an array like ``score``: measured deviations) if given.

    With M = w*group and D_j = (atol + rtol*s_j)/M (or dev_j/M) the bound on |dp_j|:
      entropy:  sum_j max_{|t - p_j| <= D_j, t >= 0} |f(t) - f(p_j)|, f = -t ln t.
                f is concave with its maximum at 1/e, so the largest change
                over the interval is at an end or at 1/e.
      variance: (1/n) sum_j D_j (2|p_j - 1/n| + D_j)   (|(a+d)^2 - a^2| <= |d|(2|a| + |d|))
      sparsity: the share of positions whose interval contains 1/n (only
                those can change side).
    Each averaged over heads like the statistic.  Returns float64 [B, 3]."""
    s = np.asarray(score, dtype=np.float64)
    h_kv = s.shape[0]
    M = float(w * group)
    segs = _segs(cu)
    out = np.zeros((len(segs), 3))
    for b, (off, n) in enumerate(segs):
        x = s[:, off:off + n]
        p = x / M
        if dev is None:
            D = (atol + rtol * np.abs(x)) / M
        else:
            D = np.abs(np.asarray(dev, dtype=np.float64)[:, off:off + n]) / M
        lo = np.maximum(p - D, 0.0)
        hi = p + D
        fp = _f(p)
        mv = np.maximum(np.abs(_f(lo) - fp), np.abs(_f(hi) - fp))
        top = (lo <= 1 / math.e) & (hi >= 1 / math.e)
        mv = np.where(top, np.maximum(mv, np.abs(1 / math.e - fp)), mv)
        ent = mv.sum() / h_kv
        var = (D * (2 * np.abs(p - 1.0 / n) + D)).sum() / (n * h_kv)
        spar = np.count_nonzero(np.abs(p - 1.0 / n) <= D) / (n * h_kv)
        out[b] = (ent, spar, var)
    return out


def stats_kernel(score, cu, w: int, group: int):
    """Rounding bound of the statistics computed in fp32 from a given fp32
    score array (what the stats kernel does), against the same statistics
    in float64 (the oracle fed the same array).

    Per position: p = fl(s * fl(1/M)) has relative error <= 2u, which moves
    f = -p ln p by <= |ln p + 1| 2u p; the logarithm (one ulp) and the
    product add <= 3u f.  Over a head (sum p = 1) that is <= 2u (E + 1) + 3u E.
    dp = fl(p - fl(1/n)) errs by <= 2u p + u/n + u|dp|, and fl(dp^2) by
    u dp^2 more.  Terms are summed in fp32 over at most 2 positions per
    thread and a 64-lane tree (8 roundings, all terms of one sign: <= 8u of
    the sum), then in double, and the result is rounded to fp32 (u).
    Entropy: (2 + 3 + 8 + 1)u E + 2u <= 16u E + 4u.  Variance:
    (1/n) sum_j [2|dp_j| (2u p_j + u/n) + (2 + 1 + 8)u dp_j^2] + u V.
    Sparsity is an exact count; its fp32 output rounds (u S).  Returns
    float64 [B, 3]."""
    s = np.asarray(score, dtype=np.float64)
    h_kv = s.shape[0]
    M = float(w * group)
    segs = _segs(cu)
    out = np.zeros((len(segs), 3))
    for b, (off, n) in enumerate(segs):
        p = s[:, off:off + n] / M
        ent = _f(p).sum() / h_kv
        dp = p - 1.0 / n
        var = (dp * dp).sum() / (n * h_kv)
        dvar = (2 * np.abs(dp) * (2 * U32 * p + U32 / n) + 11 * U32 * dp * dp).sum() / (n * h_kv)
        spar = np.count_nonzero(s[:, off:off + n] * n < M) / (n * h_kv)
        out[b] = (16 * U32 * ent + 4 * U32, U32 * spar, dvar + U32 * var + 1e-30)
    return out


# ---- row entropy --------------------------------------------------------------
#
# The kernel forms a window row's entropy H = ln Z - sum_k P_k x_k from its
# logits x_k = scale * <q, k_k> computed in fp32: bf16 products are exact in
# fp32, an MFMA accumulates d of them, then one multiply by the fp32
# constant scale*log2(e).  With each addition rounded or truncated (<= 2u
# relative), |dx_k| <= eta_k = 2 (d + 2) u scale sum_t |q_t k_kt|.
#
# Logit part.  dH/dx_k = -P_k (x_k - xbar), xbar = sum P x.  Along the path
# x + t*dx (t in [0, 1]) every P_k(t) <= e^{2 eta} P_k (eta = max eta_k) and
# |x_k(t) - xbar(t)| <= |x_k - xbar| + eta_k + eta + (e^{2 eta} - 1) M1,
# M1 = sum P |x - xbar|.  So
#   |dH| <= e^{2 eta} sum_k P_k eta_k (|x_k - xbar| + eta_k + eta + (e^{2 eta} - 1) M1).
#
# Arithmetic part.  The row's sums l = sum 2^(x - m) and tt = sum 2^(x - m)(x - m)
# are accumulated in fp32 along paths of at most ROW_PATH roundings (terms
# of one sign; each term carries the exponential's and its argument's
# rounding), so each has relative error <= ROW_PATH u.  H = ln l - ln2 tt/l
# with ln l >= 0 and -ln2 tt/l = H - ln l in [0, H], so H errs by
# <= ROW_PATH u (1 + 2H).  ROW_PATH = 512 covers a chunk's longest per-lane
# tile walk (at most 60 tiles), the lane, pair and chunk merges of sequences
# up to 2^20 keys, the per-term roundings and the final log, divide and
# multiply.
ROW_PATH = 512


def row_logit_bound(x, eta):
    """The logit part for softmax rows with logits x [rows, n] (natural
    units, -inf where hidden) and per-logit error bounds eta [rows, n] (0
    where hidden).  Returns (entropy bound [rows], H [rows], lse bound
    [rows]): d lse / dx_k = P_k, so the normaliser moves by at most
    e^{2 eta} sum_k P_k eta_k."""
    x = np.asarray(x, dtype=np.float64)
    eta = np.asarray(eta, dtype=np.float64)
    hidden = ~np.isfinite(x)
    m = x.max(axis=1, keepdims=True)
    e = np.exp(x - m)
    P = e / e.sum(axis=1, keepdims=True)
    xs = np.where(hidden, 0.0, x)
    xbar = (P * xs).sum(axis=1, keepdims=True)
    ax = np.where(hidden, 0.0, np.abs(xs - xbar))
    M1 = (P * ax).sum(axis=1)
    em = eta.max(axis=1)
    g = np.exp(2 * em)
    pe = (P * eta).sum(axis=1)
    bound = g * ((P * eta * ax).sum(axis=1) + (P * eta * eta).sum(axis=1) + (em + (g - 1) * M1) * pe)
    H = -(P * np.log(np.where(P > 0, P, 1.0))).sum(axis=1)
    return bound, H, g * pe


def row_bounds(q, k, cu, h_q: int, h_kv: int, w: int, scale: float):
    """Per-row bounds on |kernel - float64| for the row entropy and for the
    row's natural-log normaliser, from the bf16 inputs promoted to float64.
    q [B, w, h_q, d], k [T, h_kv, d].  Returns two float64 [B, h_q, w].

    The normaliser's arithmetic part: lse2 = m + log2 l with l's relative
    error <= ROW_PATH u, then the sum and the multiply by ln2 round:
    ROW_PATH u + 3u |lse|."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    d = q.shape[-1]
    G = h_q // h_kv
    B = q.shape[0]
    ent_b = np.zeros((B, h_q, w))
    lse_b = np.zeros((B, h_q, w))
    for b, (off, n) in enumerate(_segs(cu)):
        pos = n - w + np.arange(w)
        hidden = np.arange(n)[None, :] > pos[:, None]
        for h in range(h_q):
            kb = k[off:off + n, h // G, :]
            x = scale * (q[b, :, h, :] @ kb.T)                          # [w, n]
            eta = 2 * (d + 2) * U32 * scale * (np.abs(q[b, :, h, :]) @ np.abs(kb).T)
            x[hidden] = -np.inf
            eta[hidden] = 0.0
            logit, H, lse_logit = row_logit_bound(x, eta)
            m = x.max(axis=1)
            lse = m + np.log(np.exp(x - m[:, None]).sum(axis=1))
            ent_b[b, h] = logit + ROW_PATH * U32 * (1 + 2 * H)
            lse_b[b, h] = lse_logit + ROW_PATH * U32 + 3 * U32 * np.abs(lse)
    return ent_b, lse_b


def row_entropy_bound(q, k, cu, h_q: int, h_kv: int, w: int, scale: float):
    """The entropy half of ``row_bounds``."""
    return row_bounds(q, k, cu, h_q, h_kv, w, scale)[0]
