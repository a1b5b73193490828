"""CPU pins of the acceptance bounds in tests/tolerances.py: perturb the
inputs within the per-element errors each derivation assumes (random,
extreme and adversarial directions) and check that the float64 result moves
by no more than the bound; emulate the kernels' fp32 arithmetic in NumPy
float32 and check that it stays within the rounding bounds."""
import math

import numpy as np
import pytest

import oracle
from tolerances import (ROW_PATH, SCORE_ATOL, SCORE_RTOL, U32, row_entropy_bound, row_logit_bound,
                        stats_kernel, stats_propagated)


def _score_cases():
    """Score arrays [h_kv, T] whose per-(sequence, head) totals are w*group,
    like a window score: peaked (hubs), near-uniform, one dominant key, one
    position at p = 1/e, and positions at exactly 1/n."""
    rng = np.random.default_rng(3)
    w, group = 4, 2
    M = w * group
    cu = np.array([0, 300, 301, 1000], dtype=np.int64)
    cases = []
    for kind in ("peaked", "uniformish", "dominant", "at_1_over_e", "at_1_over_n"):
        s = np.zeros((3, int(cu[-1])))
        for b in range(3):
            off, n = int(cu[b]), int(cu[b + 1] - cu[b])
            for g in range(3):
                if kind == "peaked":
                    x = rng.exponential(1.0, n) ** 3
                elif kind == "uniformish":
                    x = 1.0 + 1e-3 * rng.standard_normal(n)
                elif kind == "dominant":
                    x = np.full(n, 1e-9)
                    x[rng.integers(n)] = 1.0
                elif kind == "at_1_over_e":
                    x = rng.random(n) + 0.1
                else:
                    x = np.ones(n)
                p = x / x.sum()
                if kind == "at_1_over_e" and n > 1:
                    p = p * (1 - 1 / math.e) / (p.sum() - p[0])
                    p[0] = 1 / math.e
                s[g, off:off + n] = p * M
        cases.append((kind, s.astype(np.float32).astype(np.float64), cu, w, group))
    return cases


@pytest.mark.parametrize("case", _score_cases(), ids=lambda c: c[0])
def test_stats_propagated_bounds_every_perturbation(case):
    kind, s, cu, w, group = case
    bound = stats_propagated(s, cu, w, group)
    base = oracle.layer_stats(s, cu, w, group)
    D = SCORE_ATOL + SCORE_RTOL * np.abs(s)
    rng = np.random.default_rng(11)
    p = s / (w * group)
    lens = np.diff(cu)
    toward = np.zeros_like(s)
    for b in range(len(lens)):
        seg = slice(int(cu[b]), int(cu[b + 1]))
        toward[:, seg] = np.sign(1.0 / lens[b] - p[:, seg])    # every position toward the threshold
    dirs = [rng.uniform(-1, 1, s.shape), np.ones_like(s), -np.ones_like(s), np.sign(1 / math.e - p), toward,
            np.sign(rng.standard_normal(s.shape))]
    for dvec in dirs:
        t = np.maximum(s + dvec * D, 0.0)
        moved = np.abs(oracle.layer_stats(t, cu, w, group) - base)
        assert np.all(moved <= bound * (1 + 1e-9) + 1e-15), (kind, moved, bound)


def _kernel_stats_fp32(s32, cu, w, group):
    """The stats kernel's arithmetic in float32: p = s * fl(1/M), -p ln p,
    (p - fl(1/n))^2, two positions per thread, a 64-lane tree in fp32, the
    rest in double, fp32 output."""
    s32 = np.asarray(s32, dtype=np.float32)
    h_kv = s32.shape[0]
    inv_m = np.float32(1.0 / (w * group))
    out = np.zeros((len(cu) - 1, 3), dtype=np.float32)
    for b in range(len(cu) - 1):
        off, n = int(cu[b]), int(cu[b + 1] - cu[b])
        inv_n = np.float32(1.0) / np.float32(n)
        tot = np.zeros(3)
        for g in range(h_kv):
            x = s32[g, off:off + n]
            pad = (-n) % 512
            x = np.concatenate([x, np.zeros(pad, np.float32)])
            valid = np.concatenate([np.ones(n, bool), np.zeros(pad, bool)])
            p = (x * inv_m).astype(np.float32)
            with np.errstate(divide="ignore", invalid="ignore"):
                ent = np.where(p > 0, -(p * np.log(p)).astype(np.float32), np.float32(0)).astype(np.float32)
            dp = (p - inv_n).astype(np.float32)
            var = (dp * dp).astype(np.float32)
            for arr, i in ((ent, 0), (var, 2)):
                arr = np.where(valid, arr, np.float32(0)).reshape(-1, 2, 256)   # [chunk, per-thread, thread]
                t = (arr[:, 0, :] + arr[:, 1, :]).astype(np.float32)            # per thread
                t = t.reshape(-1, 4, 64)                                          # [chunk, wave, lane]
                while t.shape[-1] > 1:                                            # lane tree
                    h = t.shape[-1] // 2
                    t = (t[..., :h] + t[..., h:]).astype(np.float32)
                tot[i] += t.astype(np.float64).sum()
            tot[1] += np.count_nonzero(x[:n].astype(np.float64) * n < w * group)
        out[b] = (tot[0] / h_kv, tot[1] / (h_kv * n), tot[2] / (h_kv * n))
    return out


@pytest.mark.parametrize("case", _score_cases(), ids=lambda c: c[0])
def test_stats_kernel_bound_covers_fp32_arithmetic(case):
    kind, s, cu, w, group = case
    got = _kernel_stats_fp32(s, cu, w, group).astype(np.float64)
    want = oracle.layer_stats(s, cu, w, group)
    bound = stats_kernel(s, cu, w, group)
    assert np.all(np.abs(got - want) <= bound), (kind, got - want, bound)


def _logit_rows(rng, rows, n, spread, hubs=0, hide=0):
    x = spread * rng.standard_normal((rows, n))
    for r in range(rows):
        x[r, rng.choice(n, hubs, replace=False)] += 3 * spread
        if hide:
            x[r, n - hide + r % hide:] = -np.inf
    return x


@pytest.mark.parametrize("spread,eta_max", [(1.0, 1e-5), (3.0, 1e-3), (20.0, 1e-2), (0.01, 1e-4)])
def test_row_logit_bound_holds(spread, eta_max):
    rng = np.random.default_rng(int(spread * 100))
    x = _logit_rows(rng, 6, 2000, spread, hubs=5, hide=40)
    eta = np.where(np.isfinite(x), rng.uniform(0, eta_max, x.shape), 0.0)
    bound, H, lse_bound = row_logit_bound(x, eta)

    def ent(z):
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        P = e / e.sum(axis=1, keepdims=True)
        return -(P * np.log(np.where(P > 0, P, 1.0))).sum(axis=1)

    np.testing.assert_allclose(ent(x), H, rtol=1e-12)
    xs = np.where(np.isfinite(x), x, 0.0)
    m = x.max(axis=1, keepdims=True)
    P = np.exp(x - m)
    P /= P.sum(axis=1, keepdims=True)
    xbar = (P * xs).sum(axis=1, keepdims=True)
    sgn = np.sign(xs - xbar)
    def lse(z):
        m = z.max(axis=1)
        return m + np.log(np.exp(z - m[:, None]).sum(axis=1))

    for d in (rng.uniform(-1, 1, x.shape), sgn, -sgn, np.ones_like(x), np.sign(rng.standard_normal(x.shape))):
        moved = np.abs(ent(x + d * eta) - H)
        assert np.all(moved <= bound * (1 + 1e-9) + 1e-14), (spread, eta_max, moved, bound)
        moved = np.abs(lse(x + d * eta) - lse(x))
        assert np.all(moved <= lse_bound * (1 + 1e-9) + 1e-14), (spread, eta_max, moved, lse_bound)


def _row_entropy_fp32(x2_rows):
    """Pass A's online row statistics in float32 on logits already in log2
    units (fp32): per tile of 16 keys a running max m, l = sum 2^(x-m) and
    tt = sum 2^(x-m) (x-m), rescaled when m moves; H = ln2 (log2 l - tt/l)."""
    f = np.float32
    rows, n = x2_rows.shape
    m = np.full(rows, f(-1e30), dtype=np.float32)
    l = np.zeros(rows, np.float32)
    tt = np.zeros(rows, np.float32)
    for t0 in range(0, n, 16):
        blk = x2_rows[:, t0:t0 + 16]
        mn = np.maximum(m, blk.max(axis=1)).astype(np.float32)
        y = (blk - mn[:, None]).astype(np.float32)
        with np.errstate(invalid="ignore"):
            e = np.exp2(y).astype(np.float32)
            yt = np.maximum(y, f(-1e30)).astype(np.float32)
            s4 = e.sum(axis=1, dtype=np.float32)
            t4 = (e * yt).astype(np.float32).sum(axis=1, dtype=np.float32)
        dm = (m - mn).astype(np.float32)
        a = np.exp2(dm).astype(np.float32)
        tt = (a * (dm * l + tt).astype(np.float32) + t4).astype(np.float32)
        l = (l * a + s4).astype(np.float32)
        m = mn
    h = (f(math.log(2)) * (np.log2(l).astype(np.float32) - (tt / l).astype(np.float32))).astype(np.float32)
    return h.astype(np.float64)


@pytest.mark.parametrize("spread", [0.5, 2.0, 8.0])
def test_row_entropy_arithmetic_part_covers_fp32_path(spread):
    """The fp32 online path (300+ sequential updates per row, more than a
    kernel lane makes) against float64 entropy of the same fp32 logits:
    within ROW_PATH u (1 + 2H)."""
    rng = np.random.default_rng(7)
    x = _logit_rows(rng, 8, 5000, spread, hubs=10, hide=16)
    x2 = (x / math.log(2)).astype(np.float32)           # log2 units, as the kernel holds them
    z = x2.astype(np.float64) * math.log(2)
    m = z.max(axis=1, keepdims=True)
    P = np.exp(z - m)
    P /= P.sum(axis=1, keepdims=True)
    H = -(P * np.log(np.where(P > 0, P, 1.0))).sum(axis=1)
    got = _row_entropy_fp32(x2)
    assert np.all(np.abs(got - H) <= ROW_PATH * U32 * (1 + 2 * H)), (got - H, H)


def test_row_entropy_bound_is_tight_enough():
    """On a workload-like case the bound is a small fraction of the entropy:
    it decides something."""
    rng = np.random.default_rng(2)
    B, w, h_q, h_kv, d, n = 1, 8, 4, 2, 64, 1500
    q = rng.standard_normal((B, w, h_q, d))
    k = rng.standard_normal((n, h_kv, d))
    cu = [0, n]
    scale = 1 / math.sqrt(d)
    b1 = row_entropy_bound(q, k, cu, h_q, h_kv, w, scale)
    ent = oracle.window_row_entropy(q, k, cu, h_q, h_kv, w, scale)
    assert np.all(b1 < 2e-4 * ent) and np.all(b1 > 0)


@pytest.mark.parametrize("case", _score_cases(), ids=lambda c: c[0])
def test_stats_propagated_with_measured_deviations(case):
    """The same bound for arbitrary per-position deviations (as measured
    between a GPU score and the oracle's)."""
    kind, s, cu, w, group = case
    rng = np.random.default_rng(21)
    dev = rng.uniform(0, 1e-4, s.shape) * (s + 1e-3)
    bound = stats_propagated(s, cu, w, group, dev=dev)
    base = oracle.layer_stats(s, cu, w, group)
    for dvec in (rng.uniform(-1, 1, s.shape), np.ones_like(s), -np.ones_like(s)):
        t = np.maximum(s + dvec * dev, 0.0)
        moved = np.abs(oracle.layer_stats(t, cu, w, group) - base)
        assert np.all(moved <= bound * (1 + 1e-9) + 1e-15), (kind, moved, bound)
