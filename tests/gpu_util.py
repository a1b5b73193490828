"""Helpers shared by the GPU parity tests: device transfer of the seeded
inputs, the acceptance rules, and the oracle side of each comparison."""
from __future__ import annotations

import math
import sys

import numpy as np

import oracle
from token_selection_tsp_amd import synth

# Score acceptance: |gpu - oracle| <= ATOL + RTOL * |oracle| elementwise.
RTOL = 1e-3
ATOL = 1e-6


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev_f32(x: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def assert_close(got, want, rtol=RTOL, atol=ATOL, what="value"):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    err = np.abs(got - want)
    lim = atol + rtol * np.abs(want)
    bad = err > lim
    if bad.any():
        i = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst at {i}: "
                             f"got {got[i]!r} want {want[i]!r} (limit {lim[i]:.3g})")


def selection_agrees(got: np.ndarray, want: np.ndarray, scores: np.ndarray, n: int, w: int, k: int,
                     rtol=RTOL, atol=ATOL) -> None:
    """End-to-end index acceptance for one (row, sequence): same length, same
    window, and every position in the symmetric difference of the kept
    candidates has an oracle score within tolerance of the oracle's k-th
    largest candidate score (a near-tie at the cut)."""
    assert len(got) == len(want) == oracle.budget_length(n, w, k)
    assert got[len(got) - w:].tolist() == list(range(n - w, n))
    kept = len(got) - w
    assert np.all(np.diff(got[:kept]) > 0), "kept positions not ascending"
    a, b = set(got[:kept].tolist()), set(want[:kept].tolist())
    diff = a ^ b
    if not diff:
        return
    cand = scores[: n - w]
    tau = np.sort(cand)[::-1][kept - 1]
    for j in diff:
        assert 0 <= j < n - w, j
        assert abs(cand[j] - tau) <= atol + rtol * abs(tau), (j, cand[j], tau)


def score_oracle(x: dict, wl: synth.Workload, scale: float):
    q = oracle.bf16_to_f64(x["q"])
    k = oracle.bf16_to_f64(x["k"])
    return oracle.window_score(q, k, x["cu_seqlens"], wl.h_q, wl.h_kv, wl.w, scale)


def scale_of(d: int) -> float:
    return float(np.float32(1.0 / math.sqrt(d)))
