"""Seeded synthetic inputs shaped like long-context GQA attention layers.

This module only draws Gaussian tensors, plants "hub" structure and rounds
to bfloat16.  It holds none of the selection arithmetic, so the HIP path and
the CPU oracle can both take their inputs from it.

The workloads stand in for the long-context evaluations the FastKV and
StructKV pages describe (LLaMA-3.1-8B-class decoders on contexts up to 128K
tokens, FastKV page section 4, StructKV page section 4).  No dataset item or
trained weight is used: every tensor is N(0, 1) noise plus a planted shared
direction on a few "hub" keys and on the window queries, so that the score
has a few clear heavy hitters and a long near-uniform tail.

Every tensor is drawn from its own counter-keyed stream
``SeedSequence([seed, layer, sequence, tensor, chunk])`` so the draw order,
chunking and thread count never change the values.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass
from fractions import Fraction
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

# tensor ids inside the seed key
_T_LEN, _T_HUBS, _T_DIR, _T_Q, _T_K, _T_V, _T_HID = range(7)
_CHUNK = 1 << 22  # elements per independently seeded chunk


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return the
    16-bit patterns as uint16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 view of bfloat16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class Budget:
    """A token budget: either a rate ``num/den`` of the sequence length
    (floored exactly) or an absolute token count.  The observation window is
    not part of the budget; it is always kept on top of it."""

    rate: Optional[Fraction] = None
    absolute: Optional[int] = None

    def tokens(self, n: int) -> int:
        if self.absolute is not None:
            return int(self.absolute)
        return int((n * self.rate.numerator) // self.rate.denominator)

    def describe(self) -> str:
        if self.absolute is not None:
            return f"{self.absolute} tokens"
        return f"{float(self.rate) * 100:g}%"


def rate(num: int, den: int = 100) -> Budget:
    return Budget(rate=Fraction(num, den))


def absolute(n: int) -> Budget:
    return Budget(absolute=n)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload.

    ``lengths`` fixes the per-sequence lengths; when it is ``None`` they are
    drawn uniformly from ``length_range`` (inclusive) for ``batch`` sequences.
    Hubs: ``hub_count(n)`` positions drawn without replacement from
    ``[hub_lo, n - w)``, plus position 0 when ``sink`` is set.  Hub keys (all
    KV heads) and all window query rows get ``alpha * u`` added, ``u`` a unit
    vector drawn per layer.  ``alpha`` may ramp linearly over layers.
    """

    name: str
    seed: int
    h_q: int
    h_kv: int
    d: int
    w: int
    hidden: int
    kv_budget: Budget
    tsp_budget: Budget
    lengths: Optional[Tuple[int, ...]] = None
    batch: int = 1
    length_range: Optional[Tuple[int, int]] = None
    hub_per_mille: int = 10
    sink: bool = False
    alpha: Tuple[float, float] = (2.0, 2.0)
    layers: int = 1
    hubs_shared_across_layers: bool = False
    fixed_hubs: Optional[int] = None
    description: str = ""

    @property
    def group(self) -> int:
        return self.h_q // self.h_kv

    def seq_lengths(self) -> List[int]:
        if self.lengths is not None:
            return list(self.lengths)
        lo, hi = self.length_range
        rng = np.random.default_rng(np.random.SeedSequence([self.seed, 0, 0, _T_LEN]))
        return [int(x) for x in rng.integers(lo, hi, size=self.batch, endpoint=True)]

    def cu_seqlens(self) -> np.ndarray:
        ls = self.seq_lengths()
        return np.concatenate([[0], np.cumsum(ls)]).astype(np.int32)

    def alpha_at(self, layer: int) -> float:
        a0, a1 = self.alpha
        if self.layers <= 1:
            return a0
        return a0 + (a1 - a0) * layer / (self.layers - 1)

    def kv_tokens(self) -> np.ndarray:
        return np.array([self.kv_budget.tokens(n) for n in self.seq_lengths()], dtype=np.int32)

    def tsp_tokens(self) -> np.ndarray:
        return np.array([self.tsp_budget.tokens(n) for n in self.seq_lengths()], dtype=np.int32)

    def hub_positions(self, layer: int, b: int, n: int) -> np.ndarray:
        key_layer = 0 if self.hubs_shared_across_layers else layer
        rng = np.random.default_rng(np.random.SeedSequence([self.seed, key_layer, b, _T_HUBS]))
        lo = 1 if self.sink else 0
        count = self.fixed_hubs if self.fixed_hubs is not None else (n * self.hub_per_mille) // 1000
        hi = n - self.w
        count = max(0, min(count, hi - lo))
        pos = rng.choice(np.arange(lo, hi), size=count, replace=False) if count > 0 else np.zeros(0, np.int64)
        if self.sink:
            pos = np.concatenate([[0], pos])
        return np.sort(pos.astype(np.int64))

    def direction(self, layer: int) -> np.ndarray:
        rng = np.random.default_rng(np.random.SeedSequence([self.seed, layer, 0, _T_DIR]))
        u = rng.standard_normal(self.d).astype(np.float64)
        return (u / np.linalg.norm(u)).astype(np.float32)


def _gaussian(key: Sequence[int], n: int, threads: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    nch = (n + _CHUNK - 1) // _CHUNK

    def fill(c: int) -> None:
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        rng = np.random.default_rng(np.random.SeedSequence(list(key) + [c]))
        out[lo:hi] = rng.standard_normal(hi - lo, dtype=np.float32)

    if nch <= 1 or threads <= 1:
        for c in range(nch):
            fill(c)
    else:
        with _cf.ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(fill, range(nch)))
    return out


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def layer_inputs(wl: Workload, layer: int = 0, parts: Sequence[str] = ("q", "k"),
                 threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw one layer's inputs as bfloat16 bit patterns (uint16).

    Returns a dict with the requested parts among
      ``q``      [B, w, H_q, d]   window queries (last w positions of each sequence)
      ``k``/``v`` [T, H_kv, d]    packed keys / values
      ``hidden`` [T, D]           packed hidden states
    plus ``cu_seqlens`` (int32 [B+1]) and ``hubs`` (list of per-sequence positions).
    """
    th = threads or _threads()
    lens = wl.seq_lengths()
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    B = len(lens)
    alpha = wl.alpha_at(layer)
    u = wl.direction(layer)
    out: Dict[str, np.ndarray] = {"cu_seqlens": cu.astype(np.int32)}
    hubs = [wl.hub_positions(layer, b, lens[b]) for b in range(B)]
    out["hubs"] = hubs
    if "q" in parts:
        q = np.empty((B, wl.w, wl.h_q, wl.d), dtype=np.uint16)
        for b in range(B):
            x = _gaussian([wl.seed, layer, b, _T_Q], wl.w * wl.h_q * wl.d, th)
            x = x.reshape(wl.w, wl.h_q, wl.d) + alpha * u
            q[b] = bf16_bits(x)
        out["q"] = q
    if "k" in parts:
        k = np.empty((T, wl.h_kv, wl.d), dtype=np.uint16)
        for b in range(B):
            n = lens[b]
            x = _gaussian([wl.seed, layer, b, _T_K], n * wl.h_kv * wl.d, th).reshape(n, wl.h_kv, wl.d)
            x[hubs[b]] += alpha * u
            k[cu[b]:cu[b + 1]] = bf16_bits(x)
        out["k"] = k
    if "v" in parts:
        v = np.empty((T, wl.h_kv, wl.d), dtype=np.uint16)
        for b in range(B):
            n = lens[b]
            x = _gaussian([wl.seed, layer, b, _T_V], n * wl.h_kv * wl.d, th)
            v[cu[b]:cu[b + 1]] = bf16_bits(x).reshape(n, wl.h_kv, wl.d)
        out["v"] = v
    if "hidden" in parts:
        hid = np.empty((T, wl.hidden), dtype=np.uint16)
        for b in range(B):
            n = lens[b]
            x = _gaussian([wl.seed, layer, b, _T_HID], n * wl.hidden, th)
            hid[cu[b]:cu[b + 1]] = bf16_bits(x).reshape(n, wl.hidden)
        out["hidden"] = hid
    return out


# The five workloads.  Shapes follow a LLaMA-3.1-8B-class decoder layer
# (GQA 32 query heads over 8 KV heads, head dim 128) at 32K and 128K tokens,
# a ragged batch, and a 16-layer StructKV-style accumulation.
WORKLOADS: Dict[str, Workload] = {
    "n1k_gqa8x2_d64": Workload(
        name="n1k_gqa8x2_d64", seed=1, h_q=8, h_kv=2, d=64, w=8, hidden=512,
        kv_budget=rate(25), tsp_budget=rate(50), lengths=(1024,),
        sink=True, fixed_hubs=16, alpha=(3.0, 3.0),
        description="single layer, N=1024, 8/2 heads, d=64, w=8, sink + 16 hubs (3x), KV 25%, TSP 50%"),
    "n32k_gqa32x8_d128": Workload(
        name="n32k_gqa32x8_d128", seed=2, h_q=32, h_kv=8, d=128, w=32, hidden=4096,
        kv_budget=absolute(2048), tsp_budget=rate(20), lengths=(32768,),
        hub_per_mille=10, alpha=(2.0, 2.0),
        description="N=32768, 32/8 heads, d=128, w=32, 1% hubs (2x), KV 2048/head, TSP 20%"),
    "n128k_gqa32x8_d128": Workload(
        name="n128k_gqa32x8_d128", seed=3, h_q=32, h_kv=8, d=128, w=32, hidden=4096,
        kv_budget=absolute(4096), tsp_budget=rate(10), lengths=(131072,),
        hub_per_mille=5, sink=True, alpha=(2.0, 2.0),
        description="N=131072, 32/8 heads, d=128, w=32, sink + 0.5% hubs (2x), KV 4096/head, TSP 10%"),
    "ragged8_4k_32k": Workload(
        name="ragged8_4k_32k", seed=4, h_q=32, h_kv=8, d=128, w=32, hidden=4096,
        kv_budget=rate(10), tsp_budget=rate(20), batch=8, length_range=(4096, 32768),
        hub_per_mille=10, alpha=(2.0, 2.0),
        description="8 packed sequences, N_b ~ U[4096, 32768], 32/8 heads, d=128, w=32, 1% hubs, KV 10%, TSP 20%"),
    "structkv16_n64k": Workload(
        name="structkv16_n64k", seed=5, h_q=32, h_kv=8, d=128, w=32, hidden=4096,
        kv_budget=rate(5), tsp_budget=rate(15), lengths=(65536,), layers=16,
        hub_per_mille=10, hubs_shared_across_layers=True, alpha=(0.5, 3.0),
        description="16 layers, N=65536, 32/8 heads, d=128, w=32, 1% shared hubs ramping 0.5x..3x, R_KV 5%, R_struct 15%"),
}

WORKLOAD_ORDER = ["n1k_gqa8x2_d64", "n32k_gqa32x8_d128", "n128k_gqa32x8_d128",
                  "ragged8_4k_32k", "structkv16_n64k"]


def small(name: str, seed: int, lengths: Sequence[int], h_q: int, h_kv: int, d: int, w: int,
          hidden: int = 64, kv: Budget = rate(25), tsp: Budget = rate(50), hubs: int = 3,
          alpha: float = 3.0, sink: bool = True, layers: int = 1) -> Workload:
    """A small custom workload for tests."""
    return Workload(name=name, seed=seed, h_q=h_q, h_kv=h_kv, d=d, w=w, hidden=hidden,
                    kv_budget=kv, tsp_budget=tsp, lengths=tuple(int(x) for x in lengths),
                    fixed_hubs=hubs, sink=sink, alpha=(alpha, alpha), layers=layers,
                    hubs_shared_across_layers=True)


def random_f32_rows(seed: int, rows: int, n: int, distinct: Optional[int] = None) -> np.ndarray:
    """Non-negative float32 rows for selection tests.  With ``distinct`` the
    values come from a small set so that ties are frequent."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 77]))
    if distinct is not None:
        vals = rng.random(distinct).astype(np.float32)
        return vals[rng.integers(0, distinct, size=(rows, n))]
    return rng.random((rows, n), dtype=np.float32)
