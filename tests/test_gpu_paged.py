"""Gather into a paged cache on the GPU against the oracle, bit for bit:
every slot of every cache (written rows, untouched slots, skipped blocks)."""
import numpy as np
import pytest

import oracle
import token_selection_tsp_amd as kv
from token_selection_tsp_amd import synth
from gpu_util import dev_bf16, host, log

pytestmark = pytest.mark.gpu


def _i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _tables(rng, lengths, bs, spare_blocks, holes=True):
    """A shuffled block table covering every selection, plus spare blocks
    nothing maps to; with ``holes`` one block is unmapped (-1) and one is out
    of range, so the rows that map there are skipped."""
    need = [-(-L // bs) for L in lengths]
    max_blocks = max(need) + 1
    num_blocks = sum(need) + spare_blocks
    perm = rng.permutation(num_blocks)
    table = np.full((len(lengths), max_blocks), -1, dtype=np.int32)
    at = 0
    for b, nb in enumerate(need):
        table[b, :nb] = perm[at:at + nb]
        at += nb
    if holes:
        b = int(np.argmax(need))
        if need[b] >= 2:
            table[b, 1] = -1
            table[b, need[b] - 1] = num_blocks + 3
    return table, num_blocks


@pytest.mark.parametrize("bs", [16, 1, 7])
def test_gather_paged_matches_oracle(bs):
    lens = [300, 17, 4096, 1000]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, heads, w = int(cu[-1]), 4, 8
    rng = np.random.default_rng(40 + bs)
    kbits = rng.integers(0, 2 ** 16, size=(T, heads, 64), dtype=np.uint16)
    vbits = rng.integers(0, 2 ** 16, size=(T, heads, 24), dtype=np.uint16)
    hbits = rng.integers(0, 2 ** 16, size=(T, 1, 2056), dtype=np.uint16)
    k_kv, k_ts = [40, 3, 1000, 999], [100, 0, 2048, 5]
    lk = [oracle.budget_length(n, w, k) for n, k in zip(lens, k_kv)]
    lt = [oracle.budget_length(n, w, k) for n, k in zip(lens, k_ts)]
    ik = np.concatenate([rng.integers(0, n, size=(heads, l)) for n, l in zip(lens, lk)], axis=1)
    it = np.concatenate([rng.integers(0, n, size=(1, l)) for n, l in zip(lens, lt)], axis=1)
    tk, nk = _tables(rng, lk, bs, spare_blocks=3)
    tt, nt = _tables(rng, lt, bs, spare_blocks=2, holes=False)
    caches = [rng.integers(0, 2 ** 16, size=(nk, bs) + s.shape[1:], dtype=np.uint16) for s in (kbits, vbits)]
    caches.append(rng.integers(0, 2 ** 16, size=(nt, bs) + hbits.shape[2:], dtype=np.uint16))
    dev_caches = [dev_bf16(c) for c in caches]
    log(f"gather_paged block {bs}")
    kv.gather_paged(cu, w, [(dev_bf16(kbits), _i32(ik), k_kv, dev_caches[0], _i32(tk)),
                            (dev_bf16(vbits), _i32(ik), k_kv, dev_caches[1], _i32(tk)),
                            (dev_bf16(hbits[:, 0]), _i32(it[0]), k_ts, dev_caches[2], _i32(tt))])
    for got, src, idx, ln, tab, c0 in ((dev_caches[0], kbits, ik, lk, tk, caches[0]),
                                       (dev_caches[1], vbits, ik, lk, tk, caches[1]),
                                       (dev_caches[2], hbits, it, lt, tt, caches[2][:, :, None])):
        want = oracle.gather_paged(src, cu, idx, ln, tab, bs, c0)
        assert np.array_equal(host(got).view(np.uint16).reshape(want.shape), want)


def test_gather_paged_full_size():
    """The N=128K workload's K and V (4096 + 32 rows per KV head) into caches
    of 16-token blocks, as the benchmark runs it: the whole caches against
    the oracle."""
    wl = synth.WORKLOADS["n128k_gqa32x8_d128"]
    x = synth.layer_inputs(wl, parts=("k", "v"))
    cu = x["cu_seqlens"]
    n, w = int(cu[-1]), wl.w
    k_kv = wl.kv_tokens()
    L = oracle.budget_length(n, w, int(k_kv[0]))
    rng = np.random.default_rng(77)
    idx = np.stack([np.concatenate([np.sort(rng.choice(n - w, L - w, replace=False)), np.arange(n - w, n)])
                    for _ in range(wl.h_kv)]).astype(np.int32)
    bs = 16
    table, nb = _tables(rng, [L], bs, spare_blocks=5, holes=False)
    caches = [np.zeros((nb, bs, wl.h_kv, wl.d), dtype=np.uint16) for _ in range(2)]
    dev_caches = [dev_bf16(c) for c in caches]
    log("gather_paged full size")
    kv.gather_paged(cu, w, [(dev_bf16(x["k"]), _i32(idx), k_kv, dev_caches[0], _i32(table)),
                            (dev_bf16(x["v"]), _i32(idx), k_kv, dev_caches[1], _i32(table))])
    for got, src, c0 in ((dev_caches[0], x["k"], caches[0]), (dev_caches[1], x["v"], caches[1])):
        want = oracle.gather_paged(src, cu, idx, [L], table, bs, c0)
        assert np.array_equal(host(got).view(np.uint16), want)
