"""The C ABI: the library loads, exports what include/kvsel.h declares, and
rejects invalid arguments on the host before anything is enqueued.  None of
these calls reaches a kernel launch, so they run without a GPU."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from token_selection_tsp_amd import kvsel

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvsel.h")
FAKE = 0x10000          # 16-byte aligned stand-in device address: never dereferenced
MISALIGNED = 0x10004

EINVAL, EUNSUP, EWS = kvsel.KVSEL_EINVAL, kvsel.KVSEL_EUNSUPPORTED, kvsel.KVSEL_EWORKSPACE


@pytest.fixture(scope="module")
def lib():
    return kvsel.library()


def _v(cu):
    arr = np.ascontiguousarray(np.asarray(cu, dtype=np.int32))
    v = kvsel.Varlen(len(cu) - 1, arr.ctypes.data)
    v._keep = arr
    return v


def _k(ks):
    arr = np.ascontiguousarray(np.asarray(ks, dtype=np.int32))
    p = arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    p._keep = arr
    return p


def test_header_declarations_are_exported(lib):
    text = open(HEADER).read()
    declared = set(re.findall(r"\b(kvsel_[a-z0-9_]+)\s*\(", text))
    declared -= {"kvsel_varlen"}
    out = subprocess.run(["nm", "-D", "--defined-only", kvsel.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (kvsel_\w+)", out))
    assert declared == exported == set(kvsel.EXPORTED)
    for name in declared:
        assert hasattr(lib, name)


def test_status_strings_and_version(lib):
    assert lib.kvsel_abi_version() == 1
    assert lib.kvsel_status_string(0) == b"ok"
    for s in range(1, 5):
        assert lib.kvsel_status_string(s) not in (b"ok", b"unknown status")
    assert lib.kvsel_status_string(99) == b"unknown status"


def test_selected_length_host_math(lib):
    cu = [0, 100, 130, 1130]
    ks = [10, 500, 0]
    w = 8
    want = sum(oracle.budget_length(n, w, k) for n, k in zip(np.diff(cu), ks))
    assert lib.kvsel_selected_length(ctypes.byref(_v(cu)), _k(ks), w) == want == 18 + 30 + 8
    assert lib.kvsel_selected_length(ctypes.byref(_v(cu)), _k([1, -1, 2]), w) == -1
    assert lib.kvsel_selected_length(ctypes.byref(_v([0, 5])), _k([1]), 6) == -1   # n < w
    assert kvsel.selected_length([0, 1024], [256], 8) == 264


@pytest.mark.parametrize("seed", range(5))
def test_pivot_layer_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    for layers in (1, 2, 3, 16, 40):
        e = rng.normal(size=layers).astype(np.float32)
        if layers > 3:
            e[layers // 2] = e[layers // 2 - 1] - 5.0           # one planted sharp drop
        assert kvsel.pivot_layer(e) == oracle.pivot_layer(e.astype(np.float64))
    ties = np.array([5, 4, 3, 2, 1], dtype=np.float32)
    assert kvsel.pivot_layer(ties) == oracle.pivot_layer(ties) == 1


def test_pivot_layer_rejects(lib):
    e = np.array([1.0, np.nan], dtype=np.float32)
    ep = e.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    assert lib.kvsel_pivot_layer(ep, 2, 1) == -1
    assert lib.kvsel_pivot_layer(None, 2, 1) == -1
    assert lib.kvsel_pivot_layer(ep, 0, 1) == -1
    strided = np.array([3.0, 9.0, 1.0, 9.0], dtype=np.float32)   # entropies 3, 1 at stride 2
    assert lib.kvsel_pivot_layer(strided.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), 2, 2) == 1


def _score(lib, cu=(0, 64), h_q=8, h_kv=2, d=64, w=8, scale=0.125, q=FAKE, k=FAKE, score=FAKE,
           lse=None, ws=FAKE, ws_bytes=None):
    v = _v(cu)
    if ws_bytes is None:
        ws_bytes = lib.kvsel_window_score_workspace(ctypes.byref(v), h_q, h_kv, d, w) if d in (64, 128) else 1 << 20
    return lib.kvsel_window_score(ctypes.byref(v), q, k, h_q, h_kv, d, w, scale, score, lse, ws,
                                  ws_bytes, None)


def test_window_score_rejects(lib):
    assert _score(lib, cu=(0, 64), h_q=6, h_kv=4) == EINVAL          # h_q % h_kv
    assert _score(lib, w=0) == EINVAL
    assert _score(lib, cu=(0, 64, 70), w=8) == EINVAL                 # second sequence shorter than w
    assert _score(lib, cu=(1, 64)) == EINVAL                          # cu[0] != 0
    assert _score(lib, cu=(0, 64, 32)) == EINVAL                      # decreasing
    assert _score(lib, d=96) == EUNSUP
    assert _score(lib, d=256) == EUNSUP
    assert _score(lib, scale=0.0) == EINVAL
    assert _score(lib, scale=float("nan")) == EINVAL
    assert _score(lib, scale=float("inf")) == EINVAL
    assert _score(lib, q=None) == EINVAL
    assert _score(lib, k=MISALIGNED) == EINVAL
    assert _score(lib, score=MISALIGNED) == EINVAL
    assert _score(lib, lse=MISALIGNED) == EINVAL
    assert _score(lib, ws=None) == EWS
    assert _score(lib, ws_bytes=16) == EWS
    v0 = kvsel.Varlen(0, None)
    assert lib.kvsel_window_score(ctypes.byref(v0), FAKE, FAKE, 8, 2, 64, 8, 0.125, FAKE, None,
                                  FAKE, 1 << 20, None) == EINVAL
    assert lib.kvsel_window_score(None, FAKE, FAKE, 8, 2, 64, 8, 0.125, FAKE, None, FAKE, 1 << 20,
                                  None) == EINVAL


def test_window_score_workspace_is_pure(lib):
    v = _v((0, 131072))
    a = lib.kvsel_window_score_workspace(ctypes.byref(v), 32, 8, 128, 32)
    b = lib.kvsel_window_score_workspace(ctypes.byref(v), 32, 8, 128, 32)
    assert a == b > 0 and a % 256 == 0
    small = lib.kvsel_window_score_workspace(ctypes.byref(_v((0, 1024))), 32, 8, 128, 32)
    assert 0 < small < a
    assert lib.kvsel_window_score_workspace(ctypes.byref(v), 32, 8, 96, 32) == 0
    assert lib.kvsel_window_score_workspace(ctypes.byref(v), 30, 8, 128, 32) == 0
    assert lib.kvsel_window_score_workspace(ctypes.byref(_v((0, 16))), 32, 8, 128, 32) == 0


def _units_from_workspace(lib, cu, h_kv=8):
    """Work units (chunks) per launch of the score plan, read back from the
    workspace size: one float2 per unit, KV head and row (128 rows), rounded
    up to 256 bytes."""
    ws = lib.kvsel_window_score_workspace(ctypes.byref(_v(cu)), 32, h_kv, 128, 32)
    per_unit = h_kv * 128 * 8
    return ws // per_unit, ws


@pytest.mark.parametrize("lens,chunk", [
    ((131072,), 4096),        # one round of 256 work-groups: the benchmark's shape
    ((32768,), 1024),         # small sequences shrink the chunk to fill the GPU once
    ((65536,), 2048),
    ((1 << 20,), 6656),       # long sequences: fewer, longer rounds
    ((24925, 31136, 29368, 18757, 31061, 32087, 31917, 6413), 7424),   # one round instead of two
])
def test_score_planner_chunks(lib, lens, chunk):
    # the planner's chunk, read back through the workspace size (a pure
    # function of the lengths and shapes)
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    units, ws = _units_from_workspace(lib, cu)
    want = sum(-(-n // chunk) for n in lens)
    assert units == want, (units, want, ws)
    assert ws == -(-want * 8 * 128 * 8 // 256) * 256


def _score_ent(lib, cu=(0, 64), h_q=8, h_kv=2, d=64, w=8, scale=0.125, score=FAKE, lse=None,
               row_ent=FAKE, mean_ent=None, ws=FAKE, ws_bytes=None):
    v = _v(cu)
    if ws_bytes is None:
        ws_bytes = lib.kvsel_window_score_entropy_workspace(ctypes.byref(v), h_q, h_kv, d, w) if d in (64, 128) else 1 << 20
    return lib.kvsel_window_score_entropy(ctypes.byref(v), FAKE, FAKE, h_q, h_kv, d, w, scale, score, lse,
                                          row_ent, mean_ent, ws, ws_bytes, None)


def test_window_score_entropy_rejects(lib):
    assert _score_ent(lib, row_ent=None) == EINVAL
    assert _score_ent(lib, row_ent=MISALIGNED) == EINVAL
    assert _score_ent(lib, mean_ent=MISALIGNED) == EINVAL
    assert _score_ent(lib, cu=(0, 64), h_q=6, h_kv=4) == EINVAL
    assert _score_ent(lib, d=96) == EUNSUP
    v = _v((0, 64))
    plain = lib.kvsel_window_score_workspace(ctypes.byref(v), 8, 2, 64, 8)
    assert _score_ent(lib, ws_bytes=plain) == EWS          # the plain score's workspace is too small
    assert _score_ent(lib, ws=None) == EWS


def test_window_score_entropy_workspace(lib):
    for cu, h_q, h_kv, d, w in (((0, 131072), 32, 8, 128, 32), ((0, 1024), 8, 2, 64, 8),
                                ((0, 3000, 3100, 9000), 16, 2, 128, 24)):
        v = _v(cu)
        plain = lib.kvsel_window_score_workspace(ctypes.byref(v), h_q, h_kv, d, w)
        ent = lib.kvsel_window_score_entropy_workspace(ctypes.byref(v), h_q, h_kv, d, w)
        assert ent > plain > 0 and ent % 256 == 0
        # at least one float per KV head and window row for every chunk of keys
        assert ent - plain >= h_kv * w * (h_q // h_kv) * 4
    assert lib.kvsel_window_score_entropy_workspace(ctypes.byref(_v((0, 16))), 32, 8, 128, 32) == 0


@pytest.mark.parametrize("seed", range(5))
def test_pivot_layer_sparsity_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    for layers in (1, 2, 3, 16, 40):
        e = rng.normal(size=layers).astype(np.float32)
        sp = rng.uniform(size=layers).astype(np.float32)
        if seed % 2:
            sp = np.sort(sp)[::-1].copy()                          # sparsity never rises: fallback rule
        want = oracle.pivot_layer_sparsity(e.astype(np.float64), sp.astype(np.float64))
        assert kvsel.pivot_layer_sparsity(e, sp) == want


def test_pivot_layer_sparsity_rejects(lib):
    fp = ctypes.POINTER(ctypes.c_float)
    e = np.array([3.0, 1.0], dtype=np.float32)
    sp = np.array([0.1, np.inf], dtype=np.float32)
    ok = np.array([0.1, 0.2], dtype=np.float32)
    assert lib.kvsel_pivot_layer_sparsity(e.ctypes.data_as(fp), sp.ctypes.data_as(fp), 2, 1) == -1
    assert lib.kvsel_pivot_layer_sparsity(None, ok.ctypes.data_as(fp), 2, 1) == -1
    assert lib.kvsel_pivot_layer_sparsity(e.ctypes.data_as(fp), None, 2, 1) == -1
    assert lib.kvsel_pivot_layer_sparsity(e.ctypes.data_as(fp), ok.ctypes.data_as(fp), 0, 1) == -1
    assert lib.kvsel_pivot_layer_sparsity(e.ctypes.data_as(fp), ok.ctypes.data_as(fp), 2, 0) == -1
    assert lib.kvsel_pivot_layer_sparsity(e.ctypes.data_as(fp), ok.ctypes.data_as(fp), 2, 1) == 1
    # stats rows [entropy, sparsity, variance] read at stride 3
    st = np.array([[5.0, 0.3, 0], [4.0, 0.2, 0], [1.0, 0.25, 0]], dtype=np.float32)
    assert lib.kvsel_pivot_layer_sparsity(st[:, 0:].ctypes.data_as(fp),
                                          st[:, 1:].ctypes.data_as(fp), 3, 3) == 2


def test_accumulate_stats_rejects(lib):
    v = _v((0, 100))
    f = lib.kvsel_accumulate_stats
    need = lib.kvsel_accumulate_stats_workspace(ctypes.byref(v), 8)
    assert need > 0
    assert f(ctypes.byref(v), None, 8, 32, 4, None, FAKE, None, None, None, 0, None) == EINVAL
    assert f(ctypes.byref(v), FAKE, 0, 32, 4, None, FAKE, None, None, None, 0, None) == EINVAL
    assert f(ctypes.byref(v), FAKE, 8, 0, 4, None, FAKE, None, None, None, 0, None) == EINVAL
    assert f(ctypes.byref(v), FAKE, 8, 32, 4, MISALIGNED, FAKE, None, None, None, 0, None) == EINVAL
    assert f(ctypes.byref(v), FAKE, 8, 32, 4, None, None, None, FAKE, None, 0, None) == EWS
    assert f(ctypes.byref(v), FAKE, 8, 32, 4, None, None, None, FAKE, FAKE, need - 8, None) == EWS
    # nothing requested: a valid no-op
    assert f(ctypes.byref(v), FAKE, 8, 32, 4, None, None, None, None, None, 0, None) == 0
    # a sequence shorter than the window, or empty, has no window distribution
    for cu in ((0, 100, 131), (0, 100, 100), (0, 0)):
        vs = _v(cu)
        ws = lib.kvsel_accumulate_stats_workspace(ctypes.byref(vs), 8)
        assert f(ctypes.byref(vs), FAKE, 8, 32, 4, None, FAKE, FAKE, FAKE, FAKE, max(ws, 16), None) == EINVAL
    # n == w is the smallest valid sequence
    vs = _v((0, 32))
    assert f(ctypes.byref(vs), FAKE, 8, 32, 4, None, None, None, None, None, 0, None) == 0


def test_topk_rejects(lib):
    v = _v((0, 100, 150))
    f = lib.kvsel_topk
    assert f(ctypes.byref(v), FAKE, 1, 8, _k([5, -1]), FAKE, None, 0, None) == EINVAL
    assert f(ctypes.byref(v), FAKE, 0, 8, _k([5, 5]), FAKE, None, 0, None) == EINVAL
    assert f(ctypes.byref(v), FAKE, 1, 51, _k([5, 5]), FAKE, None, 0, None) == EINVAL   # w > n
    assert f(ctypes.byref(v), FAKE, 1, 0, _k([5, 5]), FAKE, None, 0, None) == EINVAL
    assert f(ctypes.byref(v), MISALIGNED, 1, 8, _k([5, 5]), FAKE, None, 0, None) == EINVAL
    assert f(ctypes.byref(v), FAKE, 1, 8, None, FAKE, None, 0, None) == EINVAL
    need = lib.kvsel_topk_workspace(ctypes.byref(v), 9, 8)
    assert need > 0 and need == lib.kvsel_topk_workspace(ctypes.byref(v), 9, 8)
    assert lib.kvsel_topk_workspace(ctypes.byref(v), 9, 51) == 0                       # w > n
    assert f(ctypes.byref(v), FAKE, 1, 8, _k([5, 5]), FAKE, None, 0, None) == EWS
    assert f(ctypes.byref(v), FAKE, 1, 8, _k([5, 5]), FAKE, FAKE, 16, None) == EWS
    big = _v((0, 9_000_000))
    assert f(ctypes.byref(big), FAKE, 1, 8, _k([5]), FAKE, FAKE, 1 << 30, None) == EUNSUP


def test_gather_rejects(lib):
    v = _v((0, 100))
    f = lib.kvsel_gather
    ks = _k([10])
    assert f(ctypes.byref(v), FAKE, 8, 24, FAKE, 1, ks, 8, FAKE, None) == EINVAL      # row_bytes % 16
    assert f(ctypes.byref(v), FAKE, 8, 256, FAKE, 2, ks, 8, FAKE, None) == EINVAL     # idx_per_head
    assert f(ctypes.byref(v), FAKE, 0, 256, FAKE, 1, ks, 8, FAKE, None) == EINVAL
    assert f(ctypes.byref(v), FAKE, 8, 256, FAKE, 1, _k([-2]), 8, FAKE, None) == EINVAL
    assert f(ctypes.byref(v), FAKE, 8, 256, MISALIGNED, 1, ks, 8, FAKE, None) == EINVAL
    assert f(ctypes.byref(v), None, 8, 256, FAKE, 1, ks, 8, FAKE, None) == EINVAL


def test_gather_paged_rejects(lib):
    v = _v((0, 100))
    ks = _k([10])                                          # L = 10 + 8 = 18 rows
    f = lib.kvsel_gather_paged

    def call(dst=None, cache=FAKE, table=FAKE, num_blocks=4, block_size=16, max_blocks=2, pages=True,
             row_bytes=256):
        ks_addr = ctypes.cast(ks, ctypes.c_void_p).value   # the job struct holds a bare address
        job = (kvsel.GatherJob * 1)(kvsel.GatherJob(FAKE, dst, FAKE, ks_addr, 8, row_bytes, 1, 0))
        pc = (kvsel.PagedCache * 1)(kvsel.PagedCache(cache, table, num_blocks, block_size, max_blocks, 0))
        return f(ctypes.byref(v), 8, 1, job, pc if pages else None, None)

    assert call(dst=FAKE) == EINVAL                        # the cache is the destination
    assert call(pages=False) == EINVAL
    assert call(cache=None) == EINVAL
    assert call(cache=MISALIGNED) == EINVAL
    assert call(table=None) == EINVAL
    assert call(table=FAKE + 2) == EINVAL                  # block table not 4-byte aligned
    assert call(block_size=0) == EINVAL
    assert call(num_blocks=0) == EINVAL
    assert call(max_blocks=1) == EINVAL                    # 1 * 16 < 18 rows
    assert call(row_bytes=24) == EINVAL


def test_library_path_has_no_cpu_fallback():
    """The binding only ever calls into libkvsel: no module under the package
    imports the oracle or computes the method on the host."""
    pkg = os.path.join(ROOT, "token_selection_tsp_amd")
    for name in os.listdir(pkg):
        if name.endswith(".py"):
            src = open(os.path.join(pkg, name)).read()
            assert not re.search(r"^\s*(import|from)\s+oracle\b", src, re.M), name
            assert "import numpy" not in src or name in ("kvsel.py", "synth.py"), name


def test_window_score_noalloc_rejects_before_any_gpu_call(lib):
    """Invalid arguments and inputs whose partials exceed the fixed scratch
    are refused on the host (no GPU here, so nothing can have run)."""
    f = lib.kvsel_window_score_noalloc
    v = _v((0, 1000))
    assert f(ctypes.byref(v), None, FAKE, 8, 2, 64, 8, 0.125, FAKE, None, None) == EINVAL
    assert f(ctypes.byref(v), FAKE, FAKE, 8, 3, 64, 8, 0.125, FAKE, None, None) == EINVAL     # h_q % h_kv
    assert f(ctypes.byref(v), FAKE, FAKE, 8, 2, 64, 1001, 0.125, FAKE, None, None) == EINVAL  # w > n
    assert f(ctypes.byref(v), FAKE, FAKE, 8, 2, 64, 8, 0.0, FAKE, None, None) == EINVAL
    assert f(ctypes.byref(v), FAKE, FAKE, 8, 2, 64, 8, 0.125, MISALIGNED, None, None) == EINVAL
    assert f(ctypes.byref(v), FAKE, FAKE, 8, 2, 96, 8, 0.125, FAKE, None, None) == EUNSUP
    # 2^20 keys at 64 KV heads: the partials need more than the 4 MiB scratch
    big = _v((0, 1 << 20))
    assert lib.kvsel_window_score_workspace(ctypes.byref(big), 64, 64, 128, 1) > 4 << 20
    assert f(ctypes.byref(big), FAKE, FAKE, 64, 64, 128, 1, 0.125, FAKE, None, None) == EWS

