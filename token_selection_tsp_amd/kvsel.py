"""Python binding of libkvsel (ctypes).

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI declared in ``include/kvsel.h``.  PyTorch supplies device
memory (outputs and workspaces are ``torch.empty`` on the inputs' device) and
the stream (``torch.cuda.current_stream()``).  There is no fallback: if the
library is missing or a call fails, a ``KvselError`` is raised.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvsel.so")

KVSEL_OK, KVSEL_EINVAL, KVSEL_EUNSUPPORTED, KVSEL_EWORKSPACE, KVSEL_ELAUNCH = range(5)

EXPORTED = (
    "kvsel_status_string", "kvsel_abi_version", "kvsel_selected_length",
    "kvsel_window_score_workspace", "kvsel_window_score", "kvsel_window_score_lse",
    "kvsel_accumulate_stats_workspace", "kvsel_accumulate_stats",
    "kvsel_topk_workspace", "kvsel_topk", "kvsel_topk2_workspace", "kvsel_topk2",
    "kvsel_gather", "kvsel_gather_multi", "kvsel_pivot_layer",
    "kvsel_window_score_entropy_workspace", "kvsel_window_score_entropy", "kvsel_pivot_layer_sparsity",
    "kvsel_gather_paged", "kvsel_probe_read", "kvsel_window_score_noalloc",
    "kvsel_window_score_stats_workspace", "kvsel_window_score_stats",
)

GATHER_MAX_JOBS = 4


class KvselError(RuntimeError):
    def __init__(self, func: str, status: int, msg: str = ""):
        self.status = status
        super().__init__(f"{func} failed with status {status} ({msg})")


# Host int32 arrays cross the boundary as plain addresses (c_void_p): the same
# ABI as int32_t*, without a ctypes pointer object per argument.
class Varlen(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("cu_seqlens", ctypes.c_void_p)]


class PagedCache(ctypes.Structure):
    _fields_ = [("cache", ctypes.c_void_p), ("block_table", ctypes.c_void_p), ("num_blocks", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("max_blocks", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class GatherJob(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p), ("dst", ctypes.c_void_p), ("idx", ctypes.c_void_p),
                ("k_host", ctypes.c_void_p), ("heads", ctypes.c_int32),
                ("row_bytes", ctypes.c_int32), ("idx_per_head", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


_lib = None


def library() -> ctypes.CDLL:
    """Load libkvsel.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise KvselError("load", -1, f"{LIB_PATH} is not built; run `python -m token_selection_tsp_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int32
    VP = ctypes.POINTER(Varlen)
    IP = ctypes.c_void_p   # host int32 arrays, passed by address
    S = ctypes.c_size_t
    sig = {
        "kvsel_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "kvsel_abi_version": (ctypes.c_int, []),
        "kvsel_selected_length": (ctypes.c_int64, [VP, IP, I]),
        "kvsel_window_score_workspace": (S, [VP, I, I, I, I]),
        "kvsel_window_score": (ctypes.c_int, [VP, P, P, I, I, I, I, ctypes.c_float, P, P, P, S, P]),
        "kvsel_window_score_lse": (ctypes.c_int, [VP, P, P, I, I, I, I, ctypes.c_float, P, P, P]),
        "kvsel_window_score_noalloc": (ctypes.c_int, [VP, P, P, I, I, I, I, ctypes.c_float, P, P, P]),
        "kvsel_window_score_stats_workspace": (S, [VP, I, I, I, I]),
        "kvsel_window_score_stats": (ctypes.c_int, [VP, P, P, I, I, I, I, ctypes.c_float, P, P, P, P, P, P, P, S,
                                                    P]),
        "kvsel_window_score_entropy_workspace": (S, [VP, I, I, I, I]),
        "kvsel_window_score_entropy": (ctypes.c_int, [VP, P, P, I, I, I, I, ctypes.c_float, P, P, P, P,
                                                      P, S, P]),
        "kvsel_accumulate_stats_workspace": (S, [VP, I]),
        "kvsel_accumulate_stats": (ctypes.c_int, [VP, P, I, I, I, P, P, P, P, P, S, P]),
        "kvsel_topk_workspace": (S, [VP, I, I]),
        "kvsel_topk": (ctypes.c_int, [VP, P, I, I, IP, P, P, S, P]),
        "kvsel_topk2_workspace": (S, [VP, I, I, I]),
        "kvsel_topk2": (ctypes.c_int, [VP, I, P, I, IP, P, P, I, IP, P, P, S, P]),
        "kvsel_gather": (ctypes.c_int, [VP, P, I, I, P, I, IP, I, P, P]),
        "kvsel_gather_multi": (ctypes.c_int, [VP, I, I, ctypes.POINTER(GatherJob), P]),
        "kvsel_gather_paged": (ctypes.c_int, [VP, I, I, ctypes.POINTER(GatherJob), ctypes.POINTER(PagedCache), P]),
        "kvsel_pivot_layer": (I, [ctypes.POINTER(ctypes.c_float), I, I]),
        "kvsel_probe_read": (ctypes.c_int, [P, ctypes.c_int64, I, I, ctypes.c_int64, I, P, P]),
        "kvsel_pivot_layer_sparsity": (I, [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float),
                                           I, I]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(func: str, status: int) -> None:
    if status != KVSEL_OK:
        msg = library().kvsel_status_string(status).decode()
        raise KvselError(func, status, msg)


def _int32_array(x, name: str) -> np.ndarray:
    # host int32 arrays pass through as they are (the common case: these are
    # per-call host metadata, and the conversion below would dominate a short
    # call's host time)
    if isinstance(x, np.ndarray) and x.dtype == np.int32 and x.ndim == 1 and x.flags.c_contiguous:
        return x
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    a = np.ascontiguousarray(np.asarray(x).reshape(-1), dtype=np.int64)
    if a.size and (a.min() < -2**31 or a.max() >= 2**31):
        raise ValueError(f"{name} does not fit int32")
    return np.ascontiguousarray(a.astype(np.int32))


def _varlen(cu_seqlens) -> Tuple[Varlen, np.ndarray]:
    cu = _int32_array(cu_seqlens, "cu_seqlens")
    if cu.size < 2:
        raise ValueError("cu_seqlens needs at least two entries")
    v = Varlen(cu.size - 1, cu.ctypes.data)
    v._keep = cu   # the struct holds a bare address: keep the array alive with it
    return v, cu


def _iptr(a: np.ndarray) -> int:
    """Address of a host int32 array (kept alive by the caller for the call)."""
    return a.ctypes.data


def _stream(t) -> ctypes.c_void_p:
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t, dtype, name: str):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _buf(t, dtype, shape, like, name: str):
    """A caller-supplied buffer: a contiguous CUDA tensor of ``dtype`` and
    exactly ``shape`` on ``like``'s device.  The C ABI sees a bare pointer,
    so a smaller buffer would be read or written past its end: checked here,
    before anything is launched."""
    _dev(t, dtype, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != like.device:
        raise ValueError(f"{name} is on {t.device}, the inputs on {like.device}")
    return t


def _same_device(like, *named) -> None:
    for name, t in named:
        if t is not None and t.device != like.device:
            raise ValueError(f"{name} is on {t.device}, the inputs on {like.device}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _workspace(nbytes: int, like, workspace=None):
    import torch
    if nbytes == 0:
        return None, 0
    if workspace is not None and workspace.numel() * workspace.element_size() >= nbytes:
        return workspace, workspace.numel() * workspace.element_size()
    return torch.empty(nbytes, dtype=torch.uint8, device=like.device), nbytes


# ------------------------------------------------------------------ calls

_selected_memo: dict = {}


def selected_length(cu_seqlens, k_per_seq, w: int) -> int:
    v, cu = _varlen(cu_seqlens)
    kk = _int32_array(k_per_seq, "k_per_seq")
    if kk.size != v.batch:
        raise ValueError("one budget per sequence")
    # memoised for small batches only (the key holds the arrays' bytes)
    key = (cu.tobytes(), kk.tobytes(), int(w)) if cu.size <= 1024 else None
    L = _selected_memo.get(key) if key is not None else None
    if L is None:
        L = library().kvsel_selected_length(ctypes.byref(v), _iptr(kk), w)
        if L < 0:
            raise KvselError("kvsel_selected_length", KVSEL_EINVAL, "invalid argument")
        if key is not None:
            if len(_selected_memo) >= 256:
                _selected_memo.clear()
            _selected_memo[key] = L
    return int(L)


def window_score(q_win, k, cu_seqlens, scale: Optional[float] = None, return_lse: bool = False,
                 out=None, workspace=None, lse_in=None):
    """Window-attention score per KV head and token.

    q_win bf16 [B, w, h_q, d], k bf16 [T, h_kv, d] (CUDA tensors),
    cu_seqlens host [B+1].  Returns fp32 ``score`` [h_kv, T] (and fp32
    ``lse`` [B, h_q, w] when ``return_lse``).  With ``lse_in`` (fp32
    [B, h_q, w], the rows' natural-log normalisers from the layer's own
    attention) the score takes one pass over K (kvsel_window_score_lse)."""
    import torch
    _dev(q_win, torch.bfloat16, "q_win")
    _dev(k, torch.bfloat16, "k")
    if q_win.dim() != 4 or k.dim() != 3:
        raise ValueError("q_win must be [B, w, h_q, d] and k [T, h_kv, d]")
    B, w, h_q, d = q_win.shape
    T, h_kv, dk = k.shape
    if dk != d:
        raise ValueError("head dims differ")
    v, cu = _varlen(cu_seqlens)
    if v.batch != B or int(cu[-1]) != T:
        raise ValueError("cu_seqlens does not match the tensors")
    _same_device(k, ("q_win", q_win))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    scale = float(np.float32(scale))
    if out is not None:
        score = _buf(out, torch.float32, (h_kv, T), k, "out")
    else:
        score = torch.empty((h_kv, T), dtype=torch.float32, device=k.device)
    lib = library()
    if lse_in is not None:
        if return_lse:
            raise ValueError("lse_in and return_lse exclude each other")
        _buf(lse_in, torch.float32, (B, h_q, w), k, "lse_in")
        st = lib.kvsel_window_score_lse(ctypes.byref(v), q_win.data_ptr(), k.data_ptr(), h_q, h_kv, d, w,
                                        scale, lse_in.data_ptr(), score.data_ptr(), _stream(k))
        _check("kvsel_window_score_lse", st)
        return score
    lse = torch.empty((B, h_q, w), dtype=torch.float32, device=k.device) if return_lse else None
    nbytes = lib.kvsel_window_score_workspace(ctypes.byref(v), h_q, h_kv, d, w)
    ws, wsb = _workspace(nbytes, k, workspace)
    st = lib.kvsel_window_score(ctypes.byref(v), q_win.data_ptr(), k.data_ptr(), h_q, h_kv, d, w,
                                scale, score.data_ptr(), _ptr(lse), _ptr(ws), wsb, _stream(k))
    _check("kvsel_window_score", st)
    return (score, lse) if return_lse else score


def window_score_stats(q_win, k, cu_seqlens, scale: Optional[float] = None, return_lse: bool = False,
                       c_in=None, c_out=None, want_tok: bool = True, want_stats: bool = True, out=None,
                       tok_out=None, stats_out=None, workspace=None):
    """``window_score`` with the work of ``accumulate_stats`` folded into
    its second pass (kvsel_window_score_stats).  Returns (score, c_out, tok,
    stats), or (score, lse, c_out, tok, stats) with ``return_lse``; absent
    outputs are None.  ``c_out`` is allocated when ``c_in`` is given and
    ``c_out`` is not, as ``accumulate_stats`` does; ``out``, ``tok_out``
    (fp32 [T]) and ``stats_out`` (fp32 [B, 3]) are written in place when
    given."""
    import torch
    _dev(q_win, torch.bfloat16, "q_win")
    _dev(k, torch.bfloat16, "k")
    if q_win.dim() != 4 or k.dim() != 3:
        raise ValueError("q_win must be [B, w, h_q, d] and k [T, h_kv, d]")
    B, w, h_q, d = q_win.shape
    T, h_kv, dk = k.shape
    if dk != d:
        raise ValueError("head dims differ")
    v, cu = _varlen(cu_seqlens)
    if v.batch != B or int(cu[-1]) != T:
        raise ValueError("cu_seqlens does not match the tensors")
    _same_device(k, ("q_win", q_win))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    scale = float(np.float32(scale))
    dev = k.device
    if out is not None:
        score = _buf(out, torch.float32, (h_kv, T), k, "out")
    else:
        score = torch.empty((h_kv, T), dtype=torch.float32, device=dev)
    if c_in is not None:
        _buf(c_in, torch.float32, (h_kv, T), k, "c_in")
        if c_out is None:
            c_out = torch.empty((h_kv, T), dtype=torch.float32, device=dev)
    if c_out is not None:
        _buf(c_out, torch.float32, (h_kv, T), k, "c_out")
    lse = torch.empty((B, h_q, w), dtype=torch.float32, device=dev) if return_lse else None
    if tok_out is not None:
        tok = _buf(tok_out, torch.float32, (T,), k, "tok_out")
    else:
        tok = torch.empty(T, dtype=torch.float32, device=dev) if want_tok else None
    if stats_out is not None:
        stats = _buf(stats_out, torch.float32, (B, 3), k, "stats_out")
    else:
        stats = torch.empty((B, 3), dtype=torch.float32, device=dev) if want_stats else None
    lib = library()
    nbytes = lib.kvsel_window_score_stats_workspace(ctypes.byref(v), h_q, h_kv, d, w)
    ws, wsb = _workspace(nbytes, k, workspace)
    st = lib.kvsel_window_score_stats(ctypes.byref(v), q_win.data_ptr(), k.data_ptr(), h_q, h_kv, d, w, scale,
                                      score.data_ptr(), _ptr(lse), _ptr(c_in), _ptr(c_out), _ptr(tok),
                                      _ptr(stats), _ptr(ws), wsb, _stream(k))
    _check("kvsel_window_score_stats", st)
    return (score, lse, c_out, tok, stats) if return_lse else (score, c_out, tok, stats)


def window_score_noalloc(q_win, k, cu_seqlens, out, scale: Optional[float] = None, lse_out=None):
    """``window_score`` through kvsel_window_score_noalloc: no workspace and
    no allocation, here or in the library.  ``out`` fp32 [h_kv, T] (and
    ``lse_out`` fp32 [B, h_q, w], if wanted) are the caller's; the
    library's fixed 4 MiB device scratch holds the partials.  Calls that
    overlap on one GPU race (they share that scratch).  Returns ``out``."""
    import torch
    _dev(q_win, torch.bfloat16, "q_win")
    _dev(k, torch.bfloat16, "k")
    if q_win.dim() != 4 or k.dim() != 3:
        raise ValueError("q_win must be [B, w, h_q, d] and k [T, h_kv, d]")
    B, w, h_q, d = q_win.shape
    T, h_kv, dk = k.shape
    if dk != d:
        raise ValueError("head dims differ")
    v, cu = _varlen(cu_seqlens)
    if v.batch != B or int(cu[-1]) != T:
        raise ValueError("cu_seqlens does not match the tensors")
    _same_device(k, ("q_win", q_win))
    _buf(out, torch.float32, (h_kv, T), k, "out")
    if lse_out is not None:
        _buf(lse_out, torch.float32, (B, h_q, w), k, "lse_out")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    scale = float(np.float32(scale))
    st = library().kvsel_window_score_noalloc(ctypes.byref(v), q_win.data_ptr(), k.data_ptr(), h_q, h_kv, d,
                                              w, scale, out.data_ptr(), _ptr(lse_out), _stream(k))
    _check("kvsel_window_score_noalloc", st)
    return out


def window_score_entropy(q_win, k, cu_seqlens, scale: Optional[float] = None, return_lse: bool = False,
                         want_mean: bool = True, workspace=None):
    """``window_score`` plus the entropy (nats) of every window row's softmax
    (kvsel_window_score_entropy).  Returns (score, row_ent, mean_ent), or
    (score, lse, row_ent, mean_ent) with ``return_lse``: ``row_ent`` fp32
    [B, h_q, w], ``mean_ent`` fp32 [B] (the mean over heads and rows; None
    unless ``want_mean``)."""
    import torch
    _dev(q_win, torch.bfloat16, "q_win")
    _dev(k, torch.bfloat16, "k")
    if q_win.dim() != 4 or k.dim() != 3:
        raise ValueError("q_win must be [B, w, h_q, d] and k [T, h_kv, d]")
    B, w, h_q, d = q_win.shape
    T, h_kv, dk = k.shape
    if dk != d:
        raise ValueError("head dims differ")
    v, cu = _varlen(cu_seqlens)
    if v.batch != B or int(cu[-1]) != T:
        raise ValueError("cu_seqlens does not match the tensors")
    _same_device(k, ("q_win", q_win))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    scale = float(np.float32(scale))
    dev = k.device
    score = torch.empty((h_kv, T), dtype=torch.float32, device=dev)
    lse = torch.empty((B, h_q, w), dtype=torch.float32, device=dev) if return_lse else None
    row_ent = torch.empty((B, h_q, w), dtype=torch.float32, device=dev)
    mean_ent = torch.empty((B,), dtype=torch.float32, device=dev) if want_mean else None
    lib = library()
    nbytes = lib.kvsel_window_score_entropy_workspace(ctypes.byref(v), h_q, h_kv, d, w)
    ws, wsb = _workspace(nbytes, k, workspace)
    st = lib.kvsel_window_score_entropy(ctypes.byref(v), q_win.data_ptr(), k.data_ptr(), h_q, h_kv, d, w,
                                        scale, score.data_ptr(), _ptr(lse), row_ent.data_ptr(),
                                        _ptr(mean_ent), _ptr(ws), wsb, _stream(k))
    _check("kvsel_window_score_entropy", st)
    return (score, lse, row_ent, mean_ent) if return_lse else (score, row_ent, mean_ent)


def accumulate_stats(score, cu_seqlens, w: int, group: int, c_in=None, c_out=None,
                     want_tok: bool = True, want_stats: bool = True, workspace=None):
    """Accumulated score ``c_out = c_in + score`` (when ``c_out`` is given or
    ``c_in`` is), head sum ``tok`` [T] and per-sequence stats [B, 3]
    (entropy, sparsity, variance).  Returns (c_out, tok, stats); absent
    outputs are None."""
    import torch
    _dev(score, torch.float32, "score")
    h_kv, T = score.shape
    v, cu = _varlen(cu_seqlens)
    if int(cu[-1]) != T:
        raise ValueError("cu_seqlens does not match score")
    if score.dim() != 2:
        raise ValueError("score must be [h_kv, T]")
    if c_in is not None:
        _buf(c_in, torch.float32, (h_kv, T), score, "c_in")
        if c_out is None:
            c_out = torch.empty_like(score)
    if c_out is not None:
        _buf(c_out, torch.float32, (h_kv, T), score, "c_out")
    tok = torch.empty(T, dtype=torch.float32, device=score.device) if want_tok else None
    stats = torch.empty((v.batch, 3), dtype=torch.float32, device=score.device) if want_stats else None
    lib = library()
    nbytes = lib.kvsel_accumulate_stats_workspace(ctypes.byref(v), h_kv) if want_stats else 0
    ws, wsb = _workspace(nbytes, score, workspace)
    st = lib.kvsel_accumulate_stats(ctypes.byref(v), score.data_ptr(), h_kv, w, group, _ptr(c_in),
                                    _ptr(c_out), _ptr(tok), _ptr(stats), _ptr(ws), wsb, _stream(score))
    _check("kvsel_accumulate_stats", st)
    return c_out, tok, stats


def topk(keys, cu_seqlens, w: int, k_per_seq, out=None):
    """Top-k plus window for every row of ``keys`` (fp32 [rows, T] or [T]).
    Returns int32 [rows, L] (or [L] for a 1-D input) of sequence-local
    positions, per-sequence selections concatenated."""
    import torch
    _dev(keys, torch.float32, "keys")
    one = keys.dim() == 1
    k2 = keys.view(1, -1) if one else keys
    rows, T = k2.shape
    v, cu = _varlen(cu_seqlens)
    if int(cu[-1]) != T:
        raise ValueError("cu_seqlens does not match keys")
    kk = _int32_array(k_per_seq, "k_per_seq")
    if kk.size != v.batch:
        raise ValueError("one budget per sequence")
    L = selected_length(cu, kk, w)
    if out is not None:
        idx = _buf(out, torch.int32, (L,) if one else (rows, L), keys, "out").view(rows, L)
    else:
        idx = torch.empty((rows, L), dtype=torch.int32, device=keys.device)
    lib = library()
    nbytes = lib.kvsel_topk_workspace(ctypes.byref(v), rows, w)
    ws, wsb = _workspace(nbytes, keys)
    st = lib.kvsel_topk(ctypes.byref(v), k2.data_ptr(), rows, w, _iptr(kk), idx.data_ptr(),
                        _ptr(ws), wsb, _stream(keys))
    _check("kvsel_topk", st)
    return idx.view(-1) if one else idx


def topk2(keys_a, keys_b, cu_seqlens, w: int, k_a, k_b, out_a=None, out_b=None):
    """Both budgets in one launch pair: the same results as
    ``topk(keys_a, cu, w, k_a)`` and ``topk(keys_b, cu, w, k_b)``."""
    import torch
    _dev(keys_a, torch.float32, "keys_a")
    _dev(keys_b, torch.float32, "keys_b")
    v, cu = _varlen(cu_seqlens)
    ka, kb = _int32_array(k_a, "k_a"), _int32_array(k_b, "k_b")
    if ka.size != v.batch or kb.size != v.batch:
        raise ValueError("one budget per sequence")
    outs = []
    _same_device(keys_a, ("keys_b", keys_b))
    for keys, kk, out, name in ((keys_a, ka, out_a, "out_a"), (keys_b, kb, out_b, "out_b")):
        k2 = keys.view(1, -1) if keys.dim() == 1 else keys
        if k2.shape[1] != int(cu[-1]):
            raise ValueError("cu_seqlens does not match keys")
        L = selected_length(cu, kk, w)
        if out is not None:
            shape = (L,) if keys.dim() == 1 else (k2.shape[0], L)
            idx = _buf(out, torch.int32, shape, keys_a, name).view(k2.shape[0], L)
        else:
            idx = torch.empty((k2.shape[0], L), dtype=torch.int32, device=keys.device)
        outs.append((k2, idx))
    (a2, ia), (b2, ib) = outs
    lib = library()
    nbytes = lib.kvsel_topk2_workspace(ctypes.byref(v), a2.shape[0], b2.shape[0], w)
    ws, wsb = _workspace(nbytes, keys_a)
    st = lib.kvsel_topk2(ctypes.byref(v), w, a2.data_ptr(), a2.shape[0], _iptr(ka), ia.data_ptr(),
                         b2.data_ptr(), b2.shape[0], _iptr(kb), ib.data_ptr(), _ptr(ws), wsb,
                         _stream(keys_a))
    _check("kvsel_topk2", st)
    return (ia.view(-1) if keys_a.dim() == 1 else ia), (ib.view(-1) if keys_b.dim() == 1 else ib)


def _gather_job(src, cu, idx, w: int, k_per_seq, out, alloc: bool = True):
    """Validated job fields and output tensor for one gather (no tensor
    when ``alloc`` is false: the paged gather writes into a cache)."""
    import torch
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous CUDA tensor")
    _dev(idx, torch.int32, "idx")
    _same_device(src, ("idx", idx))
    if int(cu[-1]) != src.shape[0]:
        raise ValueError("cu_seqlens does not match src")
    idx2 = idx.view(1, -1) if idx.dim() == 1 else idx
    if src.dim() < 2:
        raise ValueError("src must be [T, heads, ...] or [T, row]")
    heads = src.shape[1] if src.dim() >= 3 else 1
    row_bytes = int(np.prod(src.shape[2:] if src.dim() >= 3 else src.shape[1:])) * src.element_size()
    if idx2.shape[0] not in (1, heads):
        raise ValueError("idx must have one row per head or a single shared row")
    per_head = 1 if (idx2.shape[0] == heads and heads > 1) else 0
    kk = _int32_array(k_per_seq, "k_per_seq")
    L = selected_length(cu, kk, w)
    if idx2.shape[1] != L:
        raise ValueError("idx length does not match the budgets")
    if not alloc:
        return (src.data_ptr(), idx2.data_ptr(), kk, heads, row_bytes, per_head), None
    shape = (L,) + tuple(src.shape[1:])
    if out is not None:
        dst = _buf(out, src.dtype, shape, src, "out")
    else:
        dst = torch.empty(shape, dtype=src.dtype, device=src.device)
    return (src.data_ptr(), idx2.data_ptr(), kk, heads, row_bytes, per_head), dst


def gather(src, cu_seqlens, idx, w: int, k_per_seq, out=None):
    """Compact ``src`` [T, heads, ...] (or [T, ...] for one head) by the
    selection ``idx`` ([heads, L] per head, or [L] / [1, L] shared).
    Returns [L, heads, ...] with the same trailing shape as ``src``."""
    v, cu = _varlen(cu_seqlens)
    (sp, ip, kk, heads, row_bytes, per_head), dst = _gather_job(src, cu, idx, w, k_per_seq, out)
    st = library().kvsel_gather(ctypes.byref(v), sp, heads, row_bytes, ip, per_head, _iptr(kk), w,
                                dst.data_ptr(), _stream(src))
    _check("kvsel_gather", st)
    return dst


def gather_multi(cu_seqlens, w: int, jobs, outs=None):
    """Several gathers in one launch.  ``jobs`` is a sequence of
    (src, idx, k_per_seq); returns the compacted tensors in order, each as
    ``gather`` would."""
    if not 1 <= len(jobs) <= GATHER_MAX_JOBS:
        raise ValueError(f"1..{GATHER_MAX_JOBS} jobs")
    if outs is not None and len(outs) != len(jobs):
        raise ValueError("one output per job")
    v, cu = _varlen(cu_seqlens)
    arr = (GatherJob * len(jobs))()
    dsts, keep = [], []
    for j, (src, idx, kps) in enumerate(jobs):
        (sp, ip, kk, heads, row_bytes, per_head), dst = _gather_job(
            src, cu, idx, w, kps, None if outs is None else outs[j])
        keep.append(kk)
        arr[j] = GatherJob(sp, dst.data_ptr(), ip, _iptr(kk), heads, row_bytes, per_head, 0)
        dsts.append(dst)
    st = library().kvsel_gather_multi(ctypes.byref(v), w, len(jobs), arr, _stream(jobs[0][0]))
    _check("kvsel_gather_multi", st)
    return dsts


def gather_paged(cu_seqlens, w: int, jobs):
    """Several gathers into paged caches in one launch
    (kvsel_gather_paged).  ``jobs`` is a sequence of
    (src, idx, k_per_seq, cache, block_table): ``cache``
    [num_blocks, block_size, heads, ...] with the trailing shape of ``src``,
    ``block_table`` int32 [B, max_blocks] on the device.  The caches are
    written in place."""
    import torch
    if not 1 <= len(jobs) <= GATHER_MAX_JOBS:
        raise ValueError(f"1..{GATHER_MAX_JOBS} jobs")
    v, cu = _varlen(cu_seqlens)
    arr = (GatherJob * len(jobs))()
    pages = (PagedCache * len(jobs))()
    keep = []
    for j, (src, idx, kps, cache, table) in enumerate(jobs):
        (sp, ip, kk, heads, row_bytes, per_head), _ = _gather_job(src, cu, idx, w, kps, None, alloc=False)
        if not cache.is_cuda or not cache.is_contiguous() or cache.dtype != src.dtype:
            raise ValueError("cache must be a contiguous CUDA tensor of the source's dtype")
        _same_device(src, ("cache", cache), ("block_table", table))
        if cache.dim() < 3 or tuple(cache.shape[2:]) != tuple(src.shape[1:]):
            raise ValueError("cache must be [num_blocks, block_size] + the source's trailing shape")
        _dev(table, torch.int32, "block_table")
        if table.dim() != 2 or table.shape[0] != v.batch:
            raise ValueError("block_table must be [B, max_blocks]")
        keep.append(kk)
        arr[j] = GatherJob(sp, None, ip, _iptr(kk), heads, row_bytes, per_head, 0)
        pages[j] = PagedCache(cache.data_ptr(), table.data_ptr(), cache.shape[0], cache.shape[1],
                              table.shape[1], 0)
    st = library().kvsel_gather_paged(ctypes.byref(v), w, len(jobs), arr, pages, _stream(jobs[0][0]))
    _check("kvsel_gather_paged", st)


def pivot_layer(entropy: Sequence[float]) -> int:
    """StructKV pivot layer from per-layer entropies (host call)."""
    e = np.ascontiguousarray(np.asarray(entropy, dtype=np.float32).reshape(-1))
    r = library().kvsel_pivot_layer(e.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), e.size, 1)
    if r < 0:
        raise KvselError("kvsel_pivot_layer", KVSEL_EINVAL, "invalid argument")
    return int(r)


def pivot_layer_sparsity(entropy: Sequence[float], sparsity: Sequence[float]) -> int:
    """StructKV pivot layer: the largest entropy drop among the layers whose
    sparsity rose (host call)."""
    e = np.ascontiguousarray(np.asarray(entropy, dtype=np.float32).reshape(-1))
    sp = np.ascontiguousarray(np.asarray(sparsity, dtype=np.float32).reshape(-1))
    if e.size != sp.size:
        raise ValueError("entropy and sparsity differ in length")
    fp = ctypes.POINTER(ctypes.c_float)
    r = library().kvsel_pivot_layer_sparsity(e.ctypes.data_as(fp), sp.ctypes.data_as(fp), e.size, 1)
    if r < 0:
        raise KvselError("kvsel_pivot_layer_sparsity", KVSEL_EINVAL, "invalid argument")
    return int(r)


def probe_read(src, rows: int, heads: int, row_bytes: int, stride_bytes: int, wgs_per_head: int, out=None):
    """Streaming-read probe (kvsel_probe_read, a measurement aid): reads
    ``heads`` interleaved row sets of the device buffer ``src`` and returns
    the uint32 XOR words [heads * wgs_per_head] (int32 tensor)."""
    import torch
    if not isinstance(src, torch.Tensor) or not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous CUDA tensor")
    need = (rows - 1) * stride_bytes + heads * row_bytes
    if rows < 1 or need > src.numel() * src.element_size():
        raise ValueError("the rows read do not fit in src")
    n = heads * wgs_per_head
    if out is None:
        out = torch.empty(n, dtype=torch.int32, device=src.device)
    _dev(out, torch.int32, "out")
    if out.device != src.device or out.numel() < n:
        raise ValueError(f"out must hold {n} words on the source's device")
    st = library().kvsel_probe_read(src.data_ptr(), rows, heads, row_bytes, stride_bytes, wgs_per_head,
                                    out.data_ptr(), _stream(src))
    _check("kvsel_probe_read", st)
    return out
