"""libkvsel: attention-score token selection (FastKV Token-Selective
Propagation, StructKV pivot pruning) as hand-written HIP kernels for AMD
Instinct MI355X (gfx950) behind a C ABI, with a thin Python binding.

The shared library is loaded on first use; nothing here falls back to a
CPU implementation.
"""
from .kvsel import (KvselError, accumulate_stats, gather, gather_multi, gather_paged, library, pivot_layer,
                    pivot_layer_sparsity, probe_read, selected_length, topk, topk2, window_score,
                    window_score_entropy, window_score_noalloc, window_score_stats)

__all__ = ["KvselError", "accumulate_stats", "gather", "gather_multi", "gather_paged", "library", "pivot_layer",
           "pivot_layer_sparsity", "probe_read", "selected_length", "topk", "topk2", "window_score",
           "window_score_entropy", "window_score_noalloc",
           "window_score_stats"]
