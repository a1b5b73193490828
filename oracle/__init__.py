"""CPU oracle for attention-score token selection.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the library path.
"""
from .kvsel_oracle import (accumulate, bf16_to_f64, budget_length, gather, gather_paged, head_sum,
                           layer_stats, mean_row_entropy, pivot_layer, pivot_layer_sparsity,
                           select_rows, select_with_window, window_row_entropy, window_score)

__all__ = ["accumulate", "bf16_to_f64", "budget_length", "gather", "gather_paged", "head_sum",
           "layer_stats", "mean_row_entropy", "pivot_layer", "pivot_layer_sparsity", "select_rows",
           "select_with_window", "window_row_entropy", "window_score"]
