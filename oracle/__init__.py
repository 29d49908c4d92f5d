"""fp64 CPU oracle for the FlashAttention-2 forward pass.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  It shares no code with
the HIP path and never imports it.
"""
from .attention import attention_fp64, attention_rows_fp64, scaled_logits_fp64
from .backward import attention_bwd_fp64, delta_fp64
from .splitkv import (attention_keyrange_fp64, combine_fp64, num_splits_heuristic, split_ranges,
                      utilisation)
from .tiled import causal_block_end, fa2_forward_tiled_fp64

__all__ = [
    "attention_fp64",
    "attention_rows_fp64",
    "scaled_logits_fp64",
    "fa2_forward_tiled_fp64",
    "causal_block_end",
    "attention_keyrange_fp64",
    "combine_fp64",
    "num_splits_heuristic",
    "split_ranges",
    "utilisation",
    "attention_bwd_fp64",
    "delta_fp64",
]
