"""MI355X-native FlashAttention-2 (forward, split-KV forward, backward).

``attention(q, k, v, causal, scale) -> (o, lse)`` runs the gfx950 HIP kernels
of libfa2.so through its C ABI (include/fa2.h).  The library is loaded on
first use and its absence is an error, never a fallback.
"""
from .fa2 import (FA2Error, FlashAttention, attention, attention_backward, attention_partial,
                  fa2_bwd, fa2_bwd_workspace_size, fa2_fwd, fa2_fwd_cross, fa2_fwd_partial,
                  fa2_fwd_splitkv, fa2_fwd_splitkv_noalloc, fa2_last_error, fa2_launch_shape,
                  fa2_merge, fa2_num_splits,
                  fa2_splitkv_workspace_size, fa2_strerror, library_path, load_library,
                  merge_partials)

__all__ = ["FA2Error", "FlashAttention", "attention", "attention_backward", "attention_partial",
           "fa2_bwd", "fa2_bwd_workspace_size", "fa2_fwd", "fa2_fwd_cross", "fa2_fwd_partial",
           "fa2_fwd_splitkv", "fa2_fwd_splitkv_noalloc", "fa2_last_error", "fa2_launch_shape",
           "fa2_merge", "fa2_num_splits",
           "fa2_splitkv_workspace_size", "fa2_strerror", "library_path", "load_library",
           "merge_partials"]
