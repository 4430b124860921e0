"""Float64 CPU oracle for exact attention (test infrastructure only; see attention.py)."""
from .attention import (attn_bwd_ref, attn_decode_ref, attn_fwd_ref, attn_rows_ref,
                        attn_split_merge_ref, attn_tiled_ref, block_mask_to_elements)
from .philox import dropout_keep_ref, keep_scale, keep_threshold, philox4x32

__all__ = ["attn_fwd_ref", "attn_bwd_ref", "attn_tiled_ref", "attn_rows_ref", "philox4x32",
           "keep_threshold", "keep_scale", "dropout_keep_ref", "block_mask_to_elements", "attn_decode_ref",
           "attn_split_merge_ref"]
