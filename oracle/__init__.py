"""Float64 CPU oracle for exact attention (test infrastructure only; see attention.py)."""
from .attention import attn_bwd_ref, attn_fwd_ref, attn_rows_ref, attn_tiled_ref

__all__ = ["attn_fwd_ref", "attn_bwd_ref", "attn_tiled_ref", "attn_rows_ref"]
