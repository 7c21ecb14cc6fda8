"""Exact IO-aware attention for AMD Instinct MI355X (gfx950).

The computation lives in ``libfa_attn.so`` (hand-written HIP kernels behind the
C ABI declared in ``include/fa_attn.h``); this package only marshals tensors to
it.  Build the library with ``python -m io_aware_exact_12_amd.build``.
"""
from ._binding import (BF16, F16, F32, MASK_CAUSAL, MASK_NONE, FaError,  # noqa: F401
                       attn_bwd, attn_bwd_raw, attn_bwd_window_raw, attn_fwd, attn_fwd_kv_outer,
                       attn_fwd_kv_outer_raw, attn_fwd_raw, attn_fwd_window_raw,
                       attn_fwd_strided_raw, attn_bwd_strided_raw, attn_fwd_block_sparse_raw,
                       attn_fwd_dv_raw, attn_bwd_dv_raw,
                       attn_bwd_block_sparse_raw, attn_bwd_noalloc, attn_bwd_noalloc_raw,
                       noalloc_max_rows,
                       bwd_workspace_bytes, bwd_block_sparse_workspace_bytes, declared_symbols, kv_outer_workspace_bytes, lib,
                       status_str)
