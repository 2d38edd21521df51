"""Kimi Delta Attention (KDA) forward on AMD Instinct MI355X (gfx950).

Python front end of ``libkda.so``; the C ABI is declared in include/kda.h.

    out, final_state = chunk_fwd(q, k, v, log_alpha, beta, initial_state, cu_seqlens)
    out, final_state, snapshots = chunk_fwd_snapshots(q, k, v, log_alpha, beta, every)
    out = decode_step(q, k, v, log_alpha, beta, state)   # state updated in place
    grads = chunk_bwd(q, k, v, log_alpha, beta, d_out, d_final_state, initial_state)
"""
from ._lib import KdaError, lib
from .ops import (bwd_workspace_size, chunk_bwd, chunk_fwd, chunk_fwd_segmented,
                  chunk_fwd_segmented_noalloc, chunk_fwd_snapshots, decode_step,
                  segmented_workspace_size)

__all__ = ["chunk_fwd", "chunk_fwd_segmented", "chunk_fwd_segmented_noalloc",
           "chunk_fwd_snapshots", "chunk_bwd", "decode_step", "segmented_workspace_size",
           "bwd_workspace_size", "KdaError", "lib"]
