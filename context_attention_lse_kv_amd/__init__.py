"""MI355X-native blockwise ring attention (one GPU's share of context parallelism).

The computation lives in ``libra.so`` (HIP kernels for gfx950 behind the C ABI of
``include/ra.h``); this package only marshals torch tensors into that ABI.
"""
from .ops import (Chunks, bwd_chunk, bwd_chunk_dkdv, bwd_chunk_dq, bwd_chunk_dkdv_ds, bwd_chunk_dq_ds, bwd_delta, bwd_ds_bytes, fwd_chunk, head_to_seq, merge_lse, ring_bwd, ring_bwd_plan, ring_bwd_workspace_bytes, ring_fwd,
                  ring_order, rows_desc, seq_head_permute, seq_to_head, split_sizes, tensor_desc)

from .autograd import head_to_seq_exchange, ring_attention, seq_to_head_exchange

__all__ = ["ring_attention", "seq_to_head_exchange", "head_to_seq_exchange", "Chunks", "bwd_chunk", "bwd_chunk_dkdv", "bwd_chunk_dq", "bwd_chunk_dkdv_ds", "bwd_chunk_dq_ds", "bwd_delta", "bwd_ds_bytes", "fwd_chunk", "head_to_seq", "merge_lse", "ring_bwd", "ring_bwd_plan", "ring_bwd_workspace_bytes", "ring_fwd",
           "ring_order", "rows_desc", "seq_head_permute", "seq_to_head", "split_sizes", "tensor_desc"]
