"""Packed-sequence block-diagonal (per-document causal) attention for MI355X.

Python face of ``libpsb.so`` (HIP kernels for gfx950, C ABI in include/psb.h):

* :func:`doc_ids_from_cu_seqlens` — document boundaries -> per-position ids
* :func:`segment_cu_seqlens` — per-position ids -> run boundaries
* :func:`blockdiag_attn_fwd` — attention with the per-document causal mask,
  for a packed row (``seq_start = 0``, ``L = S``) or one context-parallel
  rank's contiguous query shard against all delivered keys/values.
* :func:`blockdiag_attn_fwd_lse` / :func:`blockdiag_attn_bwd` — the training
  path (forward with per-row log-sum-exp, then dq, dk, dv);
  :func:`blockdiag_attention` wraps both as a differentiable torch custom op.
* :func:`blockdiag_sdpa` — drop-in ``scaled_dot_product_attention`` for an armed
  packed step (:func:`enable_packed_varlen`, :func:`packed_documents`), swapped in
  around attention modules by :func:`attach_packed_varlen_hooks`.
* :func:`shard_kv_window_start`, :func:`blockdiag_attn_fwd_window` /
  :func:`blockdiag_attn_bwd_window` — a query shard run against a delivered key
  window (its own keys plus a left halo) instead of the whole row.
* :func:`blockdiag_dense_mask`, :func:`masked_attn_fwd` — the dense-mask path: the
  per-document mask materialised, and attention under any explicit mask.
* :func:`doc_ids_from_seq_lens`, :func:`unpack_row_layout`,
  :func:`validate_document_positions` — layouts from packed length tables.
"""

from ._lib import (PAD_DOC_ID, PsbError, blockdiag_attn_bwd, blockdiag_attn_fwd, blockdiag_attn_fwd_lse,
                   bwd_workspace_size, doc_ids_from_cu_seqlens, doc_ids_from_seq_lens, load,
                   blockdiag_attn_bwd_window, blockdiag_attn_fwd_window, shard_kv_window_start,
                   blockdiag_dense_mask, masked_attn_fwd, blockdiag_prepare,
                   segment_cu_seqlens, status_string, unpack_row_layout, unpack_row_layout_batch, validate_doc_ids,
                   validate_document_positions,
                   workspace_size)

from .sdpa import (PackedState, attach_packed_varlen_hooks, blockdiag_attention, blockdiag_sdpa, current_packed_state,
                   disable_packed_varlen, enable_packed_varlen, packed_documents, patched_sdpa)

__all__ = ["blockdiag_attention", "PackedState", "attach_packed_varlen_hooks", "blockdiag_sdpa",
           "current_packed_state", "disable_packed_varlen", "enable_packed_varlen", "packed_documents",
           "patched_sdpa", "PAD_DOC_ID", "PsbError", "blockdiag_attn_bwd", "blockdiag_attn_fwd", "blockdiag_attn_fwd_lse",
           "bwd_workspace_size", "doc_ids_from_cu_seqlens", "doc_ids_from_seq_lens", "load",
           "blockdiag_attn_bwd_window", "blockdiag_attn_fwd_window", "shard_kv_window_start",
           "blockdiag_dense_mask", "masked_attn_fwd", "blockdiag_prepare",
           "segment_cu_seqlens", "status_string", "unpack_row_layout", "unpack_row_layout_batch", "validate_doc_ids",
           "validate_document_positions",
           "workspace_size"]
