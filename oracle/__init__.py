"""CPU fp64 oracle for packed block-causal attention — TEST INFRASTRUCTURE.

This package is a plain, slow, obviously-correct restatement of what the
product path computes.  It exists only so that tests, ``__graft_entry__.smoke``
and the CPU-baseline leg of ``bench.py`` have something independent to compare
the HIP kernels against.  Nothing in ``packed_sequence_block_amd`` imports it,
and it imports nothing from there: the only code the two sides share is the
seeded input generator in ``workloads`` (which holds none of the method's
arithmetic).

Sources followed (cite by page title and section):

* "nemo_automodel.components.models.glm5_next.cp" page, API entries
  ``doc_ids_from_cu_seqlens`` (cumulative boundaries -> ids ``[1, sequence]``)
  and ``segment_cu_seqlens`` (boundaries of consecutive document-id runs that
  cover the full row).
* "nemo_automodel.components.models.inkling2.context_parallel" page, API entries
  ``unpack_row_layout`` (padding and positions from -1000-padded real / padded
  length tables) and ``validate_document_positions`` (the document rule).
* "nemo_automodel.components.distributed.blockdiag_cp" page: package overview
  (a packed row needs a block-causal mask per document), ``cp_blockdiag_sdpa``
  (local queries against delivered keys, mask rebuilt from document ids,
  ``scale=None`` means ``D**-0.5``, ``enable_gqa`` as in HF's sdpa path,
  output ``[B, Hq, L, D]`` for the local rows), ``BlockdiagCpModelState``
  (``packed_cu_seqlens`` has shape ``[num_documents + 1]``).

Readings where the pages are silent:

* padding document id is -1000 (the sentinel of ``doc_ids_from_seq_lens`` and
  of the inkling2 ``unpack_row_layout`` lengths); 0 is an ordinary id;
* ``doc_ids_from_cu_seqlens`` numbers document i (0-based interval) as i+1 and
  marks positions outside ``[cu[0], cu[N])`` as padding;
* a padding query row has no allowed key and outputs exactly 0;
* ``unpack_row_layout``: document j of a row takes ``seq_lens_padded[b, j]``
  positions, its first ``seq_lens[b, j]`` are real tokens with positions 0, 1,
  ...; every other position is padding (mask True, position 0).

Every function here is pinned by ``tests/test_oracle_*.py`` against facts fixed
independently of this code (library routines, closed forms, brute force,
worked examples under ``tests/golden``).
"""

from .boundary import (PAD_DOC_ID, doc_ids_from_cu_seqlens, doc_ids_from_seq_lens, document_positions_valid,
                       segment_cu_seqlens, unpack_row_layout)
from .attention import (allowed_mask, blockdiag_attn, blockdiag_attn_loop, blockdiag_attn_rows,
                        dense_mask, kv_head_of, kv_window_start, masked_attn)

__all__ = [
    "PAD_DOC_ID", "doc_ids_from_cu_seqlens", "segment_cu_seqlens", "doc_ids_from_seq_lens",
    "document_positions_valid", "unpack_row_layout",
    "allowed_mask", "blockdiag_attn", "blockdiag_attn_loop", "blockdiag_attn_rows", "kv_head_of",
    "kv_window_start", "dense_mask", "masked_attn",
]
from .attention_bwd import blockdiag_attn_bwd, blockdiag_attn_lse
