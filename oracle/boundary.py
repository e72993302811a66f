"""Oracle for the document-id / segment-boundary calls (test infrastructure).

Follows the "nemo_automodel.components.models.glm5_next.cp" page, API entries
``doc_ids_from_cu_seqlens``, ``doc_ids_from_seq_lens`` and
``segment_cu_seqlens``.  Pure Python/numpy, written for reading, not speed.
"""

from __future__ import annotations

import numpy as np

PAD_DOC_ID = -1000


def doc_ids_from_cu_seqlens(cu_seqlens, seq_len: int) -> np.ndarray:
    """Cumulative document boundaries -> per-position document ids ``[1, seq_len]``.

    glm5_next.cp page, ``doc_ids_from_cu_seqlens``: "cumulative document
    boundaries to ids [1, sequence]".  ``cu_seqlens`` has N+1 entries
    (``BlockdiagCpModelState.packed_cu_seqlens`` shape ``[num_documents + 1]``).

    Reading (the page does not say): document i, covering ``[cu[i], cu[i+1])``,
    gets id ``i + 1``; every other position is padding (-1000).  ``cu`` must be
    non-decreasing with ``0 <= cu[0]`` and ``cu[N] <= seq_len``; anything else
    raises ``ValueError`` instead of being truncated.
    """
    cu = [int(x) for x in np.asarray(cu_seqlens).reshape(-1)]
    if len(cu) < 1:
        raise ValueError("cu_seqlens needs at least one entry")
    if seq_len < 0:
        raise ValueError("negative seq_len")
    if cu[0] < 0 or cu[-1] > seq_len:
        raise ValueError("cu_seqlens outside [0, seq_len]")
    for i in range(len(cu) - 1):
        if cu[i + 1] < cu[i]:
            raise ValueError("cu_seqlens is not non-decreasing")
    ids = [PAD_DOC_ID] * seq_len
    for i in range(len(cu) - 1):
        for p in range(cu[i], cu[i + 1]):
            ids[p] = i + 1
    return np.asarray(ids, dtype=np.int32).reshape(1, seq_len)


def doc_ids_from_seq_lens(seq_lens, seq_len: int, padding_value: int = PAD_DOC_ID) -> np.ndarray:
    """Per-document lengths ``[batch, documents]`` -> ids ``[batch, seq_len]``.

    glm5_next.cp page, ``doc_ids_from_seq_lens`` (padding id defaults to -1000);
    the inkling2 ``unpack_row_layout`` entry says the length table itself is
    padded with -1000, so any negative length ends a row's document list.
    Numbering follows ``doc_ids_from_cu_seqlens``: the j-th document of a row
    gets id j + 1.  Lengths summing past ``seq_len`` raise ``ValueError``.
    """
    lens = np.asarray(seq_lens).reshape(len(seq_lens), -1) if len(seq_lens) else np.zeros((0, 0))
    out = np.full((lens.shape[0], seq_len), padding_value, dtype=np.int32)
    for b in range(lens.shape[0]):
        pos = 0
        for j, n in enumerate(int(x) for x in lens[b]):
            if n < 0:
                break
            if pos + n > seq_len:
                raise ValueError("document lengths exceed seq_len")
            for p in range(pos, pos + n):
                out[b, p] = j + 1
            pos += n
    return out


def segment_cu_seqlens(doc_ids_row) -> np.ndarray:
    """Boundaries of maximal runs of equal ids covering the whole row.

    glm5_next.cp page, ``segment_cu_seqlens``: "boundaries for consecutive
    document-id runs covering the full row".  Padding runs are segments too,
    equal ids in separate runs are separate segments.  Output int32
    ``[R + 1]`` starting at 0 and ending at the row length (``[0]`` for an
    empty row).
    """
    ids = [int(x) for x in np.asarray(doc_ids_row).reshape(-1)]
    n = len(ids)
    cu = [0]
    for p in range(1, n):
        if ids[p] != ids[p - 1]:
            cu.append(p)
    if n > 0:
        cu.append(n)
    return np.asarray(cu, dtype=np.int32)


def document_positions_valid(keep, positions) -> np.ndarray:
    """Per row: do the logical positions follow the document rule?  ``[batch]`` bool.

    inkling2 ``context_parallel`` page, ``validate_document_positions``: inside a
    document positions grow by one, a new document starts at zero, a contiguous
    shard may begin partway through a document (so the first kept token may carry
    any offset, also after left padding), and a gap never resumes an earlier
    document.  Reading, for the kept tokens of a row in order:
      * the first kept token: position >= 0;
      * a kept token right after a kept token: previous + 1 (same document) or 0
        (a new document);
      * a kept token after one or more dropped tokens: 0.
    """
    keep = np.asarray(keep).astype(bool)
    pos = np.asarray(positions).astype(np.int64)
    if keep.shape != pos.shape or keep.ndim != 2:
        raise ValueError("keep and positions must both be [batch, sequence]")
    ok = np.ones(keep.shape[0], dtype=bool)
    for b in range(keep.shape[0]):
        seen = False
        for p in range(keep.shape[1]):
            if not keep[b, p]:
                continue
            x = int(pos[b, p])
            if not seen:
                good = x >= 0
            elif keep[b, p - 1]:
                good = x == int(pos[b, p - 1]) + 1 or x == 0
            else:
                good = x == 0
            if not good:
                ok[b] = False
                break
            seen = True
    return ok


def unpack_row_layout(seq_lens, seq_lens_padded, seq_len: int):
    """Packed length tables -> ``(padding_mask [B, seq_len] bool, position_ids [B, seq_len] int32)``.

    inkling2 ``context_parallel`` page, ``unpack_row_layout``: the packer hands over
    real and padded lengths ``[batch, documents]``, both padded with -1000, and
    padding comes from those lengths alone, never from token ids; the result is a
    boolean padding mask and integer positions ``[batch, sequence]``.  Readings:
      * a row's documents are the entries before the first negative padded length;
        document j takes the next ``seq_lens_padded[b, j]`` positions of the row;
      * of those, the first ``seq_lens[b, j]`` are real tokens with positions
        0, 1, ... inside the document; the rest of the block is padding;
      * positions past the last document are padding;
      * padding positions get ``padding_mask`` True (the blockdiag_cp page's
        ``make_cp_blockdiag_batch_and_ctx`` convention, True == pad) and position 0;
      * ``0 <= seq_lens[b, j] <= seq_lens_padded[b, j]`` for every document and
        padded lengths adding up to at most ``seq_len``; anything else raises
        ``ValueError``.
    """
    real = np.asarray(seq_lens, dtype=np.int64)
    padded = np.asarray(seq_lens_padded, dtype=np.int64)
    if real.ndim != 2 or real.shape != padded.shape:
        raise ValueError("seq_lens and seq_lens_padded must both be [batch, documents]")
    if seq_len < 0:
        raise ValueError("negative seq_len")
    B, N = real.shape
    mask = np.ones((B, seq_len), dtype=bool)
    pos = np.zeros((B, seq_len), dtype=np.int32)
    for b in range(B):
        start = 0
        for j in range(N):
            n_pad = int(padded[b, j])
            if n_pad < 0:
                break
            n_real = int(real[b, j])
            if n_real < 0 or n_real > n_pad:
                raise ValueError(f"row {b} document {j}: real length {n_real} outside [0, {n_pad}]")
            if start + n_pad > seq_len:
                raise ValueError(f"row {b}: padded lengths exceed seq_len")
            for t in range(n_real):
                mask[b, start + t] = False
                pos[b, start + t] = t
            start += n_pad
    return mask, pos
