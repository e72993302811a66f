"""Pins for the boundary oracle (doc_ids_from_cu_seqlens, segment_cu_seqlens).

Each check is fixed by something other than the oracle's own code: a worked
example derived by hand, numpy brute force written a different way
(``np.repeat`` / ``np.diff``), and round trips.
"""

import numpy as np
import pytest

import oracle
from oracle import PAD_DOC_ID


def _runs_to_ids(spec):
    ids = []
    for tok in spec.split():
        val, cnt = tok.split(":")
        ids += [int(val)] * int(cnt)
    return np.asarray(ids, dtype=np.int32)


def test_worked_example(golden):
    g = golden("boundary_cfg1.txt")
    seq_len = int(g["seq_len"])
    cu = np.asarray([int(x) for x in g["cu_seqlens"].split()], dtype=np.int32)
    ids = oracle.doc_ids_from_cu_seqlens(cu, seq_len)
    assert ids.shape == (1, seq_len) and ids.dtype == np.int32
    np.testing.assert_array_equal(ids[0], _runs_to_ids(g["doc_ids_runs"]))
    seg = oracle.segment_cu_seqlens(ids[0])
    np.testing.assert_array_equal(seg, [int(x) for x in g["segments"].split()])


def _brute_ids(cu, seq_len):
    # ids by repetition: lead padding, one block per document, trailing padding
    lens = np.diff(cu)
    body = np.repeat(np.arange(1, len(lens) + 1, dtype=np.int64), lens)
    return np.concatenate([np.full(cu[0], PAD_DOC_ID), body,
                           np.full(seq_len - cu[-1], PAD_DOC_ID)]).astype(np.int32)


def _brute_segments(ids):
    if len(ids) == 0:
        return np.zeros(1, dtype=np.int32)
    starts = np.flatnonzero(np.diff(ids.astype(np.int64))) + 1
    return np.concatenate([[0], starts, [len(ids)]]).astype(np.int32)


@pytest.mark.parametrize("seed", range(40))
def test_random_against_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 12))
    lens = rng.integers(0, 9, size=n)          # zero-length documents included
    lead = int(rng.integers(0, 4))
    tail = int(rng.integers(0, 5))
    cu = np.concatenate([[lead], lead + np.cumsum(lens)]).astype(np.int32)
    seq_len = int(cu[-1]) + tail
    ids = oracle.doc_ids_from_cu_seqlens(cu, seq_len)[0]
    np.testing.assert_array_equal(ids, _brute_ids(cu, seq_len))
    np.testing.assert_array_equal(oracle.segment_cu_seqlens(ids), _brute_segments(ids))


@pytest.mark.parametrize("seed", range(20))
def test_round_trip(seed):
    rng = np.random.default_rng(100 + seed)
    lens = rng.integers(1, 30, size=int(rng.integers(1, 10)))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ids = oracle.doc_ids_from_cu_seqlens(cu, int(cu[-1]))
    np.testing.assert_array_equal(oracle.segment_cu_seqlens(ids[0]), cu)


def test_segments_split_repeated_ids_and_count_padding():
    ids = np.asarray([5, 5, PAD_DOC_ID, PAD_DOC_ID, 5, 0, 0], dtype=np.int32)
    np.testing.assert_array_equal(oracle.segment_cu_seqlens(ids), [0, 2, 4, 5, 7])


def test_empty_and_degenerate():
    np.testing.assert_array_equal(oracle.segment_cu_seqlens(np.zeros(0, np.int32)), [0])
    assert oracle.doc_ids_from_cu_seqlens([0], 0).shape == (1, 0)
    np.testing.assert_array_equal(oracle.doc_ids_from_cu_seqlens([0], 3)[0], [PAD_DOC_ID] * 3)
    np.testing.assert_array_equal(oracle.doc_ids_from_cu_seqlens([0, 0, 2], 2)[0], [2, 2])
    np.testing.assert_array_equal(oracle.segment_cu_seqlens([9]), [0, 1])


@pytest.mark.parametrize("cu,seq_len", [([0, 5, 3], 6), ([0, 7], 6), ([-1, 2], 4), ([], 4)])
def test_invalid_cu_raises(cu, seq_len):
    with pytest.raises(ValueError):
        oracle.doc_ids_from_cu_seqlens(np.asarray(cu, dtype=np.int64), seq_len)


def test_seq_lens_variant_matches_cu_variant():
    seq_lens = np.asarray([[3, 2, -1000], [1, 1, 4]])
    ids = oracle.doc_ids_from_seq_lens(seq_lens, 7)
    np.testing.assert_array_equal(ids[0], oracle.doc_ids_from_cu_seqlens([0, 3, 5], 7)[0])
    np.testing.assert_array_equal(ids[1], oracle.doc_ids_from_cu_seqlens([0, 1, 2, 6], 7)[0])
    with pytest.raises(ValueError):
        oracle.doc_ids_from_seq_lens(np.asarray([[5, 5]]), 7)


# ---- document positions (inkling2 context_parallel page, validate_document_positions) ----

POS_CASES = [
    # (keep, positions, valid) — hand-derived from the rule
    ([1, 1, 1, 1, 1, 1], [0, 1, 2, 0, 1, 2], True),          # two documents
    ([0, 0, 1, 1, 1, 1], [9, 9, 7, 8, 0, 1], True),          # shard starts mid-document after left padding
    ([1, 1, 0, 0, 1, 1], [0, 1, 5, 5, 0, 1], True),          # dropped tokens, then a new document
    ([1, 1, 0, 1, 1, 1], [0, 1, 0, 2, 3, 4], False),         # a gap resumes the old document
    ([1, 1, 1, 1], [0, 1, 3, 4], False),                     # skipped increment
    ([1, 1, 1, 1], [4, 5, 2, 3], False),                     # reset to a non-zero position
    ([1, 1, 1], [-1, 0, 1], False),                          # negative first position
    ([0, 0, 0], [3, -2, 7], True),                           # nothing kept
    ([1, 0, 1], [5, 0, 0], True),                            # gap then reset
]


@pytest.mark.parametrize("keep,pos,valid", POS_CASES)
def test_document_positions_hand_cases(keep, pos, valid):
    got = oracle.document_positions_valid(np.asarray([keep]), np.asarray([pos]))
    assert got.tolist() == [valid]


def _layout_positions(rng, S):
    """Positions built from document lengths with dropped tokens between documents:
    valid by construction; the first document may start mid-way (a shard)."""
    keep = np.zeros(S, dtype=bool)
    pos = np.full(S, 77, dtype=np.int64)
    p = int(rng.integers(0, 4))
    first = True
    while p < S:
        n = int(rng.integers(1, 9))
        off = int(rng.integers(0, 5)) if first else 0
        for i in range(min(n, S - p)):
            keep[p + i] = True
            pos[p + i] = off + i
        p += n + int(rng.integers(0, 3))
        first = False
    return keep, pos


@pytest.mark.parametrize("seed", range(20))
def test_document_positions_constructed_and_broken(seed):
    rng = np.random.default_rng(seed)
    keep, pos = _layout_positions(rng, 40)
    assert oracle.document_positions_valid(keep[None], pos[None]).tolist() == [True]
    kept = np.nonzero(keep)[0]
    if kept.size > 1:
        bad = pos.copy()
        i = int(rng.choice(kept[1:]))
        # neither 0 nor previous + 1 (after a kept token), not 0 after a gap
        bad[i] = bad[i - 1] + 2 if keep[i - 1] else 5
        assert oracle.document_positions_valid(keep[None], bad[None]).tolist() == [False]


# ---- row layout from length tables (inkling2 context_parallel page, unpack_row_layout) ----

def test_unpack_row_layout_hand_example():
    # row 0: a 3-token document padded to 4, a 1-token document padded to 2, table end;
    # row 1: an empty document padded to 1, then 2 real of 2
    real = np.asarray([[3, 1, -1000], [0, 2, -1000]])
    padded = np.asarray([[4, 2, -1000], [1, 2, -1000]])
    mask, pos = oracle.unpack_row_layout(real, padded, 8)
    assert mask.dtype == bool and pos.dtype == np.int32 and mask.shape == pos.shape == (2, 8)
    np.testing.assert_array_equal(mask[0], [0, 0, 0, 1, 0, 1, 1, 1])
    np.testing.assert_array_equal(pos[0], [0, 1, 2, 0, 0, 0, 0, 0])
    np.testing.assert_array_equal(mask[1], [1, 0, 0, 1, 1, 1, 1, 1])
    np.testing.assert_array_equal(pos[1], [0, 0, 1, 0, 0, 0, 0, 0])


def _random_tables(rng, B, N, S):
    real = np.full((B, N), -1000, dtype=np.int64)
    padded = np.full((B, N), -1000, dtype=np.int64)
    for b in range(B):
        left = S
        for j in range(int(rng.integers(0, N + 1))):
            n_pad = int(rng.integers(0, 12))
            if n_pad > left:
                break
            real[b, j], padded[b, j] = int(rng.integers(0, n_pad + 1)), n_pad
            left -= n_pad
    return real, padded


def _brute_unpack(real, padded, S):
    # per row: concatenate, document by document, "real tokens" then "padding" blocks
    B = real.shape[0]
    mask = np.ones((B, S), dtype=bool)
    pos = np.zeros((B, S), dtype=np.int32)
    for b in range(B):
        n = int(np.argmax(padded[b] < 0)) if (padded[b] < 0).any() else padded.shape[1]
        m_parts = [np.concatenate([np.zeros(r, bool), np.ones(q - r, bool)]) for r, q in zip(real[b, :n], padded[b, :n])]
        p_parts = [np.concatenate([np.arange(r), np.zeros(q - r, np.int64)]) for r, q in zip(real[b, :n], padded[b, :n])]
        body_m = np.concatenate(m_parts) if m_parts else np.zeros(0, bool)
        body_p = np.concatenate(p_parts) if p_parts else np.zeros(0, np.int64)
        mask[b, :body_m.size] = body_m
        pos[b, :body_p.size] = body_p
    return mask, pos


@pytest.mark.parametrize("seed", range(12))
def test_unpack_row_layout_random_against_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    S = int(rng.integers(0, 60))
    real, padded = _random_tables(rng, 3, 7, S)
    mask, pos = oracle.unpack_row_layout(real, padded, S)
    bm, bp = _brute_unpack(real, padded, S)
    np.testing.assert_array_equal(mask, bm)
    np.testing.assert_array_equal(pos, bp)
    # invariants: as many real tokens as the real lengths say, and the kept tokens
    # follow the document rule (each document restarts at 0 after its padding)
    for b in range(3):
        n = int(np.argmax(padded[b] < 0)) if (padded[b] < 0).any() else padded.shape[1]
        assert int((~mask[b]).sum()) == int(real[b, :n].sum())
    assert oracle.document_positions_valid(~mask, pos).all()


def test_unpack_row_layout_without_padding_matches_doc_ids():
    # equal tables: no padding inside the documents; the kept tokens are exactly the
    # positions doc_ids_from_seq_lens covers, and a token's position is its distance
    # from the first position that carries its id
    lens = np.asarray([[5, 0, 3, 4, -1000], [2, 2, 2, 2, 2]])
    mask, pos = oracle.unpack_row_layout(lens, lens, 12)
    ids = oracle.doc_ids_from_seq_lens(lens, 12)
    np.testing.assert_array_equal(mask, ids == PAD_DOC_ID)
    for b in range(2):
        for p in range(12):
            if ids[b, p] != PAD_DOC_ID:
                assert pos[b, p] == p - int(np.argmax(ids[b] == ids[b, p]))


@pytest.mark.parametrize("real,padded,S", [
    ([[3, 2]], [[2, 2]], 8),          # more real tokens than the padded block
    ([[-1, 2]], [[2, 2]], 8),         # real table ends before the padded one
    ([[3, 3]], [[4, 5]], 8),          # padded lengths exceed seq_len
])
def test_unpack_row_layout_invalid_raises(real, padded, S):
    with pytest.raises(ValueError):
        oracle.unpack_row_layout(np.asarray(real), np.asarray(padded), S)


def test_unpack_row_layout_empty():
    mask, pos = oracle.unpack_row_layout(np.zeros((2, 0), np.int64), np.zeros((2, 0), np.int64), 3)
    assert mask.all() and (pos == 0).all()
    mask, pos = oracle.unpack_row_layout(np.asarray([[0]]), np.asarray([[0]]), 0)
    assert mask.shape == (1, 0)
