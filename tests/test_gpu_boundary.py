"""GPU boundary calls vs the oracle, bit-exact."""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import say
from workloads import make_layout

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def psb():
    import packed_sequence_block_amd as m
    m.load()
    return m


def _dev(x):
    return torch.as_tensor(np.asarray(x)).to(torch.int32).cuda()


@pytest.mark.parametrize("c", [1, 2, 3, 4, 5])
def test_named_layouts(psb, c):
    lay = make_layout(c)
    for b in range(lay.B):
        cu = lay.cu_seqlens(b)
        say("boundary cfg", c, "row", b, "S", lay.S)
        ids = psb.doc_ids_from_cu_seqlens(_dev(cu), lay.S, validate=True)
        ref = oracle.doc_ids_from_cu_seqlens(cu, lay.S)
        assert np.array_equal(ids.cpu().numpy(), ref)
        seg = psb.segment_cu_seqlens(ids[0])
        assert np.array_equal(seg.cpu().numpy(), oracle.segment_cu_seqlens(ref[0]))


@pytest.mark.parametrize("seed", range(24))
def test_random_boundaries(psb, seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 40))
    lens = rng.integers(0, 1 + int(rng.choice([3, 50, 3000])), size=n)
    lead = int(rng.integers(0, 5))
    cu = np.concatenate([[lead], lead + np.cumsum(lens)]).astype(np.int32)
    S = int(cu[-1]) + int(rng.integers(0, 70))
    say("boundary random seed", seed, "S", S, "n", n)
    ids = psb.doc_ids_from_cu_seqlens(_dev(cu), S, validate=True)
    ref = oracle.doc_ids_from_cu_seqlens(cu, S)
    assert np.array_equal(ids.cpu().numpy(), ref)
    assert np.array_equal(psb.segment_cu_seqlens(ids[0]).cpu().numpy(), oracle.segment_cu_seqlens(ref[0]))


@pytest.mark.parametrize("n", [4094, 4095, 4096, 9000])
def test_many_documents(psb, n):
    # boundary lists around the size that the kernel stages in LDS (4096 entries)
    rng = np.random.default_rng(n)
    lens = rng.integers(0, 4, size=n)
    cu = np.concatenate([[3], 3 + np.cumsum(lens)]).astype(np.int32)
    S = int(cu[-1]) + 11
    say("boundary many documents n", n, "S", S)
    ids = psb.doc_ids_from_cu_seqlens(_dev(cu), S, validate=True)
    ref = oracle.doc_ids_from_cu_seqlens(cu, S)
    assert np.array_equal(ids.cpu().numpy(), ref)


@pytest.mark.parametrize("S", [0, 1, 2, 15, 16, 17, 16383, 16384, 16385, 40000, 100003])
def test_segments_of_arbitrary_ids(psb, S):
    rng = np.random.default_rng(S)
    # runs of random length with ids drawn from a small alphabet (repeats, padding, 0)
    vals, out = [-1000, 0, 1, 2, 7], []
    while len(out) < S:
        out += [int(rng.choice(vals))] * int(rng.integers(1, 40))
    ids = np.asarray(out[:S], dtype=np.int32)
    say("segments S", S)
    got = psb.segment_cu_seqlens(_dev(ids))
    assert np.array_equal(got.cpu().numpy(), oracle.segment_cu_seqlens(ids))


def test_segments_on_unaligned_view(psb):
    ids = torch.arange(1, 1002, dtype=torch.int32).cuda() // 3
    view = ids[1:]       # 4-byte offset: not 16-byte aligned
    got = psb.segment_cu_seqlens(view)
    assert np.array_equal(got.cpu().numpy(), oracle.segment_cu_seqlens(view.cpu().numpy()))


@pytest.mark.parametrize("cu,S,bits", [([0, 5, 3], 6, 1), ([0, 7], 6, 2), ([-1, 2], 4, 2), ([0, 2, 4], 4, 0)])
def test_invalid_cu_sets_status(psb, cu, S, bits):
    from packed_sequence_block_amd import _lib
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.empty(S, dtype=torch.int32, device="cuda")
    c = _dev(cu)
    lib = _lib.load()
    assert lib.psb_doc_ids_from_cu_seqlens(_lib._ptr(c), len(cu) - 1, S, _lib._ptr(out), _lib._ptr(status),
                                           None) == 0
    torch.cuda.synchronize()
    assert int(status.item()) == bits
    if bits:
        with pytest.raises(ValueError):
            psb.doc_ids_from_cu_seqlens(c, S, validate=True)


def test_contiguity_validation(psb):
    good = _dev([[1, 1, 2, 2, 2, -1000, 3], [5, 5, -1000, -1000, 0, 0, 0]])
    psb.validate_doc_ids(good)
    bad = _dev([[1, 1, 2, 2, 1, -1000, 3]])
    with pytest.raises(ValueError):
        psb.validate_doc_ids(bad)
    bad2 = _dev([[4, -1000, 4]])
    with pytest.raises(ValueError):
        psb.validate_doc_ids(bad2)


# ---- boundary variants: lengths table, document positions ------------------------------

@pytest.mark.parametrize("seed", range(12))
def test_doc_ids_from_seq_lens(psb, seed):
    rng = np.random.default_rng(300 + seed)
    B = int(rng.integers(1, 5))
    n = int(rng.choice([1, 5, 40, 700]))
    S = int(rng.integers(1, 5000))
    lens = rng.integers(0, max(2, 2 * S // max(n, 1)), size=(B, n)).astype(np.int32)
    for b in range(B):  # some rows end early with the -1000 sentinel; keep sums <= S
        cut = int(rng.integers(0, n + 1))
        lens[b, cut:] = -1000
        c = np.cumsum(np.maximum(lens[b], 0))
        lens[b, c > S] = -1000
    say("seq_lens ids seed", seed, "B", B, "n", n, "S", S)
    got = psb.doc_ids_from_seq_lens(_dev(lens), S, validate=True)
    assert np.array_equal(got.cpu().numpy(), oracle.doc_ids_from_seq_lens(lens, S))


def test_doc_ids_from_seq_lens_overflow_sets_status(psb):
    with pytest.raises(ValueError):
        psb.doc_ids_from_seq_lens(_dev(np.asarray([[5, 5]], dtype=np.int32)), 7, validate=True)


@pytest.mark.parametrize("seed", range(16))
def test_document_positions(psb, seed):
    rng = np.random.default_rng(400 + seed)
    B, S = int(rng.integers(1, 4)), int(rng.integers(1, 3000))
    keep = np.zeros((B, S), dtype=bool)
    pos = np.zeros((B, S), dtype=np.int32)
    for b in range(B):
        p, first = int(rng.integers(0, 4)), True
        while p < S:
            n = int(rng.integers(1, 300))
            off = int(rng.integers(0, 50)) if first else 0
            m = min(n, S - p)
            keep[b, p:p + m] = True
            pos[b, p:p + m] = off + np.arange(m)
            p += n + int(rng.integers(0, 3))
            first = False
        if seed % 2 == 1:  # break one row at one kept position
            kept = np.nonzero(keep[b])[0]
            if kept.size > 1:
                i = int(rng.choice(kept[1:]))
                pos[b, i] = pos[b, i - 1] + 2 if keep[b, i - 1] else 5
    say("positions seed", seed, "B", B, "S", S)
    want = bool(np.all(oracle.document_positions_valid(keep, pos)))
    ok = True
    try:
        psb.validate_document_positions(torch.as_tensor(keep).cuda(), torch.as_tensor(pos).cuda())
    except ValueError:
        ok = False
    assert ok == want


def _unpack_tables(rng, B, n, S):
    """Real / padded length tables that fit S, -1000 after each row's last document."""
    real = np.full((B, n), -1000, dtype=np.int32)
    padded = np.full((B, n), -1000, dtype=np.int32)
    for b in range(B):
        left = S
        for j in range(int(rng.integers(0, n + 1))):
            q = int(rng.integers(0, max(2, 3 * S // max(n, 1))))
            if q > left:
                break
            real[b, j], padded[b, j] = int(rng.integers(0, q + 1)), q
            left -= q
    return real, padded


@pytest.mark.parametrize("seed", range(12))
def test_unpack_row_layout(psb, seed):
    rng = np.random.default_rng(500 + seed)
    B = int(rng.integers(1, 5))
    n = int(rng.choice([1, 6, 90, 1000]))
    S = int(rng.integers(1, 6000))
    real, padded = _unpack_tables(rng, B, n, S)
    say("unpack seed", seed, "B", B, "n", n, "S", S)
    mask, pos = psb.unpack_row_layout(_dev(real), _dev(padded), S, validate=True)
    want_m, want_p = oracle.unpack_row_layout(real, padded, S)
    assert mask.dtype == torch.bool and pos.dtype == torch.int32
    assert np.array_equal(mask.cpu().numpy(), want_m)
    assert np.array_equal(pos.cpu().numpy(), want_p)


def test_unpack_row_layout_full_rows_and_many_documents(psb):
    # tables that fill the row exactly, 4096 documents (the largest table), zero lengths
    rng = np.random.default_rng(77)
    n, S = 4096, 4096 * 3
    padded = rng.integers(0, 6, size=(2, n)).astype(np.int32)
    padded[:, -1] += S - padded.sum(axis=1).astype(np.int32)
    assert (padded >= 0).all() and (padded.sum(axis=1) == S).all()
    real = np.minimum(padded, rng.integers(0, 6, size=(2, n))).astype(np.int32)
    say("unpack 4096 documents")
    mask, pos = psb.unpack_row_layout(_dev(real), _dev(padded), S, validate=True)
    want_m, want_p = oracle.unpack_row_layout(real, padded, S)
    assert np.array_equal(mask.cpu().numpy(), want_m) and np.array_equal(pos.cpu().numpy(), want_p)
    with pytest.raises(psb.PsbError):
        psb.unpack_row_layout(_dev(np.zeros((1, n + 1), np.int32)), _dev(np.zeros((1, n + 1), np.int32)), 8)


@pytest.mark.parametrize("real,padded,S,bits", [
    ([[3, 2]], [[2, 2]], 8, 32),          # more real tokens than the padded block
    ([[-1, 2]], [[2, 2]], 8, 32),         # negative real length inside the table
    ([[3, 3]], [[4, 5]], 8, 8),           # padded lengths exceed seq_len
])
def test_unpack_row_layout_bad_tables_set_status(psb, real, padded, S, bits):
    lib = psb.load()
    r, q = _dev(np.asarray(real, np.int32)), _dev(np.asarray(padded, np.int32))
    mask = torch.empty((1, S), dtype=torch.bool, device="cuda")
    pos = torch.empty((1, S), dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    import ctypes
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    say("unpack bad table", real, padded, S)
    st = lib.psb_unpack_row_layout(P(r), P(q), 1, r.shape[1], S, P(mask), P(pos), P(status),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0 and int(status.item()) == bits
    with pytest.raises(ValueError):
        psb.unpack_row_layout(r, q, S, validate=True)


def test_unpack_then_positions_rule(psb):
    # the unpacked layout passes the document rule with keep = not padding
    rng = np.random.default_rng(5)
    real, padded = _unpack_tables(rng, 3, 50, 3000)
    mask, pos = psb.unpack_row_layout(_dev(real), _dev(padded), 3000)
    say("unpack then positions")
    psb.validate_document_positions(~mask, pos)
    batch = {"input_ids": torch.zeros((3, 3000), dtype=torch.int64, device="cuda"),
             "seq_lens": _dev(real), "seq_lens_padded": _dev(padded)}
    psb.unpack_row_layout_batch(batch)
    assert "seq_lens" not in batch and torch.equal(batch["padding_mask"], mask)
    assert torch.equal(batch["position_ids"], pos)
