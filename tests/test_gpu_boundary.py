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
