"""The seeded workloads reproduce their stated layouts; pair counts agree with the mask."""

import numpy as np
import pytest
import torch

import oracle
from workloads import make_layout, random_layout, make_qkv

# documents, allowed pairs, padding per row (numpy 2.2 default_rng(index))
EXPECTED = {
    1: (3, 10_120, [16]),
    2: (10, 4_121_156, [107]),
    3: (22, 6_143_439, [0]),
    4: (119, 37_334_127, [185, 241, 24, 109]),
    5: (19, 455_863_500, [0]),
}


@pytest.mark.parametrize("c", sorted(EXPECTED))
def test_layout_counts(c):
    lay = make_layout(c)
    ndocs, pairs, pads = EXPECTED[c]
    assert sum(len(r) for r in lay.doc_lens) == ndocs
    assert lay.allowed_pairs() == pairs
    assert lay.pad == pads
    for b in range(lay.B):
        assert sum(lay.doc_lens[b]) + lay.pad[b] == lay.S
        assert min(lay.doc_lens[b]) >= 1


def test_cp_shard_has_crossing_documents():
    lay = make_layout(3)
    cu = lay.cu_seqlens(0)
    lo, hi = lay.seq_start, lay.seq_start + lay.L
    assert any(a < lo < e for a, e in zip(cu[:-1], cu[1:]))
    assert any(a < hi < e for a, e in zip(cu[:-1], cu[1:]))


def _mask_pairs(lay):
    total = 0
    for b in range(lay.B):
        ids = torch.as_tensor(oracle.doc_ids_from_cu_seqlens(lay.cu_seqlens(b), lay.S)[0]).long()
        for i0 in range(0, lay.L, 512):
            qpos = torch.arange(lay.seq_start + i0, lay.seq_start + min(lay.L, i0 + 512))
            total += int(oracle.allowed_mask(ids, qpos).sum())
    return total


@pytest.mark.parametrize("c", [1, 2])
def test_pairs_equal_mask_count_named(c):
    lay = make_layout(c)
    assert _mask_pairs(lay) == lay.allowed_pairs()


@pytest.mark.parametrize("seed", range(8))
def test_pairs_equal_mask_count_random(seed):
    lay = random_layout(seed, B=3, S=97, L=40, seq_start=seed * 7, max_doc=30, max_pad=10)
    assert _mask_pairs(lay) == lay.allowed_pairs()


def test_qkv_deterministic_bf16():
    lay = make_layout(1)
    a = make_qkv(lay)
    b = make_qkv(lay)
    for x, y, shp in zip(a, b, lay.shapes()):
        assert x.dtype == torch.bfloat16 and tuple(x.shape) == shp
        assert torch.equal(x, y)
    assert not torch.equal(a[1], a[2])
