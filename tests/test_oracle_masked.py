"""Pins for the dense-mask oracle (``dense_mask``, ``masked_attn``).

Fixed independently of its code: the library SDPA routine (no mask, causal), the
separately pinned block-diagonal oracle, literal Python loops on a tiny input, and
closed forms (a row with no key is 0, a row with one key copies that key's value).
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import PAD_DOC_ID
from gpu_common import oracle_doc_ids
from workloads import make_qkv, random_layout

P = PAD_DOC_ID


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64)


def test_dense_mask_hand_example():
    m = oracle.dense_mask(np.asarray([[3, 3, P, 4, 4]]), 1, 4)   # rows at positions 1..4
    want = [[1, 1, 0, 0, 0],
            [0, 0, 0, 0, 0],
            [0, 0, 0, 1, 0],
            [0, 0, 0, 1, 1]]
    assert m.dtype == torch.bool and m.tolist() == [[[bool(x) for x in r] for r in want]]


def test_dense_mask_equals_block_diagonal_oracle():
    lay = random_layout(61, B=2, S=200, L=120, seq_start=50, Hq=4, Hkv=2, D=16, max_doc=60, max_pad=15)
    q, k, v = make_qkv(lay, seed_base=6100)
    ids = oracle_doc_ids(lay)
    got = oracle.masked_attn(q, k, v, oracle.dense_mask(ids, 50, 120), None, True)
    ref = oracle.blockdiag_attn(q, k, v, ids, 50, None, True)
    assert (got - ref).abs().max().item() < 1e-12


def test_all_true_and_causal_masks_match_library_sdpa():
    q, k, v = _rand((2, 4, 9, 8), 1), _rand((2, 2, 9, 8), 2), _rand((2, 2, 9, 8), 3)
    full = oracle.masked_attn(q, k, v, torch.ones((1, 9, 9), dtype=torch.bool), 0.3, True)
    assert (full - F.scaled_dot_product_attention(q, k, v, scale=0.3, enable_gqa=True)).abs().max().item() < 1e-12
    tri = torch.tril(torch.ones((9, 9), dtype=torch.bool))[None].expand(2, 9, 9)
    causal = oracle.masked_attn(q, k, v, tri, None, True)
    ref = F.scaled_dot_product_attention(q, k, v, is_causal=True, enable_gqa=True)
    assert (causal - ref).abs().max().item() < 1e-12


def test_random_mask_against_literal_loops():
    q, k, v = _rand((1, 2, 5, 3), 4), _rand((1, 2, 7, 3), 5), _rand((1, 2, 7, 3), 6)
    mask = torch.rand((1, 5, 7), generator=torch.Generator().manual_seed(7)) < 0.5
    mask[0, 2] = False
    got = oracle.masked_attn(q, k, v, mask, 0.7)
    for h in range(2):
        for i in range(5):
            keys = [j for j in range(7) if mask[0, i, j]]
            if not keys:
                assert got[0, h, i].abs().max().item() == 0.0
                continue
            s = [0.7 * sum(float(q[0, h, i, d]) * float(k[0, h, j, d]) for d in range(3)) for j in keys]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            for d in range(3):
                want = sum(wj * float(v[0, h, j, d]) for wj, j in zip(w, keys)) / sum(w)
                assert abs(float(got[0, h, i, d]) - want) < 1e-12


def test_single_key_row_copies_value():
    q, k, v = _rand((1, 1, 3, 4), 8), _rand((1, 1, 6, 4), 9), _rand((1, 1, 6, 4), 10)
    mask = torch.zeros((1, 3, 6), dtype=torch.bool)
    mask[0, 1, 4] = True
    got = oracle.masked_attn(q, k, v, mask)
    assert torch.equal(got[0, 0, 1], v[0, 0, 4]) and (got[0, 0, 0] == 0).all() and (got[0, 0, 2] == 0).all()


def test_bad_shapes_raise():
    q, k = _rand((1, 2, 3, 4), 1), _rand((1, 2, 5, 4), 2)
    with pytest.raises(ValueError):
        oracle.masked_attn(q, k, k, torch.ones((1, 5, 3), dtype=torch.bool))
    with pytest.raises(ValueError):
        oracle.masked_attn(q, _rand((1, 1, 5, 4), 3), _rand((1, 1, 5, 4), 3), torch.ones((1, 3, 5), dtype=torch.bool))
