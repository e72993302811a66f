"""Pins for the oracle's key window of a query shard (``kv_window_start``).

Fixed independently of its mask-based code: hand-derived cases, a walk back over
document runs written separately, and the fact that defines a window — keys before
it never change the shard's attention output.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import PAD_DOC_ID
from gpu_common import oracle_doc_ids
from workloads import make_qkv, random_layout

P = PAD_DOC_ID


@pytest.mark.parametrize("ids,seq_start,L,want", [
    ([1, 1, 1, 2, 2, 2, 2, 3, 3], 4, 3, 3),        # the shard starts inside document 2
    ([1, 1, 1, 2, 2, 2, 2, 3, 3], 3, 3, 3),        # ... exactly at its start
    ([5, 5, P, P, P, 7], 2, 3, 2),                 # only padding rows: no halo
    ([4, 4, 4, 4, P, P, 9, 9], 4, 4, 4),           # padding then a new document
    ([8, 8, 8, 8, 8, 8, 8, 8], 6, 2, 0),           # one long document
    ([8, 8, 8, 8, 8, 8, 8, 8], 6, 0, 6),           # empty shard
])
def test_hand_cases(ids, seq_start, L, want):
    assert oracle.kv_window_start(np.asarray([ids]), seq_start, L).tolist() == [want]


def _walk_back(row, seq_start, L):
    lo = seq_start
    for q in range(seq_start, seq_start + L):
        if row[q] == PAD_DOC_ID:
            continue
        p = q
        while p > 0 and row[p - 1] == row[q]:
            p -= 1
        lo = min(lo, p)
    return lo


@pytest.mark.parametrize("seed", range(10))
def test_random_against_run_walk(seed):
    rng = np.random.default_rng(seed)
    S = int(rng.integers(20, 300))
    s0 = int(rng.integers(0, S))
    L = int(rng.integers(0, S - s0 + 1))
    lay = random_layout(200 + seed, B=3, S=S, L=L, seq_start=s0, max_pad=S // 4)
    ids = oracle_doc_ids(lay)
    got = oracle.kv_window_start(ids, s0, L)
    assert got.tolist() == [_walk_back(ids[b].tolist(), s0, L) for b in range(3)]


@pytest.mark.parametrize("seed", range(4))
def test_keys_before_the_window_never_matter(seed):
    # replace every key / value before the window with large garbage: the shard's
    # output does not move (and one key earlier than the window would)
    lay = random_layout(300 + seed, B=2, S=160, L=60, seq_start=70, max_doc=50, max_pad=10)
    q, k, v = make_qkv(lay, seed_base=900 + seed)
    ids = oracle_doc_ids(lay)
    w = oracle.kv_window_start(ids, 70, 60)
    ref = oracle.blockdiag_attn(q, k, v, ids, 70, None, True)
    k2, v2 = k.clone(), v.clone()
    for b in range(2):
        k2[b, :, :w[b]] = 40.0
        v2[b, :, :w[b]] = -300.0
    got = oracle.blockdiag_attn(q, k2, v2, ids, 70, None, True)
    assert torch.equal(got, ref)
    for b in range(2):
        if w[b] < 70:  # the window's first key is needed by some row
            qpos = torch.arange(70, 130)
            assert bool(oracle.allowed_mask(torch.as_tensor(ids[b]).long(), qpos)[:, w[b]].any())
