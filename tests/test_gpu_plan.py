"""The tile plan (psb_blockdiag_attn_plan) against a host reference of its tables.

The plan is the step between the document ids and the attention kernel: for every
32-row query block, the key range [start of the first valid row's document, last
valid row + 1), and the list of row-tile records ordered by key-range length (or
in row order when the longest record is short next to the share of all records that
each concurrent workgroup slot of the attention kernel gets).  Its tables are checked
directly here, exactly (integers) except for the order of records with equal length,
which the counting sort leaves open.
"""

import ctypes

import numpy as np
import pytest
import torch

from gpu_common import oracle_doc_ids, say
from workloads import make_layout

pytestmark = pytest.mark.gpu

PAD = -1000
ROWS, KEYS = 32, 64


@pytest.fixture(scope="module")
def lib():
    from packed_sequence_block_amd import _lib
    return _lib.load()


def ref_blocks(ids, L, seq_start):
    """Key range (lo, hi) of every 32-row query block, from the definition."""
    B, S = ids.shape
    nblk = (L + ROWS - 1) // ROWS
    lo = np.zeros((B, nblk), np.int64)
    hi = np.zeros((B, nblk), np.int64)
    pos = np.arange(S)
    for b in range(B):
        row = ids[b]
        starts = np.where(np.concatenate([[True], row[1:] != row[:-1]]), pos, 0)
        run_start = np.maximum.accumulate(starts)      # first position of each position's run
        for j in range(nblk):
            q = seq_start + np.arange(j * ROWS, min(L, (j + 1) * ROWS))
            q = q[row[q] != PAD]
            if q.size:
                lo[b, j], hi[b, j] = run_start[q[0]], q[-1] + 1
    return lo, hi


def pad256(n):
    return (n + 255) // 256 * 256


def run_plan(lib, ids_np, Hq, Hkv, L, seq_start, D=128):
    B, S = ids_np.shape
    ids = torch.as_tensor(ids_np, dtype=torch.int32).cuda()
    n = lib.psb_blockdiag_attn_fwd_workspace_size(B, Hq, Hkv, L, D)
    ws = torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")  # stale bytes must not matter
    st = lib.psb_blockdiag_attn_plan(ctypes.c_void_p(ids.data_ptr()), B, Hq, Hkv, L, S, D, seq_start,
                                     1 if Hq != Hkv else 0, ctypes.c_void_p(ws.data_ptr()), n, None)
    assert st == 0, st
    torch.cuda.synchronize()
    return ws.cpu().numpy().view(np.int32)


def check_plan(lib, ids_np, Hq, Hkv, L, seq_start):
    check_plan_words(run_plan(lib, ids_np, Hq, Hkv, L, seq_start), ids_np, Hq, Hkv, L, seq_start)


def concurrent_slots(D=128):
    """Workgroups the attention kernel runs at once: CUs x 2 at D = 128, x 3 at D = 64."""
    return torch.cuda.get_device_properties(0).multi_processor_count * (2 if D == 128 else 3)


def check_plan_words(words, ids_np, Hq, Hkv, L, seq_start, D=128):
    """The plan tables in a workspace (as int32 words) against the definition."""
    B = ids_np.shape[0]
    group = Hq // Hkv
    nh = 4 if group % 4 == 0 else (2 if group % 2 == 0 else 1)
    nr = 4 // nh
    nblk = (L + ROWS - 1) // ROWS
    ntile_row = (nblk + nr - 1) // nr
    lo, hi = ref_blocks(ids_np, L, seq_start)
    off = pad256(4 * B * nblk) // 4
    got_lo = words[:B * nblk].reshape(B, nblk)
    got_hi = words[off:off + B * nblk].reshape(B, nblk)
    assert np.array_equal(got_lo, lo), "block lo"
    assert np.array_equal(got_hi, hi), "block hi"
    rec = words[2 * off:2 * off + 16 * B * ntile_row].reshape(-1, 16)
    seen = set()
    iters, full_iters, order = [], [], []
    for r in rec:
        b, rt = int(r[0]), int(r[1])
        assert 0 <= b < B and 0 <= rt < ntile_row
        seen.add((b, rt))
        blo, bhi = np.zeros(4, np.int64), np.zeros(4, np.int64)
        for j in range(nr):
            if rt * nr + j < nblk:
                blo[j], bhi[j] = lo[b, rt * nr + j], hi[b, rt * nr + j]
        nz = bhi > blo
        want_lo = int(blo[nz].min()) if nz.any() else 0
        want_hi = int(bhi[nz].max()) if nz.any() else 0
        assert (int(r[2]), int(r[3])) == (want_lo, want_hi), (b, rt)
        assert np.array_equal(r[4:8], blo) and np.array_equal(r[8:12], bhi), (b, rt)
        n = -(-(want_hi - want_lo) // KEYS) if want_hi > want_lo else 0
        full_iters.append(n)
        iters.append(min(n, 2047))
        order.append(b * ntile_row + rt)
    assert len(seen) == B * ntile_row, "every row tile exactly once"
    units = Hq // nh
    if 4 * max(full_iters) * concurrent_slots(D) <= sum(full_iters) * units:
        assert order == list(range(B * ntile_row)), "row order"
    else:
        assert all(a >= b for a, b in zip(iters, iters[1:])), "longest key range first"
    return order


@pytest.mark.parametrize("c", [1, 2, 3, 4, 5])
def test_named_layouts(lib, c):
    lay = make_layout(c)
    say("plan cfg", c)
    check_plan(lib, oracle_doc_ids(lay), lay.Hq, lay.Hkv, lay.L, lay.seq_start)


@pytest.mark.parametrize("c,row_order", [(2, False), (3, False), (4, True)])
def test_order_choice(lib, c, row_order):
    # short documents against a large grid keep row order (workload 4); long single
    # records next to a small grid are ordered longest first (workloads 2, 3)
    lay = make_layout(c)
    say("plan order cfg", c)
    order = check_plan_words(run_plan(lib, oracle_doc_ids(lay), lay.Hq, lay.Hkv, lay.L, lay.seq_start),
                             oracle_doc_ids(lay), lay.Hq, lay.Hkv, lay.L, lay.seq_start)
    assert (order == sorted(order)) == row_order


def random_ids(rng, B, S):
    ids = np.full((B, S), PAD, np.int32)
    for b in range(B):
        p = int(rng.integers(0, 40))  # leading padding
        d = 1
        while p < S:
            n = int(rng.choice([1, 7, 31, 32, 33, 64, 200, 1500]))
            ids[b, p:p + n] = d if rng.random() > 0.15 else PAD
            p += n
            d += 1
    return ids


@pytest.mark.parametrize("seed", range(10))
def test_random_layouts(lib, seed):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 4))
    S = int(rng.integers(1, 6000))
    L = int(rng.integers(1, S + 1))
    seq_start = int(rng.integers(0, S - L + 1))
    Hq, Hkv = [(8, 2), (4, 4), (6, 3)][seed % 3]
    ids = random_ids(rng, B, S)
    say("plan random seed", seed, "B", B, "S", S, "L", L, "seq_start", seq_start, "heads", Hq, Hkv)
    check_plan(lib, ids, Hq, Hkv, L, seq_start)


@pytest.mark.parametrize("B,S,L,seq_start", [(1, 16384, 16384, 0), (2, 9000, 8224, 700), (1, 16416, 16416, 0)])
def test_larger_rows(lib, B, S, L, seq_start):
    # several hundred query blocks per row, a shard of two rows, a ragged last block
    rng = np.random.default_rng(S + L)
    ids = random_ids(rng, B, S)
    say("plan two-kernel B", B, "S", S, "L", L)
    check_plan(lib, ids, 8, 2, L, seq_start)
