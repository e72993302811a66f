"""The one-launch step preparation (psb_blockdiag_prepare) on the GPU: document ids and
run boundaries bit-exact against the oracle, plan tables against their definition (as
for psb_blockdiag_attn_plan), and attention run on its plan equal to the separate path."""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import say
from test_gpu_plan import check_plan_words
from workloads import make_layout, make_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def psb():
    import packed_sequence_block_amd as m
    m.load()
    return m


def padded_cu(rows):
    """[B, N + 1] boundaries, shorter rows repeating their last boundary."""
    n1 = max(len(r) for r in rows)
    return np.stack([np.concatenate([r, np.full(n1 - len(r), r[-1])]) for r in rows]).astype(np.int32)


def random_cu(rng, S):
    """Boundaries with lead / tail padding and zero-length documents."""
    cu = [int(rng.integers(0, max(1, S // 10)))]
    while True:
        n = int(rng.choice([0, 1, 5, 31, 32, 33, 64, 200, 900]))
        if cu[-1] + n > S - int(rng.integers(0, 3)):
            break
        cu.append(cu[-1] + n)
    return np.asarray(cu, dtype=np.int32)


def check(psb, rows, S, L, s0, Hq, Hkv, D):
    cu = padded_cu(rows)
    B = cu.shape[0]
    ids, seg, n, ws = psb.blockdiag_prepare(torch.as_tensor(cu).cuda(), S, Hq, Hkv, D, s0, L, Hq != Hkv,
                                            validate=True)
    torch.cuda.synchronize()
    ids_c, seg_c, n_c = ids.cpu().numpy(), seg.cpu().numpy(), n.cpu().numpy()
    for b in range(B):
        assert np.array_equal(ids_c[b], oracle.doc_ids_from_cu_seqlens(rows[b], S)[0]), f"ids row {b}"
        want = oracle.segment_cu_seqlens(ids_c[b])
        assert n_c[b] == len(want) - 1 and np.array_equal(seg_c[b, :n_c[b] + 1], want), f"segments row {b}"
    if L > 0:
        words = ws.cpu().numpy().view(np.int32)
        check_plan_words(words, ids_c, Hq, Hkv, L, s0, D)
    return ids, ws


@pytest.mark.parametrize("c", [1, 2, 3, 4, 5])
def test_named_layouts(psb, c):
    lay = make_layout(c)
    say("prepare", lay.name)
    check(psb, [np.asarray(lay.cu_seqlens(b), np.int32) for b in range(lay.B)], lay.S, lay.L, lay.seq_start,
          lay.Hq, lay.Hkv, lay.D)


@pytest.mark.parametrize("seed", range(10))
def test_random(psb, seed):
    rng = np.random.default_rng(1500 + seed)
    B = int(rng.integers(1, 5))
    S = int(rng.integers(1, 7000))
    L = int(rng.integers(0, S + 1))
    s0 = int(rng.integers(0, S - L + 1))
    Hq, Hkv = [(8, 2), (4, 4), (6, 3), (16, 1)][seed % 4]
    rows = [random_cu(rng, S) for _ in range(B)]
    say("prepare random", seed, "B", B, "S", S, "L", L, "s0", s0, "docs", [len(r) - 1 for r in rows])
    check(psb, rows, S, L, s0, Hq, Hkv, 128)


def test_degenerate(psb):
    say("prepare degenerate")
    check(psb, [np.asarray([0], np.int32)], 1, 1, 0, 4, 4, 64)             # no document: all padding
    check(psb, [np.asarray([3, 3, 3], np.int32)], 10, 10, 0, 4, 4, 64)     # only empty documents
    check(psb, [np.asarray([0, 10], np.int32)], 10, 0, 10, 4, 4, 64)       # empty shard at the end
    check(psb, [np.asarray([2, 7], np.int32), np.asarray([0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10], np.int32)],
          10, 10, 0, 8, 2, 128)
    ids, seg, n, _ = psb.blockdiag_prepare(torch.zeros((1, 1), dtype=torch.int32, device="cuda"), 0, 4, 4, 64, 0, 0)
    torch.cuda.synchronize()
    assert int(n.item()) == 0 and int(seg[0, 0].item()) == 0


def test_invalid_boundaries_set_status(psb):
    say("prepare invalid")
    for cu in ([0, 5, 3], [0, 12], [-1, 4]):
        with pytest.raises(ValueError):
            psb.blockdiag_prepare(torch.as_tensor([cu], dtype=torch.int32).cuda(), 10, 4, 4, 64, validate=True)


def test_attention_on_prepared_plan(psb):
    # the attention kernel run on this plan gives exactly the separate path's output
    lay = make_layout(3)
    q, k, v = (t.cuda() for t in make_qkv(lay))
    cu = torch.as_tensor(padded_cu([np.asarray(lay.cu_seqlens(0), np.int32)])).cuda()
    say("prepare + attention", lay.name)
    ids, _, _, ws = psb.blockdiag_prepare(cu, lay.S, lay.Hq, lay.Hkv, lay.D, lay.seq_start, lay.L, lay.enable_gqa)
    import ctypes
    lib = psb.load()
    out = torch.empty((lay.B, lay.Hq, lay.L, lay.D), dtype=torch.bfloat16, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = lib.psb_blockdiag_attn_fwd_planned(P(q), P(k), P(v), P(ids), lay.B, lay.Hq, lay.Hkv, lay.L, lay.S, lay.D,
                                            None, None, lay.seq_start, lay.D ** -0.5, 1, P(out), P(ws),
                                            ws.numel(), None, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    ref = psb.blockdiag_attn_fwd(q, k, v, ids, lay.seq_start, None, lay.enable_gqa)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_plan_sizes_around_the_single_launch_limit(psb):
    # one launch orders the plan while B * ceil(L / 32) <= 2048; past that a second kernel
    # does; both must give a valid plan and the same attention
    rng = np.random.default_rng(1601)
    for B, S in ((1, 65536), (1, 65537), (3, 22000)):
        rows = [random_cu(rng, S) for _ in range(B)]
        say("prepare limit", "B", B, "S", S, "blocks", B * ((S + 31) // 32))
        check(psb, rows, S, S, 0, 8, 2, 128)


def test_plan_with_boundaries_too_many_to_stage(psb):
    # B * (documents + 1) above the 4096 boundaries the plan workgroup stages in LDS: it reads
    # them from memory instead
    B, S = 3, 6000
    rows = [np.arange(0, S + 1, 1 + b, dtype=np.int32) for b in range(B)]
    say("prepare many documents", [len(r) - 1 for r in rows])
    check(psb, rows, S, S, 0, 4, 4, 64)
    check(psb, rows, S, 1000, 2500, 4, 4, 64)
