"""Query shard against a delivered key window (left-halo delivery) on the GPU.

The window start is bit-exact against the oracle's; the windowed forward is checked
against the oracle run on the WHOLE rows' keys (the window must not change the result)
and, when the window covers every needed key, must equal the whole-row kernel bit for
bit (the same tiles are visited); the windowed backward is checked against the oracle's
gradients and against the whole-row backward.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import compare, oracle_doc_ids, say
from test_gpu_backward import check_grad
from workloads import make_layout, make_qkv, random_layout

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def psb():
    import packed_sequence_block_amd as m
    m.load()
    return m


def _pad_rows(ids, s0, L, B, Hq):
    pad = torch.as_tensor(np.asarray(ids)[:, s0:s0 + L] == oracle.PAD_DOC_ID)
    return pad.unsqueeze(1).expand(B, Hq, L)


@pytest.mark.parametrize("c", [2, 3, 4, 5])
def test_window_start_named(psb, c):
    lay = make_layout(c)
    ids = oracle_doc_ids(lay)
    for s0, L in [(lay.seq_start, lay.L), (lay.S // 2 + 37, lay.S // 4), (lay.S - 100, 100), (0, 0)]:
        say("window start", lay.name, s0, L)
        got = psb.shard_kv_window_start(torch.as_tensor(ids).cuda(), s0, L).cpu().numpy()
        assert got.tolist() == oracle.kv_window_start(ids, s0, L).tolist()


@pytest.mark.parametrize("seed", range(8))
def test_window_start_random(psb, seed):
    rng = np.random.default_rng(600 + seed)
    S = int(rng.integers(1, 5000))
    s0 = int(rng.integers(0, S))
    L = int(rng.integers(0, S - s0 + 1))
    lay = random_layout(700 + seed, B=3, S=S, L=L, seq_start=s0, max_doc=int(rng.integers(1, 2000)),
                        max_pad=S // 3)
    ids = oracle_doc_ids(lay)
    say("window start random", seed, S, s0, L)
    got = psb.shard_kv_window_start(torch.as_tensor(ids).cuda(), s0, L).cpu().numpy()
    assert got.tolist() == oracle.kv_window_start(ids, s0, L).tolist()


WIN = [
    # (seed, B, S, L, seq_start, Hq, Hkv, D, max_doc, max_pad, extra keys past the shard)
    (1, 1, 700, 200, 300, 4, 2, 128, 250, 0, 0),
    (2, 2, 1000, 256, 512, 8, 8, 64, 400, 30, 100),
    (3, 1, 900, 129, 640, 16, 1, 128, 900, 0, 131),
    (4, 3, 500, 100, 100, 4, 4, 64, 60, 20, 0),
]


def _window(psb, ids, s0, L):
    w = psb.shard_kv_window_start(torch.as_tensor(ids).cuda(), s0, L)
    return int(w.min().item())


@pytest.mark.parametrize("case", WIN, ids=lambda c: f"seed{c[0]}")
def test_forward_window(psb, case):
    seed, B, S, L, s0, Hq, Hkv, D, md, mp, extra = case
    lay = random_layout(800 + seed, B=B, S=S, L=L, seq_start=s0, Hq=Hq, Hkv=Hkv, D=D, max_doc=md, max_pad=mp)
    q, k, v = make_qkv(lay, seed_base=8000 + 10 * seed)
    ids = oracle_doc_ids(lay)
    w = _window(psb, ids, s0, L)
    kv_end = min(S, s0 + L + extra)
    say("fwd window", seed, "w", w, "kv_end", kv_end)
    qd, idd = q.cuda(), torch.as_tensor(ids).cuda()
    kw, vw = k[:, :, w:kv_end].contiguous().cuda(), v[:, :, w:kv_end].contiguous().cuda()
    out = psb.blockdiag_attn_fwd_window(qd, kw, vw, idd, s0, w, None, Hq != Hkv, validate=True)
    full = psb.blockdiag_attn_fwd(qd, k.cuda(), v.cuda(), idd, s0, None, Hq != Hkv)
    torch.cuda.synchronize()
    assert torch.equal(out, full), "window forward differs from the whole-row forward"
    ref = oracle.blockdiag_attn(q, k, v, ids, s0, None, Hq != Hkv)
    compare(out, ref, _pad_rows(ids, s0, L, B, Hq), f"window-{seed}")


def test_forward_window_full_size_cp_shard(psb):
    # the context-parallel shard workload at its real shape, with only its own keys
    # plus the left halo delivered
    lay = make_layout(3)
    q, k, v = make_qkv(lay)
    ids = oracle_doc_ids(lay)
    s0, L = lay.seq_start, lay.L
    w = _window(psb, ids, s0, L)
    say("fwd window", lay.name, "w", w, "keys", s0 + L - w, "of", lay.S)
    assert w < s0  # this layout's shard starts inside a document
    qd, idd = q.cuda(), torch.as_tensor(ids).cuda()
    out, lse, _ = psb.blockdiag_attn_fwd_window(qd, k[:, :, w:s0 + L].contiguous().cuda(),
                                                v[:, :, w:s0 + L].contiguous().cuda(), idd, s0, w, None,
                                                lay.enable_gqa, with_lse=True, validate=True)
    full, lse_full, _ = psb.blockdiag_attn_fwd_lse(qd, k.cuda(), v.cuda(), idd, s0, None, lay.enable_gqa)
    torch.cuda.synchronize()
    assert torch.equal(out, full) and torch.equal(lse, lse_full)
    rows = [0, 1, 577, 2048, L - 1]
    ref = oracle.blockdiag_attn_rows(q, k, v, ids, s0, None, lay.enable_gqa, 0, rows)
    compare(out[0][:, rows].permute(1, 0, 2), ref, None, "cfg3 window rows")


def test_window_too_late_is_reported(psb):
    # a window that starts after the first needed key: status raised, no fault
    ids = np.asarray([[1] * 100 + [2] * 500], dtype=np.int32)   # the shard [300, 500) sits in [100, 600)
    g = torch.Generator().manual_seed(9100)
    q = torch.randn((1, 2, 200, 64), generator=g).to(torch.bfloat16)
    k, v = (torch.randn((1, 2, 600, 64), generator=g).to(torch.bfloat16) for _ in range(2))
    w = _window(psb, ids, 300, 200)
    assert w == 100
    say("fwd window too late", w, 200)
    with pytest.raises(ValueError):
        psb.blockdiag_attn_fwd_window(q.cuda(), k[:, :, 200:].contiguous().cuda(), v[:, :, 200:].contiguous().cuda(),
                                      torch.as_tensor(ids).cuda(), 300, 200, None, False, validate=True)


def test_window_shape_errors(psb):
    q = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16, device="cuda")
    ids = torch.ones((1, 256), dtype=torch.int32, device="cuda")
    kv = torch.zeros((1, 2, 100, 64), dtype=torch.bfloat16, device="cuda")
    say("window shape errors")
    with pytest.raises(psb.PsbError):   # window starts after the shard
        psb.blockdiag_attn_fwd_window(q, kv, kv, ids, 100, 101)
    with pytest.raises(psb.PsbError):   # window ends before the shard does
        psb.blockdiag_attn_fwd_window(q, kv[:, :, :50].contiguous(), kv[:, :, :50].contiguous(), ids, 100, 100)
    with pytest.raises(psb.PsbError):   # window runs past the row
        psb.blockdiag_attn_fwd_window(q, kv, kv, ids, 200, 190)


@pytest.mark.parametrize("case", WIN, ids=lambda c: f"seed{c[0]}")
def test_backward_window(psb, case):
    seed, B, S, L, s0, Hq, Hkv, D, md, mp, extra = case
    lay = random_layout(800 + seed, B=B, S=S, L=L, seq_start=s0, Hq=Hq, Hkv=Hkv, D=D, max_doc=md, max_pad=mp)
    q, k, v = make_qkv(lay, seed_base=8000 + 10 * seed)
    ids = oracle_doc_ids(lay)
    w = _window(psb, ids, s0, L)
    kv_end = min(S, s0 + L + extra)
    g = torch.Generator().manual_seed(70 + seed)
    dout = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    gqa = Hq != Hkv
    say("bwd window", seed, "w", w, "kv_end", kv_end)
    qd, idd = q.cuda(), torch.as_tensor(ids).cuda()
    kw, vw = k[:, :, w:kv_end].contiguous().cuda(), v[:, :, w:kv_end].contiguous().cuda()
    out, lse, ws = psb.blockdiag_attn_fwd_window(qd, kw, vw, idd, s0, w, None, gqa, with_lse=True)
    dq, dk, dv = psb.blockdiag_attn_bwd_window(qd, kw, vw, out, dout.cuda(), lse, idd, ws, s0, w, None, gqa,
                                               validate=True)
    out_f, lse_f, ws_f = psb.blockdiag_attn_fwd_lse(qd, k.cuda(), v.cuda(), idd, s0, None, gqa)
    dq_f, dk_f, dv_f = psb.blockdiag_attn_bwd(qd, k.cuda(), v.cuda(), out_f, dout.cuda(), lse_f, idd, ws_f, s0,
                                              None, gqa)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq_f), "window dq differs from the whole-row dq"
    # keys outside the window get no gradient from this shard
    assert torch.count_nonzero(dk_f[:, :, :w]).item() == 0 and torch.count_nonzero(dk_f[:, :, kv_end:]).item() == 0
    rq, rk, rv = oracle.blockdiag_attn_bwd(q, k, v, dout, ids, s0, None, gqa)
    check_grad(dq.cpu(), rq, f"window-{seed} dq")
    check_grad(dk.cpu(), rk[:, :, w:kv_end], f"window-{seed} dk")
    check_grad(dv.cpu(), rv[:, :, w:kv_end], f"window-{seed} dv")
