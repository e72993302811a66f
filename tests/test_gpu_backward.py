"""GPU training path vs the CPU fp64 oracle: forward log-sum-exp and the backward.

Tolerances, from the arithmetic:
* lse: the kernel sums the bf16-rounded probabilities (relative rounding <= 2^-8
  each), so |lse - oracle| <= 2^-8 + fp32 rounding; the test allows 5e-3.
* dq, dk, dv: every term carries relative rounding of order 2^-8 (P and dS rounded
  to bf16 before their products, lse as above, the bf16 output O inside
  rowsum(dO * O), and the final bf16 rounding), so the error scales with the
  gradient itself: max |gpu - oracle| <= 2e-2 * max |oracle| and mean |gpu - oracle|
  <= 5e-3 * mean |oracle|, per tensor.
The oracle gets the same bf16 inputs (q, k, v, dout) upcast exactly.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import oracle_doc_ids, say
from workloads import make_layout, make_qkv, random_layout

pytestmark = pytest.mark.gpu

LSE_TOL = 5e-3
REL_MAX = 2e-2
REL_MEAN = 5e-3


@pytest.fixture(scope="module")
def psb():
    import packed_sequence_block_amd as m
    m.load()
    return m


def check_grad(got, ref, what):
    g = got.detach().float().cpu().double()
    r = torch.as_tensor(ref, dtype=torch.float64)
    assert torch.isfinite(g).all(), f"{what}: non-finite"
    d = (g - r).abs()
    scale_max = max(r.abs().max().item(), 1e-6)
    scale_mean = max(r.abs().mean().item(), 1e-9)
    assert d.max().item() <= REL_MAX * scale_max, f"{what}: max err {d.max().item():.3e} vs {scale_max:.3e}"
    assert d.mean().item() <= REL_MEAN * scale_mean, f"{what}: mean err {d.mean().item():.3e} vs {scale_mean:.3e}"


def run_case(psb, q, k, v, ids, seq_start, scale, gqa, seed, what):
    dev = "cuda"
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    idd = torch.as_tensor(ids, dtype=torch.int32).to(dev)
    say(what, "B", q.shape[0], "Hq", q.shape[1], "Hkv", k.shape[1], "L", q.shape[2], "S", k.shape[2],
        "D", q.shape[3], "seq_start", seq_start)
    out, lse, ws = psb.blockdiag_attn_fwd_lse(qd, kd, vd, idd, seq_start, scale, gqa)
    # forward output equals the plain forward's
    plain = psb.blockdiag_attn_fwd(qd, kd, vd, idd, seq_start, scale, gqa)
    assert torch.equal(out, plain), f"{what}: training forward output differs from the forward"
    lse_ref = oracle.blockdiag_attn_lse(q, k, ids, seq_start, scale, gqa)
    lg = lse.cpu().double()
    fin = torch.isfinite(lse_ref)
    assert torch.equal(torch.isfinite(lg), fin), f"{what}: lse -inf pattern"
    assert (lg[fin] - lse_ref[fin]).abs().max().item() <= LSE_TOL if fin.any() else True, f"{what}: lse"
    g = torch.Generator().manual_seed(seed)
    dout = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    dq, dk, dv = psb.blockdiag_attn_bwd(qd, kd, vd, out, dout.to(dev), lse, idd, ws, seq_start, scale, gqa)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.blockdiag_attn_bwd(q, k, v, dout, ids, seq_start, scale, gqa)
    check_grad(dq, rq, what + " dq")
    check_grad(dk, rk, what + " dk")
    check_grad(dv, rv, what + " dv")
    return dq, dk, dv


def test_config1(psb):
    lay = make_layout(1)
    q, k, v = make_qkv(lay)
    run_case(psb, q, k, v, oracle_doc_ids(lay), lay.seq_start, None, lay.enable_gqa, 11, "bwd cfg1")


SMALL = [
    # (seed, B, S, L, seq_start, Hq, Hkv, D, pad)
    (1, 1, 300, 300, 0, 4, 4, 64, 20),
    (2, 2, 520, 520, 0, 8, 2, 128, 0),
    (3, 1, 700, 256, 300, 4, 1, 128, 0),
    (4, 1, 1100, 1100, 0, 16, 1, 64, 37),
    (5, 1, 640, 200, 190, 8, 8, 128, 5),
    (6, 3, 260, 260, 0, 2, 2, 64, 60),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"seed{c[0]}" for c in SMALL])
def test_random_small(psb, case):
    seed, B, S, L, s0, Hq, Hkv, D, pad = case
    lay = random_layout(seed, B=B, S=S, L=L, seq_start=s0, Hq=Hq, Hkv=Hkv, D=D, max_pad=pad)
    q, k, v = make_qkv(lay, seed_base=5000 + 10 * seed)
    run_case(psb, q, k, v, oracle_doc_ids(lay), s0, None, Hq != Hkv, 100 + seed, f"bwd random-{seed}")


def test_negative_scale_and_lead_padding(psb):
    B, S, H, D = 1, 200, 2, 64
    ids = np.full((1, S), -1000, dtype=np.int64)
    ids[0, 13:90] = 4
    ids[0, 90:170] = 9
    g = torch.Generator().manual_seed(7)
    q, k, v = (torch.randn((B, H, S, D), generator=g).to(torch.bfloat16) for _ in range(3))
    run_case(psb, q, k, v, ids, 0, -0.2, False, 8, "bwd negative scale")


def gpu_fwd_bwd(psb, q, k, v, ids, seq_start, dout, gqa):
    dev = "cuda"
    qd, kd, vd = q.contiguous().to(dev), k.to(dev), v.to(dev)
    idd = torch.as_tensor(ids, dtype=torch.int32).to(dev)
    out, lse, ws = psb.blockdiag_attn_fwd_lse(qd, kd, vd, idd, seq_start, None, gqa)
    res = psb.blockdiag_attn_bwd(qd, kd, vd, out, dout.contiguous().to(dev), lse, idd, ws, seq_start, None, gqa)
    torch.cuda.synchronize()
    return [t.float().cpu() for t in res]


def test_shards_sum_to_full(psb):
    # a partition of the rows into two shards: dq is the concatenation and dk / dv
    # the sum of the shards' results (the pages' per-rank gradient routing)
    lay = random_layout(21, B=1, S=600, L=600, seq_start=0, Hq=4, Hkv=2, D=128)
    q, k, v = make_qkv(lay, seed_base=6000)
    ids = oracle_doc_ids(lay)
    g = torch.Generator().manual_seed(31)
    dout = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    a = 256
    say("bwd shards at", a)
    s1 = gpu_fwd_bwd(psb, q[:, :, :a], k, v, ids, 0, dout[:, :, :a], True)
    s2 = gpu_fwd_bwd(psb, q[:, :, a:], k, v, ids, a, dout[:, :, a:], True)
    rq, rk, rv = oracle.blockdiag_attn_bwd(q, k, v, dout, ids, 0, None, True)
    check_grad(torch.cat([s1[0], s2[0]], dim=2), rq, "shards dq")
    check_grad(s1[1] + s2[1], rk, "shards dk")
    check_grad(s1[2] + s2[2], rv, "shards dv")


def test_no_query_rows_gives_zero_kv_gradients(psb):
    # an empty query shard: dq is empty and no key receives a gradient
    dev = "cuda"
    g = torch.Generator().manual_seed(3)
    q = torch.zeros((1, 2, 0, 64), dtype=torch.bfloat16, device=dev)
    k, v = (torch.randn((1, 2, 50, 64), generator=g).to(torch.bfloat16).to(dev) for _ in range(2))
    ids = torch.ones((1, 50), dtype=torch.int32, device=dev)
    say("bwd empty shard")
    out, lse, ws = psb.blockdiag_attn_fwd_lse(q, k, v, ids, 20, None, False)
    dq, dk, dv = psb.blockdiag_attn_bwd(q, k, v, out, torch.zeros_like(q), lse, ids, ws, 20, None, False)
    torch.cuda.synchronize()
    assert dq.numel() == 0
    assert torch.count_nonzero(dk).item() == 0 and torch.count_nonzero(dv).item() == 0


def test_autograd_function(psb):
    # loss.backward() through the autograd wrapper gives the oracle's gradients
    lay = random_layout(41, B=1, S=400, L=400, seq_start=0, Hq=4, Hkv=2, D=64)
    q, k, v = make_qkv(lay, seed_base=7000)
    ids = oracle_doc_ids(lay)
    g = torch.Generator().manual_seed(9)
    dout = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    dev = "cuda"
    qd, kd, vd = (t.to(dev).requires_grad_(True) for t in (q, k, v))
    say("bwd autograd")
    out = psb.blockdiag_attention(qd, kd, vd, torch.as_tensor(ids, dtype=torch.int32).to(dev), 0, None, True)
    (out.float() * dout.to(dev).float()).sum().backward()
    torch.cuda.synchronize()
    rq, rk, rv = oracle.blockdiag_attn_bwd(q, k, v, dout, ids, 0, None, True)
    check_grad(qd.grad, rq, "autograd dq")
    check_grad(kd.grad, rk, "autograd dk")
    check_grad(vd.grad, rv, "autograd dv")


@pytest.mark.parametrize("c", [2, 3, 4, 5])
def test_full_size_one_document(psb, c):
    # the full-size training path (all rows, all heads, the bench's configuration), checked
    # on one document: its rows' dq depend only on those rows, and its keys' dk / dv only
    # on the rows of the same document, so the oracle on that document alone gives them
    lay = make_layout(c)
    q, k, v = make_qkv(lay)
    ids = oracle_doc_ids(lay)
    g = torch.Generator().manual_seed(50 + c)
    dout = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    dev = "cuda"
    say("bwd full size", lay.name)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    idd = torch.as_tensor(ids, dtype=torch.int32).to(dev)
    out, lse, ws = psb.blockdiag_attn_fwd_lse(qd, kd, vd, idd, lay.seq_start, None, lay.enable_gqa)
    dq, dk, dv = psb.blockdiag_attn_bwd(qd, kd, vd, out, dout.to(dev), lse, idd, ws, lay.seq_start, None,
                                        lay.enable_gqa)
    torch.cuda.synchronize()
    # a document that lies inside the query shard, of moderate length
    b = 0
    cu = lay.cu_seqlens(b)
    lo_q, hi_q = lay.seq_start, lay.seq_start + lay.L
    cands = [(int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)
             if cu[i] >= lo_q and cu[i + 1] <= hi_q and 64 <= cu[i + 1] - cu[i] <= 1500]
    assert cands, "no document of moderate length inside the shard"
    d0, d1 = cands[len(cands) // 2]
    r0, r1 = d0 - lay.seq_start, d1 - lay.seq_start
    sub = np.asarray(ids[b:b + 1])
    rq, rk, rv = oracle.blockdiag_attn_bwd(q[b:b + 1, :, r0:r1], k[b:b + 1], v[b:b + 1], dout[b:b + 1, :, r0:r1],
                                           sub, d0, None, lay.enable_gqa)
    check_grad(dq[b:b + 1, :, r0:r1].cpu(), rq, f"{lay.name} dq")
    check_grad(dk[b:b + 1, :, d0:d1].cpu(), rk[:, :, d0:d1], f"{lay.name} dk")
    check_grad(dv[b:b + 1, :, d0:d1].cpu(), rv[:, :, d0:d1], f"{lay.name} dv")


def test_long_documents_split_key_tiles(psb):
    # one 4096-token document and a short one: the long document's key tiles see thousands
    # of rows, so the key-side plan cuts them into row chunks and spends its whole slot
    # budget (the rest stay whole); gradients still match the oracle and repeat bit for bit
    S = 4600
    ids = np.full((1, S), 2, dtype=np.int32)
    ids[0, :4096] = 1
    ids[0, 4550:] = oracle.PAD_DOC_ID
    g = torch.Generator().manual_seed(601)
    q = torch.randn((1, 4, S, 64), generator=g).to(torch.bfloat16)
    k = torch.randn((1, 2, S, 64), generator=g).to(torch.bfloat16)
    v = torch.randn((1, 2, S, 64), generator=g).to(torch.bfloat16)
    grads = run_case(psb, q, k, v, ids, 0, None, True, 602, "bwd split tiles")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    idd = torch.as_tensor(ids).cuda()
    out, lse, ws = psb.blockdiag_attn_fwd_lse(qd, kd, vd, idd, 0, None, True)
    dout = torch.randn(q.shape, generator=torch.Generator().manual_seed(602)).to(torch.bfloat16).cuda()
    again = psb.blockdiag_attn_bwd(qd, kd, vd, out, dout, lse, idd, ws, 0, None, True)
    torch.cuda.synchronize()
    for a, b in zip(grads, again):
        assert torch.equal(a, b)


def _full_size_grads(psb, lay, seed):
    q, k, v = make_qkv(lay)
    ids = oracle_doc_ids(lay)
    dout = torch.randn(q.shape, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)
    dev = "cuda"
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    idd = torch.as_tensor(ids, dtype=torch.int32).to(dev)
    out, lse, ws = psb.blockdiag_attn_fwd_lse(qd, kd, vd, idd, lay.seq_start, None, lay.enable_gqa)
    dq, dk, dv = psb.blockdiag_attn_bwd(qd, kd, vd, out, dout.to(dev), lse, idd, ws, lay.seq_start, None,
                                        lay.enable_gqa)
    torch.cuda.synchronize()
    return q, k, v, ids, dout, dq.cpu(), dk.cpu(), dv.cpu()


@pytest.mark.parametrize("c", [2, 3, 4])
def test_whole_gradients(psb, c):
    # every element of dq, dk, dv at full size against the oracle (one batch row at a time)
    lay = make_layout(c)
    say("bwd whole gradients", lay.name)
    q, k, v, ids, dout, dq, dk, dv = _full_size_grads(psb, lay, 60 + c)
    for b in range(lay.B):
        rq, rk, rv = oracle.blockdiag_attn_bwd(q[b:b + 1], k[b:b + 1], v[b:b + 1], dout[b:b + 1],
                                               np.asarray(ids[b:b + 1]), lay.seq_start, None, lay.enable_gqa)
        check_grad(dq[b:b + 1], rq, f"{lay.name} row {b} dq")
        check_grad(dk[b:b + 1], rk, f"{lay.name} row {b} dk")
        check_grad(dv[b:b + 1], rv, f"{lay.name} row {b} dv")


def test_whole_gradients_cfg5_kv_head(psb):
    # workload 5 (S = 65536): every element of the gradients of kv head 1 and its 16 query
    # heads (heads never mix, so the oracle on that slice alone gives them)
    lay = make_layout(5)
    g, G = 1, lay.Hq // lay.Hkv
    say("bwd whole gradients", lay.name, "kv head", g)
    q, k, v, ids, dout, dq, dk, dv = _full_size_grads(psb, lay, 65)
    hs = slice(g * G, (g + 1) * G)
    rq, rk, rv = oracle.blockdiag_attn_bwd(q[:, hs], k[:, g:g + 1], v[:, g:g + 1], dout[:, hs], np.asarray(ids),
                                           lay.seq_start, None, True)
    check_grad(dq[:, hs], rq, f"{lay.name} kv head {g} dq")
    check_grad(dk[:, g:g + 1], rk, f"{lay.name} kv head {g} dk")
    check_grad(dv[:, g:g + 1], rv, f"{lay.name} kv head {g} dv")


def _extreme_case(D, regime):
    lay = random_layout(1400 + D, B=1, S=700, L=None, seq_start=0, Hq=4, Hkv=2, D=D, max_doc=300, max_pad=20)
    q, k, v = make_qkv(lay, seed_base=7300 + D)
    scale = 1.0
    if regime == "wide":  # scores of magnitude in the hundreds: rows close to one-hot
        q = (q.float() * 6).to(torch.bfloat16)
        k = (k.float() * 6).to(torch.bfloat16)
    elif regime == "growing_steep":  # key j scaled by 1 + j / 40
        k = (k.float() * (1.0 + torch.arange(lay.S, dtype=torch.float32) / 40.0)[None, None, :, None]).to(torch.bfloat16)
    elif regime == "growing_mild":  # key j scaled by 1 + j / 300, the default scale
        k = (k.float() * (1.0 + torch.arange(lay.S, dtype=torch.float32) / 300.0)[None, None, :, None]).to(torch.bfloat16)
        scale = D ** -0.5
    else:  # far below zero: q . k near -8 D for every pair
        q = torch.full_like(q, 2.0)
        k = (torch.full_like(k, -2.0).float() + 0.05 * k.float()).to(torch.bfloat16)
    return lay, q, k, v, oracle_doc_ids(lay), scale


@pytest.mark.parametrize("D", [64, 128])
def test_growing_scores_gradients(psb, D):
    # scores that grow along the keys move the forward's exp2 offset on many tiles; the
    # backward recomputes P from the forward's lse and must still give the oracle's gradients
    lay, q, k, v, ids, scale = _extreme_case(D, "growing_mild")
    run_case(psb, q, k, v, ids, 0, scale, True, 7400 + D, f"growing scores D{D}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("regime", ["wide", "growing_steep", "far_below"])
def test_extreme_score_ranges_lse(psb, D, regime):
    # The lse the backward consumes, in the forward's extreme regimes (the forward output is
    # checked by the forward test of the same inputs).  Gradients are not compared here: when
    # rows are close to one-hot, or all keys share a large common component, dS = P (dP -
    # delta) is a small difference of order-one terms, and delta comes from the bf16 output
    # that the method stores.  That rounding alone moves dQ by 2-7 times the relative
    # tolerance in the fp64 oracle's own arithmetic.  It is a property of the method's
    # storage, not of this kernel.
    lay, q, k, v, ids, scale = _extreme_case(D, regime)
    idd = torch.as_tensor(ids, dtype=torch.int32).cuda()
    say(regime, "D", D)
    _, lse, _ = psb.blockdiag_attn_fwd_lse(q.cuda(), k.cuda(), v.cuda(), idd, 0, scale, True)
    torch.cuda.synchronize()
    lse_ref = oracle.blockdiag_attn_lse(q, k, ids, 0, scale, True)
    lg = lse.cpu().double()
    fin = torch.isfinite(lse_ref)
    assert torch.equal(torch.isfinite(lg), fin), f"{regime} D{D}: lse -inf pattern"
    err = (lg[fin] - lse_ref[fin]).abs().max().item()
    say(regime, "lse max abs err", err)
    # lse is of the order of the largest score (up to about 3000 here): fp32 keeps it to a
    # relative 2^-23 of that, so the bound scales with it
    bound = max(LSE_TOL, 4e-7 * lse_ref[fin].abs().max().item())
    assert err <= bound, f"{regime} D{D}: lse err {err:.3e} > {bound:.3e}"
