"""HIP attention vs the fp64 oracle: full outputs on small/ragged problems."""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import compare, oracle_doc_ids, say
from workloads import Layout, make_layout, make_qkv, random_layout

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def psb():
    import packed_sequence_block_amd as m
    m.load()
    return m


def run_case(psb, lay, seed_base=None, scale=None, ids=None):
    q, k, v = make_qkv(lay, seed_base=seed_base)
    if ids is None:
        ids = oracle_doc_ids(lay)
    say(lay.name, "B", lay.B, "S", lay.S, "L", lay.L, "s0", lay.seq_start, "Hq", lay.Hq, "Hkv", lay.Hkv,
        "D", lay.D)
    out = psb.blockdiag_attn_fwd(q.cuda(), k.cuda(), v.cuda(), torch.as_tensor(ids).cuda(), lay.seq_start,
                                 scale, lay.enable_gqa)
    torch.cuda.synchronize()
    ref = oracle.blockdiag_attn(q, k, v, ids, lay.seq_start, scale, lay.enable_gqa)
    qpos = np.arange(lay.seq_start, lay.seq_start + lay.L)
    pad = torch.as_tensor(np.asarray(ids)[:, qpos] == oracle.PAD_DOC_ID)       # [B, L]
    pad_rows = pad.unsqueeze(1).expand(lay.B, lay.Hq, lay.L)
    return compare(out, ref, pad_rows, lay.name)


def test_config1_full(psb):
    mx, mean = run_case(psb, make_layout(1))
    say("config 1 whole output max/mean abs err", mx, mean)


SMALL = [
    # (seed, B, S, L, seq_start, Hq, Hkv, D, max_doc, max_pad)
    (1, 1, 1, None, 0, 1, 1, 64, 1, 0),
    (2, 1, 31, None, 0, 4, 2, 64, 40, 0),
    (3, 1, 33, None, 0, 4, 4, 128, 40, 0),
    (4, 2, 100, None, 0, 8, 2, 128, 30, 9),
    (5, 1, 257, None, 0, 16, 1, 64, 300, 17),
    (6, 3, 300, None, 0, 6, 3, 128, 70, 40),
    (7, 1, 1000, None, 0, 32, 8, 128, 400, 100),
    (8, 1, 1000, 333, 411, 8, 8, 64, 250, 0),
    (9, 2, 700, 129, 64, 16, 4, 128, 1000, 0),
    (10, 1, 513, None, 0, 2, 2, 128, 5, 3),
    (11, 1, 640, 96, 544, 4, 1, 128, 200, 60),
    (12, 2, 2048, None, 0, 8, 8, 128, 2048, 0),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"seed{c[0]}")
def test_random_small(psb, case):
    seed, B, S, L, s0, Hq, Hkv, D, md, mp = case
    lay = random_layout(seed, B=B, S=S, L=L, seq_start=s0, Hq=Hq, Hkv=Hkv, D=D, max_doc=md, max_pad=mp,
                        enable_gqa=Hq != Hkv)
    run_case(psb, lay, seed_base=seed * 11)


def test_lead_and_mid_padding(psb):
    # padding before the first document and between documents
    lay = Layout("lead-mid-pad", 0, B=1, S=300, L=300, seq_start=0, Hq=4, Hkv=2, D=128)
    ids = np.full((1, 300), oracle.PAD_DOC_ID, dtype=np.int32)
    ids[0, 20:90] = 1
    ids[0, 90:130] = 2
    ids[0, 170:260] = 3
    ids[0, 261:262] = 4
    run_case(psb, lay, seed_base=77, ids=ids)


def test_all_padding(psb):
    lay = Layout("all-pad", 0, B=2, S=150, L=150, seq_start=0, Hq=2, Hkv=1, D=64)
    ids = np.full((2, 150), oracle.PAD_DOC_ID, dtype=np.int32)
    run_case(psb, lay, seed_base=78, ids=ids)


def test_arbitrary_ids_and_explicit_scale(psb):
    # ids need not come from doc_ids_from_cu_seqlens: any values, 0 included, one run each
    lay = Layout("arb-ids", 0, B=1, S=200, L=200, seq_start=0, Hq=4, Hkv=4, D=64, enable_gqa=False)
    ids = np.asarray([[0] * 50 + [99] * 70 + [-1000] * 5 + [-7] * 75], dtype=np.int32)
    run_case(psb, lay, seed_base=79, ids=ids, scale=0.37)
    run_case(psb, lay, seed_base=80, ids=ids, scale=-0.2)


def test_strided_q_and_kv(psb):
    lay = random_layout(21, B=2, S=400, L=400, Hq=8, Hkv=2, D=128, max_doc=150, max_pad=20)
    q, k, v = make_qkv(lay, seed_base=5)
    ids = oracle_doc_ids(lay)
    # [B, S, H, D] storage viewed as [B, H, S, D]
    qd = q.permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3)
    kd = k.permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3)
    vd = v.permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3)
    assert not qd.is_contiguous()
    say("strided q/kv")
    out = psb.blockdiag_attn_fwd(qd, kd, vd, torch.as_tensor(ids).cuda(), 0, None, True)
    ref = oracle.blockdiag_attn(q, k, v, ids, 0, None, True)
    compare(out, ref, None, "strided")


def test_deterministic(psb):
    lay = random_layout(31, B=1, S=1500, Hq=8, Hkv=2, D=128, max_doc=600, max_pad=30)
    q, k, v = (t.cuda() for t in make_qkv(lay, seed_base=3))
    ids = torch.as_tensor(oracle_doc_ids(lay)).cuda()
    say("determinism")
    a = psb.blockdiag_attn_fwd(q, k, v, ids, 0, None, True)
    b = psb.blockdiag_attn_fwd(q, k, v, ids, 0, None, True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_gpu_doc_ids_feed_attention(psb):
    # whole path on the device: cu_seqlens -> doc ids -> attention
    lay = make_layout(1)
    q, k, v = make_qkv(lay)
    cu = torch.as_tensor(lay.cu_seqlens(0)).cuda()
    ids = psb.doc_ids_from_cu_seqlens(cu, lay.S)
    say("device ids -> attention")
    out = psb.blockdiag_attn_fwd(q.cuda(), k.cuda(), v.cuda(), ids, 0, None, True)
    ref = oracle.blockdiag_attn(q, k, v, oracle_doc_ids(lay), 0, None, True)
    compare(out, ref, None, "device-ids")


def _run_qkv(psb, lay, q, k, v, scale):
    ids = oracle_doc_ids(lay)
    out = psb.blockdiag_attn_fwd(q.cuda(), k.cuda(), v.cuda(), torch.as_tensor(ids).cuda(), lay.seq_start,
                                 scale, lay.enable_gqa)
    torch.cuda.synchronize()
    ref = oracle.blockdiag_attn(q, k, v, ids, lay.seq_start, scale, lay.enable_gqa)
    qpos = np.arange(lay.seq_start, lay.seq_start + lay.L)
    pad = torch.as_tensor(np.asarray(ids)[:, qpos] == oracle.PAD_DOC_ID)
    return compare(out, ref, pad.unsqueeze(1).expand(lay.B, lay.Hq, lay.L), lay.name)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("regime", ["wide", "growing", "far_below"])
def test_extreme_score_ranges(psb, D, regime):
    # The kernel keeps an exp2 offset per row and moves it only when a lane's P for a tile
    # sums past 2^8, starting from FLT_MAX so that a row's first keys set it.  These inputs
    # drive that logic hard; the fp64 oracle is exact for them.
    #   wide:      q and k scaled by 6 at scale 1: scores of magnitude in the hundreds, the
    #              softmax close to one-hot, most weights far below fp32 range;
    #   growing:   key j scaled by 1 + j / 40: each later tile's scores outgrow the offset,
    #              so it moves on most tiles;
    #   far_below: q . k near -500 for every pair: with an offset that started at 0 every
    #              weight would underflow.
    lay = random_layout(1300 + D, B=1, S=900, L=None, seq_start=0, Hq=4, Hkv=2, D=D, max_doc=400, max_pad=30)
    q, k, v = make_qkv(lay, seed_base=7100 + D)
    say(regime, "D", D, "S", lay.S)
    if regime == "wide":
        q = (q.float() * 6).to(torch.bfloat16)
        k = (k.float() * 6).to(torch.bfloat16)
        scale = 1.0
    elif regime == "growing":
        grow = 1.0 + torch.arange(lay.S, dtype=torch.float32) / 40.0
        k = (k.float() * grow[None, None, :, None]).to(torch.bfloat16)
        scale = 1.0
    else:
        q = torch.full_like(q, 2.0)
        k = (torch.full_like(k, -2.0).float() + 0.05 * k.float()).to(torch.bfloat16)
        scale = 1.0
    mx, mean = _run_qkv(psb, lay, q, k, v, scale)
    say(regime, "max/mean abs err", mx, mean)


@pytest.mark.parametrize("scale", [None, -0.3])
def test_many_items_d128(psb, scale):
    # a grid of several rounds of items per workgroup slot (6 x 64 row tiles x 8 head units =
    # 3072 items) with random documents and padding tails, at D = 128
    lay = random_layout(1500, B=6, S=2048, L=None, seq_start=0, Hq=32, Hkv=8, D=128, max_doc=700, max_pad=90)
    mx, mean = run_case(psb, lay, seed_base=7600, scale=scale)
    say("many items D128 scale", scale, "max/mean abs err", mx, mean)
