"""scale = 0 and -0.0 on the GPU (cp_blockdiag_sdpa on the blockdiag_cp page takes any
float scale).  With a zero scale every allowed key gets the same weight, so each row
is the mean of v over its document prefix; the oracle computes exactly that from the
definition.  Checked for the varlen forward (with and without lse), the backward,
the key-window forward and attention under an explicit mask."""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import compare, oracle_doc_ids, say
from test_gpu_backward import LSE_TOL, check_grad
from workloads import make_layout, make_qkv, random_layout

pytestmark = pytest.mark.gpu

ZEROS = [0.0, -0.0]


@pytest.fixture(scope="module")
def psb():
    import packed_sequence_block_amd as m
    m.load()
    return m


def _layouts():
    return [make_layout(1),
            random_layout(401, B=2, S=700, L=300, seq_start=250, Hq=8, Hkv=2, D=128, max_doc=260, max_pad=0),
            random_layout(402, B=1, S=1000, Hq=4, Hkv=4, D=64, max_doc=400, max_pad=90, enable_gqa=False)]


def _pad_rows(lay, ids):
    qpos = np.arange(lay.seq_start, lay.seq_start + lay.L)
    pad = torch.as_tensor(np.asarray(ids)[:, qpos] == oracle.PAD_DOC_ID)
    return pad.unsqueeze(1).expand(lay.B, lay.Hq, lay.L)


@pytest.mark.parametrize("scale", ZEROS, ids=["plus0", "minus0"])
@pytest.mark.parametrize("li", [0, 1, 2])
def test_forward_scale_zero(psb, scale, li):
    lay = _layouts()[li]
    q, k, v = make_qkv(lay, seed_base=9100 + li)
    ids = oracle_doc_ids(lay)
    say("scale zero forward", lay.name, scale)
    idd = torch.as_tensor(ids).cuda()
    out = psb.blockdiag_attn_fwd(q.cuda(), k.cuda(), v.cuda(), idd, lay.seq_start, scale, lay.enable_gqa)
    torch.cuda.synchronize()
    ref = oracle.blockdiag_attn(q, k, v, ids, lay.seq_start, scale, lay.enable_gqa)
    compare(out, ref, _pad_rows(lay, ids), f"{lay.name} scale {scale}")


@pytest.mark.parametrize("scale", ZEROS, ids=["plus0", "minus0"])
def test_training_path_scale_zero(psb, scale):
    lay = _layouts()[1]
    q, k, v = make_qkv(lay, seed_base=9200)
    ids = oracle_doc_ids(lay)
    qd, kd, vd, idd = q.cuda(), k.cuda(), v.cuda(), torch.as_tensor(ids).cuda()
    say("scale zero lse + backward", scale)
    out, lse, ws = psb.blockdiag_attn_fwd_lse(qd, kd, vd, idd, lay.seq_start, scale, True)
    lse_ref = oracle.blockdiag_attn_lse(q, k, ids, lay.seq_start, scale, True)
    lg = lse.cpu().double()
    fin = torch.isfinite(lse_ref)
    assert torch.equal(torch.isfinite(lg), fin)
    assert (lg[fin] - lse_ref[fin]).abs().max().item() <= LSE_TOL
    compare(out, oracle.blockdiag_attn(q, k, v, ids, lay.seq_start, scale, True), _pad_rows(lay, ids), "lse fwd")
    g = torch.Generator().manual_seed(9201)
    dout = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    dq, dk, dv = psb.blockdiag_attn_bwd(qd, kd, vd, out, dout.cuda(), lse, idd, ws, lay.seq_start, scale, True)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.blockdiag_attn_bwd(q, k, v, dout, ids, lay.seq_start, scale, True)
    # a zero scale multiplies dq and dk: both are exactly zero
    assert torch.count_nonzero(dq).item() == 0 and torch.count_nonzero(dk).item() == 0
    assert float(rq.abs().max()) == 0.0 and float(rk.abs().max()) == 0.0
    check_grad(dv, rv, f"dv scale {scale}")


@pytest.mark.parametrize("scale", ZEROS, ids=["plus0", "minus0"])
def test_window_forward_scale_zero(psb, scale):
    lay = _layouts()[1]
    q, k, v = make_qkv(lay, seed_base=9300)
    ids = oracle_doc_ids(lay)
    idd = torch.as_tensor(ids).cuda()
    w = int(psb.shard_kv_window_start(idd, lay.seq_start, lay.L).min().item())
    kv_len = lay.seq_start + lay.L - w
    say("scale zero window forward", scale, w, kv_len)
    kw = k[:, :, w:w + kv_len].contiguous().cuda()
    vw = v[:, :, w:w + kv_len].contiguous().cuda()
    out = psb.blockdiag_attn_fwd_window(q.cuda(), kw, vw, idd, lay.seq_start, w, scale, True, validate=True)
    torch.cuda.synchronize()
    compare(out, oracle.blockdiag_attn(q, k, v, ids, lay.seq_start, scale, True), _pad_rows(lay, ids), "window")


@pytest.mark.parametrize("scale", ZEROS, ids=["plus0", "minus0"])
def test_masked_attention_scale_zero(psb, scale):
    g = torch.Generator().manual_seed(9400)
    B, Hq, Hkv, L, S, D = 2, 4, 2, 150, 260, 128
    q = torch.randn((B, Hq, L, D), generator=g).to(torch.bfloat16)
    k = torch.randn((B, Hkv, S, D), generator=g).to(torch.bfloat16)
    v = torch.randn((B, Hkv, S, D), generator=g).to(torch.bfloat16)
    mask = torch.rand((B, L, S), generator=g) < 0.3
    mask[:, ::9] = False   # rows without a key: exactly 0
    say("scale zero masked attention", scale)
    out, lse = psb.masked_attn_fwd(q.cuda(), k.cuda(), v.cuda(), mask.cuda(), scale, True, with_lse=True)
    torch.cuda.synchronize()
    ref = oracle.masked_attn(q, k, v, mask, scale, True)
    empty = ~mask.any(dim=2)
    compare(out, ref, empty.unsqueeze(1).expand(B, Hq, L), f"masked scale {scale}")
    # lse = log(number of allowed keys) at scale 0
    cnt = mask.sum(dim=2).double().unsqueeze(1).expand(B, Hq, L)
    lg = lse.cpu().double()
    has = cnt > 0
    assert torch.all(torch.isneginf(lg[~has]))
    assert (lg[has] - torch.log(cnt[has])).abs().max().item() <= LSE_TOL
