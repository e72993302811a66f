"""Dense-mask path on the GPU: the materialised per-document mask (bit-exact against
the oracle's) and attention under explicit masks (against the oracle's masked
attention, at the forward's tolerances; rows without a key exactly 0)."""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import compare, oracle_doc_ids, say
from workloads import make_layout, make_qkv, random_layout

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def psb():
    import packed_sequence_block_amd as m
    m.load()
    return m


@pytest.mark.parametrize("seed,S,s0,L", [(1, 100, 0, 100), (2, 257, 40, 150), (3, 1000, 999, 1), (4, 64, 10, 0)])
def test_dense_mask_bit_exact(psb, seed, S, s0, L):
    lay = random_layout(1100 + seed, B=2, S=S, L=L, seq_start=s0, max_doc=max(1, S // 4), max_pad=S // 5)
    ids = oracle_doc_ids(lay)
    say("dense mask", seed, S, s0, L)
    got = psb.blockdiag_dense_mask(torch.as_tensor(ids).cuda(), s0, L)
    torch.cuda.synchronize()
    assert got.shape == (2, L, S)
    assert torch.equal(got.cpu(), oracle.dense_mask(ids, s0, L))
    if L:
        assert not got._base[:, :, S:].any()  # row padding written as 0


def _rand_mask(seed, B, L, S, p):
    g = torch.Generator().manual_seed(seed)
    m = torch.rand((B, L, S), generator=g) < p
    m[:, ::7] = False  # rows without any key
    return m


def _qkv(seed, B, Hq, Hkv, L, S, D):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn((B, Hq, L, D), generator=g).to(torch.bfloat16),
            torch.randn((B, Hkv, S, D), generator=g).to(torch.bfloat16),
            torch.randn((B, Hkv, S, D), generator=g).to(torch.bfloat16))


MASKED = [
    # (seed, B, Hq, Hkv, L, S, D, density, mask form)
    (1, 1, 2, 2, 64, 64, 64, 0.5, "full"),
    (2, 2, 8, 2, 100, 300, 128, 0.1, "full"),
    (3, 1, 4, 1, 333, 37, 64, 0.9, "full"),      # L > S, S not a multiple of 4 (copied)
    (4, 3, 4, 4, 70, 130, 128, 0.5, "shared"),   # one mask for the batch
    (5, 2, 4, 2, 65, 200, 64, 0.3, "heads"),     # [B, 1, L, S]
    (6, 1, 16, 8, 256, 1024, 128, 0.02, "2d"),   # [L, S], sparse
]


@pytest.mark.parametrize("case", MASKED, ids=lambda c: f"seed{c[0]}")
def test_masked_attention_random(psb, case):
    seed, B, Hq, Hkv, L, S, D, dens, form = case
    q, k, v = _qkv(1200 + seed, B, Hq, Hkv, L, S, D)
    m = _rand_mask(1300 + seed, 1 if form in ("shared", "2d") else B, L, S, dens)
    mk = {"full": m, "shared": m, "heads": m[:, None], "2d": m[0]}[form]
    say("masked attn", seed, B, Hq, Hkv, L, S, D, dens, form)
    out = psb.masked_attn_fwd(q.cuda(), k.cuda(), v.cuda(), mk.cuda(), None, Hq != Hkv)
    torch.cuda.synchronize()
    ref = oracle.masked_attn(q, k, v, m, None, Hq != Hkv)
    empty = ~m.any(dim=2)                                    # [B or 1, L]
    compare(out, ref, empty.unsqueeze(1).expand(B, Hq, L), f"masked-{seed}")


@pytest.mark.parametrize("seed", [1, 2])
def test_dense_path_equals_block_diagonal(psb, seed):
    lay = random_layout(1400 + seed, B=2, S=700, L=500, seq_start=150, Hq=8, Hkv=2, D=128, max_doc=200,
                        max_pad=40)
    q, k, v = make_qkv(lay, seed_base=14000 + seed)
    ids = oracle_doc_ids(lay)
    say("dense path", seed)
    idd = torch.as_tensor(ids).cuda()
    mask = psb.blockdiag_dense_mask(idd, 150, 500)
    out, lse = psb.masked_attn_fwd(q.cuda(), k.cuda(), v.cuda(), mask, None, True, with_lse=True)
    torch.cuda.synchronize()
    ref = oracle.blockdiag_attn(q, k, v, ids, 150, None, True)
    pad = torch.as_tensor(ids[:, 150:650] == oracle.PAD_DOC_ID).unsqueeze(1).expand(2, 8, 500)
    compare(out, ref, pad, f"dense-{seed}")
    lse_ref = oracle.blockdiag_attn_lse(q, k, ids, 150, None, True)
    lg = lse.cpu().double()
    fin = torch.isfinite(lse_ref)
    assert torch.equal(torch.isfinite(lg), fin)
    assert (lg[fin] - lse_ref[fin]).abs().max().item() <= 5e-3


def test_dense_path_full_size_packed_row(psb):
    # the packed-row workload at full size through the dense path: equal to the varlen
    # kernel within the forward tolerance, and to the oracle on sampled rows
    lay = make_layout(2)
    q, k, v = make_qkv(lay)
    ids = oracle_doc_ids(lay)
    say("dense path full size", lay.name)
    qd, kd, vd, idd = q.cuda(), k.cuda(), v.cuda(), torch.as_tensor(ids).cuda()
    mask = psb.blockdiag_dense_mask(idd, 0, lay.L)
    out = psb.masked_attn_fwd(qd, kd, vd, mask, None, lay.enable_gqa)
    var = psb.blockdiag_attn_fwd(qd, kd, vd, idd, 0, None, lay.enable_gqa)
    torch.cuda.synchronize()
    d = (out.float() - var.float()).abs()
    assert d.max().item() <= 2e-2 and d.mean().item() <= 2e-3
    rows = [0, 1, 1000, 4095, 8191]
    ref = oracle.blockdiag_attn_rows(q, k, v, ids, 0, None, lay.enable_gqa, 0, rows)
    compare(out[0][:, rows].permute(1, 0, 2), ref, None, "dense full-size rows")


def test_masked_attention_argument_errors(psb):
    q = torch.zeros((1, 2, 8, 64), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 2, 16, 64), dtype=torch.bfloat16, device="cuda")
    say("masked attn errors")
    with pytest.raises(ValueError):
        psb.masked_attn_fwd(q, kv, kv, torch.ones((1, 8, 15), dtype=torch.bool, device="cuda"))
    with pytest.raises(ValueError):
        psb.masked_attn_fwd(q, kv, kv, torch.ones((1, 2, 8, 16), dtype=torch.bool, device="cuda"))
