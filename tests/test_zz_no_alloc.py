"""The no-allocation forward (psb_blockdiag_attn_fwd_noalloc, for callers that cannot
allocate device memory) through the C ABI: two calls in a row, the second on a smaller
problem, each equal bit for bit to psb_blockdiag_attn_fwd on the same inputs and within
the oracle's tolerance; a problem whose plan tables exceed the static buffer is refused
on the host before anything is enqueued."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from gpu_common import compare, oracle_doc_ids, say
from workloads import make_qkv, random_layout

pytestmark = pytest.mark.gpu

SCRATCH_LIMIT = -6


@pytest.fixture(scope="module")
def psb():
    import packed_sequence_block_amd as m
    m.load()
    return m


def _P(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _both(psb, lay, seed):
    lib = psb.load()
    q, k, v = make_qkv(lay, seed_base=seed)
    ids = oracle_doc_ids(lay)
    qd, kd, vd, idd = q.cuda(), k.cuda(), v.cuda(), torch.as_tensor(ids).cuda()
    B, Hq, Hkv, L, S, D = lay.B, lay.Hq, lay.Hkv, lay.L, lay.S, lay.D
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sc = float(D) ** -0.5
    gqa = 1 if lay.enable_gqa else 0
    out_na = torch.full((B, Hq, L, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    word = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("no-alloc forward", lay.name, B, Hq, Hkv, L, S, D, lay.seq_start)
    r = lib.psb_blockdiag_attn_fwd_noalloc(_P(qd), _P(kd), _P(vd), _P(idd), B, Hq, Hkv, L, S, D, None, None,
                                           lay.seq_start, sc, gqa, _P(out_na), _P(word), st)
    assert r == 0, r
    out_ref = torch.empty_like(out_na)
    nb = psb.workspace_size(B, Hq, Hkv, L, D)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    r = lib.psb_blockdiag_attn_fwd(_P(qd), _P(kd), _P(vd), _P(idd), B, Hq, Hkv, L, S, D, None, None, lay.seq_start,
                                   sc, gqa, _P(out_ref), _P(ws), nb, None, st)
    assert r == 0, r
    torch.cuda.synchronize()
    assert int(word.item()) == 0
    assert torch.equal(out_na, out_ref), f"{lay.name}: no-alloc output differs from the workspace call"
    qpos = np.arange(lay.seq_start, lay.seq_start + L)
    pad = torch.as_tensor(ids[:, qpos] == oracle.PAD_DOC_ID).unsqueeze(1).expand(B, Hq, L)
    compare(out_na, oracle.blockdiag_attn(q, k, v, ids, lay.seq_start, None, lay.enable_gqa), pad, lay.name)


def test_two_calls_second_smaller(psb):
    big = random_layout(801, B=2, S=3000, L=2000, seq_start=1000, Hq=8, Hkv=2, D=128, max_doc=900, max_pad=0)
    small = random_layout(802, B=1, S=700, Hq=4, Hkv=4, D=64, max_doc=200, max_pad=40, enable_gqa=False)
    _both(psb, big, 8010)
    _both(psb, small, 8020)


def test_oversized_plan_is_refused(psb):
    lib = psb.load()
    cap = int(lib.psb_blockdiag_attn_fwd_noalloc_max_workspace())
    assert cap == 4 << 20
    # B * L large enough that the plan tables exceed the buffer; the host check returns
    # before any pointer is used (none of these dummy addresses is ever read)
    B, Hq, Hkv, D = 64, 4, 4, 64
    L = S = 1 << 16
    while psb.workspace_size(B, Hq, Hkv, L, D) <= cap:
        B *= 2
    assert B <= 65536
    fake = ctypes.c_void_p(1 << 20)
    say("no-alloc oversized refusal")
    r = lib.psb_blockdiag_attn_fwd_noalloc(fake, fake, fake, fake, B, Hq, Hkv, L, S, D, None, None, 0, 0.125, 0,
                                           fake, None, None)
    assert r == SCRATCH_LIMIT
    assert "static buffer" in psb.status_string(r)
