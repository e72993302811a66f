"""Large and extreme layouts beyond the named workloads: a 131072-token row that is one
document (the longest key ranges: 2048 tiles for the last rows), the same row cut into
4096 documents of 32 tokens (every tile on a document boundary), and a row that is
padding except for one token.  Checked on sampled rows against the oracle, row by row."""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import compare, say

pytestmark = pytest.mark.gpu

S = 131072


@pytest.fixture(scope="module")
def psb():
    import packed_sequence_block_amd as m
    m.load()
    return m


@pytest.fixture(scope="module")
def qkv():
    g = torch.Generator().manual_seed(4242)
    q = torch.randn((1, 2, S, 64), generator=g).to(torch.bfloat16)
    k = torch.randn((1, 1, S, 64), generator=g).to(torch.bfloat16)
    v = torch.randn((1, 1, S, 64), generator=g).to(torch.bfloat16)
    return q, k, v


def check_rows(psb, q, k, v, ids, rows, what):
    say(what)
    out = psb.blockdiag_attn_fwd(q.cuda(), k.cuda(), v.cuda(), torch.as_tensor(ids).cuda(), 0, None, True)
    torch.cuda.synchronize()
    ref = oracle.blockdiag_attn_rows(q, k, v, ids, 0, None, True, 0, rows)
    got = out[0, :, rows].permute(1, 0, 2).cpu()
    pad = torch.as_tensor(ids[0, np.asarray(rows)] == oracle.PAD_DOC_ID)
    compare(got, ref, pad, what)


def test_one_document_of_131072(psb, qkv):
    ids = np.ones((1, S), dtype=np.int32)
    rows = [0, 1, 63, 64, 65535, 65536, S - 65, S - 2, S - 1]
    check_rows(psb, *qkv, ids, rows, "one document of 131072 tokens")


def test_4096_documents_of_32(psb, qkv):
    ids = (np.arange(S, dtype=np.int32) // 32 + 1).reshape(1, S)
    rows = [0, 31, 32, 33, 4095, 4096, S // 2 + 7, S - 33, S - 32, S - 1]
    check_rows(psb, *qkv, ids, rows, "4096 documents of 32 tokens")


def test_single_token_document_in_padding(psb, qkv):
    ids = np.full((1, S), oracle.PAD_DOC_ID, dtype=np.int32)
    ids[0, 70000] = 5
    rows = [0, 69999, 70000, 70001, S - 1]
    check_rows(psb, *qkv, ids, rows, "one token in a padding row")
