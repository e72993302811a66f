"""The attention calls' device status word (C ABI): given a word, each call also checks
that every non-padding id is one contiguous run of its row (inkling2 context_parallel
page, validate_document_positions: a gap never resumes a document) and sets
PSB_DATA_DOC_NOT_CONTIGUOUS for an id split across runs; a layout that keeps the rule
leaves the word 0, and a NULL word skips the check."""

import ctypes

import numpy as np
import pytest
import torch

from gpu_common import say
from workloads import make_qkv, random_layout

pytestmark = pytest.mark.gpu

NOT_CONTIGUOUS = 4


@pytest.fixture(scope="module")
def psb():
    import packed_sequence_block_amd as m
    m.load()
    return m


def _P(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _problem(split):
    lay = random_layout(77, B=2, S=256, Hq=4, Hkv=2, D=64, max_doc=90, max_pad=0)
    q, k, v = (t.cuda() for t in make_qkv(lay, seed_base=7700))
    ids = np.zeros((2, 256), dtype=np.int32)
    ids[:, :100] = 5
    ids[:, 100:180] = 6
    ids[:, 180:] = 7
    if split:
        ids[1, 200:220] = 5   # id 5 again after other documents in row 1
    return lay, q, k, v, torch.as_tensor(ids).cuda()


def _calls(psb, lay, q, k, v, ids, word):
    """Each attention entry point with the given status word; returns the statuses."""
    lib = psb.load()
    B, Hq, Hkv, S, D = 2, 4, 2, 256, 64
    L = S
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sc = float(D) ** -0.5
    out = torch.empty((B, Hq, L, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda")
    nb = psb.bwd_workspace_size(B, Hq, Hkv, L, S, D)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    res = {}
    res["fwd"] = lib.psb_blockdiag_attn_fwd(_P(q), _P(k), _P(v), _P(ids), B, Hq, Hkv, L, S, D, None, None, 0, sc, 1,
                                            _P(out), _P(ws), nb, _P(word), st)
    res["plan"] = lib.psb_blockdiag_attn_plan(_P(ids), B, Hq, Hkv, L, S, D, 0, 1, _P(ws), nb, st)
    res["planned"] = lib.psb_blockdiag_attn_fwd_planned(_P(q), _P(k), _P(v), _P(ids), B, Hq, Hkv, L, S, D, None,
                                                        None, 0, sc, 1, _P(out), _P(ws), nb, _P(word), st)
    res["lse_planned"] = lib.psb_blockdiag_attn_fwd_lse_planned(_P(q), _P(k), _P(v), _P(ids), B, Hq, Hkv, L, S, D,
                                                                None, None, 0, sc, 1, _P(out), _P(lse), _P(ws), nb,
                                                                _P(word), st)
    dout = torch.ones_like(out)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    res["bwd_planned"] = lib.psb_blockdiag_attn_bwd_planned(_P(q), _P(k), _P(v), _P(out), _P(dout), _P(lse), _P(ids),
                                                            B, Hq, Hkv, L, S, D, 0, sc, 1, _P(dq), _P(dk), _P(dv),
                                                            _P(ws), nb, _P(word), st)
    res["window_planned"] = lib.psb_blockdiag_attn_fwd_window_planned(
        _P(q), _P(k), _P(v), _P(ids), B, Hq, Hkv, L, S, D, None, None, 0, 0, S, sc, 1, _P(out), None, _P(ws), nb,
        _P(word), st)
    return res


ENTRY_POINTS = ["fwd", "planned", "lse_planned", "bwd_planned", "window_planned"]


@pytest.mark.parametrize("which", ENTRY_POINTS)
def test_split_id_sets_the_bit(psb, which):
    lay, q, k, v, ids = _problem(split=True)
    say("status word, split id", which)
    word = torch.zeros(1, dtype=torch.int32, device="cuda")
    res = _calls_one(psb, lay, q, k, v, ids, word, which)
    torch.cuda.synchronize()
    assert res == 0
    assert int(word.item()) == NOT_CONTIGUOUS, (which, int(word.item()))


def _calls_one(psb, lay, q, k, v, ids, word, which):
    # run the full sequence with NULL words except the named entry point
    lib = psb.load()
    B, Hq, Hkv, S, D = 2, 4, 2, 256, 64
    L = S
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sc = float(D) ** -0.5
    out = torch.empty((B, Hq, L, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda")
    nb = psb.bwd_workspace_size(B, Hq, Hkv, L, S, D)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    w = lambda name: _P(word) if name == which else None  # noqa: E731
    assert lib.psb_blockdiag_attn_plan(_P(ids), B, Hq, Hkv, L, S, D, 0, 1, _P(ws), nb, st) == 0
    assert lib.psb_blockdiag_attn_fwd_lse_planned(_P(q), _P(k), _P(v), _P(ids), B, Hq, Hkv, L, S, D, None, None, 0,
                                                  sc, 1, _P(out), _P(lse), _P(ws), nb, w("lse_planned"), st) == 0
    if which == "fwd":
        return lib.psb_blockdiag_attn_fwd(_P(q), _P(k), _P(v), _P(ids), B, Hq, Hkv, L, S, D, None, None, 0, sc, 1,
                                          _P(out), _P(ws), nb, w("fwd"), st)
    if which == "planned":
        return lib.psb_blockdiag_attn_fwd_planned(_P(q), _P(k), _P(v), _P(ids), B, Hq, Hkv, L, S, D, None, None, 0,
                                                  sc, 1, _P(out), _P(ws), nb, w("planned"), st)
    if which == "bwd_planned":
        dout = torch.ones_like(out)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        return lib.psb_blockdiag_attn_bwd_planned(_P(q), _P(k), _P(v), _P(out), _P(dout), _P(lse), _P(ids), B, Hq,
                                                  Hkv, L, S, D, 0, sc, 1, _P(dq), _P(dk), _P(dv), _P(ws), nb,
                                                  w("bwd_planned"), st)
    if which == "window_planned":
        return lib.psb_blockdiag_attn_fwd_window_planned(
            _P(q), _P(k), _P(v), _P(ids), B, Hq, Hkv, L, S, D, None, None, 0, 0, S, sc, 1, _P(out), None, _P(ws), nb,
            w("window_planned"), st)
    return 0


def test_contiguous_ids_leave_the_word_zero(psb):
    lay, q, k, v, ids = _problem(split=False)
    word = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("status word, contiguous ids")
    res = _calls(psb, lay, q, k, v, ids, word)
    torch.cuda.synchronize()
    assert all(s == 0 for s in res.values()), res
    assert int(word.item()) == 0


def test_binding_validate_raises_on_split_id(psb):
    lay, q, k, v, ids = _problem(split=True)
    say("binding validate=True, split id")
    with pytest.raises(ValueError, match="more than one run"):
        psb.blockdiag_attn_fwd(q, k, v, ids, 0, None, True, validate=True)
    _, _, _, _, good = _problem(split=False)
    psb.blockdiag_attn_fwd(q, k, v, good, 0, None, True, validate=True)
