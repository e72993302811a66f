"""The C-ABI library loads without a GPU, exports every declared symbol, and
rejects bad arguments on the host (these calls return before any launch and
never dereference the fake, aligned pointers they are given)."""

import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "psb.h")
LIB = os.path.join(ROOT, "packed_sequence_block_amd", "libpsb.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__.build()
    from packed_sequence_block_amd import _lib
    return _lib.load()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(psb_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_three_calls():
    syms = declared_symbols()
    for name in ("psb_doc_ids_from_cu_seqlens", "psb_segment_cu_seqlens", "psb_blockdiag_attn_fwd"):
        assert name in syms


def test_every_declared_symbol_is_exported(lib):
    missing = [s for s in declared_symbols() if not hasattr(lib, s)]
    assert not missing, missing


def test_binding_signatures_cover_header(lib):
    from packed_sequence_block_amd import _lib
    assert sorted(_lib.SIGNATURES) == declared_symbols()


def test_status_strings(lib):
    from packed_sequence_block_amd import _lib
    for code in (0, -1, -2, -3, -4, -5):
        assert _lib.status_string(code)
    assert _lib.status_string(0) == "ok"
    assert "unknown" in _lib.status_string(17)
    assert lib.psb_version() >= 100


FAKE = ctypes.c_void_p(0x100000)   # aligned, never dereferenced by the calls below
NULL = None


def attn(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, doc=FAKE, B=1, Hq=4, Hkv=2, L=64, S=64, D=128, qs=None, kvs=None,
             seq_start=0, scale=0.125, gqa=1, out=FAKE, ws=FAKE, ws_bytes=1 << 20)
    a.update(over)
    return lib.psb_blockdiag_attn_fwd(a["q"], a["k"], a["v"], a["doc"], a["B"], a["Hq"], a["Hkv"], a["L"],
                                      a["S"], a["D"], a["qs"], a["kvs"], a["seq_start"], a["scale"],
                                      a["gqa"], a["out"], a["ws"], a["ws_bytes"], None, None)


@pytest.mark.parametrize("over,code", [
    (dict(D=96), -3),
    (dict(D=32), -3),
    (dict(Hq=6, Hkv=4), -2),
    (dict(gqa=0), -2),
    (dict(seq_start=1), -2),
    (dict(L=65), -2),
    (dict(Hkv=0), -2),
    (dict(B=-1), -1),
    (dict(seq_start=-1), -1),
    (dict(scale=float("nan")), -1),
    (dict(scale=float("inf")), -1),
    (dict(q=NULL), -1),
    (dict(doc=NULL), -1),
    (dict(ws=NULL), -1),
    (dict(out=ctypes.c_void_p(0x100002)), -1),
    (dict(ws_bytes=16), -4),
    (dict(qs=(ctypes.c_int64 * 3)(64 * 128 * 4, 64 * 128, 100)), -2),
    (dict(kvs=(ctypes.c_int64 * 3)(64 * 128 * 2, 64 * 128, 64)), -2),
])
def test_attention_argument_errors(lib, over, code):
    assert attn(lib, **over) == code


@pytest.mark.parametrize("over", [dict(B=0), dict(L=0, S=0), dict(Hq=0, Hkv=1)])
def test_empty_attention_is_ok_without_launch(lib, over):
    assert attn(lib, q=NULL, k=NULL, v=NULL, doc=NULL, out=NULL, ws=NULL, **over) == 0


def test_workspace_size_is_positive(lib):
    assert lib.psb_blockdiag_attn_fwd_workspace_size(1, 32, 8, 8192, 128) >= 4 * (2 * 256 + 3 * 256)
    assert lib.psb_blockdiag_attn_fwd_workspace_size(0, 0, 0, 0, 128) > 0


def test_boundary_argument_errors(lib):
    f = lib.psb_doc_ids_from_cu_seqlens
    assert f(NULL, 3, 10, FAKE, NULL, NULL) == -1
    assert f(FAKE, -1, 10, FAKE, NULL, NULL) == -1
    assert f(FAKE, 3, -5, FAKE, NULL, NULL) == -1
    assert f(FAKE, 3, 10, NULL, NULL, NULL) == -1
    g = lib.psb_segment_cu_seqlens
    assert g(FAKE, 100, FAKE, 100, FAKE, NULL) == -4   # capacity must be >= S + 1
    assert g(FAKE, -1, FAKE, 100, FAKE, NULL) == -1
    assert g(FAKE, 10, NULL, 11, FAKE, NULL) == -1
    assert g(FAKE, 10, FAKE, 11, NULL, NULL) == -1
    h = lib.psb_validate_doc_ids
    assert h(FAKE, 1, 10, 10, NULL, NULL) == -1       # status word is required
    assert h(FAKE, 1, 10, 5, FAKE, NULL) == -2        # row stride shorter than a row
    assert h(NULL, 0, 10, 10, FAKE, NULL) == 0        # empty: nothing to check
