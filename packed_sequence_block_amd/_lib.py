"""ctypes binding of libpsb.so (argument marshalling only).

Every computation runs in the library's HIP kernels; torch provides device
memory and the current stream.  Loading fails loudly when the library has not
been built: there is no other implementation behind these functions.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpsb.so")

PSB_OK = 0
PSB_ERR_INVALID_ARG = -1
PSB_ERR_SHAPE = -2
PSB_ERR_UNSUPPORTED = -3
PSB_ERR_CAPACITY = -4
PSB_ERR_HIP = -5
PSB_ERR_SCRATCH_LIMIT = -6
PAD_DOC_ID = -1000
DATA_CU_NOT_MONOTONE = 1
DATA_CU_OUT_OF_RANGE = 2
DATA_DOC_NOT_CONTIGUOUS = 4
DATA_LENS_EXCEED_SEQ = 8
DATA_BAD_POSITIONS = 16
DATA_BAD_LENGTHS = 32
DATA_KV_WINDOW = 64

_c_i64 = ctypes.c_int64
_c_i32 = ctypes.c_int32
_vp = ctypes.c_void_p

# name -> (restype, argtypes); mirrors include/psb.h
SIGNATURES = {
    "psb_status_string": (ctypes.c_char_p, [_c_i32]),
    "psb_version": (_c_i32, []),
    "psb_doc_ids_from_cu_seqlens": (_c_i32, [_vp, _c_i64, _c_i64, _vp, _vp, _vp]),
    "psb_segment_cu_seqlens": (_c_i32, [_vp, _c_i64, _vp, _c_i64, _vp, _vp]),
    "psb_validate_doc_ids": (_c_i32, [_vp, _c_i64, _c_i64, _c_i64, _vp, _vp]),
    "psb_doc_ids_from_seq_lens": (_c_i32, [_vp, _c_i64, _c_i64, _c_i64, _c_i32, _vp, _vp, _vp]),
    "psb_validate_document_positions": (_c_i32, [_vp, _vp, _c_i64, _c_i64, _vp, _vp]),
    "psb_unpack_row_layout": (_c_i32, [_vp, _vp, _c_i64, _c_i64, _c_i64, _vp, _vp, _vp, _vp]),
    "psb_shard_kv_window_start": (_c_i32, [_vp, _c_i64, _c_i64, _c_i64, _c_i64, _vp, _vp]),
    "psb_blockdiag_prepare": (_c_i32, [_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                       _c_i32, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp, _vp]),
    "psb_blockdiag_dense_mask": (_c_i32, [_vp, _c_i64, _c_i64, _c_i64, _c_i64, _vp, _c_i64, _vp]),
    "psb_masked_attn_fwd": (_c_i32, [_vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                     _c_i64, _vp, _vp, ctypes.c_float, _c_i32, _vp, _vp, _vp]),
    "psb_blockdiag_attn_fwd_window_planned": (_c_i32, [_vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                                       _c_i64, _vp, _vp, _c_i64, _c_i64, _c_i64, ctypes.c_float,
                                                       _c_i32, _vp, _vp, _vp, ctypes.c_size_t, _vp, _vp]),
    "psb_blockdiag_attn_bwd_window_planned": (_c_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64,
                                                       _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                                       ctypes.c_float, _c_i32, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                                       _vp, _vp]),
    "psb_blockdiag_attn_fwd_workspace_size": (ctypes.c_size_t, [_c_i64, _c_i64, _c_i64, _c_i64, _c_i64]),
    "psb_blockdiag_attn_fwd": (_c_i32, [_vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                        _vp, _vp, _c_i64, ctypes.c_float, _c_i32, _vp, _vp, ctypes.c_size_t,
                                        _vp, _vp]),
    "psb_blockdiag_attn_fwd_noalloc_max_workspace": (ctypes.c_size_t, []),
    "psb_blockdiag_attn_fwd_noalloc": (_c_i32, [_vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                                _vp, _vp, _c_i64, ctypes.c_float, _c_i32, _vp, _vp, _vp]),
    "psb_blockdiag_attn_plan": (_c_i32, [_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i32,
                                         _vp, ctypes.c_size_t, _vp]),
    "psb_blockdiag_attn_fwd_planned": (_c_i32, [_vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                                _c_i64, _vp, _vp, _c_i64, ctypes.c_float, _c_i32, _vp, _vp,
                                                ctypes.c_size_t, _vp, _vp]),
    "psb_blockdiag_attn_fwd_lse_planned": (_c_i32, [_vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                                    _c_i64, _vp, _vp, _c_i64, ctypes.c_float, _c_i32, _vp, _vp,
                                                    _vp, ctypes.c_size_t, _vp, _vp]),
    "psb_blockdiag_attn_bwd_workspace_size": (ctypes.c_size_t, [_c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                                                _c_i64]),
    "psb_blockdiag_attn_bwd_planned": (_c_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _c_i64,
                                                _c_i64, _c_i64, _c_i64, ctypes.c_float, _c_i32, _vp, _vp, _vp,
                                                _vp, ctypes.c_size_t, _vp, _vp]),
}

_lib = None


class PsbError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def load() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m packed_sequence_block_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().psb_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != PSB_OK:
        raise PsbError(status, where)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need_gpu(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("psb runs on the GPU only: pass device tensors")


def doc_ids_from_cu_seqlens(cu_seqlens: torch.Tensor, seq_len: int,
                            validate: bool = False) -> torch.Tensor:
    """Document ids ``[1, seq_len]`` (int32) from boundaries ``[N + 1]``.

    Document i gets id i + 1; uncovered positions get -1000.  With
    ``validate=True`` the call synchronizes and raises ``ValueError`` when the
    boundaries are not non-decreasing inside ``[0, seq_len]``.
    """
    _need_gpu(cu_seqlens)
    cu = cu_seqlens.reshape(-1)
    if cu.dtype != torch.int32:
        cu = cu.to(torch.int32)
    cu = cu.contiguous()
    if cu.numel() < 1:
        raise ValueError("cu_seqlens needs at least one entry")
    out = torch.empty((1, int(seq_len)), dtype=torch.int32, device=cu.device)
    status = torch.zeros(1, dtype=torch.int32, device=cu.device) if validate else None
    _check(load().psb_doc_ids_from_cu_seqlens(_ptr(cu), cu.numel() - 1, int(seq_len), _ptr(out),
                                              _ptr(status), _vp(_stream(cu))),
           "doc_ids_from_cu_seqlens")
    if validate and int(status.item()) != 0:
        raise ValueError(f"cu_seqlens invalid (status bits {int(status.item())})")
    return out


def segment_cu_seqlens(doc_ids_row: torch.Tensor) -> torch.Tensor:
    """Run boundaries ``[R + 1]`` (int32) of one row; synchronizes once to size the result."""
    _need_gpu(doc_ids_row)
    ids = doc_ids_row.reshape(-1)
    if ids.dtype != torch.int32:
        ids = ids.to(torch.int32)
    ids = ids.contiguous()
    S = ids.numel()
    cu = torch.empty(S + 1, dtype=torch.int32, device=ids.device)
    n = torch.empty(1, dtype=torch.int32, device=ids.device)
    _check(load().psb_segment_cu_seqlens(_ptr(ids), S, _ptr(cu), S + 1, _ptr(n), _vp(_stream(ids))),
           "segment_cu_seqlens")
    return cu[: int(n.item()) + 1]


def validate_doc_ids(doc_ids: torch.Tensor) -> None:
    """Raises ``ValueError`` unless every non-padding id is one contiguous run per row."""
    _need_gpu(doc_ids)
    ids = doc_ids.reshape(doc_ids.shape[0] if doc_ids.dim() > 1 else 1, -1).to(torch.int32).contiguous()
    status = torch.zeros(1, dtype=torch.int32, device=ids.device)
    _check(load().psb_validate_doc_ids(_ptr(ids), ids.shape[0], ids.shape[1], ids.shape[1], _ptr(status),
                                       _vp(_stream(ids))), "validate_doc_ids")
    if int(status.item()) & DATA_DOC_NOT_CONTIGUOUS:
        raise ValueError("a non-padding document id occurs in more than one run of a row")


def workspace_size(B: int, Hq: int, Hkv: int, L: int, D: int) -> int:
    return int(load().psb_blockdiag_attn_fwd_workspace_size(B, Hq, Hkv, L, D))


def blockdiag_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, doc_ids: torch.Tensor,
                       seq_start: int = 0, scale: float | None = None, enable_gqa: bool = False,
                       out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                       validate: bool = False) -> torch.Tensor:
    """Block-diagonal causal attention forward: ``out [B, Hq, L, D]`` (bf16).

    ``q [B, Hq, L, D]`` and ``k, v [B, Hkv, S, D]`` are bf16 with the last dim
    contiguous; ``doc_ids [B, S]`` int32 (global positions, -1000 = padding).
    ``scale=None`` means ``D ** -0.5``.  ``workspace`` (uint8, at least
    :func:`workspace_size` bytes) may be passed to avoid an allocation per call.
    ``validate=True`` has the call check that every non-padding id is one run of its
    row (through the call's status word), synchronizes and raises ``ValueError`` if not.
    """
    _need_gpu(q, k, v, doc_ids)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or t.dim() != 4:
            raise ValueError(f"{name} must be a 4-D bfloat16 tensor")
        if t.stride(3) != 1:
            raise ValueError(f"{name} must have a contiguous last dimension")
    if k.stride() != v.stride() or k.shape != v.shape:
        raise ValueError("k and v must share shape and strides")
    B, Hq, L, D = q.shape
    S = k.shape[2]
    Hkv = k.shape[1]
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError("k/v shape does not match q")
    ids = doc_ids.reshape(B, -1) if doc_ids.dim() != 2 else doc_ids
    if ids.dtype != torch.int32:
        ids = ids.to(torch.int32)
    ids = ids.contiguous()
    if tuple(ids.shape) != (B, S):
        raise ValueError(f"doc_ids must be [B, S] = [{B}, {S}]")
    if out is None:
        out = torch.empty((B, Hq, L, D), dtype=torch.bfloat16, device=q.device)
    elif out.shape != (B, Hq, L, D) or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 [B, Hq, L, D] tensor")
    need = workspace_size(B, Hq, Hkv, L, D)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    sc = float(D) ** -0.5 if scale is None else float(scale)
    qs = (ctypes.c_int64 * 3)(*q.stride()[:3])
    kvs = (ctypes.c_int64 * 3)(*k.stride()[:3])
    word = torch.zeros(1, dtype=torch.int32, device=q.device) if validate else None
    status = load().psb_blockdiag_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(ids), B, Hq, Hkv, L, S, D, qs, kvs, int(seq_start), sc,
        1 if enable_gqa else 0, _ptr(out), _ptr(workspace), need, _ptr(word), _vp(_stream(q)))
    _check(status, "blockdiag_attn_fwd")
    if validate and int(word.item()) & DATA_DOC_NOT_CONTIGUOUS:
        raise ValueError("a non-padding document id occurs in more than one run of a row")
    return out


def _check_qkv(q, k, v, contiguous=False):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or t.dim() != 4:
            raise ValueError(f"{name} must be a 4-D bfloat16 tensor")
        if contiguous and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3]:
        raise ValueError("k/v shape does not match q")


def _ids(doc_ids, B, S):
    ids = doc_ids.reshape(B, -1) if doc_ids.dim() != 2 else doc_ids
    ids = (ids if ids.dtype == torch.int32 else ids.to(torch.int32)).contiguous()
    if tuple(ids.shape) != (B, S):
        raise ValueError(f"doc_ids must be [B, S] = [{B}, {S}]")
    return ids


def bwd_workspace_size(B: int, Hq: int, Hkv: int, L: int, S: int, D: int) -> int:
    return int(load().psb_blockdiag_attn_bwd_workspace_size(B, Hq, Hkv, L, S, D))


def blockdiag_attn_fwd_lse(q, k, v, doc_ids, seq_start: int = 0, scale: float | None = None,
                           enable_gqa: bool = False, workspace: torch.Tensor | None = None):
    """Training forward: ``(out [B,Hq,L,D] bf16, lse [B,Hq,L] fp32, workspace)``.

    All tensors contiguous.  The returned workspace holds the tile plan and is
    what :func:`blockdiag_attn_bwd` needs for the same arguments.
    """
    _need_gpu(q, k, v, doc_ids)
    _check_qkv(q, k, v, contiguous=True)
    B, Hq, L, D = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    ids = _ids(doc_ids, B, S)
    need = bwd_workspace_size(B, Hq, Hkv, L, S, D)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    out = torch.empty((B, Hq, L, D), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device)
    sc = float(D) ** -0.5 if scale is None else float(scale)
    gqa = 1 if enable_gqa else 0
    st = _vp(_stream(q))
    lib = load()
    _check(lib.psb_blockdiag_attn_plan(_ptr(ids), B, Hq, Hkv, L, S, D, int(seq_start), gqa, _ptr(workspace),
                                       need, st), "blockdiag_attn_plan")
    _check(lib.psb_blockdiag_attn_fwd_lse_planned(_ptr(q), _ptr(k), _ptr(v), _ptr(ids), B, Hq, Hkv, L, S, D,
                                                  None, None, int(seq_start), sc, gqa, _ptr(out), _ptr(lse),
                                                  _ptr(workspace), need, None, st),
           "blockdiag_attn_fwd_lse_planned")
    return out, lse, workspace


def blockdiag_attn_bwd(q, k, v, out, dout, lse, doc_ids, workspace, seq_start: int = 0,
                       scale: float | None = None, enable_gqa: bool = False):
    """Gradients ``(dq, dk, dv)`` (bf16) of ``sum(out * dout)``; ``workspace`` from
    :func:`blockdiag_attn_fwd_lse` with the same arguments."""
    _need_gpu(q, k, v, out, dout, lse, doc_ids, workspace)
    _check_qkv(q, k, v, contiguous=True)
    B, Hq, L, D = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    for name, t in (("out", out), ("dout", dout)):
        if t.shape != q.shape or t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 tensor shaped like q")
    if lse.shape != (B, Hq, L) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, Hq, L] tensor")
    ids = _ids(doc_ids, B, S)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    sc = float(D) ** -0.5 if scale is None else float(scale)
    nbytes = workspace.numel() * workspace.element_size()
    _check(load().psb_blockdiag_attn_bwd_planned(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(ids), B, Hq, Hkv, L, S, D,
        int(seq_start), sc, 1 if enable_gqa else 0, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), nbytes,
        None, _vp(_stream(q))), "blockdiag_attn_bwd_planned")
    return dq, dk, dv


def doc_ids_from_seq_lens(seq_lens: torch.Tensor, seq_len: int, padding_value: int = PAD_DOC_ID,
                          validate: bool = False) -> torch.Tensor:
    """Document ids ``[batch, seq_len]`` (int32) from lengths ``[batch, documents]``.

    In each row the lengths up to the first negative entry are documents; the j-th
    covers the next ``seq_lens[b, j]`` positions with id j + 1, the rest of the row
    gets ``padding_value``.  ``validate=True`` synchronizes and raises
    ``ValueError`` when a row's lengths add up past ``seq_len``.
    """
    _need_gpu(seq_lens)
    lens = seq_lens if seq_lens.dim() == 2 else seq_lens.reshape(1, -1)
    lens = (lens if lens.dtype == torch.int32 else lens.to(torch.int32)).contiguous()
    B, n = lens.shape
    out = torch.empty((B, int(seq_len)), dtype=torch.int32, device=lens.device)
    status = torch.zeros(1, dtype=torch.int32, device=lens.device) if validate else None
    _check(load().psb_doc_ids_from_seq_lens(_ptr(lens), B, n, int(seq_len), int(padding_value), _ptr(out),
                                            _ptr(status), _vp(_stream(lens))), "doc_ids_from_seq_lens")
    if validate and int(status.item()) != 0:
        raise ValueError(f"document lengths exceed seq_len (status bits {int(status.item())})")
    return out


def unpack_row_layout(seq_lens: torch.Tensor, seq_lens_padded: torch.Tensor, seq_len: int,
                      validate: bool = False):
    """``(padding_mask [B, seq_len] bool, position_ids [B, seq_len] int32)`` from the
    packer's real / padded length tables ``[batch, documents]`` (-1000-padded).

    Document j of a row takes the next ``seq_lens_padded[b, j]`` positions; its first
    ``seq_lens[b, j]`` are real tokens at positions 0, 1, ...; every other position is
    padding (mask True, position 0).  ``validate=True`` synchronizes and raises
    ``ValueError`` for a real length outside ``[0, padded]`` or padded lengths that add
    up past ``seq_len``.
    """
    _need_gpu(seq_lens, seq_lens_padded)
    if seq_lens.shape != seq_lens_padded.shape:
        raise ValueError("seq_lens and seq_lens_padded must have one shape")
    tabs = []
    for t in (seq_lens, seq_lens_padded):
        t = t if t.dim() == 2 else t.reshape(1, -1)
        tabs.append((t if t.dtype == torch.int32 else t.to(torch.int32)).contiguous())
    B, n = tabs[0].shape
    dev = tabs[0].device
    mask = torch.empty((B, int(seq_len)), dtype=torch.bool, device=dev)
    pos = torch.empty((B, int(seq_len)), dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev) if validate else None
    _check(load().psb_unpack_row_layout(_ptr(tabs[0]), _ptr(tabs[1]), B, n, int(seq_len), _ptr(mask), _ptr(pos),
                                        _ptr(status), _vp(_stream(tabs[0]))), "unpack_row_layout")
    if validate and int(status.item()) != 0:
        raise ValueError(f"bad length tables (status bits {int(status.item())})")
    return mask, pos


def unpack_row_layout_batch(batch: dict, validate: bool = False) -> None:
    """In place on a batch mapping: replaces ``seq_lens`` / ``seq_lens_padded`` with a
    boolean ``padding_mask`` and ``position_ids`` of the shape of ``input_ids``; token
    ids and labels are left as they are."""
    S = batch["input_ids"].shape[-1]
    mask, pos = unpack_row_layout(batch.pop("seq_lens"), batch.pop("seq_lens_padded"), S, validate)
    batch["padding_mask"] = mask
    batch["position_ids"] = pos


def validate_document_positions(keep: torch.Tensor, positions: torch.Tensor) -> None:
    """Raises ``ValueError`` unless every row's logical positions follow the document
    rule (synchronizes once)."""
    _need_gpu(keep, positions)
    if keep.shape != positions.shape or keep.dim() != 2:
        raise ValueError("keep and positions must both be [batch, sequence]")
    k = keep.to(torch.uint8).contiguous()
    p = (positions if positions.dtype == torch.int32 else positions.to(torch.int32)).contiguous()
    status = torch.zeros(1, dtype=torch.int32, device=keep.device)
    _check(load().psb_validate_document_positions(_ptr(k), _ptr(p), k.shape[0], k.shape[1], _ptr(status),
                                                  _vp(_stream(k))), "validate_document_positions")
    if int(status.item()) != 0:
        raise ValueError("positions break the document rule")


# ---- query shard against a delivered key window (left-halo delivery) -------------------

def shard_kv_window_start(doc_ids: torch.Tensor, seq_start: int, L: int) -> torch.Tensor:
    """Per row, the first key position the query shard ``[seq_start, seq_start + L)``
    needs (``[B]`` int32, on the device): ``min(seq_start, start of the document of the
    shard's first non-padding row)``."""
    _need_gpu(doc_ids)
    ids = doc_ids.reshape(doc_ids.shape[0] if doc_ids.dim() > 1 else 1, -1)
    ids = (ids if ids.dtype == torch.int32 else ids.to(torch.int32)).contiguous()
    B, S = ids.shape
    out = torch.empty(B, dtype=torch.int32, device=ids.device)
    _check(load().psb_shard_kv_window_start(_ptr(ids), B, S, int(seq_start), int(L), _ptr(out), _vp(_stream(ids))),
           "shard_kv_window_start")
    return out


def _window_status(status, where):
    if status is not None and int(status.item()) & DATA_KV_WINDOW:
        raise ValueError(f"{where}: a query row needs a key before the delivered window")


def blockdiag_attn_fwd_window(q, k, v, doc_ids, seq_start: int, kv_start: int, scale: float | None = None,
                              enable_gqa: bool = False, with_lse: bool = False,
                              workspace: torch.Tensor | None = None, validate: bool = False):
    """Forward of a query shard against the keys ``[kv_start, kv_start + kv_len)``.

    ``k, v [B, Hkv, kv_len, D]`` (contiguous) hold just that window; ``doc_ids [B, S]``
    covers the whole rows.  Returns ``out``, or ``(out, lse, workspace)`` with
    ``with_lse=True`` (the workspace then serves :func:`blockdiag_attn_bwd_window`).
    ``validate=True`` synchronizes and raises ``ValueError`` when some row needs a key
    before ``kv_start``.
    """
    _need_gpu(q, k, v, doc_ids)
    _check_qkv(q, k, v, contiguous=True)
    B, Hq, L, D = q.shape
    Hkv, kv_len = k.shape[1], k.shape[2]
    S = doc_ids.shape[-1]
    ids = _ids(doc_ids, B, S)
    need = bwd_workspace_size(B, Hq, Hkv, L, S, D) if with_lse else workspace_size(B, Hq, Hkv, L, D)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    out = torch.empty((B, Hq, L, D), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device) if with_lse else None
    status = torch.zeros(1, dtype=torch.int32, device=q.device) if validate else None
    sc = float(D) ** -0.5 if scale is None else float(scale)
    gqa = 1 if enable_gqa else 0
    st = _vp(_stream(q))
    lib = load()
    _check(lib.psb_blockdiag_attn_plan(_ptr(ids), B, Hq, Hkv, L, S, D, int(seq_start), gqa, _ptr(workspace),
                                       need, st), "blockdiag_attn_plan")
    _check(lib.psb_blockdiag_attn_fwd_window_planned(
        _ptr(q), _ptr(k), _ptr(v), _ptr(ids), B, Hq, Hkv, L, S, D, None, None, int(seq_start), int(kv_start),
        kv_len, sc, gqa, _ptr(out), _ptr(lse), _ptr(workspace), need, _ptr(status), st),
        "blockdiag_attn_fwd_window_planned")
    _window_status(status, "blockdiag_attn_fwd_window")
    return (out, lse, workspace) if with_lse else out


def blockdiag_attn_bwd_window(q, k, v, out, dout, lse, doc_ids, workspace, seq_start: int, kv_start: int,
                              scale: float | None = None, enable_gqa: bool = False, validate: bool = False):
    """Gradients ``(dq, dk, dv)`` of the windowed forward; ``dk, dv [B, Hkv, kv_len, D]``
    are the gradients of the window's keys (this shard's rows only)."""
    _need_gpu(q, k, v, out, dout, lse, doc_ids, workspace)
    _check_qkv(q, k, v, contiguous=True)
    B, Hq, L, D = q.shape
    Hkv, kv_len = k.shape[1], k.shape[2]
    S = doc_ids.shape[-1]
    for name, t in (("out", out), ("dout", dout)):
        if t.shape != q.shape or t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 tensor shaped like q")
    if lse.shape != (B, Hq, L) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, Hq, L] tensor")
    ids = _ids(doc_ids, B, S)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    status = torch.zeros(1, dtype=torch.int32, device=q.device) if validate else None
    sc = float(D) ** -0.5 if scale is None else float(scale)
    nbytes = workspace.numel() * workspace.element_size()
    _check(load().psb_blockdiag_attn_bwd_window_planned(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(ids), B, Hq, Hkv, L, S, D,
        int(seq_start), int(kv_start), kv_len, sc, 1 if enable_gqa else 0, _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(workspace), nbytes, _ptr(status), _vp(_stream(q))), "blockdiag_attn_bwd_window_planned")
    _window_status(status, "blockdiag_attn_bwd_window")
    return dq, dk, dv


# ---- dense-mask path -------------------------------------------------------------------

def blockdiag_dense_mask(doc_ids: torch.Tensor, seq_start: int = 0, L: int | None = None) -> torch.Tensor:
    """The per-document causal mask of the query rows ``[seq_start, seq_start + L)``:
    bool ``[B, L, S]`` (True = may attend), a view of rows padded to a multiple of 16
    bytes (the layout :func:`masked_attn_fwd` reads without a copy)."""
    _need_gpu(doc_ids)
    ids = doc_ids.reshape(doc_ids.shape[0] if doc_ids.dim() > 1 else 1, -1)
    ids = (ids if ids.dtype == torch.int32 else ids.to(torch.int32)).contiguous()
    B, S = ids.shape
    L = S - int(seq_start) if L is None else int(L)
    stride = (S + 15) // 16 * 16
    buf = torch.empty((B, L, stride), dtype=torch.bool, device=ids.device)
    _check(load().psb_blockdiag_dense_mask(_ptr(ids), B, S, int(seq_start), L, _ptr(buf), stride,
                                           _vp(_stream(ids))), "blockdiag_dense_mask")
    return buf[:, :, :S]


def _mask_operand(mask: torch.Tensor, B: int, L: int, S: int):
    """(tensor, batch stride, row stride) the kernel can read: rows 4-byte aligned and
    readable up to S rounded up to 4; anything else is copied into such a layout."""
    m = mask
    if m.dim() == 4:
        if m.shape[1] != 1:
            raise ValueError("a 4-D mask must be [B or 1, 1, L, S] (one mask for all heads)")
        m = m[:, 0]
    if m.dim() == 2:
        m = m.unsqueeze(0)
    if m.dim() != 3 or m.shape[1:] != (L, S) or m.shape[0] not in (1, B):
        raise ValueError(f"mask must be [B or 1, L, S] = [{B}, {L}, {S}]")
    if m.dtype not in (torch.bool, torch.uint8):
        raise ValueError("mask must be bool (True = may attend)")
    sb = 0 if m.shape[0] == 1 else m.stride(0)
    ss = m.stride(1)
    S4 = (S + 3) // 4 * 4
    end = m.storage_offset() + (m.shape[0] - 1) * sb + (L - 1) * ss + S4
    ok = (m.stride(2) == 1 or S <= 1) and sb % 4 == 0 and ss % 4 == 0 and ss >= S4 and \
        m.data_ptr() % 4 == 0 and end <= m.untyped_storage().nbytes()
    if not ok:
        stride = (S + 15) // 16 * 16
        buf = torch.zeros((m.shape[0], L, stride), dtype=torch.bool, device=m.device)
        buf[:, :, :S] = m != 0
        m, sb, ss = buf, (0 if m.shape[0] == 1 else L * stride), stride
    return m, sb, ss


def masked_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: torch.Tensor,
                    scale: float | None = None, enable_gqa: bool = False, with_lse: bool = False):
    """Attention under an explicit boolean mask ``[B or 1, L, S]`` (True = may attend,
    the same for every head); rows without an allowed key give 0.  ``q [B, Hq, L, D]``,
    ``k, v [B, Hkv, S, D]`` bf16 with a contiguous last dim.  Returns ``out`` or
    ``(out, lse)``."""
    _need_gpu(q, k, v, mask)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or t.dim() != 4 or t.stride(3) != 1:
            raise ValueError(f"{name} must be a 4-D bfloat16 tensor with a contiguous last dimension")
    if k.stride() != v.stride() or k.shape != v.shape:
        raise ValueError("k and v must share shape and strides")
    B, Hq, L, D = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError("k/v shape does not match q")
    m, sb, ss = _mask_operand(mask, B, L, S)
    out = torch.empty((B, Hq, L, D), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device) if with_lse else None
    sc = float(D) ** -0.5 if scale is None else float(scale)
    qs = (ctypes.c_int64 * 3)(*q.stride()[:3])
    kvs = (ctypes.c_int64 * 3)(*k.stride()[:3])
    _check(load().psb_masked_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(m), sb, ss, B, Hq, Hkv, L, S, D, qs, kvs,
                                      sc, 1 if enable_gqa else 0, _ptr(out), _ptr(lse), _vp(_stream(q))),
           "masked_attn_fwd")
    return (out, lse) if with_lse else out


def blockdiag_prepare(cu_seqlens: torch.Tensor, seq_len: int, Hq: int, Hkv: int, D: int, seq_start: int = 0,
                      L: int | None = None, enable_gqa: bool = False, workspace: torch.Tensor | None = None,
                      validate: bool = False):
    """One step's preparation for B rows in one launch, from boundaries ``[B, N + 1]``
    (rows with fewer documents repeat their last boundary): returns ``(doc_ids [B, S],
    seg_cu [B, S + 1], seg_n [B], workspace)``; row b's run boundaries are
    ``seg_cu[b, :seg_n[b] + 1]`` and the workspace holds the attention plan for
    :func:`blockdiag_attn_fwd`-style planned calls with these shapes."""
    _need_gpu(cu_seqlens)
    cu = cu_seqlens if cu_seqlens.dim() == 2 else cu_seqlens.reshape(1, -1)
    cu = (cu if cu.dtype == torch.int32 else cu.to(torch.int32)).contiguous()
    B, n1 = cu.shape
    S = int(seq_len)
    L = S - int(seq_start) if L is None else int(L)
    dev = cu.device
    ids = torch.empty((B, S), dtype=torch.int32, device=dev)
    seg = torch.empty((B, S + 1), dtype=torch.int32, device=dev)
    n = torch.empty(B, dtype=torch.int32, device=dev)
    need = workspace_size(B, Hq, Hkv, L, D)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev) if validate else None
    _check(load().psb_blockdiag_prepare(_ptr(cu), n1, n1 - 1, B, Hq, Hkv, L, S, D, int(seq_start),
                                        1 if enable_gqa else 0, _ptr(ids), _ptr(seg), _ptr(n), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _ptr(status),
                                        _vp(_stream(cu))), "blockdiag_prepare")
    if validate and int(status.item()) != 0:
        raise ValueError(f"cu_seqlens invalid (status bits {int(status.item())})")
    return ids, seg, n, workspace
