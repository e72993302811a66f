"""Oracle for block-diagonal (per-document causal) attention — test infrastructure.

Definition followed ("nemo_automodel.components.distributed.blockdiag_cp"
page: the package overview and the ``cp_blockdiag_sdpa`` entry):

* a packed row concatenates documents, and the correct mask is causal inside
  each document and blocks every pair across documents;
* the local queries ``q[B, Hq, L, D]`` are rows ``seq_start + i`` of the global
  sequence and run against the delivered keys/values ``[B, Hkv, S, D]``;
* the mask is rebuilt from the document ids alone (``attn_mask``/``is_causal``
  play no part);
* ``scale=None`` means ``D ** -0.5``; ``enable_gqa`` is PyTorch/HF sdpa
  grouped-query attention, i.e. each kv head serves ``Hq // Hkv`` consecutive
  query heads;
* the result has the query's shape ``[B, Hq, L, D]``.

So, for row i of batch b and query head h, with ``qpos = seq_start + i`` and
kv head ``g``: key k is allowed iff ``doc[b,k] == doc[b,qpos]``,
``doc[b,qpos] != -1000`` and ``k <= qpos``; the output is the softmax-weighted
mean of the allowed values, computed in fp64 from the exactly-upcast bf16
inputs.  A row with no allowed key (a padding query) outputs exactly 0.
"""

from __future__ import annotations

import numpy as np
import torch

from .boundary import PAD_DOC_ID


def _check(q, k, v, doc_ids, seq_start, enable_gqa):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, seq, D]")
    B, Hq, L, D = q.shape
    Bk, Hkv, S, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or Dk != D:
        raise ValueError("k/v shape does not match q")
    if tuple(doc_ids.shape) != (B, S):
        raise ValueError("doc_ids must be [B, S]")
    if seq_start < 0 or seq_start + L > S:
        raise ValueError("query shard [seq_start, seq_start+L) outside [0, S)")
    if Hq != Hkv and not enable_gqa:
        raise ValueError("Hq != Hkv needs enable_gqa")
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hkv, L, S, D


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """KV head serving query head h under sdpa's grouped-query convention.

    sdpa with ``enable_gqa`` repeats each kv head ``Hq // Hkv`` times along the
    head axis (repeat_interleave), so query head h reads kv head
    ``h // (Hq // Hkv)``.
    """
    return h // (Hq // Hkv)


def allowed_mask(doc_row: torch.Tensor, qpos: torch.Tensor) -> torch.Tensor:
    """Explicit block-causal mask ``[len(qpos), S]`` from one row's doc ids.

    Allowed iff same document, the query is not padding, and key <= query.
    """
    S = doc_row.shape[0]
    kpos = torch.arange(S, dtype=torch.int64)
    dq = doc_row[qpos].unsqueeze(1)
    dk = doc_row.unsqueeze(0)
    return (dq == dk) & (dq != PAD_DOC_ID) & (kpos.unsqueeze(0) <= qpos.unsqueeze(1))


def _softmax_weighted_mean(scores: torch.Tensor, mask: torch.Tensor, vals: torch.Tensor) -> torch.Tensor:
    """Rows of softmax(scores restricted to mask) @ vals; empty rows give 0.

    ``scores`` [r, c] fp64, ``mask`` [r, c] bool, ``vals`` [c, D] fp64.
    """
    has = mask.any(dim=1)
    s = scores.masked_fill(~mask, float("-inf"))
    m = s.max(dim=1, keepdim=True).values
    m = torch.where(has.unsqueeze(1), m, torch.zeros_like(m))
    p = torch.exp(s - m)                       # exp(-inf) == 0 on masked keys
    denom = p.sum(dim=1, keepdim=True)
    out = (p @ vals) / torch.where(has.unsqueeze(1), denom, torch.ones_like(denom))
    out[~has] = 0.0
    return out


def _as_f64(t):
    return t.detach().to("cpu").to(torch.float64)


def blockdiag_attn(q, k, v, doc_ids, seq_start: int = 0, scale: float | None = None,
                   enable_gqa: bool = False, chunk: int = 128) -> torch.Tensor:
    """Block-causal attention, fp64, ``[B, Hq, L, D]``.

    Rows are taken ``chunk`` at a time; for each chunk the explicit mask is
    built from the document ids and only the key columns that some row of the
    chunk may see are multiplied (a masked column contributes exp(-inf) = 0,
    so leaving it out changes nothing).
    """
    doc_ids = torch.as_tensor(np.asarray(doc_ids)).to(torch.int64).reshape(q.shape[0], -1)
    B, Hq, Hkv, L, S, D = _check(q, k, v, doc_ids, seq_start, enable_gqa)
    sc = float(D) ** -0.5 if scale is None else float(scale)
    qf, kf, vf = _as_f64(q), _as_f64(k), _as_f64(v)
    out = torch.zeros((B, Hq, L, D), dtype=torch.float64)
    for b in range(B):
        for i0 in range(0, L, chunk):
            i1 = min(L, i0 + chunk)
            qpos = torch.arange(seq_start + i0, seq_start + i1, dtype=torch.int64)
            mask = allowed_mask(doc_ids[b], qpos)
            cols = torch.nonzero(mask.any(dim=0)).reshape(-1)
            if cols.numel() == 0:
                continue
            mc = mask[:, cols]
            for h in range(Hq):
                g = kv_head_of(h, Hq, Hkv)
                scores = (qf[b, h, i0:i1] @ kf[b, g, cols].T) * sc
                out[b, h, i0:i1] = _softmax_weighted_mean(scores, mc, vf[b, g, cols])
    return out


def blockdiag_attn_rows(q, k, v, doc_ids, seq_start: int, scale: float | None,
                        enable_gqa: bool, b: int, rows) -> torch.Tensor:
    """Oracle output for selected local rows of batch ``b``: ``[len(rows), Hq, D]``.

    Same definition as :func:`blockdiag_attn`, one row at a time, for checking
    sampled outputs of full-size problems.
    """
    doc_ids = torch.as_tensor(np.asarray(doc_ids)).to(torch.int64).reshape(q.shape[0], -1)
    B, Hq, Hkv, L, S, D = _check(q, k, v, doc_ids, seq_start, enable_gqa)
    sc = float(D) ** -0.5 if scale is None else float(scale)
    res = torch.zeros((len(rows), Hq, D), dtype=torch.float64)
    for n, i in enumerate(rows):
        qpos = torch.tensor([seq_start + int(i)], dtype=torch.int64)
        mask = allowed_mask(doc_ids[b], qpos)
        cols = torch.nonzero(mask[0]).reshape(-1)
        if cols.numel() == 0:
            continue
        mc = mask[:, cols]
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            qrow = _as_f64(q[b, h, int(i)]).unsqueeze(0)
            kk, vv = _as_f64(k[b, g, cols]), _as_f64(v[b, g, cols])
            res[n, h] = _softmax_weighted_mean((qrow @ kk.T) * sc, mc, vv)[0]
    return res


def blockdiag_attn_loop(q, k, v, doc_ids, seq_start: int = 0, scale: float | None = None,
                        enable_gqa: bool = False) -> np.ndarray:
    """The same definition as literal loops in Python floats — tiny inputs only."""
    doc_np = np.asarray(doc_ids).reshape(q.shape[0], -1)
    B, Hq, Hkv, L, S, D = _check(q, k, v, torch.as_tensor(doc_np), seq_start, enable_gqa)
    sc = float(D) ** -0.5 if scale is None else float(scale)
    qn, kn, vn = (_as_f64(t).numpy() for t in (q, k, v))
    out = np.zeros((B, Hq, L, D), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            for i in range(L):
                qpos = seq_start + i
                dq = int(doc_np[b, qpos])
                keys = [kk for kk in range(S)
                        if int(doc_np[b, kk]) == dq and dq != PAD_DOC_ID and kk <= qpos]
                if not keys:
                    continue
                s = [sc * sum(float(qn[b, h, i, d]) * float(kn[b, g, kk, d]) for d in range(D))
                     for kk in keys]
                mx = max(s)
                w = [np.exp(x - mx) for x in s]
                tot = sum(w)
                for d in range(D):
                    out[b, h, i, d] = sum(wj * float(vn[b, g, kk, d]) for wj, kk in zip(w, keys)) / tot
    return out


def kv_window_start(doc_ids, seq_start: int, L: int) -> np.ndarray:
    """First key position a query shard needs, per batch row: ``[B]`` int64.

    blockdiag_cp page, package overview (the ``.exchange`` layer can deliver only
    the needed keys through a left halo instead of an all-gather) and
    ``cp_blockdiag_sdpa`` (the local rows at ``seq_start + i``): the shard's keys
    are its own ``[seq_start, seq_start + L)`` plus the earlier keys some local
    query may attend to.  Taken straight from the explicit mask: the smallest
    key column with an allowed pair for any local row, or ``seq_start`` when that
    is smaller (or no row has a key).
    """
    doc_ids = torch.as_tensor(np.asarray(doc_ids)).to(torch.int64)
    doc_ids = doc_ids.reshape(doc_ids.shape[0], -1) if doc_ids.dim() > 0 else doc_ids.reshape(1, -1)
    out = np.full(doc_ids.shape[0], seq_start, dtype=np.int64)
    qpos = torch.arange(seq_start, seq_start + L, dtype=torch.int64)
    for b in range(doc_ids.shape[0]):
        if L == 0:
            continue
        cols = torch.nonzero(allowed_mask(doc_ids[b], qpos).any(dim=0)).reshape(-1)
        if cols.numel() > 0:
            out[b] = min(seq_start, int(cols[0]))
    return out


def dense_mask(doc_ids, seq_start: int, L: int) -> torch.Tensor:
    """The per-document causal mask materialised, bool ``[B, L, S]`` (True = may attend).

    blockdiag_cp page, package overview: the ``.kernels`` layer has a dense-mask path
    next to the varlen kernels; this is the mask such a path consumes, row i of the
    shard being global position ``seq_start + i``.
    """
    doc_ids = torch.as_tensor(np.asarray(doc_ids)).to(torch.int64)
    doc_ids = doc_ids.reshape(doc_ids.shape[0], -1)
    qpos = torch.arange(seq_start, seq_start + L, dtype=torch.int64)
    return torch.stack([allowed_mask(doc_ids[b], qpos) for b in range(doc_ids.shape[0])])


def masked_attn(q, k, v, mask, scale: float | None = None, enable_gqa: bool = False) -> torch.Tensor:
    """Attention under an explicit boolean mask, fp64 ``[B, Hq, L, D]``.

    ``mask`` is ``[B, L, S]`` (or ``[1, L, S]``, shared by the batch), True where
    query row i may attend to key j, the same for every head; a row with no allowed
    key outputs 0.  Scale and GQA as in ``blockdiag_attn``.
    """
    mask = torch.as_tensor(np.asarray(mask)).to(torch.bool)
    B, Hq, L, D = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("k / v shape does not match q")
    if enable_gqa:
        if Hq % Hkv != 0:
            raise ValueError("Hq must be a multiple of Hkv")
    elif Hq != Hkv:
        raise ValueError("Hq != Hkv needs enable_gqa")
    if mask.dim() != 3 or mask.shape[1:] != (L, S) or mask.shape[0] not in (1, B):
        raise ValueError("mask must be [B or 1, L, S]")
    sc = float(D) ** -0.5 if scale is None else float(scale)
    qf, kf, vf = _as_f64(q), _as_f64(k), _as_f64(v)
    out = torch.zeros((B, Hq, L, D), dtype=torch.float64)
    for b in range(B):
        mb = mask[b if mask.shape[0] == B else 0]
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            out[b, h] = _softmax_weighted_mean((qf[b, h] @ kf[b, g].T) * sc, mb, vf[b, g])
    return out
