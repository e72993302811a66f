"""Oracle for the gradients of block-diagonal attention — test infrastructure.

The pages treat this attention as part of a training step: the
"nemo_automodel.components.distributed.blockdiag_cp" page (package overview and
``attach_cp1_packed_varlen_hooks``) keeps the packed block-diagonal path active
while backward recomputes checkpointed forwards, and the
"nemo_automodel.components.models.glm5_next.cp" page (``all_gather_sequence``,
``gather_sequence``) keeps K/V gradient flow across shards, routing each
gradient back to the rank that owns the shard.  They print no gradient
formula, so the oracle is the derivative of the forward definition itself
(see ``attention.py``), written out in fp64 for each (batch, query head):

    s   = scale * Q K^T            over allowed keys only (same mask as forward)
    P   = softmax(s) row-wise      (rows without an allowed key: P = 0, out = 0)
    O   = P V
    dV  = P^T dO                   summed over the query heads of a kv head
    dP  = dO V^T
    dS  = P * (dP - rowsum(dO * O))
    dQ  = scale * dS K
    dK  = scale * dS^T Q           summed over the query heads of a kv head

``rowsum(dO * O)`` equals ``rowsum(P * dP)`` because each row of P sums to 1.
The log-sum-exp that a forward keeps for this backward is
``lse = log(sum over allowed keys of exp(s))``, -inf for a row without keys.

For a query shard (``seq_start``, ``L``) the gradients are those of the shard's
own loss: dK and dV collect only what the shard's rows contribute, and the
full-sequence dK / dV is the sum over the shards of a partition of the rows
(the same sum the pages' differentiable gathers perform across ranks).
"""

from __future__ import annotations

import numpy as np
import torch

from .attention import _check, _as_f64, allowed_mask, kv_head_of


def blockdiag_attn_lse(q, k, doc_ids, seq_start: int = 0, scale: float | None = None,
                       enable_gqa: bool = False, chunk: int = 128) -> torch.Tensor:
    """Natural-log sum of exp(scale * q.k) over each row's allowed keys, fp64 ``[B, Hq, L]``.

    Rows without an allowed key (padding queries) get -inf.
    """
    doc_ids = torch.as_tensor(np.asarray(doc_ids)).to(torch.int64).reshape(q.shape[0], -1)
    B, Hq, Hkv, L, S, D = _check(q, k, k, doc_ids, seq_start, enable_gqa)
    sc = float(D) ** -0.5 if scale is None else float(scale)
    qf, kf = _as_f64(q), _as_f64(k)
    lse = torch.full((B, Hq, L), float("-inf"), dtype=torch.float64)
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
                s = ((qf[b, h, i0:i1] @ kf[b, g, cols].T) * sc).masked_fill(~mc, float("-inf"))
                lse[b, h, i0:i1] = torch.logsumexp(s, dim=1)
    return lse


def blockdiag_attn_bwd(q, k, v, dout, doc_ids, seq_start: int = 0, scale: float | None = None,
                       enable_gqa: bool = False, chunk: int = 128):
    """Gradients ``(dq [B,Hq,L,D], dk [B,Hkv,S,D], dv [B,Hkv,S,D])`` of ``sum(out * dout)``, fp64.

    Rows are taken ``chunk`` at a time with the explicit mask, as in the forward
    oracle; masked entries of P are exactly 0, so they add nothing anywhere.
    """
    doc_ids = torch.as_tensor(np.asarray(doc_ids)).to(torch.int64).reshape(q.shape[0], -1)
    B, Hq, Hkv, L, S, D = _check(q, k, v, doc_ids, seq_start, enable_gqa)
    if tuple(dout.shape) != tuple(q.shape):
        raise ValueError("dout must have the shape of q")
    sc = float(D) ** -0.5 if scale is None else float(scale)
    qf, kf, vf, dof = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    dq = torch.zeros((B, Hq, L, D), dtype=torch.float64)
    dk = torch.zeros((B, Hkv, S, D), dtype=torch.float64)
    dv = torch.zeros((B, Hkv, S, D), dtype=torch.float64)
    for b in range(B):
        for i0 in range(0, L, chunk):
            i1 = min(L, i0 + chunk)
            qpos = torch.arange(seq_start + i0, seq_start + i1, dtype=torch.int64)
            mask = allowed_mask(doc_ids[b], qpos)
            cols = torch.nonzero(mask.any(dim=0)).reshape(-1)
            if cols.numel() == 0:
                continue
            mc = mask[:, cols]
            has = mc.any(dim=1, keepdim=True)
            for h in range(Hq):
                g = kv_head_of(h, Hq, Hkv)
                kk, vv = kf[b, g, cols], vf[b, g, cols]
                s = ((qf[b, h, i0:i1] @ kk.T) * sc).masked_fill(~mc, float("-inf"))
                m = torch.where(has, s.max(dim=1, keepdim=True).values, torch.zeros_like(has, dtype=s.dtype))
                e = torch.exp(s - m)
                p = e / torch.where(has, e.sum(dim=1, keepdim=True), torch.ones_like(m))
                o = p @ vv
                do = dof[b, h, i0:i1]
                dp = do @ vv.T
                delta = (do * o).sum(dim=1, keepdim=True)
                ds = p * (dp - delta)
                dq[b, h, i0:i1] = sc * (ds @ kk)
                dk[b, g, cols] += sc * (ds.T @ qf[b, h, i0:i1])
                dv[b, g, cols] += p.T @ do
    return dq, dk, dv
