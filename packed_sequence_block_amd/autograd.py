"""PyTorch autograd face of the training path (argument marshalling only).

``blockdiag_attention(q, k, v, doc_ids, seq_start=0, scale=None, enable_gqa=False)``
returns the block-diagonal attention output and, on backward, the gradients for
q, k and v from the library's HIP kernels (forward with the per-row log-sum-exp,
then the dq / dk-dv kernels).  For a query shard, the k / v gradients are the
shard's own contributions, which the caller sums across ranks (the glm5_next.cp
page's differentiable gathers route them back the same way).

Inputs must be contiguous bf16 on the GPU; doc_ids int32 [B, S].
"""

from __future__ import annotations

import torch

from . import _lib


class _BlockDiagAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, doc_ids, seq_start, scale, enable_gqa):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        out, lse, ws = _lib.blockdiag_attn_fwd_lse(q, k, v, doc_ids, seq_start, scale, enable_gqa)
        ctx.save_for_backward(q, k, v, out, lse, doc_ids, ws)
        ctx.args = (seq_start, scale, enable_gqa)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, lse, doc_ids, ws = ctx.saved_tensors
        seq_start, scale, enable_gqa = ctx.args
        dq, dk, dv = _lib.blockdiag_attn_bwd(q, k, v, out, dout.to(torch.bfloat16).contiguous(), lse, doc_ids, ws,
                                             seq_start, scale, enable_gqa)
        return dq, dk, dv, None, None, None, None


def blockdiag_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, doc_ids: torch.Tensor,
                        seq_start: int = 0, scale: float | None = None, enable_gqa: bool = False) -> torch.Tensor:
    """Differentiable block-diagonal (per-document causal) attention, ``[B, Hq, L, D]`` bf16."""
    return _BlockDiagAttention.apply(q, k, v, doc_ids, int(seq_start), scale, bool(enable_gqa))
