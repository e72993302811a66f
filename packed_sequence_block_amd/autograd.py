"""PyTorch autograd face of the training path (argument marshalling only).

``blockdiag_attention(q, k, v, doc_ids, seq_start=0, scale=None, enable_gqa=False)``
returns the block-diagonal attention output and, on backward, the gradients for
q, k and v from the library's HIP kernels (forward with the per-row log-sum-exp,
then the dq / dk-dv kernels), through the custom ops of ``sdpa.py``.  For a query
shard, the k / v gradients are the shard's own contributions, which the caller sums
across ranks (the glm5_next.cp page's differentiable gathers route them back the
same way).

Inputs are bf16 on the GPU; doc_ids int32 [B, S].
"""

from __future__ import annotations

import torch

from .sdpa import blockdiag_attn_fwd_op


def blockdiag_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, doc_ids: torch.Tensor,
                        seq_start: int = 0, scale: float | None = None, enable_gqa: bool = False) -> torch.Tensor:
    """Differentiable block-diagonal (per-document causal) attention, ``[B, Hq, L, D]`` bf16."""
    sc = float(q.shape[-1]) ** -0.5 if scale is None else float(scale)
    out, _, _ = blockdiag_attn_fwd_op(q, k, v, doc_ids, int(seq_start), sc, bool(enable_gqa))
    return out
