"""Drop-in scaled-dot-product attention for packed rows (argument marshalling only).

Follows the "nemo_automodel.components.distributed.blockdiag_cp" page:
* ``cp_blockdiag_sdpa`` — the SDPA signature; the mask comes from the document ids
  of the armed step, so ``attn_mask`` and ``is_causal`` are ignored; ``scale=None``
  means ``D**-0.5``; ``enable_gqa`` as in sdpa; output ``[B, Hq, L, D]``;
* ``enable_cp1_packed_varlen`` / ``disable_cp1_packed_varlen`` /
  ``current_blockdiag_cp_state`` — the packed layout is armed for one outer step
  (``doc_ids [1, S]`` or ``[S]`` over the whole packed row) and cleared afterwards;
* ``attach_cp1_packed_varlen_hooks`` — forward pre/post hooks on each attention
  module swap ``torch.nn.functional.scaled_dot_product_attention`` for the packed
  call and put the stock one back, also when the forward raises, so activation-
  checkpoint recomputation inside backward takes the packed path as long as the
  step is armed.

The attention itself is the library's HIP forward / backward, registered as the
torch custom ops ``psb::blockdiag_attn_fwd`` and ``psb::blockdiag_attn_bwd`` (with
shape functions and an autograd formula), so graph tracers see one opaque op.
"""

from __future__ import annotations

import contextlib
from dataclasses import dataclass

import torch
import torch.nn.functional as F

from . import _lib

# ---- custom ops ---------------------------------------------------------------------


@torch.library.custom_op("psb::blockdiag_attn_fwd", mutates_args=(), device_types="cuda")
def blockdiag_attn_fwd_op(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, doc_ids: torch.Tensor,
                          seq_start: int, scale: float, enable_gqa: bool
                          ) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """``(out [B,Hq,L,D] bf16, lse [B,Hq,L] fp32, workspace uint8)``; the workspace holds
    the tile plan the backward reads."""
    out, lse, ws = _lib.blockdiag_attn_fwd_lse(q.contiguous(), k.contiguous(), v.contiguous(), doc_ids,
                                               seq_start, scale, enable_gqa)
    return out, lse, ws


@blockdiag_attn_fwd_op.register_fake
def _fwd_fake(q, k, v, doc_ids, seq_start, scale, enable_gqa):
    B, Hq, L, D = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    n = _lib.bwd_workspace_size(B, Hq, Hkv, L, S, D)
    return (q.new_empty((B, Hq, L, D)), q.new_empty((B, Hq, L), dtype=torch.float32),
            q.new_empty((n,), dtype=torch.uint8))


@torch.library.custom_op("psb::blockdiag_attn_bwd", mutates_args=(), device_types="cuda")
def blockdiag_attn_bwd_op(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                          dout: torch.Tensor, lse: torch.Tensor, doc_ids: torch.Tensor, workspace: torch.Tensor,
                          seq_start: int, scale: float, enable_gqa: bool
                          ) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    # The library's backward writes its per-row table and key-side tile order after the
    # plan (the first workspace_size bytes).  It gets a fresh buffer holding a copy of the
    # plan, so the forward's saved workspace is never written and the op mutates nothing.
    B, Hq, L, D = q.shape
    n = _lib.workspace_size(B, Hq, k.shape[1], L, D)
    ws = torch.empty_like(workspace)
    ws[:n].copy_(workspace[:n])
    return _lib.blockdiag_attn_bwd(q.contiguous(), k.contiguous(), v.contiguous(), out,
                                   dout.to(torch.bfloat16).contiguous(), lse, doc_ids, ws, seq_start, scale,
                                   enable_gqa)


@blockdiag_attn_bwd_op.register_fake
def _bwd_fake(q, k, v, out, dout, lse, doc_ids, workspace, seq_start, scale, enable_gqa):
    return (q.new_empty(q.shape), k.new_empty(k.shape), v.new_empty(v.shape))


def _setup_context(ctx, inputs, output):
    ctx.set_materialize_grads(False)  # lse and workspace get no gradient: no zero tensors for them
    q, k, v, doc_ids, seq_start, scale, enable_gqa = inputs
    out, lse, ws = output
    ctx.save_for_backward(q, k, v, out, lse, doc_ids, ws)
    ctx.args = (seq_start, scale, enable_gqa)


def _backward(ctx, dout, dlse, dws):
    q, k, v, out, lse, doc_ids, ws = ctx.saved_tensors
    if dout is None:  # the output was not used by the loss
        return None, None, None, None, None, None, None
    seq_start, scale, enable_gqa = ctx.args
    dq, dk, dv = blockdiag_attn_bwd_op(q, k, v, out, dout, lse, doc_ids, ws, seq_start, scale, enable_gqa)
    return dq, dk, dv, None, None, None, None


blockdiag_attn_fwd_op.register_autograd(_backward, setup_context=_setup_context)


def blockdiag_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, doc_ids: torch.Tensor,
                        seq_start: int = 0, scale: float | None = None, enable_gqa: bool = False) -> torch.Tensor:
    """Differentiable block-diagonal (per-document causal) attention, ``[B, Hq, L, D]`` bf16,
    with explicit document ids ``[B, S]`` (no armed state).  For a query shard the k / v
    gradients are the shard's own contributions, which the caller sums across ranks (the
    glm5_next.cp page's differentiable gathers route them back the same way)."""
    sc = float(q.shape[-1]) ** -0.5 if scale is None else float(scale)
    out, _, _ = blockdiag_attn_fwd_op(q, k, v, doc_ids, int(seq_start), sc, bool(enable_gqa))
    return out


def _ids_2d(doc_ids: torch.Tensor, B: int) -> torch.Tensor:
    ids = doc_ids.reshape(1, -1) if doc_ids.dim() == 1 else doc_ids
    if ids.shape[0] == 1 and B > 1:
        ids = ids.expand(B, -1)
    return (ids if ids.dtype == torch.int32 else ids.to(torch.int32)).contiguous()


# ---- the armed packed step ------------------------------------------------------------


@dataclass(frozen=True)
class PackedState:
    """Document ids ``[B or 1, S]`` of the whole packed rows (-1000 = padding) and the
    global position of the local query rows' first row."""
    doc_ids: torch.Tensor
    seq_start: int = 0


_state: PackedState | None = None


def enable_packed_varlen(doc_ids: torch.Tensor, seq_start: int = 0) -> PackedState:
    """Arms the packed path for the next forward (and its backward recomputation)."""
    global _state
    if not doc_ids.is_cuda:
        raise ValueError("doc_ids must live on the GPU")
    _state = PackedState(doc_ids, int(seq_start))
    return _state


def disable_packed_varlen() -> None:
    """Clears the armed state (call before the next outer forward)."""
    global _state
    _state = None


def current_packed_state() -> PackedState | None:
    return _state


@contextlib.contextmanager
def packed_documents(doc_ids: torch.Tensor, seq_start: int = 0):
    """``with packed_documents(ids): ...`` arms the packed path for the block and puts
    the previous state back afterwards."""
    global _state
    prev = _state
    enable_packed_varlen(doc_ids, seq_start)
    try:
        yield _state
    finally:
        _state = prev


# ---- the drop-in -----------------------------------------------------------------------


def blockdiag_sdpa(query: torch.Tensor, key: torch.Tensor, value: torch.Tensor, attn_mask=None,
                   dropout_p: float = 0.0, is_causal: bool = False, scale: float | None = None,
                   enable_gqa: bool = False, **kwargs) -> torch.Tensor:
    """``F.scaled_dot_product_attention`` with the armed step's per-document causal mask.

    ``attn_mask`` and ``is_causal`` are ignored (the mask is rebuilt from the document
    ids); dropout is not supported.  Differentiable.
    """
    del attn_mask, is_causal, kwargs
    st = _state
    if st is None:
        raise RuntimeError("no packed layout armed: call enable_packed_varlen(doc_ids) first")
    if dropout_p != 0.0:
        raise ValueError("blockdiag_sdpa does not support dropout")
    if query.dtype != torch.bfloat16:
        raise ValueError("blockdiag_sdpa computes in bfloat16: pass bf16 query, key and value")
    D = query.shape[-1]
    sc = float(D) ** -0.5 if scale is None else float(scale)
    ids = _ids_2d(st.doc_ids, query.shape[0])
    out, _, _ = blockdiag_attn_fwd_op(query, key, value, ids, st.seq_start, sc, bool(enable_gqa))
    return out


_stock_sdpa = F.scaled_dot_product_attention


@contextlib.contextmanager
def patched_sdpa():
    """Within the block ``F.scaled_dot_product_attention`` is :func:`blockdiag_sdpa`."""
    prev = F.scaled_dot_product_attention
    F.scaled_dot_product_attention = blockdiag_sdpa
    try:
        yield
    finally:
        F.scaled_dot_product_attention = prev


def attach_packed_varlen_hooks(model: torch.nn.Module, suffix: str = "self_attn") -> list:
    """Pre/post forward hooks on every submodule whose name ends with ``suffix``: while a
    packed layout is armed, each such forward sees :func:`blockdiag_sdpa` as
    ``F.scaled_dot_product_attention``; the stock function is restored after the
    forward, also when it raises.  Returns the hook handles."""
    handles = []
    for name, mod in model.named_modules():
        if not name.endswith(suffix):
            continue

        def pre(module, args, kwargs):
            module._psb_prev_sdpa = F.scaled_dot_product_attention
            if _state is not None:
                F.scaled_dot_product_attention = blockdiag_sdpa

        def post(module, args, kwargs, output):
            F.scaled_dot_product_attention = getattr(module, "_psb_prev_sdpa", _stock_sdpa)

        handles.append(mod.register_forward_pre_hook(pre, with_kwargs=True))
        handles.append(mod.register_forward_hook(post, with_kwargs=True, always_call=True))
    return handles
