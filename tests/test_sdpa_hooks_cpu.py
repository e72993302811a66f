"""Host-side mechanics of the SDPA drop-in: arming, the hook swap and its restore,
argument checks, and the custom ops' registration (no GPU call is made)."""

import pytest
import torch
import torch.nn.functional as F

import packed_sequence_block_amd as psb
from packed_sequence_block_amd import sdpa


class _Attn(torch.nn.Module):
    def __init__(self, fail=False):
        super().__init__()
        self.fail = fail
        self.seen = []

    def forward(self, x):
        self.seen.append(F.scaled_dot_product_attention is psb.blockdiag_sdpa)
        if self.fail:
            raise RuntimeError("forward failed")
        return x


class _Layer(torch.nn.Module):
    def __init__(self, fail=False):
        super().__init__()
        self.self_attn = _Attn(fail)
        self.mlp = torch.nn.Identity()

    def forward(self, x):
        return self.mlp(self.self_attn(x))


@pytest.fixture
def armed(monkeypatch):
    # a CPU stand-in for the armed state: the hooks only look at whether one is set
    monkeypatch.setattr(sdpa, "_state", sdpa.PackedState(torch.zeros((1, 4), dtype=torch.int32)))


def test_hooks_swap_only_while_armed():
    model = torch.nn.Sequential(_Layer(), _Layer())
    handles = psb.attach_packed_varlen_hooks(model)
    assert len(handles) == 4  # a pre and a post hook per attention module
    stock = F.scaled_dot_product_attention
    model(torch.ones(2))
    assert [m.self_attn.seen for m in model] == [[False], [False]]
    sdpa._state = sdpa.PackedState(torch.zeros((1, 4), dtype=torch.int32))
    try:
        model(torch.ones(2))
    finally:
        sdpa._state = None
    assert [m.self_attn.seen[-1] for m in model] == [True, True]
    assert F.scaled_dot_product_attention is stock
    for h in handles:
        h.remove()


def test_hook_restores_stock_sdpa_when_forward_raises(armed):
    model = torch.nn.Sequential(_Layer(fail=True))
    psb.attach_packed_varlen_hooks(model)
    stock = F.scaled_dot_product_attention
    with pytest.raises(RuntimeError):
        model(torch.ones(2))
    assert model[0].self_attn.seen == [True]
    assert F.scaled_dot_product_attention is stock


def test_patched_sdpa_context_restores():
    stock = F.scaled_dot_product_attention
    with pytest.raises(KeyError):
        with psb.patched_sdpa():
            assert F.scaled_dot_product_attention is psb.blockdiag_sdpa
            raise KeyError
    assert F.scaled_dot_product_attention is stock


def test_sdpa_needs_armed_state_and_no_dropout(armed):
    x = torch.zeros((1, 1, 4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        psb.blockdiag_sdpa(x, x, x, dropout_p=0.1)
    with pytest.raises(ValueError):
        psb.blockdiag_sdpa(x.float(), x.float(), x.float())
    sdpa._state = None
    with pytest.raises(RuntimeError):
        psb.blockdiag_sdpa(x, x, x)


def test_arming_requires_device_ids_and_context_restores():
    with pytest.raises(ValueError):
        psb.enable_packed_varlen(torch.zeros(8, dtype=torch.int32))
    assert psb.current_packed_state() is None
    psb.disable_packed_varlen()
    assert psb.current_packed_state() is None


def test_custom_ops_registered():
    assert hasattr(torch.ops.psb, "blockdiag_attn_fwd") and hasattr(torch.ops.psb, "blockdiag_attn_bwd")
    schema = str(torch.ops.psb.blockdiag_attn_fwd.default._schema)
    assert "seq_start" in schema and "enable_gqa" in schema
