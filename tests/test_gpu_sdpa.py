"""The SDPA drop-in on the GPU: a module that calls the stock
``F.scaled_dot_product_attention`` gets the per-document causal attention while a
packed step is armed (forward and gradients vs the oracle), also through activation-
checkpoint recomputation, and the stock call when it is not; opcheck on the custom op."""

import pytest
import torch
import torch.nn.functional as F
import torch.utils.checkpoint as ckpt

import oracle
from gpu_common import compare, oracle_doc_ids, say
from test_gpu_backward import check_grad
from workloads import make_qkv, random_layout

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def psb():
    import packed_sequence_block_amd as m
    m.load()
    return m


class Attn(torch.nn.Module):
    def __init__(self, gqa):
        super().__init__()
        self.gqa = gqa

    def forward(self, q, k, v):
        return F.scaled_dot_product_attention(q, k, v, is_causal=True, enable_gqa=self.gqa)


class Block(torch.nn.Module):
    def __init__(self, gqa):
        super().__init__()
        self.self_attn = Attn(gqa)

    def forward(self, q, k, v):
        return self.self_attn(q, k, v)


def _case(seed):
    lay = random_layout(seed, B=1, S=384, L=384, seq_start=0, Hq=4, Hkv=2, D=64, max_doc=150, max_pad=20)
    q, k, v = make_qkv(lay, seed_base=4000 + seed)
    return lay, q, k, v, oracle_doc_ids(lay)


@pytest.mark.parametrize("use_ckpt", [False, True])
def test_hooked_module_forward_and_grads(psb, use_ckpt):
    lay, q, k, v, ids = _case(51)
    g = torch.Generator().manual_seed(52)
    dout = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    model = Block(True)
    handles = psb.attach_packed_varlen_hooks(model)
    qd, kd, vd = (t.cuda().requires_grad_(True) for t in (q, k, v))
    say("sdpa drop-in", "checkpoint" if use_ckpt else "plain")
    with psb.packed_documents(torch.as_tensor(ids).cuda()):
        out = ckpt.checkpoint(model, qd, kd, vd, use_reentrant=False) if use_ckpt else model(qd, kd, vd)
        (out.float() * dout.cuda().float()).sum().backward()  # recomputation runs while still armed
    torch.cuda.synchronize()
    for h in handles:
        h.remove()
    ref = oracle.blockdiag_attn(q, k, v, ids, 0, None, True)
    compare(out, ref, None, "drop-in forward")
    rq, rk, rv = oracle.blockdiag_attn_bwd(q, k, v, dout, ids, 0, None, True)
    check_grad(qd.grad, rq, "drop-in dq")
    check_grad(kd.grad, rk, "drop-in dk")
    check_grad(vd.grad, rv, "drop-in dv")


def test_unarmed_module_runs_stock_sdpa(psb):
    lay, q, k, v, ids = _case(53)
    model = Block(True)
    handles = psb.attach_packed_varlen_hooks(model)
    say("sdpa unarmed")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out = model(qd, kd, vd)
    stock = F.scaled_dot_product_attention(qd.float(), kd.float().repeat_interleave(2, dim=1).contiguous(),
                                           vd.float().repeat_interleave(2, dim=1).contiguous(), is_causal=True)
    with psb.packed_documents(torch.as_tensor(ids).cuda()):
        packed = model(qd, kd, vd)
    torch.cuda.synchronize()
    for h in handles:
        h.remove()
    assert (out.float() - stock).abs().max().item() < 2e-2   # whole-row causal: the stock call ran
    assert not torch.equal(out, packed)


def test_opcheck_custom_op(psb):
    lay, q, k, v, ids = _case(54)
    args = (q.cuda(), k.cuda(), v.cuda(), torch.as_tensor(ids, dtype=torch.int32).cuda(), 0, 64 ** -0.5, True)
    say("opcheck")
    torch.library.opcheck(torch.ops.psb.blockdiag_attn_fwd.default, args,
                          test_utils=("test_schema", "test_autograd_registration", "test_faketensor"))


def test_opcheck_backward_op(psb):
    lay, q, k, v, ids = _case(55)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    idd = torch.as_tensor(ids, dtype=torch.int32).cuda()
    out, lse, ws = torch.ops.psb.blockdiag_attn_fwd(qd, kd, vd, idd, 0, 64 ** -0.5, True)
    g = torch.Generator().manual_seed(56)
    dout = torch.randn(q.shape, generator=g).to(torch.bfloat16).cuda()
    args = (qd, kd, vd, out, dout, lse, idd, ws, 0, 64 ** -0.5, True)
    say("opcheck backward op")
    torch.library.opcheck(torch.ops.psb.blockdiag_attn_bwd.default, args,
                          test_utils=("test_schema", "test_faketensor"))


def test_backward_twice_leaves_saved_workspace_intact(psb):
    # retain_graph: the second backward reads the same saved plan and gives the same grads
    lay, q, k, v, ids = _case(57)
    qd, kd, vd = (t.cuda().requires_grad_(True) for t in (q, k, v))
    g = torch.Generator().manual_seed(58)
    dout = torch.randn(q.shape, generator=g).to(torch.bfloat16).cuda()
    say("backward twice")
    with psb.packed_documents(torch.as_tensor(ids).cuda()):
        out = psb.blockdiag_sdpa(qd, kd, vd, enable_gqa=True)
    out.backward(dout, retain_graph=True)
    first = [t.grad.clone() for t in (qd, kd, vd)]
    for t in (qd, kd, vd):
        t.grad = None
    out.backward(dout)
    torch.cuda.synchronize()
    for a, t in zip(first, (qd, kd, vd)):
        assert torch.equal(a, t.grad)
