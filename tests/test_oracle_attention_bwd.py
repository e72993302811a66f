"""Pins for the backward oracle (oracle/attention_bwd.py), plus planted mistakes.

Each pin checks the oracle's gradients against something fixed independently of
its formulas: PyTorch autograd through the library SDPA routine, central finite
differences of the (separately pinned) forward oracle, the partition identity of
a sharded sequence, and closed forms.  Every planted mistake must fail at least
one pin.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import attention_bwd as ab

PAD = -1000


def rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64)


def ids_from_lengths(lengths, pad=0):
    out = []
    for i, n in enumerate(lengths):
        out += [i + 1] * n
    return np.asarray(out + [PAD] * pad, dtype=np.int64)[None, :]


def sdpa_grads(q, k, v, dout, scale, gqa):
    """Autograd of the library routine (causal, one document), fp64."""
    q, k, v = (t.clone().requires_grad_(True) for t in (q, k, v))
    out = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale, enable_gqa=gqa)
    (out * dout).sum().backward()
    return q.grad, k.grad, v.grad


def close(a, b, tol=1e-10):
    return torch.allclose(torch.as_tensor(a, dtype=torch.float64), torch.as_tensor(b, dtype=torch.float64),
                          atol=tol, rtol=tol)


# ---- pins: each takes a backward implementation and asserts -----------------------------

def pin_single_document(bwd):
    B, Hq, Hkv, S, D = 1, 4, 2, 23, 8
    q, k, v, do = rand((B, Hq, S, D), 1), rand((B, Hkv, S, D), 2), rand((B, Hkv, S, D), 3), rand((B, Hq, S, D), 4)
    ids = np.ones((1, S), dtype=np.int64) * 7
    got = bwd(q, k, v, do, ids, 0, 0.3, True)
    want = sdpa_grads(q, k, v, do, 0.3, True)
    for a, b in zip(got, want):
        assert close(a, b), "single document != SDPA autograd"


def pin_packed_equals_separate(bwd):
    B, H, D = 1, 2, 4
    lens, pad = [5, 9, 3], 4
    ids = ids_from_lengths(lens, pad)
    S = ids.shape[1]
    q, k, v, do = rand((B, H, S, D), 5), rand((B, H, S, D), 6), rand((B, H, S, D), 7), rand((B, H, S, D), 8)
    dq, dk, dv = bwd(q, k, v, do, ids, 0, None, False)
    p = 0
    for n in lens:
        sl = slice(p, p + n)
        w = sdpa_grads(q[:, :, sl], k[:, :, sl], v[:, :, sl], do[:, :, sl], D ** -0.5, False)
        assert close(dq[:, :, sl], w[0]) and close(dk[:, :, sl], w[1]) and close(dv[:, :, sl], w[2]), \
            "packed row != documents run alone"
        p += n
    tail = slice(p, S)  # padding: no gradient anywhere
    assert torch.all(dq[:, :, tail] == 0) and torch.all(dk[:, :, tail] == 0) and torch.all(dv[:, :, tail] == 0)


def pin_finite_differences(bwd):
    B, Hq, Hkv, S, D = 1, 2, 1, 10, 3
    ids = np.asarray([[1, 1, 1, 2, 2, 2, 2, PAD, 3, 3]], dtype=np.int64)
    q, k, v, do = rand((B, Hq, S, D), 9), rand((B, Hkv, S, D), 10), rand((B, Hkv, S, D), 11), rand((B, Hq, S, D), 12)
    dq, dk, dv = bwd(q, k, v, do, ids, 0, 0.7, True)

    def loss(qq, kk, vv):
        return float((oracle.blockdiag_attn(qq, kk, vv, ids, 0, 0.7, True) * do).sum())

    eps = 1e-6
    rng = np.random.default_rng(0)
    for which, grad in (("q", dq), ("k", dk), ("v", dv)):
        for _ in range(6):
            t = {"q": q, "k": k, "v": v}[which]
            idx = tuple(int(rng.integers(0, n)) for n in t.shape)
            plus, minus = t.clone(), t.clone()
            plus[idx] += eps
            minus[idx] -= eps
            args_p = {"q": q, "k": k, "v": v, which: plus}
            args_m = {"q": q, "k": k, "v": v, which: minus}
            fd = (loss(args_p["q"], args_p["k"], args_p["v"]) - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
            assert abs(fd - float(grad[idx])) < 1e-6, f"finite difference mismatch in d{which} at {idx}"


def pin_shards_partition(bwd):
    B, Hq, Hkv, S, D = 1, 2, 2, 20, 4
    ids = ids_from_lengths([6, 8, 4], 2)
    q, k, v, do = rand((B, Hq, S, D), 13), rand((B, Hkv, S, D), 14), rand((B, Hkv, S, D), 15), rand((B, Hq, S, D), 16)
    full = bwd(q, k, v, do, ids, 0, None, False)
    a = 9  # cuts the second document
    s1 = bwd(q[:, :, :a], k, v, do[:, :, :a], ids, 0, None, False)
    s2 = bwd(q[:, :, a:], k, v, do[:, :, a:], ids, a, None, False)
    assert close(full[0][:, :, :a], s1[0]) and close(full[0][:, :, a:], s2[0]), "shard dq != rows of full dq"
    assert close(full[1], s1[1] + s2[1]) and close(full[2], s1[2] + s2[2]), "dk/dv != sum over shards"


def pin_gqa_sums_heads(bwd):
    B, Hq, Hkv, S, D = 1, 6, 2, 9, 4
    ids = ids_from_lengths([4, 5])
    q, k, v, do = rand((B, Hq, S, D), 17), rand((B, Hkv, S, D), 18), rand((B, Hkv, S, D), 19), rand((B, Hq, S, D), 20)
    dq, dk, dv = bwd(q, k, v, do, ids, 0, None, True)
    r = Hq // Hkv
    ke, ve = k.repeat_interleave(r, dim=1), v.repeat_interleave(r, dim=1)
    w = sdpa_grads(q[:, :, :4], ke[:, :, :4], ve[:, :, :4], do[:, :, :4], D ** -0.5, False)
    assert close(dq[:, :, :4], w[0]), "GQA dq"
    assert close(dk[:, :, :4], w[1].reshape(B, Hkv, r, 4, D).sum(2)), "GQA dk is the sum over the group"
    assert close(dv[:, :, :4], w[2].reshape(B, Hkv, r, 4, D).sum(2)), "GQA dv is the sum over the group"


def pin_zero_queries(bwd):
    # q = 0: uniform weights over each row's allowed keys, so dv[k] = sum over rows r that
    # see k of do[r] / (number of keys row r sees)  (closed form)
    B, H, D = 1, 1, 3
    ids = ids_from_lengths([3, 4], 1)
    S = ids.shape[1]
    q = torch.zeros((B, H, S, D), dtype=torch.float64)
    k, v, do = rand((B, H, S, D), 21), rand((B, H, S, D), 22), rand((B, H, S, D), 23)
    _, _, dv = bwd(q, k, v, do, ids, 0, None, False)
    want = torch.zeros_like(dv)
    starts = {1: 0, 2: 3}
    for r in range(S):
        d = int(ids[0, r])
        if d == PAD:
            continue
        n = r - starts[d] + 1
        for kk in range(starts[d], r + 1):
            want[0, 0, kk] += do[0, 0, r] / n
    assert close(dv, want), "q = 0 closed form for dv"


PINS = [pin_single_document, pin_packed_equals_separate, pin_finite_differences, pin_shards_partition,
        pin_gqa_sums_heads, pin_zero_queries]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_backward_pins(pin):
    pin(ab.blockdiag_attn_bwd)


def test_lse_closed_form_and_consistency():
    B, H, D = 1, 2, 4
    ids = ids_from_lengths([5, 7], 3)
    S = ids.shape[1]
    # q = 0: every allowed score is 0, so lse = log(number of allowed keys)
    k = rand((B, H, S, D), 30)
    lse = ab.blockdiag_attn_lse(torch.zeros((B, H, S, D), dtype=torch.float64), k, ids)
    starts = {1: 0, 2: 5}
    for r in range(S):
        d = int(ids[0, r])
        want = float("-inf") if d == PAD else np.log(r - starts[d] + 1)
        assert np.all(lse[0, :, r].numpy() == want) or np.allclose(lse[0, :, r].numpy(), want, atol=1e-14)
    # random q: exp(s - lse) over the allowed keys reproduces the forward oracle
    q, v = rand((B, H, S, D), 31), rand((B, H, S, D), 32)
    lse = ab.blockdiag_attn_lse(q, k, ids, 0, 0.4)
    out = oracle.blockdiag_attn(q, k, v, ids, 0, 0.4)
    mask = oracle.allowed_mask(torch.as_tensor(ids[0]), torch.arange(S))
    for h in range(H):
        s = (q[0, h] @ k[0, h].T) * 0.4
        p = torch.where(mask, torch.exp(s - lse[0, h].unsqueeze(1)), torch.zeros_like(s))
        rows = mask.any(dim=1)
        assert torch.allclose(p.sum(dim=1)[rows], torch.ones(int(rows.sum()), dtype=torch.float64), atol=1e-12)
        assert torch.allclose(p @ v[0, h], out[0, h], atol=1e-12)


# ---- planted mistakes -------------------------------------------------------------------

def _mutant(kind):
    def bwd(q, k, v, dout, doc_ids, seq_start=0, scale=None, enable_gqa=False):
        dq, dk, dv = ab.blockdiag_attn_bwd(q, k, v, dout, doc_ids, seq_start, scale, enable_gqa)
        if kind == "dq_scale_dropped":
            D = q.shape[-1]
            sc = D ** -0.5 if scale is None else scale
            return dq / sc, dk, dv
        if kind == "dk_dv_swapped":
            return dq, dv, dk
        if kind == "no_gqa_sum":  # keep only the first query head of each group
            Hq, Hkv = q.shape[1], k.shape[1]
            if Hq == Hkv:
                return dq, dk, dv
            r = Hq // Hkv
            one = ab.blockdiag_attn_bwd(q[:, ::r], k, v, dout[:, ::r], doc_ids, seq_start, scale, True)
            return dq, one[1], one[2]
        raise AssertionError(kind)
    return bwd


def _delta_dropped(q, k, v, dout, doc_ids, seq_start=0, scale=None, enable_gqa=False):
    # the gradient formulas with dS = P * dP: the rowsum(dO * O) term forgotten
    doc = torch.as_tensor(np.asarray(doc_ids)).to(torch.int64).reshape(q.shape[0], -1)
    B, Hq, Hkv, L, S, D = oracle.attention._check(q, k, v, doc, seq_start, enable_gqa)
    sc = D ** -0.5 if scale is None else scale
    dq = torch.zeros((B, Hq, L, D), dtype=torch.float64)
    dk = torch.zeros((B, Hkv, S, D), dtype=torch.float64)
    dv = torch.zeros((B, Hkv, S, D), dtype=torch.float64)
    qpos = torch.arange(seq_start, seq_start + L)
    for b in range(B):
        mask = oracle.allowed_mask(doc[b], qpos)
        has = mask.any(dim=1, keepdim=True)
        for h in range(Hq):
            g = oracle.kv_head_of(h, Hq, Hkv)
            s = ((q[b, h].double() @ k[b, g].double().T) * sc).masked_fill(~mask, float("-inf"))
            m = torch.where(has, s.max(dim=1, keepdim=True).values, torch.zeros_like(has, dtype=s.dtype))
            e = torch.exp(s - m)
            p = e / torch.where(has, e.sum(dim=1, keepdim=True), torch.ones_like(m))
            dp = dout[b, h].double() @ v[b, g].double().T
            ds = p * dp
            dq[b, h] = sc * (ds @ k[b, g].double())
            dk[b, g] += sc * (ds.T @ q[b, h].double())
            dv[b, g] += p.T @ dout[b, h].double()
    return dq, dk, dv


MUTANTS = {
    "dq_scale_dropped": _mutant("dq_scale_dropped"),
    "dk_dv_swapped": _mutant("dk_dv_swapped"),
    "no_gqa_sum": _mutant("no_gqa_sum"),
    "delta_dropped": _delta_dropped,
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_backward_mistake_is_caught(name):
    caught = []
    for pin in PINS:
        try:
            pin(MUTANTS[name])
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name} passes every pin"
