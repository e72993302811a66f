"""Independent pins for the attention oracle.

Each pin takes an attention function with the oracle's signature
``attn(q, k, v, doc_ids, seq_start, scale, enable_gqa) -> [B, Hq, L, D]`` and
raises ``AssertionError`` when the function disagrees with a fact that is fixed
without the oracle: PyTorch's own causal sdpa (a library routine), closed
forms, or invariants of the definition on the blockdiag_cp page (package
overview, ``cp_blockdiag_sdpa``).  ``tests/test_oracle_attention.py`` runs them
on the oracle and on planted mistakes, which must each fail at least one pin.
"""

from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

PAD = -1000
TOL = 1e-10


def _bf16_randn(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, dtype=torch.float32, generator=g).to(torch.bfloat16)


def _ids(lens, pad, lead_pad=0):
    ids = [PAD] * lead_pad
    for j, n in enumerate(lens):
        ids += [j + 1] * n
    ids += [PAD] * pad
    return torch.tensor([ids], dtype=torch.int32)


def _close(a, b, tol=TOL):
    a = torch.as_tensor(np.asarray(a), dtype=torch.float64)
    b = torch.as_tensor(np.asarray(b), dtype=torch.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    err = (a - b).abs().max().item() if a.numel() else 0.0
    assert err <= tol, f"max abs diff {err}"


def _sdpa_causal(q, k, v, scale, gqa):
    """Library routine: ordinary causal attention in fp64 on the CPU."""
    return F.scaled_dot_product_attention(q.double(), k.double(), v.double(), is_causal=True,
                                          scale=scale, enable_gqa=gqa)


def pin_single_document(attn):
    """One document filling the row == ordinary causal attention (sdpa)."""
    for (Hq, Hkv, S, D, seed) in [(2, 2, 37, 16, 1), (4, 2, 29, 8, 2), (6, 3, 20, 4, 3)]:
        q, k, v = (_bf16_randn(s, seed * 10 + j) for j, s in
                   enumerate([(1, Hq, S, D), (1, Hkv, S, D), (1, Hkv, S, D)]))
        ids = torch.full((1, S), 5, dtype=torch.int32)
        sc = float(D) ** -0.5
        out = attn(q, k, v, ids, 0, sc, Hq != Hkv)
        _close(out, _sdpa_causal(q, k, v, sc, Hq != Hkv))


def pin_packed_equals_per_document(attn):
    """Packed row == each document run alone through causal sdpa; padding -> 0."""
    lens, pad = [5, 1, 9, 3, 7], 4
    S = sum(lens) + pad
    Hq, Hkv, D = 4, 2, 8
    q, k, v = (_bf16_randn(s, 77 + j) for j, s in
               enumerate([(2, Hq, S, D), (2, Hkv, S, D), (2, Hkv, S, D)]))
    ids = torch.cat([_ids(lens, pad), _ids(lens[::-1], pad)], dim=0)
    sc = 0.3
    out = torch.as_tensor(np.asarray(attn(q, k, v, ids, 0, sc, True)))
    ref = torch.zeros_like(out, dtype=torch.float64)
    for b, row_lens in enumerate([lens, lens[::-1]]):
        a = 0
        for n in row_lens:
            sl = slice(a, a + n)
            ref[b:b + 1, :, sl] = _sdpa_causal(q[b:b + 1, :, sl], k[b:b + 1, :, sl],
                                               v[b:b + 1, :, sl], sc, True)
            a += n
    _close(out, ref)


def pin_shard_equals_rows(attn):
    """A query shard at seq_start == the same rows of the unsharded result."""
    lens = [6, 11, 4, 9]
    S = sum(lens)
    Hq, Hkv, D = 2, 1, 8
    q, k, v = (_bf16_randn(s, 300 + j) for j, s in
               enumerate([(1, Hq, S, D), (1, Hkv, S, D), (1, Hkv, S, D)]))
    ids = _ids(lens, 0)
    full = torch.as_tensor(np.asarray(attn(q, k, v, ids, 0, 0.5, True)))
    for s0, L in [(8, 10), (3, 1), (0, 5), (S - 7, 7)]:
        part = attn(q[:, :, s0:s0 + L].contiguous(), k, v, ids, s0, 0.5, True)
        _close(part, full[:, :, s0:s0 + L])


def pin_padding_rows_zero(attn):
    """Queries with the padding id output exactly 0 (also lead and mid-row padding)."""
    ids = torch.tensor([[PAD, PAD, 1, 1, 1, PAD, 2, 2, PAD, PAD]], dtype=torch.int32)
    q, k, v = (_bf16_randn(s, 500 + j) for j, s in enumerate([(1, 2, 10, 4)] * 3))
    out = torch.as_tensor(np.asarray(attn(q, k, v, ids, 0, 1.0, False)))
    pad_rows = (ids[0] == PAD).nonzero().reshape(-1)
    assert torch.all(out[:, :, pad_rows] == 0)
    assert torch.all(out[:, :, (ids[0] != PAD).nonzero().reshape(-1)].abs().sum(-1) > 0)


def pin_zero_query_prefix_mean(attn):
    """q = 0: every allowed score is 0, so a row is the plain mean of V over
    ``[doc_start, qpos]`` — written here as a cumulative sum."""
    lens, pad = [7, 3, 12], 2
    S = sum(lens) + pad
    D = 4
    v = _bf16_randn((1, 1, S, D), 901)
    k = _bf16_randn((1, 1, S, D), 902)
    q = torch.zeros((1, 1, S, D), dtype=torch.bfloat16)
    out = torch.as_tensor(np.asarray(attn(q, k, v, _ids(lens, pad), 0, 0.7, False)))
    ref = torch.zeros((S, D), dtype=torch.float64)
    a = 0
    vv = v[0, 0].double()
    for n in lens:
        cs = torch.cumsum(vv[a:a + n], dim=0)
        ref[a:a + n] = cs / torch.arange(1, n + 1, dtype=torch.float64).unsqueeze(1)
        a += n
    _close(out[0, 0], ref)


def pin_zero_scale_prefix_mean(attn):
    """scale = 0 (either sign) with arbitrary q: every allowed score is 0, so a row is
    again the plain mean of V over ``[doc_start, qpos]``, with padding rows 0."""
    lens, pad = [6, 1, 9], 3
    S = sum(lens) + pad
    D = 4
    q, k, v = _bf16_randn((1, 2, S, D), 911), _bf16_randn((1, 1, S, D), 912), _bf16_randn((1, 1, S, D), 913)
    ref = torch.zeros((S, D), dtype=torch.float64)
    a = 0
    vv = v[0, 0].double()
    for n in lens:
        cs = torch.cumsum(vv[a:a + n], dim=0)
        ref[a:a + n] = cs / torch.arange(1, n + 1, dtype=torch.float64).unsqueeze(1)
        a += n
    for sc in (0.0, -0.0):
        out = torch.as_tensor(np.asarray(attn(q, k, v, _ids(lens, pad), 0, sc, True)))
        _close(out[0, 0], ref)
        _close(out[0, 1], ref)


def pin_constant_value_per_document(attn):
    """V constant inside each document => output equals that constant."""
    lens = [5, 8, 3]
    S = sum(lens)
    D = 4
    q, k = _bf16_randn((1, 2, S, D), 11), _bf16_randn((1, 2, S, D), 12)
    consts = torch.tensor([1.5, -2.25, 0.125], dtype=torch.float64)
    v = torch.cat([consts[j].repeat(n) for j, n in enumerate(lens)]).reshape(1, 1, S, 1)
    v = (v * torch.tensor([1.0, -1.0, 2.0, 0.5], dtype=torch.float64)).repeat(1, 2, 1, 1)
    v = v.to(torch.bfloat16)
    out = torch.as_tensor(np.asarray(attn(q, k, v, _ids(lens, 0), 0, 1.3, False)))
    _close(out, v.double(), 1e-12)


def pin_gqa_equals_repeat_interleave(attn):
    """GQA == multi-head attention on kv heads repeated Hq/Hkv times (interleaved)."""
    lens = [4, 10, 6]
    S = sum(lens)
    Hq, Hkv, D = 6, 2, 8
    q = _bf16_randn((1, Hq, S, D), 41)
    k, v = _bf16_randn((1, Hkv, S, D), 42), _bf16_randn((1, Hkv, S, D), 43)
    ids = _ids(lens, 0)
    a = attn(q, k, v, ids, 0, 0.4, True)
    r = Hq // Hkv
    b = attn(q, k.repeat_interleave(r, dim=1), v.repeat_interleave(r, dim=1), ids, 0, 0.4, False)
    _close(a, b)
    # and each head group against sdpa's own grouped path on one document
    one = torch.full((1, S), 2, dtype=torch.int32)
    _close(attn(q, k, v, one, 0, 0.4, True), _sdpa_causal(q, k, v, 0.4, True))


def pin_hand_example(attn, golden):
    """The hand-derived 4-token example in tests/golden/attention_hand.txt."""
    def mat(s):
        return [[float(x) for x in row.split()] for row in s.split("|")]
    ids = torch.tensor([[int(x) for x in golden["doc_ids"].split()]], dtype=torch.int32)
    q, k, v = (torch.tensor(mat(golden[n])).to(torch.bfloat16).reshape(1, 1, 4, 2)
               for n in ("q", "k", "v"))
    out = attn(q, k, v, ids, 0, 1.0, False)
    _close(np.asarray(out).reshape(4, 2), np.asarray(mat(golden["out"])), 1e-12)


ALL_PINS = [pin_single_document, pin_packed_equals_per_document, pin_shard_equals_rows,
            pin_padding_rows_zero, pin_zero_query_prefix_mean, pin_zero_scale_prefix_mean,
            pin_constant_value_per_document,
            pin_gqa_equals_repeat_interleave]
