"""Pins for the attention oracle, plus planted mistakes that the pins must catch."""

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as oa
import pins
from workloads import random_layout, make_qkv


def _oracle(q, k, v, ids, s0, sc, gqa):
    return oracle.blockdiag_attn(q, k, v, ids, s0, sc, gqa, chunk=7)


def _loop(q, k, v, ids, s0, sc, gqa):
    return oracle.blockdiag_attn_loop(q, k, v, ids, s0, sc, gqa)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_meets_pin(pin):
    pin(_oracle)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_loop_oracle_meets_pin(pin):
    pin(_loop)


def test_hand_example(golden):
    g = golden("attention_hand.txt")
    pins.pin_hand_example(_oracle, g)
    pins.pin_hand_example(_loop, g)


@pytest.mark.parametrize("seed", range(6))
def test_loop_equals_chunked(seed):
    lay = random_layout(seed, B=2, S=23, L=15, seq_start=seed % 9, Hq=4, Hkv=2, D=8,
                        max_doc=9, max_pad=5)
    q, k, v = make_qkv(lay, seed_base=seed * 7)
    ids = np.stack([oracle.doc_ids_from_cu_seqlens(lay.cu_seqlens(b), lay.S)[0]
                    for b in range(lay.B)])
    a = oracle.blockdiag_attn(q, k, v, ids, lay.seq_start, None, True, chunk=4)
    b = oracle.blockdiag_attn_loop(q, k, v, ids, lay.seq_start, None, True)
    assert np.abs(a.numpy() - b).max() < 1e-12


def test_rows_equal_full():
    lay = random_layout(9, B=2, S=40, L=25, seq_start=10, Hq=4, Hkv=1, D=16, max_doc=12,
                        max_pad=6)
    q, k, v = make_qkv(lay, seed_base=5)
    ids = np.stack([oracle.doc_ids_from_cu_seqlens(lay.cu_seqlens(b), lay.S)[0]
                    for b in range(lay.B)])
    full = oracle.blockdiag_attn(q, k, v, ids, 10, 0.2, True)
    rows = [0, 3, 24, 11]
    for b in range(2):
        r = oracle.blockdiag_attn_rows(q, k, v, ids, 10, 0.2, True, b, rows)
        assert torch.allclose(r, full[b, :, rows].permute(1, 0, 2), atol=1e-13, rtol=0)


def test_default_scale_is_inverse_sqrt_d():
    lay = random_layout(3, B=1, S=12, Hq=2, Hkv=2, D=16, max_doc=5)
    q, k, v = make_qkv(lay, seed_base=1)
    ids = oracle.doc_ids_from_cu_seqlens(lay.cu_seqlens(0), 12)
    a = oracle.blockdiag_attn(q, k, v, ids, 0, None, False)
    b = oracle.blockdiag_attn(q, k, v, ids, 0, 0.25, False)
    assert torch.equal(a, b)


@pytest.mark.parametrize("bad", ["gqa_off", "ratio", "shard", "ids"])
def test_argument_errors(bad):
    q = torch.zeros(1, 4, 8, 4)
    k = torch.zeros(1, 2, 8, 4)
    ids = torch.ones(1, 8, dtype=torch.int32)
    kw = dict(seq_start=0, scale=None, enable_gqa=True)
    if bad == "gqa_off":
        kw["enable_gqa"] = False
    elif bad == "ratio":
        k = torch.zeros(1, 3, 8, 4)
    elif bad == "shard":
        kw["seq_start"] = 1
    elif bad == "ids":
        ids = torch.ones(1, 7, dtype=torch.int32)
    with pytest.raises(ValueError):
        oracle.blockdiag_attn(q, k, k, ids, **kw)


# ---- planted mistakes: each must fail at least one pin --------------------------

def _mask_k_lt_q(doc_row, qpos):
    S = doc_row.shape[0]
    kpos = torch.arange(S)
    dq, dk = doc_row[qpos].unsqueeze(1), doc_row.unsqueeze(0)
    return (dq == dk) & (dq != oracle.PAD_DOC_ID) & (kpos.unsqueeze(0) < qpos.unsqueeze(1))


def _mask_no_causal(doc_row, qpos):
    dq, dk = doc_row[qpos].unsqueeze(1), doc_row.unsqueeze(0)
    return (dq == dk) & (dq != oracle.PAD_DOC_ID)


def _mask_no_doc(doc_row, qpos):
    S = doc_row.shape[0]
    kpos = torch.arange(S)
    dq = doc_row[qpos].unsqueeze(1)
    return (dq != oracle.PAD_DOC_ID) & (kpos.unsqueeze(0) <= qpos.unsqueeze(1))


def _mask_pad_attends(doc_row, qpos):
    S = doc_row.shape[0]
    kpos = torch.arange(S)
    dq, dk = doc_row[qpos].unsqueeze(1), doc_row.unsqueeze(0)
    return (dq == dk) & (kpos.unsqueeze(0) <= qpos.unsqueeze(1))


def _swm_no_denominator(scores, mask, vals):
    s = scores.masked_fill(~mask, float("-inf"))
    m = s.max(dim=1, keepdim=True).values
    m = torch.where(mask.any(1, keepdim=True), m, torch.zeros_like(m))
    out = torch.exp(s - m) @ vals
    out[~mask.any(1)] = 0
    return out


# name -> (oracle attribute, factory(original) -> planted replacement)
MUTANTS = {
    "causal_off_by_one": ("allowed_mask", lambda orig: _mask_k_lt_q),
    "no_causality": ("allowed_mask", lambda orig: _mask_no_causal),
    "no_document_equality": ("allowed_mask", lambda orig: _mask_no_doc),
    "padding_attends": ("allowed_mask", lambda orig: _mask_pad_attends),
    "gqa_modulo_mapping": ("kv_head_of", lambda orig: (lambda h, Hq, Hkv: h % Hkv)),
    "dropped_denominator": ("_softmax_weighted_mean", lambda orig: _swm_no_denominator),
    "wrong_sign": ("_softmax_weighted_mean", lambda orig: (lambda s, m, v: orig(-s, m, v))),
    "values_reversed": ("_softmax_weighted_mean", lambda orig: (lambda s, m, v: orig(s, m, v.flip(0)))),
}

WRAPPED = {
    "k_v_swapped": lambda q, k, v, ids, s0, sc, g: _oracle(q, v, k, ids, s0, sc, g),
    "scale_ignored": lambda q, k, v, ids, s0, sc, g: _oracle(q, k, v, ids, s0, 1.0, g),
    "shard_offset_ignored": lambda q, k, v, ids, s0, sc, g: _oracle(q, k, v, ids, 0, sc, g),
    # a falsy test on the scale turns 0 into the default D ** -0.5
    "zero_scale_as_default": lambda q, k, v, ids, s0, sc, g: _oracle(q, k, v, ids, s0, sc or None, g),
}


def _count_failures(attn):
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(attn)
        except (AssertionError, RuntimeError, ValueError, IndexError):
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, factory = MUTANTS[name]
    monkeypatch.setattr(oa, attr, factory(getattr(oa, attr)))
    assert _count_failures(_oracle), f"mutant {name} passed every pin"


@pytest.mark.parametrize("name", sorted(WRAPPED))
def test_wrapped_mistake_is_caught(name):
    assert _count_failures(WRAPPED[name]), f"mutant {name} passed every pin"
