"""A CPU model of the forward kernel's per-row softmax arithmetic, against the oracle.

The forward kernel walks 64-key tiles and keeps, per query row, an exp2 offset nmsc,
a running sum l and an fp32 accumulator o (online softmax in the exp2 domain with
sc = |scale| * log2(e)):
  * masked scores become -inf;
  * e = exp2(s sc + nmsc) (one fused multiply-add) in fp32 for the whole tile, and
    p = e rounded to bf16;
  * if the e held by one lane (half of the tile's keys: key % 8 < 4, or the rest) sum
    to more than 2^8, the offset is retuned: with m the tile's maximum raw score,
    nmsc' = -m sc replaces nmsc wherever it is smaller; l and o are multiplied by
    exp2(nmsc' - nmsc) and the tile's e and p are recomputed;
  * on the first tile, nmsc' = -m sc is taken before any e is made (where smaller than
    nmsc), which is what the retune does there with l and o still 0;
  * nmsc starts at FLT_MAX, so that a row's first finite score in a later tile gives
    p = inf and forces the exact maximum (masked scores still give exp2(-inf) = 0);
  * l adds the fp32 e, o adds the bf16 p times v; the output is o / l (0 when
    l == 0), rounded to bf16.
A negative scale flips the sign of q; sc is held at least at the smallest normal
float, so that scale = 0 gives equal weights instead of exp2(-inf * 0) = NaN on the
masked keys.  This model runs the same steps in numpy float32 (the MFMA dot products
in float32 too, in another summation order) and must meet the oracle's tolerance;
with sc = 0 allowed through it produces NaN, which is why the kernel holds sc up.
(The kernel takes the retune decision for a whole wave of 32 rows at once; a retune
that another row asked for moves this row's offset only when its maximum lies above
it, which is as exact.)
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import make_qkv, random_layout

TILE = 64
RETUNE_SUM = np.float32(256.0)
LOG2E = np.float32(1.4426950408889634)
FLT_MIN = np.float32(np.finfo(np.float32).tiny)
FLT_MAX = np.float32(np.finfo(np.float32).max)


def _bf16(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def _fma32(a, b, c):
    # float32 fused multiply-add: the product of two floats is exact in float64
    return (a.astype(np.float64) * np.float64(b) + np.float64(c)).astype(np.float32)


def model_row(qrow, keys, vals, allowed, scale, clamp=True):
    """One query row: qrow [D], keys / vals [S, D], allowed [S] bool; float32 result [D]."""
    sc = np.float32(abs(scale)) * LOG2E
    if clamp:
        sc = max(sc, FLT_MIN)
    q = -qrow if np.signbit(np.float32(scale)) and scale != 0 else qrow
    s_all = (keys.astype(np.float32) @ q.astype(np.float32)).astype(np.float32)
    nmsc = FLT_MAX
    l = np.float32(0.0)
    o = np.zeros(vals.shape[1], dtype=np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        for t0 in range(0, keys.shape[0], TILE):
            s = np.where(allowed[t0:t0 + TILE], s_all[t0:t0 + TILE], np.float32(-np.inf)).astype(np.float32)
            lane = (np.arange(t0, t0 + len(s)) % 8) < 4
            if t0 == 0:
                nm = np.float32(-np.float32(s.max()) * sc)
                nmsc = nm if nm < nmsc else nmsc
            e = np.exp2(_fma32(s, sc, nmsc)).astype(np.float32)
            if e[lane].sum(dtype=np.float32) > RETUNE_SUM or e[~lane].sum(dtype=np.float32) > RETUNE_SUM:
                nm = np.float32(-np.float32(s.max()) * sc)
                if nm < nmsc:
                    alpha = np.float32(np.exp2(np.float32(nm - nmsc)))
                    nmsc = nm
                    l = np.float32(l * alpha)
                    o = (o * alpha).astype(np.float32)
                e = np.exp2(_fma32(s, sc, nmsc)).astype(np.float32)
            p = _bf16(e)
            l = np.float32(l + e.sum(dtype=np.float32))
            o = (o + p @ vals[t0:t0 + TILE].astype(np.float32)).astype(np.float32)
    inv = np.float32(1.0) / l if l > 0 else np.float32(0.0)
    return _bf16(o * inv)


def model_attn(q, k, v, ids, seq_start, scale, clamp=True):
    B, Hq, L, D = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    qf, kf, vf = (t.float().numpy() for t in (q, k, v))
    out = np.zeros((B, Hq, L, D), dtype=np.float32)
    for b in range(B):
        qpos = torch.arange(seq_start, seq_start + L)
        mask = oracle.allowed_mask(torch.as_tensor(ids[b]).long(), qpos).numpy()
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for i in range(L):
                out[b, h, i] = model_row(qf[b, h, i], kf[b, g], vf[b, g], mask[i], scale, clamp)
    return out


def _case(seed):
    lay = random_layout(seed, B=1, S=300, L=200, seq_start=100, Hq=2, Hkv=1, D=16, max_doc=130, max_pad=25)
    q, k, v = make_qkv(lay, seed_base=6100 + seed)
    ids = np.stack([oracle.doc_ids_from_cu_seqlens(lay.cu_seqlens(b), lay.S)[0] for b in range(lay.B)])
    return lay, q, k, v, ids


@pytest.mark.parametrize("scale", [0.25, 0.37, -0.2, 3.0, 0.0, -0.0])
def test_model_meets_oracle(scale):
    lay, q, k, v, ids = _case(3)
    got = model_attn(q, k, v, ids, lay.seq_start, scale)
    ref = oracle.blockdiag_attn(q, k, v, ids, lay.seq_start, scale, True).numpy()
    assert np.isfinite(got).all()
    d = np.abs(got - ref)
    assert d.max() <= 2e-2 and d.mean() <= 2e-3, (d.max(), d.mean())
    pad = ids[0, lay.seq_start:lay.seq_start + lay.L] == oracle.PAD_DOC_ID
    assert pad.any() and np.all(got[:, :, pad] == 0)


def test_first_key_sets_the_offset():
    # every score far below zero: an offset that started at 0 would underflow every p
    # (exp2(-720) = 0) and return zeros; the FLT_MAX start forces the exact maximum first
    rng = np.random.default_rng(5)
    S, D = 150, 16
    qrow = np.full(D, 4.0, dtype=np.float32)
    keys = np.full((S, D), -8.0, dtype=np.float32)  # q.k = -512 for every key
    vals = _bf16(rng.standard_normal((S, D)))
    allowed = np.zeros(S, dtype=bool)
    allowed[70:131] = True  # the first allowed key sits in the second tile
    got = model_row(qrow, keys, vals, allowed, 1.0)
    ref = _bf16(vals[allowed].mean(axis=0))
    assert np.abs(got - ref).max() <= 2e-2


def test_zero_scale_weights_are_exactly_one():
    # the exp2 arguments at sc = FLT_MIN are tiny: every allowed weight is bf16 1.0
    s = np.asarray([-300.0, -1.0, 0.0, 2.5, 900.0], dtype=np.float32)
    m = np.float32(900.0)
    p = _bf16(np.exp2(_fma32(s, FLT_MIN, np.float32(-m * FLT_MIN))))
    assert np.all(p == 1.0)
    masked = _bf16(np.exp2(_fma32(np.asarray([-np.inf], dtype=np.float32), FLT_MIN, np.float32(-m * FLT_MIN))))
    assert masked[0] == 0.0


def test_unclamped_zero_scale_gives_nan():
    lay, q, k, v, ids = _case(4)
    got = model_attn(q[:, :, :40], k, v, ids, lay.seq_start, 0.0, clamp=False)
    assert np.isnan(got).any()
