"""Seeded synthetic inputs for packed block-causal attention.

This module only draws inputs: document-length layouts of packed rows and
bf16 q/k/v tensors.  It holds none of the arithmetic of the method (no doc-id
construction, no masking, no attention); both the CPU oracle and the HIP path
consume what it returns.

The five named workloads follow the packed-row shapes that the block-diagonal
context-parallel page (nemo_automodel.components.distributed.blockdiag_cp,
package overview and ``cp_blockdiag_sdpa``) is about: documents concatenated
into one row, an optional padding tail, and either the whole row as queries
(cp_size == 1) or one rank's contiguous query shard against all keys.

Recipe (all layouts use ``numpy.random.default_rng(index)``):

* "fill": draw document lengths until their running sum reaches the content
  length C, then shorten the last one so the sum is exactly C.  Padding is the
  tail ``[C, S)`` of the row.
* q, k, v: ``torch.randn(shape, float32, generator=manual_seed(1000*index+j))``
  with j = 0, 1, 2, rounded to bfloat16 (round-to-nearest-even).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

PAD_DOC_ID = -1000


@dataclass
class Layout:
    """Document layout of a packed batch plus the attention problem shape.

    ``doc_lens[b]`` lists the lengths of the documents packed into row b, in
    order from position 0; ``pad[b]`` trailing positions of the row are padding.
    Queries are the ``L`` rows starting at global position ``seq_start``.
    """

    name: str
    index: int
    B: int
    S: int
    L: int
    seq_start: int
    Hq: int
    Hkv: int
    D: int
    doc_lens: list = field(default_factory=list)
    pad: list = field(default_factory=list)
    enable_gqa: bool = True

    @property
    def scale(self) -> float:
        return float(self.D) ** -0.5

    def cu_seqlens(self, b: int) -> np.ndarray:
        """Cumulative document boundaries of row ``b`` (int32, ``[N+1]``).

        This is the packing metadata format the pages take as input
        (``packed_cu_seqlens`` of shape ``[num_documents + 1]``).
        """
        lens = np.asarray(self.doc_lens[b], dtype=np.int64)
        out = np.zeros(len(lens) + 1, dtype=np.int64)
        np.cumsum(lens, out=out[1:])
        return out.astype(np.int32)

    def allowed_pairs(self) -> int:
        """Number of (query, key) pairs the block-causal mask allows.

        Counted from the lengths: a query at offset j inside its document sees
        j + 1 keys; only queries in ``[seq_start, seq_start + L)`` count.
        """
        total = 0
        lo, hi = self.seq_start, self.seq_start + self.L
        for b in range(self.B):
            start = 0
            for n in self.doc_lens[b]:
                a, e = max(start, lo), min(start + n, hi)
                if a < e:
                    # sum over q in [a, e) of (q - start + 1)
                    first, last = a - start + 1, e - start
                    total += (first + last) * (last - first + 1) // 2
                start += n
        return int(total)

    def useful_flops(self) -> int:
        """4 * D * Hq flops per allowed pair: 2*D for q.k and 2*D for p.v."""
        return 4 * self.D * self.Hq * self.allowed_pairs()

    def shapes(self):
        return ((self.B, self.Hq, self.L, self.D),
                (self.B, self.Hkv, self.S, self.D),
                (self.B, self.Hkv, self.S, self.D))


def _fill(draw, content: int) -> list:
    lens, total = [], 0
    while total < content:
        n = int(draw())
        lens.append(n)
        total += n
    if lens:
        lens[-1] -= total - content
    return lens


CONFIG_NAMES = {
    1: "tiny-packed-S256-Hq4-Hkv2-D64",
    2: "packed-row-S8192-Hq32-Hkv8-D128",
    3: "cp-shard-S32768-L4096-at12288-Hq32-Hkv8-D128",
    4: "short-docs-B4-S16384-Hq64-Hkv8-D128",
    5: "long-mixed-S65536-Hq64-Hkv4-D64",
}


def make_layout(index: int) -> Layout:
    """The five named workloads (1-based index)."""
    name = CONFIG_NAMES[index]
    if index == 1:
        return Layout(name, 1, B=1, S=256, L=256, seq_start=0, Hq=4, Hkv=2, D=64,
                      doc_lens=[[100, 60, 80]], pad=[16])
    rng = np.random.default_rng(index)
    if index == 2:
        pad = int(rng.integers(0, 128))
        lens = _fill(lambda: rng.integers(128, 2049), 8192 - pad)
        return Layout(name, 2, B=1, S=8192, L=8192, seq_start=0, Hq=32, Hkv=8, D=128,
                      doc_lens=[lens], pad=[pad])
    if index == 3:
        mu = math.log(1024.0)
        lens = _fill(lambda: min(8192, max(1, round(rng.lognormal(mu, 1.0)))), 32768)
        lay = Layout(name, 3, B=1, S=32768, L=4096, seq_start=12288, Hq=32, Hkv=8,
                     D=128, doc_lens=[lens], pad=[0])
        return lay
    if index == 4:
        lens_rows, pads = [], []
        for _ in range(4):
            pad = int(rng.integers(0, 256))
            lens_rows.append(_fill(lambda: 16 + rng.geometric(1.0 / 497.0) - 1, 16384 - pad))
            pads.append(pad)
        return Layout(name, 4, B=4, S=16384, L=16384, seq_start=0, Hq=64, Hkv=8, D=128,
                      doc_lens=lens_rows, pad=pads)
    if index == 5:
        def draw():
            if rng.random() < 0.8:
                return rng.integers(64, 1025)
            return rng.integers(8192, 24577)
        lens = _fill(draw, 65536)
        return Layout(name, 5, B=1, S=65536, L=65536, seq_start=0, Hq=64, Hkv=4, D=64,
                      doc_lens=[lens], pad=[0])
    raise KeyError(index)


def random_layout(seed: int, B: int, S: int, L: int | None = None, seq_start: int = 0,
                  Hq: int = 4, Hkv: int = 2, D: int = 64, max_doc: int | None = None,
                  max_pad: int = 0, enable_gqa: bool = True) -> Layout:
    """Small random layouts for parity sweeps: uniform lengths in [1, max_doc]."""
    rng = np.random.default_rng(seed)
    L = S - seq_start if L is None else L
    max_doc = max(1, S // 3) if max_doc is None else max_doc
    lens_rows, pads = [], []
    for _ in range(B):
        pad = int(rng.integers(0, max_pad + 1)) if max_pad > 0 else 0
        pad = min(pad, S)
        lens_rows.append(_fill(lambda: rng.integers(1, max_doc + 1), S - pad))
        pads.append(pad)
    return Layout(f"random-{seed}", 0, B=B, S=S, L=L, seq_start=seq_start, Hq=Hq,
                  Hkv=Hkv, D=D, doc_lens=lens_rows, pad=pads, enable_gqa=enable_gqa)


def make_qkv(layout: Layout, seed_base: int | None = None):
    """bf16 q [B,Hq,L,D], k/v [B,Hkv,S,D] on the CPU, i.i.d. N(0,1) then RNE."""
    base = 1000 * layout.index if seed_base is None else seed_base
    out = []
    for j, shape in enumerate(layout.shapes()):
        g = torch.Generator().manual_seed(base + j)
        out.append(torch.randn(shape, dtype=torch.float32, generator=g).to(torch.bfloat16))
    return tuple(out)
