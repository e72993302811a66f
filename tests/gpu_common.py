"""Helpers for the GPU parity tests (HIP path vs the CPU oracle)."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

MAX_ABS = 2e-2   # attention tolerance for bf16 inputs: max |gpu - oracle| over all outputs
MEAN_ABS = 2e-3  # and mean |gpu - oracle|


def say(*a):
    """Names the case before a GPU step (flushed, so a fault still leaves a trace)."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def oracle_doc_ids(layout) -> np.ndarray:
    return np.stack([oracle.doc_ids_from_cu_seqlens(layout.cu_seqlens(b), layout.S)[0]
                     for b in range(layout.B)])


def compare(gpu_out: torch.Tensor, ref: torch.Tensor, pad_rows=None, what=""):
    """Element-wise comparison at the stated tolerances; padding rows must be exactly 0."""
    g = gpu_out.detach().to("cpu").to(torch.float64)
    r = torch.as_tensor(ref).to(torch.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert torch.isfinite(g).all(), f"{what}: non-finite output"
    diff = (g - r).abs()
    mx = diff.max().item() if diff.numel() else 0.0
    mean = diff.mean().item() if diff.numel() else 0.0
    assert mx <= MAX_ABS, f"{what}: max abs err {mx:.3e} > {MAX_ABS}"
    assert mean <= MEAN_ABS, f"{what}: mean abs err {mean:.3e} > {MEAN_ABS}"
    if pad_rows is not None:
        sel = g[pad_rows]
        assert torch.all(sel == 0), f"{what}: padding rows not exactly zero"
    return mx, mean
