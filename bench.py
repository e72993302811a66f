"""Benchmark of the packed block-causal attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C] [--no-cpu-baseline]

One step = the whole device path over one batch of synthetic packed rows that
is already resident in HBM:
  step preparation for all rows (document ids, run boundaries, tile plan: one
  kernel, one of whose workgroups orders the row tiles) -> block-diagonal
  attention kernel.
The metric is useful TFLOP/s = 4 * D * Hq * allowed_pairs / step time.

Default workload: the packed LLM row (B=1, S=L=8192, Hq=32, Hkv=8, D=128,
uniform[128, 2048] document lengths, 107-token padding tail, seed 2).
Prints ONE JSON line.  The timed steps carry no events (an event record between
two launches costs the queue a few microseconds).  `roofline` describes the
attention kernel alone, timed with HIP events on the stream it is launched on
around K back-to-back launches after the timed steps; `phase_ms` times the
preparation the same way, and for reference the separate per-row boundary calls
and plan call that compute the same outputs.  `traffic` is HBM bytes per launch
from the committed rocprofv3 counter runs, reported only while the kernel
source is unchanged; `backward` times the training path's backward (dq, dk, dv)
on the same workload; `cpu_baseline` times the CPU fp64 oracle on the host cores
over the same workload.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
METRIC = "useful TFLOP/s packed block-causal attention fwd; % of bf16 MFMA peak"
ATTN_SOURCE = os.path.join(ROOT, "packed_sequence_block_amd", "csrc", "attn_fwd.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_traffic.json")


def attn_source_hash() -> str:
    with open(ATTN_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per attention launch from the committed rocprofv3 counter runs,
    or None when they were taken on another kernel source or workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256_16") != attn_source_hash() or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(lay, q, k, v, budget_s: float = 10.0, max_passes: int = 40):
    import torch
    import oracle
    ids = [oracle.doc_ids_from_cu_seqlens(lay.cu_seqlens(b), lay.S)[0] for b in range(lay.B)]
    import numpy as np
    ids = np.stack(ids)
    passes, t0 = 0, time.perf_counter()
    while True:
        oracle.blockdiag_attn(q, k, v, ids, lay.seq_start, None, lay.enable_gqa)
        passes += 1
        el = time.perf_counter() - t0
        if el >= budget_s or passes >= max_passes:
            break
    flops = lay.useful_flops() * passes
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": torch.get_num_threads(),
            "kind": "oracle",
            "sample": f"whole workload x{passes} (all {lay.B} rows, {lay.Hq} heads), {el:.1f} s, fp64 torch-CPU"}


def backward_leg(psb, lib, lay, q, k, v, doc_ids, stream, steps, timed):
    """Training path on the same workload: forward with log-sum-exp, then the backward
    (dq, dk, dv).  Useful flops of the backward are counted as 2.5x the forward's
    (recomputed Q K^T plus the four gradient products, as attention backward is
    conventionally counted), over the same allowed pairs."""
    import torch
    B, Hq, Hkv, L, S, D = lay.B, lay.Hq, lay.Hkv, lay.L, lay.S, lay.D
    g = torch.Generator().manual_seed(77)
    dout = torch.randn((B, Hq, L, D), generator=g).to(torch.bfloat16).to(q.device)
    out, lse, ws = psb.blockdiag_attn_fwd_lse(q, k, v, doc_ids, lay.seq_start, None, lay.enable_gqa)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nb = ws.numel()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    args = (P(q), P(k), P(v), P(out), P(dout), P(lse), P(doc_ids), B, Hq, Hkv, L, S, D, lay.seq_start,
            float(D) ** -0.5, 1 if lay.enable_gqa else 0, P(dq), P(dk), P(dv), P(ws), nb, None, sptr)

    def bwd():
        st = lib.psb_blockdiag_attn_bwd_planned(*args)
        assert st == 0, st

    for _ in range(3):
        bwd()
    torch.cuda.synchronize()
    ms = timed(bwd, max(5, steps // 2))
    flops = 2.5 * lay.useful_flops()
    return {"what": "dq, dk, dv from dout (dq with delta, then dk/dv kernels)", "ms": round(ms, 5),
            "useful_tflops": round(flops / (ms * 1e-3) / 1e12, 3),
            "pct_of_bf16_peak": round(100 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "flop_convention": "2.5 x forward useful flops"}


def window_leg(psb, lib, lay, q, k, v, doc_ids, stream, steps, timed):
    """The same forward with only the keys the shard needs delivered: its own
    [seq_start, seq_start + L) plus the left halo back to the start of the document
    crossing its first row (window start from the library's own kernel)."""
    import torch
    B, Hq, Hkv, L, S, D = lay.B, lay.Hq, lay.Hkv, lay.L, lay.S, lay.D
    w = int(psb.shard_kv_window_start(doc_ids, lay.seq_start, L).min().item())
    kv_len = lay.seq_start + L - w
    kw, vw = k[:, :, w:w + kv_len].contiguous(), v[:, :, w:w + kv_len].contiguous()
    out = torch.empty((B, Hq, L, D), dtype=torch.bfloat16, device=q.device)
    need = psb.workspace_size(B, Hq, Hkv, L, D)
    ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    sptr = ctypes.c_void_p(stream.cuda_stream)
    gqa = 1 if lay.enable_gqa else 0
    assert lib.psb_blockdiag_attn_plan(P(doc_ids), B, Hq, Hkv, L, S, D, lay.seq_start, gqa, P(ws), need, sptr) == 0

    def fwd():
        st = lib.psb_blockdiag_attn_fwd_window_planned(P(q), P(kw), P(vw), P(doc_ids), B, Hq, Hkv, L, S, D, None,
                                                       None, lay.seq_start, w, kv_len, float(D) ** -0.5, gqa,
                                                       P(out), None, P(ws), need, None, sptr)
        assert st == 0, st

    for _ in range(3):
        fwd()
    torch.cuda.synchronize()
    ms = timed(fwd, steps)
    kv_bytes = 2 * B * Hkv * kv_len * D * 2
    return {"what": "forward against the delivered key window (own keys + left halo)", "kv_start": w,
            "keys": kv_len, "of": S, "kv_bytes": kv_bytes, "kv_bytes_whole_row": 2 * B * Hkv * S * D * 2,
            "ms": round(ms, 5), "useful_tflops": round(lay.useful_flops() / (ms * 1e-3) / 1e12, 3)}


def dense_leg(psb, lib, lay, q, k, v, doc_ids, stream, steps, timed):
    """The dense-mask path on the same workload: the per-document mask materialised,
    then attention under that explicit mask (every key tile of every row visited)."""
    import torch
    B, Hq, Hkv, L, S, D = lay.B, lay.Hq, lay.Hkv, lay.L, lay.S, lay.D
    stride = (S + 15) // 16 * 16
    mask = torch.empty((B, L, stride), dtype=torch.bool, device=q.device)
    out = torch.empty((B, Hq, L, D), dtype=torch.bfloat16, device=q.device)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    sptr = ctypes.c_void_p(stream.cuda_stream)

    def build():
        assert lib.psb_blockdiag_dense_mask(P(doc_ids), B, S, lay.seq_start, L, P(mask), stride, sptr) == 0

    def attn():
        st = lib.psb_masked_attn_fwd(P(q), P(k), P(v), P(mask), L * stride, stride, B, Hq, Hkv, L, S, D, None, None,
                                     float(D) ** -0.5, 1 if lay.enable_gqa else 0, P(out), None, sptr)
        assert st == 0, st

    build()
    attn()
    torch.cuda.synchronize()
    n = max(3, steps // 5)
    mask_ms, attn_ms = timed(build, n), timed(attn, n)
    visited = 4.0 * D * Hq * B * L * S
    return {"what": "materialised per-document mask + attention under it", "mask_ms": round(mask_ms, 5),
            "attention_ms": round(attn_ms, 5), "mask_bytes": B * L * stride,
            "useful_tflops": round(lay.useful_flops() / ((mask_ms + attn_ms) * 1e-3) / 1e12, 3),
            "visited_tflops": round(visited / (attn_ms * 1e-3) / 1e12, 3)}


def variants_leg(psb, lay, stream, steps, timed):
    """The boundary variants on the workload's rows: ids from a -1000-padded length table,
    the row layout (padding mask, positions) from real / padded lengths (each document
    padded up to a multiple of 8 tokens), and the document-position check on that layout."""
    import torch
    B, S = lay.B, lay.S
    n = max(len(r) for r in lay.doc_lens)
    real = torch.full((B, n), -1000, dtype=torch.int32)
    padded = torch.full((B, n), -1000, dtype=torch.int32)
    for b, row in enumerate(lay.doc_lens):
        left = S
        for j, d in enumerate(row):
            q = min((int(d) + 7) // 8 * 8, left)
            real[b, j], padded[b, j] = min(int(d), q), q
            left -= q
    real, padded = real.to("cuda"), padded.to("cuda")
    ids = psb.doc_ids_from_seq_lens(real, S)
    mask, pos = psb.unpack_row_layout(real, padded, S)
    keep = (~mask).to(torch.uint8)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    lib = psb.load()
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    sptr = ctypes.c_void_p(stream.cuda_stream)

    def f_ids():
        assert lib.psb_doc_ids_from_seq_lens(P(real), B, n, S, -1000, P(ids), None, sptr) == 0

    def f_unpack():
        assert lib.psb_unpack_row_layout(P(real), P(padded), B, n, S, P(mask), P(pos), None, sptr) == 0

    def f_check():
        assert lib.psb_validate_document_positions(P(keep), P(pos), B, S, P(status), sptr) == 0

    for f in (f_ids, f_unpack, f_check):
        f()
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "unpacked layout breaks the document rule"
    return {"what": "boundary variants on the workload's rows (ms per call)",
            "doc_ids_from_seq_lens": round(timed(f_ids, steps), 5),
            "unpack_row_layout": round(timed(f_unpack, steps), 5),
            "validate_document_positions": round(timed(f_check, steps), 5)}


def dropin_leg(psb, lay, q, k, v, doc_ids, steps):
    """The SDPA drop-in as a model would call it (module code calls the stock
    scaled_dot_product_attention while a packed step is armed): forward, and forward +
    backward through autograd, wall-clock per call including the custom-op dispatch."""
    import torch
    import torch.nn.functional as F
    g = torch.Generator().manual_seed(78)
    dout = torch.randn(q.shape, generator=g).to(torch.bfloat16).to(q.device)
    qg, kg, vg = (t.detach().clone().requires_grad_(True) for t in (q, k, v))
    n = max(3, steps // 5)

    def fwd():
        with torch.no_grad(), psb.packed_documents(doc_ids, lay.seq_start), psb.patched_sdpa():
            return F.scaled_dot_product_attention(q, k, v, is_causal=True, enable_gqa=lay.enable_gqa)

    def fwd_bwd():
        with psb.packed_documents(doc_ids, lay.seq_start), psb.patched_sdpa():
            out = F.scaled_dot_product_attention(qg, kg, vg, is_causal=True, enable_gqa=lay.enable_gqa)
        out.backward(dout)

    res = {}
    for name, fn in (("forward_ms", fwd), ("forward_backward_ms", fwd_bwd)):
        for _ in range(3):  # the first backward also starts autograd's device thread
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        res[name] = round((time.perf_counter() - t0) * 1e3 / n, 5)
    res["what"] = "F.scaled_dot_product_attention swapped for the packed path (custom ops), wall clock"
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the training-path (backward) timing")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-mask path timing")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": n, "bytes_written": n}))
        return
    import packed_sequence_block_amd as psb
    from workloads import make_layout, make_qkv

    lib = psb.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lay = make_layout(args.config)
    q_cpu, k_cpu, v_cpu = make_qkv(lay)
    q, k, v = q_cpu.to(dev), k_cpu.to(dev), v_cpu.to(dev)
    B, Hq, Hkv, L, S, D = lay.B, lay.Hq, lay.Hkv, lay.L, lay.S, lay.D
    cus = [torch.as_tensor(lay.cu_seqlens(b)).to(dev) for b in range(B)]
    doc_ids = torch.empty((B, S), dtype=torch.int32, device=dev)
    seg_cu = torch.empty((B, S + 1), dtype=torch.int32, device=dev)
    seg_n = torch.empty((B,), dtype=torch.int32, device=dev)
    ws_bytes = psb.workspace_size(B, Hq, Hkv, L, D)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, L, D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    sptr = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    scale = float(D) ** -0.5
    gqa = 1 if lay.enable_gqa else 0
    row_ptrs = [(P(cus[b]), cus[b].numel() - 1, ctypes.c_void_p(doc_ids[b].data_ptr()),
                 ctypes.c_void_p(seg_cu[b].data_ptr()), ctypes.c_void_p(seg_n[b:].data_ptr()))
                for b in range(B)]
    qp, kp, vp, dp, op, wp = P(q), P(k), P(v), P(doc_ids), P(out), P(ws)
    # all rows' boundaries as one [B, N + 1] table (shorter rows repeat their last boundary)
    n1 = max(c.numel() for c in cus)
    cu_all = torch.stack([torch.cat([c, c[-1:].expand(n1 - c.numel())]) for c in cus]).to(torch.int32).contiguous()
    cup, segp, segnp = P(cu_all), P(seg_cu), P(seg_n)

    def prepare():
        # the step's ids, run boundaries and plan for all rows: one launch
        st = lib.psb_blockdiag_prepare(cup, n1, n1 - 1, B, Hq, Hkv, L, S, D, lay.seq_start, gqa, dp, segp, segnp,
                                       wp, ws_bytes, None, sptr)
        assert st == 0, st

    def boundary():
        for cu_p, nd, ids_p, scu_p, sn_p in row_ptrs:
            st = lib.psb_doc_ids_from_cu_seqlens(cu_p, nd, S, ids_p, None, sptr)
            assert st == 0, st
            st = lib.psb_segment_cu_seqlens(ids_p, S, scu_p, S + 1, sn_p, sptr)
            assert st == 0, st

    def plan():
        st = lib.psb_blockdiag_attn_plan(dp, B, Hq, Hkv, L, S, D, lay.seq_start, gqa, wp, ws_bytes, sptr)
        assert st == 0, st

    def attention():
        st = lib.psb_blockdiag_attn_fwd_planned(qp, kp, vp, dp, B, Hq, Hkv, L, S, D, None, None, lay.seq_start,
                                                scale, gqa, op, wp, ws_bytes, None, sptr)
        assert st == 0, st

    def step():
        prepare()
        attention()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps

    def timed(fn, n):
        # n back-to-back calls between one pair of events on the launch stream
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for _ in range(n):
            fn()
        a1.record(stream)
        torch.cuda.synchronize(dev)
        return a0.elapsed_time(a1) / n

    attn_ms = timed(attention, args.steps)
    phase_ms = {"prepare": round(timed(prepare, args.steps), 5), "attention": round(attn_ms, 5),
                "separate_calls": {"boundary_per_row": round(timed(boundary, args.steps), 5),
                                   "plan": round(timed(plan, args.steps), 5)}}
    flops = lay.useful_flops()
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (attn_ms * 1e-3) / 1e12
    traffic = measured_traffic(lay.name)
    rec = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": lay.name, "B": B, "S": S, "L": L, "seq_start": lay.seq_start, "Hq": Hq,
                   "Hkv": Hkv, "D": D, "documents": sum(len(r) for r in lay.doc_lens),
                   "allowed_pairs": lay.allowed_pairs(), "useful_gflop_per_step": round(flops / 1e9, 3),
                   "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": "attn_fwd_kernel", "kernel_ms": round(attn_ms, 5)},
        "phase_ms": phase_ms,
    }
    if not args.no_dense:
        rec["dense_mask"] = dense_leg(psb, lib, lay, q, k, v, doc_ids, stream, args.steps, timed)
    rec["boundary_variants"] = variants_leg(psb, lay, stream, args.steps, timed)
    rec["drop_in"] = dropin_leg(psb, lay, q, k, v, doc_ids, args.steps)
    rec["kv_window"] = window_leg(psb, lib, lay, q, k, v, doc_ids, stream, args.steps, timed)
    if not args.no_backward:
        rec["backward"] = backward_leg(psb, lib, lay, q, k, v, doc_ids, stream, args.steps, timed)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(lay, q_cpu, k_cpu, v_cpu)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
