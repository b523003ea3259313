#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--settle-ms T] [--workload dense] [--no-cpu-baseline] [--pass bwd]

One step is the whole hot path on one batch: build the block mask for the
workload's mask, then run the attention forward (both kernels, enqueued on
torch's current stream). Inputs are seeded synthetic tensors resident in HBM
before timing starts. The metric is effective TFLOPS counting only admitted
(unmasked) pairs: 4 * D * pairs * B * H per forward (two products, 2 FLOP per
multiply-add). Prints one JSON line.

Before the W warm-up steps the step runs untimed for --settle-ms (300 by
default): under sustained load the GPU raises its clock over the first ~50 ms
(a cold dense run takes ~547 us a step over steps 5-25 and ~478 us from step
50 on), so timing right after a few warm-up steps would measure that ramp,
not the kernels' steady rate. The K timed steps follow the W warm-up steps.

With --pass bwd the step is the block-mask build plus the backward call
(flexattn_bwd: dQ, then dK/dV) on the forward's O and LSE, counted by the usual
convention as 2.5 times the forward's FLOPs (five products per tile).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU (the published 2.5 PFLOP/s)
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = ["attention_tiled_attn_amd/csrc/attn_fwd_pp.hip",
                  "attention_tiled_attn_amd/csrc/attn_fwd.hip",
                  "attention_tiled_attn_amd/csrc/device_util.h",
                  "attention_tiled_attn_amd/csrc/exp2_poly.h",
                  "attention_tiled_attn_amd/csrc/variants.h",
                  "attention_tiled_attn_amd/csrc/variant_args.h",
                  "attention_tiled_attn_amd/csrc/launch.h"]


def admitted_pairs(wl, doc_ids) -> int:
    """Admitted (query, key) pairs per head, summed over batch rows.

    For the query at position p every mask admits an interval of keys: the
    causal part [0, p] (with a prefix P: [0, max(p, P - 1)]), the window part
    [p - W + 1, inf), the document part the run of positions that carry p's
    label, and the key range [0, Skv - 1]. Their intersection is an interval,
    so each row's count is hi - lo + 1 (or 0)."""
    import numpy as np
    pos = np.arange(wl.Sq, dtype=np.int64) + wl.q_offset
    tot = 0
    for b in range(wl.B):
        lo = np.zeros_like(pos)
        hi = np.full_like(pos, wl.Skv - 1)
        if wl.causal:
            reach = pos if wl.prefix is None else np.maximum(pos, wl.prefix - 1)
            hi = np.minimum(hi, reach)
        if wl.window:
            lo = np.maximum(lo, pos - wl.window + 1)
        if wl.documents:
            lab = np.asarray(doc_ids[b], dtype=np.int64)
            n = lab.size
            starts = np.r_[0, np.flatnonzero(np.diff(lab) != 0) + 1]
            ends = np.r_[starts[1:], n] - 1
            run = np.repeat(np.arange(starts.size), np.diff(np.r_[starts, n]))
            lo = np.maximum(lo, starts[run[pos]])
            hi = np.minimum(hi, ends[run[pos]])
        tot += int(np.maximum(hi - lo + 1, 0).sum())
    return tot


def kernel_sha() -> str:
    """Hash of the forward kernel's sources with comments and blank lines
    dropped, so that it changes with the code, not with its commentary."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [ln.rstrip() for ln in text.splitlines() if ln.strip()]
        h.update("\n".join(lines).encode())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str):
    """HBM bytes per launch of the attention kernel from the committed counter
    summary (lines `kernel_sha: ...` and `hbm_bytes_per_launch: ...`), or None
    when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"attn_fwd_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(("#", "|", " ")):
                k, v = line.split(":", 1)
                fields[k.strip().strip("`-* ")] = v.strip().strip("`")
    if fields.get("kernel_sha") != kernel_sha():
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _host() -> dict:
    """Cores this process may use and the CPU model (from /proc/cpuinfo)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return {"affinity_cpus": n, "cpu_model": model}


def _slice_sample(wl, doc_ids, pair_budget: float):
    """Whole (batch row, query head) slices in order, as many as fit the
    admitted-pair budget (at least one): (batches, heads, pairs)."""
    per_b = [_pairs_in_rows(wl, np.arange(wl.Sq), None if doc_ids is None else doc_ids[b])
             for b in range(wl.B)]
    total = sum(per_b) * wl.H
    if total <= pair_budget:
        return list(range(wl.B)), list(range(wl.H)), total
    n_heads = max(1, min(wl.H, int(pair_budget // max(per_b[0], 1))))
    if n_heads < wl.H:
        return [0], list(range(n_heads)), per_b[0] * n_heads
    n_b = max(1, int(pair_budget // (per_b[0] * wl.H)))
    return list(range(n_b)), list(range(wl.H)), sum(per_b[:n_b]) * wl.H


def _oracle_kwargs(inp) -> dict:
    wl = inp.wl
    return dict(causal=wl.causal, window=wl.window or None, doc_ids=inp.doc_ids,
                alibi_slopes=None if inp.slopes is None else inp.slopes.astype(np.float64),
                softcap=wl.softcap if wl.mod == "softcap" else None, q_offset=wl.q_offset,
                prefix=wl.prefix,
                rel_bias=None if inp.rel_bias is None else inp.rel_bias.astype(np.float64))


def cpu_baseline(inp, pair_budget: float = 4e9):
    """The oracle, as it is, in a pool of host processes (one per usable core,
    at most 16, one BLAS thread each), on whole (batch, head) slices of the
    same workload: the whole workload when its admitted pairs fit the budget,
    else its first slices. Rate in the unit of the GPU metric."""
    from oracle.pool import attention_parallel
    from workload import bf16_values
    wl = inp.wl
    batches, heads, pairs = _slice_sample(wl, inp.doc_ids, pair_budget)
    q, k, v = (bf16_values(t) for t in (inp.q, inp.k, inp.v))
    st = {}
    attention_parallel(q, k, v, wl.scale, heads=heads, batches=batches, stats=st, **_oracle_kwargs(inp))
    dt = st["seconds"]
    whole = len(batches) * len(heads) == wl.B * wl.H
    return {"value": 4.0 * wl.D * pairs / dt / 1e12, "unit": "TFLOPS", "cores": st["workers"],
            "kind": "oracle", **_host(),
            "sample": (f"{'the whole workload' if whole else 'a bounded sample'}: "
                       f"{len(batches) * len(heads)} of {wl.B * wl.H} (batch, head) slices, "
                       f"{pairs} admitted pairs; fp64 numpy oracle in {st['workers']} processes "
                       f"(1 BLAS thread each, {st['tasks']} row blocks), {dt:.1f} s wall")}


def cpu_baseline_bwd(inp, dout, pair_budget: float = 1e9):
    """The oracle's gradients, as they are, per (batch, query head) slice in
    a pool of host processes, on whole slices of the same workload up to the
    pair budget; rate in the unit of the GPU metric (2.5 x the forward FLOPs
    of the admitted pairs done)."""
    from oracle.pool import attention_backward_slices
    from workload import bf16_values
    wl = inp.wl
    batches, heads, pairs = _slice_sample(wl, inp.doc_ids, pair_budget)
    q, k, v, g = (bf16_values(t) for t in (inp.q, inp.k, inp.v, dout))
    st = {}
    attention_backward_slices(q, k, v, g, wl.scale, [(b, h) for b in batches for h in heads], stats=st,
                              **_oracle_kwargs(inp))
    dt = st["seconds"]
    return {"value": 2.5 * 4.0 * wl.D * pairs / dt / 1e12, "unit": "TFLOPS", "cores": st["workers"],
            "kind": "oracle", **_host(),
            "sample": (f"{len(batches) * len(heads)} of {wl.B * wl.H} whole (batch, head) slices, "
                       f"{pairs} admitted pairs; fp64 numpy oracle gradients in {st['workers']} "
                       f"processes (1 BLAS thread each), {dt:.1f} s wall")}


def _pairs_in_rows(wl, rows, doc_row) -> int:
    import oracle
    tot = 0
    keys = np.arange(wl.Skv)
    for r0 in range(0, rows.size, 256):
        r = rows[r0:r0 + 256]
        tot += int(oracle.admitted(r[:, None] + wl.q_offset, keys[None, :], causal=wl.causal,
                                   window=wl.window or None, doc_row=doc_row,
                                   prefix=wl.prefix).sum())
    return tot


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed load before the warm-up steps, so the clock settles")
    ap.add_argument("--workload", default="dense")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pass", dest="which", choices=["fwd", "bwd"], default="fwd",
                    help="time the forward (default) or the backward")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (for counter scaling)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU only; sharding is design-only",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import attention_tiled_attn_amd as fa
    from workload import WORKLOADS, make_inputs

    wl = WORKLOADS[args.workload]
    inp = make_inputs(wl)
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    var = fa.Variant(causal=wl.causal, window=wl.window,
                     doc_ids=torch.from_numpy(inp.doc_ids).to(dev) if inp.doc_ids is not None else None,
                     alibi_slopes=torch.from_numpy(inp.slopes).to(dev) if inp.slopes is not None else None,
                     softcap=wl.softcap if wl.mod == "softcap" else None,
                     q_offset=wl.q_offset, prefix=wl.prefix,
                     rel_bias=torch.from_numpy(inp.rel_bias).to(dev) if inp.rel_bias is not None else None)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    if args.copy_calibration_mb:
        n = args.copy_calibration_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4}), file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)
    bwd = args.which == "bwd"
    if bwd:
        from workload import draw_dout
        if wl.dtype != "bf16":
            print(json.dumps({"error": "the backward takes bf16 inputs"}))
            sys.exit(2)
        dout_cpu = draw_dout(wl.B, wl.H, wl.Sq, wl.D, wl.seed).to(torch.bfloat16)
        dout = dout_cpu.to(dev)
        fa.attention(q, k, v, var, scale=wl.scale, out=out, lse=lse)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        torch.cuda.synchronize()

    splits = workspace = None
    if wl.decode or wl.split:
        splits = fa.flexattn_split_count(wl.B, wl.H, wl.Hkv, wl.Sq, wl.Skv)
        nbytes = fa.flexattn_decode_workspace_bytes(wl.B, wl.H, wl.Hkv, wl.Sq, wl.D, splits)
        workspace = torch.empty(max(nbytes, 4) // 4, dtype=torch.float32, device=dev)

    # A variant with no mask needs no block mask: the kernels take every key
    # tile inside Skv as full without one. Otherwise the step builds it.
    needs_bm = var.mask_kind != 0

    def step(ev=None):
        bm = fa.build_block_mask(var, wl.B, wl.Sq, wl.Skv, dev) if needs_bm else None
        if ev is not None:
            ev[0].record(stream)
        if bwd:
            fa.attention_backward(q, k, v, out, lse, dout, var, scale=wl.scale, block_mask=bm,
                                  dq=dq, dk=dk, dv=dv, delta=delta)
        elif wl.decode or wl.split:
            fa.decode(q, k, v, var, scale=wl.scale, block_mask=bm, out=out, lse=lse,
                      splits=splits, workspace=workspace)
        else:
            fa.attention(q, k, v, var, scale=wl.scale, block_mask=bm, out=out, lse=lse)
        if ev is not None:
            ev[1].record(stream)
        return bm

    settle_steps = 0
    t_end = time.perf_counter() + args.settle_ms * 1e-3
    while time.perf_counter() < t_end:
        for _ in range(4):
            step()
        settle_steps += 4
        torch.cuda.synchronize()      # keep the host within a few steps of the GPU
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kern_ms = [a.elapsed_time(b) for a, b in evs]
    kern_avg_ms = sum(kern_ms) / len(kern_ms)
    ms_per_step = elapsed * 1e3 / args.steps

    pairs = admitted_pairs(wl, inp.doc_ids)            # summed over batch rows
    flop = 4.0 * wl.D * pairs * wl.H                   # per forward
    if bwd:
        flop *= 2.5                                    # per backward, by convention
    value = flop / (ms_per_step * 1e-3) / 1e12
    achieved = flop / (kern_avg_ms * 1e-3) / 1e12

    # tile FLOPs: every computed (128-row half, 128-key) tile counts in full
    bm = fa.build_block_mask(var, wl.B, wl.Sq, wl.Skv, dev)
    torch.cuda.synchronize()
    cnt, lst = bm.counts().cpu(), bm.lists().cpu()
    halves = 0
    for bb in range(cnt.shape[0]):
        for qp in range(cnt.shape[1]):
            e = lst[bb, qp, :int(cnt[bb, qp])]
            halves += int(((e & 1) + ((e >> 2) & 1)).sum())
    halves *= wl.B if bm.struct.num_b == 1 else 1
    tile_flop = 4.0 * wl.D * 128 * 128 * halves * wl.H * (2.5 if bwd else 1.0)

    bytes_alg = (q.numel() + k.numel() + v.numel() + out.numel()) * q.element_size() + lse.numel() * 4
    if bwd:   # also reads dO and O, writes dQ, dK, dV and delta
        bytes_alg += (2 * q.numel() + q.numel() + k.numel() + v.numel()) * q.element_size() + lse.numel() * 4
    traffic = None if bwd else traffic_from_profile(wl.name)
    # where `traffic` comes from: counters taken with rocprofv3 on this same
    # kernel source (matched by kernel_sha), not measured in this run
    traffic_src = f"profiles/attn_fwd_{wl.name}_traffic.md (rocprofv3 FETCH_SIZE + WRITE_SIZE)" if traffic else None
    if wl.decode:
        # HBM-bound: K and V are read once, Q read and O, LSE written once
        roof = {"bound": "hbm", "achieved": round(bytes_alg / (kern_avg_ms * 1e-3) / 1e9, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(bytes_alg / (kern_avg_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "traffic": traffic, "traffic_source": traffic_src, "algorithmic_bytes": bytes_alg,
                "kernel": "attn_fwd_pp_kernel (decode mode) + attn_decode_merge_kernel",
                "splits": splits}
    else:
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "traffic_source": traffic_src, "algorithmic_bytes": bytes_alg,
                "kernel": ("attn_bwd_dq_kernel + attn_bwd_dkdv_kernel" if bwd else
                           "attn_fwd_pp_kernel (split keys) + attn_decode_merge_kernel" if wl.split else
                           "attn_fwd_pp_kernel" if wl.dtype == "bf16" else "attn_fwd_kernel")}
        if wl.split:
            roof["splits"] = splits

    rec = {
        "metric": ("attention bwd effective TFLOPS (2.5x forward unmasked FLOPs), 1 GPU" if bwd else
                   "attention fwd effective TFLOPS (unmasked FLOPs) + % bf16 MFMA peak, 1 GPU"),
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "settle_steps": settle_steps,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "bf16 (fp32 in/out)",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "Hkv": wl.Hkv, "Sq": wl.Sq,
                   "Skv": wl.Skv, "D": wl.D, "causal": wl.causal, "window": wl.window,
                   "documents": wl.documents, "mod": wl.mod, "q_offset": wl.q_offset,
                   "prefix": wl.prefix, "rel_max": wl.rel_max, "seed": wl.seed},
        "pct_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "attn_kernel_ms": round(kern_avg_ms, 4),
        "attn_kernel_ms_min": round(min(kern_ms), 4),
        "tile_tflops": round(tile_flop / (kern_avg_ms * 1e-3) / 1e12, 2),
        "admitted_pairs_per_head": pairs // wl.B,
        "roofline": roof,
        "kernel_sha": kernel_sha(),
        "gpu": torch.cuda.get_device_name(dev),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_bwd(inp, dout_cpu) if bwd else cpu_baseline(inp)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
