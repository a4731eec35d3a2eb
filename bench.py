#!/usr/bin/env python3
"""Benchmark of one device's share of ring attention on one MI355X.

A step is one pass of the whole path over one batch of synthetic input that
is already resident in HBM:
  * prefill workloads: the device's query chunk against every KV chunk in
    ring order, each received chunk staged through the double buffer on the
    side stream (RA_FLAG_STAGE), causal chunks skipped/masked, output and
    normalisation fused;
  * decode workloads: split-KV partials over the cache, then the merge.

Prints ONE JSON line.  `value` is the headline workload's algorithmic
TFLOP/s (unmasked query-key pairs x 4 x d per head, no dense-tile flops).
`roofline` prices the dominant kernel against the bf16 MFMA peak (prefill)
or HBM bandwidth (decode) with its average launch time from HIP events on the
launch stream; `cpu_baseline` times the CPU oracle on a bounded row sample of
the same workload.  `secondary` holds the other workloads timed in the run.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--secondary NAMES]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published peaks
PEAK_BF16_TFLOPS = 2516.6  # dense bf16 MFMA, 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0

# HBM bytes per launch of each workload's dominant kernel (for the backward:
# per step, summed over its bwd_pre, bwd_dq and bwd_dkdv launches), from rocprofv3
# --pmc FETCH_SIZE and WRITE_SIZE runs of this script, scaled by what the same
# counters read for a plain 1 GiB elementwise copy (--copy-calibration):
# FETCH_SIZE x 2.000, WRITE_SIZE x 1.000.  Valid only for the kernel sources
# they were taken on; any change to them voids the figures (traffic -> null).
KERNEL_SOURCES = ("long_context_blockwise_amd/csrc/attn_fwd_bf16.hip", "long_context_blockwise_amd/csrc/attn_bwd_bf16.hip",
                  "long_context_blockwise_amd/csrc/tile_common.h", "long_context_blockwise_amd/csrc/ra_internal.h",
                  "long_context_blockwise_amd/csrc/ring_attn.cpp", "long_context_blockwise_amd/csrc/merge.hip")
MEASURED_TRAFFIC = {
    "digest": "2f121dd3a9a8dce6",
    "prefill_bf16_h32_d128": 5.8531e8,
    "decode_b4_gqa32x8_cache1m": 1.7250e10,
    "decode_b4_gqa32x8_cache1m_fp8": 8.6614e9,
    "bwd:prefill_bf16_h32_d128": 8.2409e9,
    "local_w4096_s4096_h32_d128": 8.4241e8,
    "docs4096_h32_d128": 2.0920e8,
    "bwd:docs4096_h32_d128": 2.9350e9,
}

HEADLINE = "prefill_bf16_h32_d128"
SECONDARY = ("decode_b4_gqa32x8_cache1m,decode_b4_gqa32x8_cache1m_fp8,bwd:prefill_bf16_h32_d128,"
             "local_w4096_s4096_h32_d128,docs4096_h32_d128,bwd:docs4096_h32_d128")


def visible_pairs_per_head(wl, rows=None):
    """Unmasked (query, key) pairs of one (batch, head) for the given rows."""
    rows = range(wl.Lq) if rows is None else rows
    total = 0
    for start, n in zip(wl.starts(), wl.lens()):
        for r in rows:
            pos = wl.q_offset + r
            if not wl.causal:
                total += n
            else:
                total += max(0, min(n, pos - start + 1))
    return total


def visible_pairs_fast(wl):
    """Same as visible_pairs_per_head over all rows, in closed form."""
    total = 0
    for start, n in zip(wl.starts(), wl.lens()):
        if not wl.causal:
            total += n * wl.Lq
            continue
        for_lo = wl.q_offset - start + 1  # visible keys of row 0 (unclipped)
        # sum over r of clip(for_lo + r, 0, n)
        r_full = max(0, min(wl.Lq, n - for_lo))  # rows with for_lo + r < n
        acc = 0
        # rows 0..r_full-1 contribute max(0, for_lo + r)
        lo = max(0, -for_lo + 1) if for_lo <= 0 else 0
        lo = min(lo, r_full)
        if r_full > lo:
            a, b = for_lo + lo, for_lo + r_full - 1
            acc += (a + b) * (r_full - lo) // 2
        acc += (wl.Lq - r_full) * n
        total += acc
    return total


def masked(wl):
    return bool(wl.window or wl.anchor or wl.doc_mean)


def visible_pairs(wl, rows=None):
    """Unmasked (query, key) pairs of one query head, summed over batches,
    for the given rows (default all).  A key at position k is visible to the
    query at p when it carries p's segment label (packed documents) and
    either is one of p's anchors (A - 1, A, A + S with A = S floor(p / S))
    or passes the causal rule (k <= p) and the window (|p - k| <= W)."""
    if not masked(wl):
        per = visible_pairs_fast(wl) if rows is None else visible_pairs_per_head(wl, rows)
        return per * wl.B
    import numpy as np

    from long_context_blockwise_amd import inputs

    rows = np.arange(wl.Lq, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    N = sum(wl.lens())  # chunks are contiguous: key position = index over all chunks
    p = wl.q_offset + rows
    W, S = wl.window, wl.anchor
    lo = np.maximum(0, p - W) if W else np.zeros_like(p)
    if wl.causal:
        hi = np.minimum(p, N - 1)
    else:
        hi = np.minimum(p + W, N - 1) if W else np.full_like(p, N - 1)
    q_seg, k_segs = inputs.segment_labels(wl)
    total = 0
    for b in range(wl.B):
        if q_seg is not None:  # packed documents: labels never decrease along the sequence
            lab = np.concatenate([k[b].numpy() for k in k_segs])
            ql = q_seg[b].numpy()[rows]
            first, last = np.searchsorted(lab, ql, "left"), np.searchsorted(lab, ql, "right")
        else:
            first, last = np.zeros_like(p), np.full_like(p, N)
        cnt = np.maximum(0, np.minimum(hi, last - 1) - np.maximum(lo, first) + 1)
        if S:
            A = p // S * S
            for k in (A - 1, A, A + S):
                cnt = cnt + ((k >= 0) & (k < N) & (k >= first) & (k < last) & ~((k >= lo) & (k <= hi)))
        total += int(cnt.sum())
    return total


def kernel_digest():
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(name):
    """HBM bytes per launch measured on the current kernel sources, else None."""
    if name not in MEASURED_TRAFFIC or kernel_digest() != MEASURED_TRAFFIC["digest"]:
        return None
    return MEASURED_TRAFFIC[name]


def algorithmic(wl):
    pairs = visible_pairs(wl) * wl.Hq
    flops = pairs * 2 * (wl.d_qk + wl.d_v)
    es = 2 if wl.dtype == "bf16" else 4
    if wl.kv_dtype == "fp8":  # 1-byte codes plus one exponent byte per 64 tokens for K and for V
        nblk = sum((n + 63) // 64 for n in wl.lens())
        kv_bytes = sum(wl.lens()) * wl.B * wl.Hkv * (wl.d_qk + wl.d_v) + nblk * wl.B * wl.Hkv * 2
    else:
        kv_bytes = sum(wl.lens()) * wl.B * wl.Hkv * (wl.d_qk + wl.d_v) * es
    qo_bytes = wl.B * wl.Lq * wl.Hq * (wl.d_qk + wl.d_v) * es
    return flops, kv_bytes + qo_bytes


class WorkloadRun:
    """Inputs resident on the GPU plus the exact call bench.py times."""

    def __init__(self, name, device="cuda:0"):
        import torch

        from long_context_blockwise_amd import inputs
        import long_context_blockwise_amd as ra

        self.ra = ra
        self.torch = torch
        self.wl = inputs.WORKLOADS[name]
        wl = self.wl
        self.decode = wl.Lq <= 16
        self.x = inputs.make(wl, device)
        if self.decode:
            self.order = list(range(wl.P))
            self.flags = 0  # split-KV + merge
        else:
            dev_index = wl.q_offset // wl.chunk_len  # this device's chunk index
            self.order = ra.ring_attn_ring_order(dev_index, wl.P)
            self.flags = ra.RA_FLAG_STAGE
        self.chunks = self.x.chunks(self.order)
        q_seg, k_segs = inputs.segment_labels(wl, device)
        # local window, anchors and segment labels of the workload (if any)
        self.masks = dict(window=wl.window, anchor=wl.anchor, q_seg=q_seg,
                          k_segs=None if k_segs is None else [k_segs[c] for c in self.order])
        self.out = torch.empty((wl.B, wl.Lq, wl.Hq, wl.d_v), device=device, dtype=wl.torch_dtype)
        ws = ra.ring_attn_workspace_size(self.x.q, self.chunks, wl.causal, wl.q_offset, self.flags, **self.masks)
        self.ws = torch.empty(max(ws, 1), device=device, dtype=torch.uint8)
        self.ctx = ra.RingAttnContext(torch.device(device).index or 0)
        cls = ra.ring_attn_plan(wl.Lq, wl.q_offset, wl.causal, [c[2] for c in self.chunks],
                                [c[0].shape[1] for c in self.chunks], window=wl.window, anchor=wl.anchor)
        computed = sum(1 for c in cls if c != ra.RA_CHUNK_SKIP)
        # kernel launches of the dominant kernel per step
        self.launches = 1 if self.decode else computed
        self.flops, self.bytes = algorithmic(wl)

    def step(self):
        self.ra.ring_attn_fwd(self.x.q, self.chunks, self.wl.causal, self.wl.q_offset,
                              flags=self.flags, out=self.out, ctx=self.ctx, workspace=self.ws, **self.masks)

    def time(self, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            ev[i][0].record()
            self.step()
            ev[i][1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ev_ms = [a.elapsed_time(b) for (a, b) in ev]
        return wall / steps, sum(ev_ms) / len(ev_ms)

    def result(self, sec_per_step, ev_ms):
        wl = self.wl
        tflops = self.flops / sec_per_step / 1e12
        gbs = self.bytes / sec_per_step / 1e9
        launch_s = ev_ms / 1e3 / self.launches
        if self.decode:
            achieved = self.bytes / self.launches / launch_s / 1e9
            roof = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                        frac=round(achieved / PEAK_HBM_GBS, 4), traffic=measured_traffic(wl.name))
            metric, value, unit = "decode HBM GB/s at 1M KV", gbs, "GB/s"
            if wl.kv_dtype == "fp8":
                metric = "decode HBM GB/s at 1M KV (8-bit KV cache)"
        else:
            achieved = self.flops / self.launches / launch_s / 1e12
            peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_TFLOPS
            roof = dict(bound="mfma", achieved=round(achieved, 1), peak=peak, unit="TFLOP/s",
                        frac=round(achieved / peak, 4), traffic=measured_traffic(wl.name))
            metric, value, unit = "causal attn fwd TFLOP/s (% MFMA peak) per GPU", tflops, "TFLOP/s"
            if wl.window or wl.anchor:
                metric = "local-window + anchor attn fwd TFLOP/s over visible pairs per GPU"
            elif wl.doc_mean:
                metric = "packed-document attn fwd TFLOP/s over visible pairs per GPU"
        return dict(workload=wl.name, metric=metric, value=round(value, 2), unit=unit,
                    ms_per_step=round(sec_per_step * 1e3, 4),
                    tokens_per_s=round(wl.B * wl.Lq / sec_per_step, 1),
                    tflops=round(tflops, 2), gbs=round(gbs, 1),
                    launches_per_step=self.launches, roofline=roof)


class BackwardRun(WorkloadRun):
    """The gradients (dQ, dK, dV) of a prefill workload's ring share: one
    ring_attn_bwd call over all chunks in ring order (in place), with the
    forward's output, state and a seeded output gradient resident."""

    def __init__(self, name, device="cuda:0"):
        super().__init__(name, device)
        torch, ra, wl = self.torch, self.ra, self.wl
        from long_context_blockwise_amd import inputs

        self.out, self.state = ra.ring_attn_fwd(self.x.q, self.chunks, wl.causal, wl.q_offset,
                                                flags=ra.RA_FLAG_NO_SPLIT_KV, want_state=True, ctx=self.ctx,
                                                **self.masks)
        self.dout = inputs.output_grad(wl, device)
        self.dq = torch.empty((wl.B, wl.Lq, wl.Hq, wl.d_qk), device=device, dtype=torch.float32)
        self.grads = [(torch.empty(c[0].shape, device=device, dtype=torch.float32),
                       torch.empty(c[1].shape, device=device, dtype=torch.float32)) for c in self.chunks]
        bws = ra.ring_attn_bwd_workspace_size(self.x.q, self.chunks, window=wl.window, anchor=wl.anchor)
        self.bws = torch.empty(max(bws, 1), device=device, dtype=torch.uint8)
        pairs = visible_pairs(wl) * wl.Hq
        # S = QK^T, dP = dO V^T, dV = P^T dO, dQ = dS K, dK = dS^T Q per visible pair
        self.flops = pairs * 2 * (3 * wl.d_qk + 2 * wl.d_v)
        torch.cuda.synchronize()

    def step(self):
        self.ra.ring_attn_bwd(self.x.q, self.chunks, self.out, self.dout, self.state, self.wl.causal,
                              self.wl.q_offset, dq=self.dq, grads=self.grads, ctx=self.ctx, workspace=self.bws,
                              **self.masks)

    def result(self, sec_per_step, ev_ms):
        wl = self.wl
        tflops = self.flops / sec_per_step / 1e12
        achieved = self.flops / (ev_ms / 1e3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / PEAK_BF16_TFLOPS, 4), traffic=measured_traffic("bwd:" + wl.name),
                    kernels="bwd_pre + bwd_dq + bwd_dkdv per step (traffic: per step)")
        metric = "causal attn bwd TFLOP/s (dQ, dK, dV) per GPU"
        if wl.doc_mean:
            metric = "packed-document attn bwd TFLOP/s (dQ, dK, dV) over visible pairs per GPU"
        elif wl.window or wl.anchor:
            metric = "local-window + anchor attn bwd TFLOP/s (dQ, dK, dV) over visible pairs per GPU"
        return dict(workload="bwd:" + wl.name, metric=metric,
                    value=round(tflops, 2), unit="TFLOP/s", ms_per_step=round(sec_per_step * 1e3, 4),
                    tokens_per_s=round(wl.B * wl.Lq / sec_per_step, 1), tflops=round(tflops, 2),
                    launches_per_step=2 + len(self.chunks), roofline=roof)


def cpu_baseline(name, budget_s=20.0):
    """Time the CPU oracle on a bounded, stratified row sample of a workload
    (all heads and batches of the sampled rows) and scale to TFLOP/s."""
    import numpy as np

    import oracle
    from long_context_blockwise_amd import inputs

    wl = inputs.WORKLOADS[name]
    x = inputs.make(wl, "cpu")
    chunks = x.chunks()
    rows_all = inputs.sample_rows(wl.Lq, tile=max(1, wl.Lq // 2048), seed=1)
    rng = np.random.default_rng(0)
    rng.shuffle(rows_all)
    n, spent, done_rows, t_total = 1, 0.0, [], 0.0
    while spent < budget_s / 2 and len(done_rows) < len(rows_all):
        rows = sorted(rows_all[len(done_rows):len(done_rows) + n])
        t0 = time.perf_counter()
        oracle.attention(x.q, chunks, wl.q_offset, wl.causal, rows=rows)
        dt = time.perf_counter() - t0
        done_rows += rows
        t_total += dt
        spent += dt
        n *= 2
    pairs = visible_pairs(wl, done_rows) * wl.Hq
    flops = pairs * 2 * (wl.d_qk + wl.d_v)
    return dict(value=round(flops / t_total / 1e12, 6), unit="TFLOP/s", cores=oracle.threads(),
                kind="oracle",
                sample=f"{len(done_rows)} of {wl.Lq} query rows (all {wl.B}x{wl.Hq} batch-heads) of "
                       f"{wl.name}, fp64 C oracle, {t_total:.1f} s, {flops / 1e9:.1f} GFLOP")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--secondary", default=SECONDARY, help="comma list, '' for none")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run one plain elementwise copy of BYTES bytes (reads BYTES, writes "
                         "BYTES) to calibrate the FETCH_SIZE / WRITE_SIZE counters, then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one device's ring share on one GPU; --gpus must be 1 "
              "(the multi-GPU ring is not part of this build)", file=sys.stderr)
        sys.exit(2)

    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        n = args.copy_calibration // 4
        src = torch.ones(n, device="cuda:0", dtype=torch.float32)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4}), flush=True)
        return
    props = torch.cuda.get_device_properties(0)
    run = WorkloadRun(args.workload)
    sec, ev_ms = run.time(args.steps, args.warmup)
    head = run.result(sec, ev_ms)
    print(f"[bench] {head}", file=sys.stderr, flush=True)
    del run
    torch.cuda.empty_cache()

    secondary = []
    for name in [s for s in args.secondary.split(",") if s and s != args.workload]:
        r = BackwardRun(name[4:]) if name.startswith("bwd:") else WorkloadRun(name)
        s2, e2 = r.time(max(3, args.steps // 2), max(1, args.warmup))
        res = r.result(s2, e2)
        print(f"[bench] {res}", file=sys.stderr, flush=True)
        secondary.append(res)
        del r
        torch.cuda.empty_cache()

    cpu = None if args.no_cpu else cpu_baseline(args.workload)
    wl = head
    from long_context_blockwise_amd import inputs

    w = inputs.WORKLOADS[args.workload]
    line = {
        "metric": head["metric"],
        "value": head["value"],
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "fp32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d_qk,
                   "chunk_len": w.chunk_len, "P": w.P, "Lq": w.Lq, "q_offset": w.q_offset,
                   "causal": w.causal, "tokens_per_s": head["tokens_per_s"],
                   "gpu": props.name, "cus": props.multi_processor_count},
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
