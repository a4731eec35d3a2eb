#!/usr/bin/env python3
"""Benchmark of one device's share of ring attention on one MI355X.

A step is one pass of the whole path over one batch of synthetic input that
is already resident in HBM:
  * prefill workloads: the device's query chunk against every KV chunk in
    ring order, each received chunk staged through the double buffer on the
    side stream (RA_FLAG_STAGE), causal chunks skipped/masked, output and
    normalisation fused.  ``inplace:NAME`` runs the same share with every
    chunk read where it lies (no staging; chunks of one length share a
    launch), which prices the ring stand-in;
  * decode workloads: split-KV partials over the cache, then the merge;
  * ``bwd:NAME``: the gradients (dQ, dK, dV) of a prefill share.

The headline is the 1M-token ring share (32 query / 8 KV heads, d=128, the
last of 32 chunks of 32768 tokens, causal): the largest single-GPU prefill
configuration.  Prints ONE JSON line.  `value` is its algorithmic TFLOP/s
(unmasked query-key pairs x 2 (d_qk + d_v) per head; no dense-tile flops).
`roofline` prices the dominant kernel against the bf16 MFMA peak (prefill)
or HBM bandwidth (decode) with its average launch time from HIP events on
the launch stream; `cpu_baseline` times the CPU oracle on a bounded,
stratified row sample of the same workload; `secondary` holds the other
workloads timed in the run; `run_info` records the board clock sampled
during the headline's timed steps, the host CPU and the source digest.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--secondary NAMES]
    python bench.py --profile NAMES [--profile-out DIR]   # rocprofv3 harness

``--profile`` runs this script under rocprofv3 once per pass (kernel trace;
two counter groups for the matrix and vector pipes; FETCH_SIZE; WRITE_SIZE;
the same two for a plain copy that calibrates them) and writes one summary
per workload: MFMA utilisation and VALU activity for prefill, achieved HBM
bytes and GB/s for decode, each against the chip's published peaks.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import shlex
import statistics
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published peaks
PEAK_BF16_TFLOPS = 2516.6  # dense bf16 MFMA, 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_FP32_TFLOPS = 157.3   # fp32 vector
PEAK_HBM_GBS = 8000.0
N_CU, N_SIMD, N_XCD = 256, 1024, 8

# HBM bytes per launch of each workload's dominant kernel (for the backward:
# per step, summed over its bwd_pre, bwd_dq and bwd_dkdv launches), from rocprofv3
# --pmc FETCH_SIZE and WRITE_SIZE runs of this script (--profile), scaled by
# what the same counters read for a plain 1 GiB elementwise copy.  Valid only
# for the kernel sources they were taken on; any change to them voids the
# figures (traffic -> null).
KERNEL_SOURCES = ("long_context_blockwise_amd/csrc/attn_fwd_bf16.hip", "long_context_blockwise_amd/csrc/attn_bwd_bf16.hip",
                  "long_context_blockwise_amd/csrc/tile_common.h", "long_context_blockwise_amd/csrc/ra_internal.h",
                  "long_context_blockwise_amd/csrc/ring_attn.cpp", "long_context_blockwise_amd/csrc/merge.hip")
MEASURED_TRAFFIC = {
    "digest": "e2e31f289d21efb3",
    "ring_1m_gqa32x8_d128": 3518201363,
    "prefill_bf16_h32_d128": 600605906,
    "mla_h16_d512": 4261628265,
    "decode_b4_gqa32x8_cache1m": 17250013029,
    "decode_b4_gqa32x8_cache1m_fp8": 8661515163,
    "decode_b4_gqa32x8_cache1m_bhsd": 17250147298,
    "decode_b4_gqa32x8_cache1m_fp8_bhsd": 8661657975,
    "local_w4096_s4096_h32_d128": 947904156,
    "docs4096_h32_d128": 190502846,
    "bwd:prefill_bf16_h32_d128": 10444776712,
    "bwd:mla_h16_d512": 109414190501,
}

HEADLINE = "ring_1m_gqa32x8_d128"
# minimum GPU time of each secondary workload's warmup and of its timed steps
SECONDARY_WARMUP_S = 0.3
SECONDARY_TIMED_S = 0.2
# minimum GPU time of the warmup before the profiled (timed) steps
PROFILE_WARMUP_S = 0.3
SECONDARY = ("prefill_bf16_h32_d128,mla_h16_d512,decode_b4_gqa32x8_cache1m,decode_b4_gqa32x8_cache1m_fp8,"
             "tiny_ring_fp32,bwd:prefill_bf16_h32_d128,inplace:prefill_bf16_h32_d128,inplace:ring_1m_gqa32x8_d128,"
             "local_w4096_s4096_h32_d128,docs4096_h32_d128,bwd:docs4096_h32_d128,bwd:mla_h16_d512,"
             "decode_b4_gqa32x8_cache1m_bhsd,decode_b4_gqa32x8_cache1m_fp8_bhsd")


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


def _digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def kernel_digest():
    return _digest(KERNEL_SOURCES)


def source_digest():
    """Digest of everything the timed path runs: kernels, host runtime, header,
    binding and this script (the tree that runs carries no git metadata)."""
    files = sorted(glob.glob(os.path.join(ROOT, "long_context_blockwise_amd", "csrc", "*")))
    files = [os.path.relpath(f, ROOT) for f in files]
    files += ["include/ring_attn.h", "long_context_blockwise_amd/ring_attn.py", "long_context_blockwise_amd/inputs.py",
              "bench.py"]
    return _digest(files)


def git_revision():
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "--short=12", "HEAD"], capture_output=True, text=True,
                           timeout=10)
        return r.stdout.strip() or None if r.returncode == 0 else None
    except (OSError, subprocess.SubprocessError):
        return None


def measured_traffic(name):
    """HBM bytes per launch measured on the current kernel sources, else None."""
    if name not in MEASURED_TRAFFIC or kernel_digest() != MEASURED_TRAFFIC["digest"]:
        return None
    return MEASURED_TRAFFIC[name]


def host_cpu():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def sample_sclk_mhz():
    """Current shader clock of GPU 0 in MHz as amd-smi reports it (mean over
    the XCDs it lists), or None.  Runs amd-smi as a child process."""
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "--clock", "--json"], capture_output=True, text=True,
                           timeout=30)
    except (OSError, subprocess.SubprocessError):
        return None
    if r.returncode != 0:
        return None
    try:
        data = json.loads(r.stdout)
    except ValueError:
        return None
    vals = []

    def walk(x, key=""):
        if isinstance(x, dict):
            if key.lower().startswith("gfx") and "clk" in x:
                v = x["clk"]
                v = v.get("value") if isinstance(v, dict) else v
                try:
                    vals.append(float(v))
                except (TypeError, ValueError):
                    pass
                return
            for k, v in x.items():
                walk(v, str(k))
        elif isinstance(x, list):
            for v in x:
                walk(v, key)
    walk(data)
    return round(sum(vals) / len(vals), 1) if vals else None


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

    def __init__(self, name, device="cuda:0", inplace=False):
        import torch

        from long_context_blockwise_amd import inputs
        import long_context_blockwise_amd as ra

        self.ra = ra
        self.torch = torch
        self.wl = inputs.WORKLOADS[name]
        self.label = ("inplace:" if inplace else "") + name
        wl = self.wl
        self.decode = wl.Lq <= 16
        self.x = inputs.make(wl, device)
        if self.decode:
            self.order = list(range(wl.P))
            self.flags = 0  # split-KV + merge
        else:
            dev_index = wl.q_offset // wl.chunk_len  # this device's chunk index
            self.order = ra.ring_attn_ring_order(dev_index, wl.P)
            self.flags = ra.RA_FLAG_NO_SPLIT_KV if inplace else ra.RA_FLAG_STAGE
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
        computed = [c for c, k in zip(self.chunks, cls) if k != ra.RA_CHUNK_SKIP]
        # kernel launches of the dominant kernel per step: one per computed
        # chunk when staged; in place, chunks of one length share a launch
        if self.decode:
            self.launches = 1
        elif inplace:
            self.launches = len({c[0].shape[1] for c in computed}) if computed else 1
        else:
            self.launches = max(1, len(computed))
        self.flops, self.bytes = algorithmic(wl)

    def step(self):
        self.ra.ring_attn_fwd(self.x.q, self.chunks, self.wl.causal, self.wl.q_offset,
                              flags=self.flags, out=self.out, ctx=self.ctx, workspace=self.ws, **self.masks)

    def estimate_step_s(self):
        """Wall time of one step after one untimed step (for sizing warmup)."""
        torch = self.torch
        self.step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        self.step()
        torch.cuda.synchronize()
        return max(time.perf_counter() - t0, 1e-5)

    def time(self, steps, warmup, during=None):
        """Mean wall time per step and the per-step HIP-event times (ms) on
        the launch stream; `during` runs on a host thread meanwhile."""
        torch = self.torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        th = threading.Thread(target=during, daemon=True) if during else None
        t0 = time.perf_counter()
        if th:
            th.start()
        for i in range(steps):
            ev[i][0].record()
            self.step()
            ev[i][1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        if th:
            th.join(timeout=60)
        ev_ms = [a.elapsed_time(b) for (a, b) in ev]
        return wall / steps, ev_ms

    def _timing(self, sec_per_step, ev_ms):
        return dict(ms_per_step=round(sec_per_step * 1e3, 4),
                    ms_per_step_events_mean=round(statistics.fmean(ev_ms), 4),
                    ms_per_step_median=round(statistics.median(ev_ms), 4),
                    ms_per_step_min=round(min(ev_ms), 4))

    def result(self, sec_per_step, ev_ms):
        wl = self.wl
        tflops = self.flops / sec_per_step / 1e12
        gbs = self.bytes / sec_per_step / 1e9
        launch_s = statistics.fmean(ev_ms) / 1e3 / self.launches
        if self.decode:
            achieved = self.bytes / self.launches / launch_s / 1e9
            roof = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                        frac=round(achieved / PEAK_HBM_GBS, 4), traffic=measured_traffic(self.label))
            metric, value, unit = "decode HBM GB/s at 1M KV", gbs, "GB/s"
            if wl.kv_dtype == "fp8":
                metric = "decode HBM GB/s at 1M KV (8-bit KV cache)"
            if wl.kv_heads_major:
                metric = metric.replace("at 1M KV", "at 1M KV, head-major cache")
        elif wl.dtype == "fp32":
            # a latency-bound 16-workgroup launch on the fp32 vector ALUs
            achieved = self.flops / self.launches / launch_s / 1e12
            roof = dict(bound="alu", achieved=round(achieved, 3), peak=PEAK_FP32_TFLOPS, unit="TFLOP/s",
                        frac=round(achieved / PEAK_FP32_TFLOPS, 5), traffic=measured_traffic(self.label))
            metric, value, unit = "attn fwd TFLOP/s, fp32 inputs (latency-bound tiny ring)", tflops, "TFLOP/s"
        else:
            achieved = self.flops / self.launches / launch_s / 1e12
            roof = dict(bound="mfma", achieved=round(achieved, 1), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                        frac=round(achieved / PEAK_BF16_TFLOPS, 4), traffic=measured_traffic(self.label))
            metric, value, unit = "causal attn fwd TFLOP/s (% MFMA peak) per GPU", tflops, "TFLOP/s"
            if wl.window or wl.anchor:
                metric = "local-window + anchor attn fwd TFLOP/s over visible pairs per GPU"
            elif wl.doc_mean:
                metric = "packed-document attn fwd TFLOP/s over visible pairs per GPU"
        mode = "split-KV + merge" if self.decode else ("in place" if self.label.startswith("inplace:")
                                                      else "staged ring (side-stream double buffer)")
        return dict(workload=self.label, mode=mode, metric=metric, value=round(value, 2), unit=unit,
                    **self._timing(sec_per_step, ev_ms),
                    tokens_per_s=round(wl.B * wl.Lq / sec_per_step, 1),
                    tflops=round(tflops, 3), gbs=round(gbs, 1),
                    launches_per_step=self.launches, roofline=roof)


class BackwardRun(WorkloadRun):
    """The gradients (dQ, dK, dV) of a prefill workload's ring share: one
    ring_attn_bwd call over all chunks in ring order (in place), with the
    forward's output, state and a seeded output gradient resident."""

    def __init__(self, name, device="cuda:0"):
        super().__init__(name, device)
        torch, ra, wl = self.torch, self.ra, self.wl
        from long_context_blockwise_amd import inputs

        self.label = "bwd:" + name
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
        achieved = self.flops / (statistics.fmean(ev_ms) / 1e3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / PEAK_BF16_TFLOPS, 4), traffic=measured_traffic(self.label),
                    kernels="bwd_pre + bwd_dq + bwd_dkdv per step (traffic: per step)")
        metric = "causal attn bwd TFLOP/s (dQ, dK, dV) per GPU"
        if wl.doc_mean:
            metric = "packed-document attn bwd TFLOP/s (dQ, dK, dV) over visible pairs per GPU"
        elif wl.window or wl.anchor:
            metric = "local-window + anchor attn bwd TFLOP/s (dQ, dK, dV) over visible pairs per GPU"
        return dict(workload=self.label, mode="in place", metric=metric,
                    value=round(tflops, 2), unit="TFLOP/s", **self._timing(sec_per_step, ev_ms),
                    tokens_per_s=round(wl.B * wl.Lq / sec_per_step, 1), tflops=round(tflops, 2),
                    launches_per_step=2 + len(self.chunks), roofline=roof)


def make_run(label):
    if label.startswith("bwd:"):
        return BackwardRun(label[4:])
    if label.startswith("inplace:"):
        return WorkloadRun(label[8:], inplace=True)
    return WorkloadRun(label)


def cpu_baseline(name, x=None, budget_s=20.0):
    """Time the CPU oracle on a bounded, stratified row sample of a workload
    (all heads and batches of the sampled rows), scale to TFLOP/s, and
    extrapolate the full workload's time from the sampled pairs.  `x` are the
    workload's inputs (device tensors are copied to the host); by default
    they are drawn on the host."""
    import numpy as np

    import oracle
    from long_context_blockwise_amd import inputs

    wl = inputs.WORKLOADS[name]
    if x is None:
        x = inputs.make(wl, "cpu")
    q = x.q.cpu()
    chunks = [tuple(t.cpu() if hasattr(t, "cpu") else t for t in c) for c in x.chunks()]
    rows_all = inputs.sample_rows(wl.Lq, tile=max(1, wl.Lq // 2048), seed=1)
    rng = np.random.default_rng(0)
    rng.shuffle(rows_all)
    n, spent, done_rows, t_total = 1, 0.0, [], 0.0
    while spent < budget_s / 2 and len(done_rows) < len(rows_all):
        rows = sorted(rows_all[len(done_rows):len(done_rows) + n])
        t0 = time.perf_counter()
        oracle.attention(q, chunks, wl.q_offset, wl.causal, rows=rows)
        dt = time.perf_counter() - t0
        done_rows += rows
        t_total += dt
        spent += dt
        n *= 2
    pairs = visible_pairs(wl, done_rows) * wl.Hq
    flops = pairs * 2 * (wl.d_qk + wl.d_v)
    full_flops, _ = algorithmic(wl)
    model, affinity = host_cpu()
    return dict(value=round(flops / t_total / 1e12, 6), unit="TFLOP/s", cores=oracle.threads(),
                kind="oracle",
                sample=f"{len(done_rows)} of {wl.Lq} query rows (stratified, all {wl.B}x{wl.Hq} batch-heads) of "
                       f"{wl.name}, fp64 C oracle, {t_total:.1f} s, {flops / 1e9:.1f} GFLOP",
                extrapolated_full_s=round(t_total * full_flops / flops, 1),
                host_cpu=model, affinity_cores=affinity)


# --------------------------------------------------------------------------- #
# rocprofv3 harness (--profile)
# --------------------------------------------------------------------------- #
# Counter groups: one rocprofv3 run each (at most 8 SQ and 2 GRBM counters
# per run; FETCH_SIZE and WRITE_SIZE take 3 and 2 of the 4 TCC slots, so
# each has a run of its own).
PMC_PIPES = ("GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_ACTIVE_INST_VALU "
             "SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU SQ_INSTS_MFMA")
PMC_LDS = "GRBM_GUI_ACTIVE SQ_ACTIVE_INST_LDS SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS SQ_INSTS_VALU_TRANS_F32 SQ_WAVES"
PMC_FETCH = "FETCH_SIZE"
PMC_WRITE = "WRITE_SIZE"

# The kernel each workload's roofline is priced on (a substring of the
# demangled name rocprofv3 reports), and whether it is priced in flops or bytes.
# (alternatives: the first one the trace holds is taken)
PREFILL_D128 = ("fwd_bf16_kernel<128, 64, 4, 1, 2, 0>",)
DOMINANT = {
    "ring_1m_gqa32x8_d128": (PREFILL_D128, "mfma"),
    "prefill_bf16_h32_d128": (PREFILL_D128, "mfma"),
    "inplace:ring_1m_gqa32x8_d128": (PREFILL_D128, "mfma"),
    "inplace:prefill_bf16_h32_d128": (PREFILL_D128, "mfma"),
    "mla_h16_d512": (("fwd_bf16_wide_kernel",), "mfma"),
    "inplace:mla_h16_d512": (("fwd_bf16_wide_kernel",), "mfma"),
    "decode_b4_gqa32x8_cache1m": (("fwd_bf16_kernel<128, 64, 4, 2, 2, 0>",), "hbm"),
    "decode_b4_gqa32x8_cache1m_fp8": (("fwd_fp8kv_kernel",), "hbm"),
    "decode_b4_gqa32x8_cache1m_bhsd": (("fwd_bf16_kernel<128, 64, 4, 2, 2, 0>",), "hbm"),
    "decode_b4_gqa32x8_cache1m_fp8_bhsd": (("fwd_fp8kv_kernel",), "hbm"),
    "bwd:prefill_bf16_h32_d128": (("bwd_",), "mfma"),
    "bwd:mla_h16_d512": (("bwd_",), "mfma"),
    "local_w4096_s4096_h32_d128": (("fwd_bf16_kernel<128, 64, 4, 1, 2, 1>",), "mfma"),
    "docs4096_h32_d128": (("fwd_bf16_kernel<128, 64, 4, 1, 2, 2>",), "mfma"),
}


def _rocprof_run(args, outdir, tag, child, timeout):
    """One rocprofv3 run of `child` (argv of this script) with `args`;
    returns the output directory of the run."""
    d = os.path.join(outdir, "raw", tag)
    os.makedirs(d, exist_ok=True)
    cmd = ["rocprofv3", *args, "-d", d, "-o", tag, "--output-format", "csv", "--", sys.executable, *child]
    print("[profile] " + " ".join(shlex.quote(c) for c in cmd), file=sys.stderr, flush=True)
    env = dict(os.environ, TMPDIR=os.environ.get("TMPDIR", "/tmp"))
    r = subprocess.run(cmd, cwd=ROOT, env=env, timeout=timeout, capture_output=True, text=True)
    with open(os.path.join(d, "rocprof.log"), "w") as f:
        f.write(r.stdout + "\n---- stderr ----\n" + r.stderr)
    if r.returncode != 0:
        # rocprofv3 may exit non-zero after a complete run; the CSVs decide
        print(f"[profile] rocprofv3 exit {r.returncode} ({tag}); see {d}/rocprof.log", file=sys.stderr, flush=True)
    return d, " ".join(shlex.quote(c) for c in cmd)


def _csv_rows(d, suffix):
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(f, newline="") as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _counters(d, pattern, last=None):
    """{counter: [value per dispatch]} over the dispatches of the kernels whose
    name contains `pattern` (only the `last` ones in dispatch order, when
    given), and how many dispatches those are."""
    per = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        if pattern not in r.get("Kernel_Name", ""):
            continue
        key = int(r["Dispatch_Id"])
        per.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])
    keys = sorted(per)
    if last:
        keys = keys[-last:]
    vals = {}
    for key in keys:
        for k, v in per[key].items():
            vals.setdefault(k, []).append(v)
    return vals, len(keys)


def _child_line(d):
    """The JSON line a profiled bench.py child printed (its stdout), or None."""
    try:
        with open(os.path.join(d, "rocprof.log")) as f:
            out = f.read().split("---- stderr ----")[0]
    except OSError:
        return None
    for line in reversed(out.splitlines()):
        if line.startswith("{"):
            try:
                return json.loads(line)
            except ValueError:
                return None
    return None


def profile(names, outdir, steps):
    os.makedirs(outdir, exist_ok=True)
    me = os.path.relpath(os.path.abspath(__file__), ROOT)
    # copy calibration: a plain elementwise copy of 1 GiB (reads 1 GiB, writes 1 GiB)
    cal_bytes = 1 << 30
    calib = {}
    for tag, grp in (("copy_fetch", PMC_FETCH), ("copy_write", PMC_WRITE)):
        d, _ = _rocprof_run(["--pmc", *grp.split()], outdir, tag, [me, "--copy-calibration", str(cal_bytes)], 300)
        vals, _n = _counters(d, "neg")
        name = grp.split()[0]
        if vals.get(name):
            calib[name] = cal_bytes / (max(vals[name]) * 1024.0)  # true bytes per counted byte
    summary = {"calibration": calib, "workloads": {}}
    for name in names:
        base = name.split(":", 1)[-1]
        child = [me, "--workload", name, "--secondary", "", "--no-cpu", "--steps", str(steps), "--warmup", "1",
                 "--warmup-s", str(PROFILE_WARMUP_S), "--no-clock"]
        tagb = name.replace(":", "_")
        runs = {}
        runs["trace"] = _rocprof_run(["--kernel-trace", "--stats"], outdir, tagb + "_trace", child, 900)
        for key, grp in (("pipes", PMC_PIPES), ("lds", PMC_LDS), ("fetch", PMC_FETCH), ("write", PMC_WRITE)):
            runs[key] = _rocprof_run(["--pmc", *grp.split()], outdir, f"{tagb}_{key}", child, 900)
        summary["workloads"][name] = write_profile_summary(name, runs, calib, outdir, steps)
    with open(os.path.join(outdir, "profile_summary.json"), "w") as f:
        json.dump(summary, f, indent=1)
    print(json.dumps(summary), flush=True)


def write_profile_summary(name, runs, calib, outdir, steps):
    from long_context_blockwise_amd import inputs

    patterns, bound = DOMINANT.get(name, (("",), "mfma"))
    base = name.split(":", 1)[-1]
    wl = inputs.WORKLOADS[base]
    stats = _csv_rows(runs["trace"][0], "kernel_stats.csv")
    all_traces = _csv_rows(runs["trace"][0], "kernel_trace.csv")
    pattern = next((p for p in patterns if any(p in r.get("Kernel_Name", "") for r in all_traces)), patterns[0])
    traces = sorted((r for r in all_traces if pattern in r.get("Kernel_Name", "")),
                    key=lambda r: int(r["Start_Timestamp"]))
    # The traced command runs untimed steps (its warmup, sized to a minimum GPU
    # time, and the step-time estimate) before the timed ones; its JSON line
    # says how many.  Only the timed steps' dispatches are priced, in the trace
    # and in each counter run.
    child = _child_line(runs["trace"][0]) or {}
    untimed = (child.get("run_info") or {}).get("untimed_steps", 1)
    per_step = len(traces) / (steps + untimed) if traces else float("nan")
    n_timed = max(1, round(steps * per_step)) if traces else 0
    all_durs = len(traces)
    traces = traces[-n_timed:] if traces else traces
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) for r in traces]
    avg_ns = statistics.fmean(durs) if durs else float("nan")
    pipes, n_disp = _counters(runs["pipes"][0], pattern, n_timed)
    lds, _ = _counters(runs["lds"][0], pattern, n_timed)
    fetch, _ = _counters(runs["fetch"][0], pattern, n_timed)
    write, _ = _counters(runs["write"][0], pattern, n_timed)
    mean = lambda v: statistics.fmean(v) if v else float("nan")
    flops, kv_bytes = algorithmic(wl)
    if name.startswith("bwd:"):
        flops = visible_pairs(wl) * wl.Hq * 2 * (3 * wl.d_qk + 2 * wl.d_v)
    n_steps = steps
    grbm = mean(pipes.get("GRBM_GUI_ACTIVE", [])) / N_XCD  # cycles (the counter sums the XCDs)
    clock_ghz = grbm / avg_ns if durs else float("nan")
    mfma_busy = mean(pipes.get("SQ_VALU_MFMA_BUSY_CYCLES", [])) / (grbm * N_SIMD)
    valu_busy = mean(pipes.get("SQ_ACTIVE_INST_VALU", [])) / (grbm * N_CU)
    coexec = mean(pipes.get("SQ_VALU_MFMA_COEXEC_CYCLES", [])) / (grbm * N_SIMD)
    mops = mean(pipes.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", [])) * 512.0
    lds_busy = mean(lds.get("SQ_ACTIVE_INST_LDS", [])) / (grbm * N_CU)
    fb = mean(fetch.get("FETCH_SIZE", [])) * 1024.0 * calib.get("FETCH_SIZE", float("nan"))
    wb = mean(write.get("WRITE_SIZE", [])) * 1024.0 * calib.get("WRITE_SIZE", float("nan"))
    if name.startswith("bwd:"):
        launches = 1.0  # priced per step over all its kernels (pattern "bwd_")
        alg_flops_launch = flops
        alg_bytes_launch = kv_bytes
    else:
        launches = per_step if per_step == per_step else 1.0
        alg_flops_launch = flops / launches
        alg_bytes_launch = kv_bytes / launches
    if name.startswith("bwd:"):
        step_ns = sum(durs) / n_steps if durs else float("nan")
        achieved_tflops = alg_flops_launch / step_ns / 1e3
        fb_step, wb_step = fb * per_step, wb * per_step
    else:
        achieved_tflops = alg_flops_launch / avg_ns / 1e3
        fb_step, wb_step = fb, wb
    achieved_gbs = alg_bytes_launch / avg_ns
    kname = traces[0]["Kernel_Name"] if traces else pattern
    short = kname.replace("void ", "").replace("ra::(anonymous namespace)::", "").split("(")[0].replace(" ", "")
    if name.startswith("bwd:"):
        short = "bwd_pre+bwd_dq+bwd_dkdv"
    fname = "".join(c if c.isalnum() or c in "_-" else "_" for c in short.split("<")[0]) + "_" + name.replace(":", "_")
    path = os.path.join(outdir, fname + ".md")
    lines = [f"# {short} on `{name}`", "",
             f"Workload: {wl.name} (B={wl.B}, Hq={wl.Hq}, Hkv={wl.Hkv}, d={wl.d_qk}, {wl.P} chunks of "
             f"{wl.chunk_len}, Lq={wl.Lq}, q_offset={wl.q_offset}, causal={wl.causal}, "
             f"kv={wl.kv_dtype or wl.dtype}).", "",
             "Made by `python bench.py --profile " + name + "`, which ran:", ""]
    for key, (_d, cmd) in runs.items():
        lines.append(f"- {key}: `{cmd}`")
    lines += ["", "## Kernel trace (rocprofv3 --stats, raw rows)", "",
              "| Name | Calls | TotalDurationNs | AverageNs | MinNs | MaxNs |", "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| `{r.get('Name', '')[:110]}` | {r.get('Calls')} | {r.get('TotalDurationNs')} | "
                     f"{r.get('AverageNs')} | {r.get('MinNs')} | {r.get('MaxNs')} |")
    fmt = lambda v, p=3: "n/a" if v != v else f"{v:.{p}g}" if abs(v) < 1e4 else f"{v:.4e}"
    lines += ["", f"## Dominant kernel `{short}` (derived over the {len(durs)} dispatches of the {steps} timed "
                  f"steps: the last of {all_durs} in the trace, and of each counter run)", "",
              "| Quantity | Value | How |", "|---|---|---|",
              f"| average duration | {fmt(avg_ns / 1e3, 5)} µs | kernel trace, timed dispatches matching `{pattern}` |",
              f"| launches per step | {fmt(per_step)} | dispatches / ({steps} timed + {untimed} untimed steps) |",
              f"| shader clock | {fmt(clock_ghz, 4)} GHz | GRBM_GUI_ACTIVE / {N_XCD} XCDs / average duration |",
              f"| MFMA busy | {fmt(100 * mfma_busy, 4)} % | SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE/{N_XCD} x "
              f"{N_SIMD} SIMDs) |",
              f"| VALU active | {fmt(100 * valu_busy, 4)} % | SQ_ACTIVE_INST_VALU / (GRBM_GUI_ACTIVE/{N_XCD} x "
              f"{N_CU} CUs) |",
              f"| MFMA and VALU together | {fmt(100 * coexec, 4)} % | SQ_VALU_MFMA_COEXEC_CYCLES / "
              f"(GRBM_GUI_ACTIVE/{N_XCD} x {N_SIMD}) |",
              f"| LDS active | {fmt(100 * lds_busy, 4)} % | SQ_ACTIVE_INST_LDS / (GRBM_GUI_ACTIVE/{N_XCD} x {N_CU}) |",
              f"| MFMA flops executed per dispatch | {fmt(mops)} | SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 |",
              f"| algorithmic flops per launch | {fmt(alg_flops_launch)} | visible pairs x 2(d_qk+d_v) per head |",
              f"| VALU instructions per MFMA | {fmt(mean(pipes.get('SQ_INSTS_VALU', [])) / max(mean(pipes.get('SQ_INSTS_MFMA', [])), 1))} | SQ_INSTS_VALU / SQ_INSTS_MFMA |",
              f"| transcendental (exp) per MFMA | {fmt(mean(lds.get('SQ_INSTS_VALU_TRANS_F32', [])) / max(mean(pipes.get('SQ_INSTS_MFMA', [])), 1))} | SQ_INSTS_VALU_TRANS_F32 / SQ_INSTS_MFMA |",
              f"| LDS bank conflicts / LDS instructions | {fmt(mean(lds.get('SQ_LDS_BANK_CONFLICT', [])) / max(mean(lds.get('SQ_INSTS_LDS', [])), 1))} | cycles per instruction |",
              f"| HBM read bytes per dispatch | {fmt(fb)} | FETCH_SIZE KiB x 1024 x {fmt(calib.get('FETCH_SIZE', float('nan')), 4)} (copy calibration) |",
              f"| HBM write bytes per dispatch | {fmt(wb)} | WRITE_SIZE KiB x 1024 x {fmt(calib.get('WRITE_SIZE', float('nan')), 4)} (copy calibration) |",
              f"| algorithmic K/V+Q+out bytes per launch | {fmt(alg_bytes_launch)} | K+V once, Q, out |"]
    # the staging copies of the ring stand-in: their time and how much of it
    # overlaps the attention kernels (kernel-trace intervals)
    t_timed = int(traces[0]["Start_Timestamp"]) if traces else 0
    copies = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in all_traces
              if "copyBuffer" in r.get("Kernel_Name", "") and int(r["End_Timestamp"]) > t_timed]
    attn = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in traces)
    copy_ns = sum(e - b for b, e in copies)
    over_ns = 0
    for b, e in copies:
        for ab, ae in attn:
            if ab >= e:
                break
            over_ns += max(0, min(e, ae) - max(b, ab))
    stage = dict(copies=len(copies), copy_ns=copy_ns, overlap_ns=over_ns,
                 copy_frac_of_kernel_time=copy_ns / max(sum(durs), 1))
    if copies:
        lines += [f"| staging copies (ring stand-in) | {len(copies)} copies, {fmt(copy_ns / 1e3, 5)} µs in all, "
                  f"{fmt(100 * over_ns / max(copy_ns, 1), 4)} % of it while an attention kernel ran | "
                  f"kernel trace: `copyBuffer` intervals against `{pattern}` intervals |",
                  f"| staging copy time / attention kernel time | {fmt(100 * copy_ns / max(sum(durs), 1), 4)} % | "
                  "both from the kernel trace (copies run on the side stream) |"]
    # the bench's own HIP-event timing of the traced command (its JSON line),
    # the figure the bench line reports, for comparison with the trace
    ev = (child.get("roofline") or {}).get("achieved")
    if ev:
        ev_ns = (alg_flops_launch / ev * 1e-3) if bound == "mfma" else (alg_bytes_launch / ev)
        unit = "TFLOP/s" if bound == "mfma" else "GB/s"
        what = "step" if name.startswith("bwd:") else "launch"
        lines += [f"| bench events in the traced command | {fmt(ev_ns / 1e3, 5)} µs per {what} ({fmt(ev, 5)} {unit}) | "
                  "HIP events on the launch stream around the timed steps of the trace run (its JSON line) |"]
    if bound == "mfma":
        lines += [f"| **achieved (algorithmic)** | **{fmt(achieved_tflops, 5)} TFLOP/s = "
                  f"{fmt(100 * achieved_tflops / PEAK_BF16_TFLOPS, 4)} % of {PEAK_BF16_TFLOPS}** | "
                  "algorithmic flops per launch / average duration |"]
    else:
        lines += [f"| **achieved (algorithmic)** | **{fmt(achieved_gbs, 5)} GB/s = "
                  f"{fmt(100 * achieved_gbs / PEAK_HBM_GBS, 4)} % of {PEAK_HBM_GBS:.0f}** | "
                  "algorithmic bytes per launch / average duration |",
                  f"| measured HBM rate | {fmt((fb + wb) / avg_ns, 5)} GB/s | (read + write bytes) / average duration |"]
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return dict(file=path, kernel=short, avg_us=avg_ns / 1e3, launches_per_step=per_step, clock_ghz=clock_ghz,
                mfma_busy=mfma_busy, valu_busy=valu_busy, coexec=coexec, lds_busy=lds_busy,
                fetch_bytes=fb_step, write_bytes=wb_step, traffic_bytes=fb_step + wb_step,
                achieved_tflops=achieved_tflops, achieved_gbs=achieved_gbs, staging=stage,
                kernel_digest=kernel_digest())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--secondary", default=SECONDARY, help="comma list, '' for none")
    ap.add_argument("--secondary-steps", type=int, default=0, help="timed steps of each secondary (default steps/2)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--warmup-s", type=float, default=0.0, metavar="SECONDS",
                    help="warm the headline workload up for at least this much GPU time (more steps than "
                         "--warmup when its steps are short; the profile runs use it)")
    ap.add_argument("--no-clock", action="store_true", help="do not sample the board clock")
    ap.add_argument("--profile", default="", metavar="NAMES",
                    help="run the rocprofv3 harness on these workloads (comma list) and write summaries")
    ap.add_argument("--profile-out", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--profile-steps", type=int, default=2)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run one plain elementwise copy of BYTES bytes (reads BYTES, writes "
                         "BYTES) to calibrate the FETCH_SIZE / WRITE_SIZE counters, then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one device's ring share on one GPU; --gpus must be 1 "
              "(the ring across GPUs is not implemented: each device's share runs on one GPU)", file=sys.stderr)
        sys.exit(2)
    if args.profile:  # the parent only starts rocprofv3 runs; it never touches the GPU itself
        profile([s for s in args.profile.split(",") if s], args.profile_out, args.profile_steps)
        return

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
    run = make_run(args.workload)
    clock = {}

    def sample():  # the board clock half a second into the timed steps
        time.sleep(0.5)
        t0 = time.perf_counter()
        clock["sclk_mhz"] = sample_sclk_mhz()
        clock["t"] = (t0, time.perf_counter())
    warm, est_steps = args.warmup, 0
    if args.warmup_s > 0:
        warm = max(warm, math.ceil(args.warmup_s / run.estimate_step_s()))
        est_steps = 2  # the two untimed steps of the estimate
    t_start = time.perf_counter()
    sec, ev_ms = run.time(args.steps, warm, during=None if args.no_clock else sample)
    t_end = time.perf_counter()
    head = run.result(sec, ev_ms)
    print(f"[bench] {head}", file=sys.stderr, flush=True)
    x_head = None if args.no_cpu else run.x
    run.x = None
    del run
    torch.cuda.empty_cache()
    # was the clock read while the timed steps were still running?
    t_timed0 = t_end - sec * args.steps
    clock_inside = bool(clock.get("t")) and clock["t"][0] >= t_timed0 and clock["t"][1] <= t_end

    secondary = []
    sec_steps = args.secondary_steps or max(3, args.steps // 2)
    for name in [s for s in args.secondary.split(",") if s and s != args.workload]:
        r = make_run(name)
        # Short steps are warmed up and timed for a minimum span of GPU time:
        # after the idle gap of setting a workload up, the board takes tens of
        # milliseconds of load to reach its steady clocks, which a few steps
        # of a millisecond or two do not cover.
        est = r.estimate_step_s()
        warm = max(1, args.warmup, math.ceil(SECONDARY_WARMUP_S / est))
        steps2 = max(sec_steps, math.ceil(SECONDARY_TIMED_S / est))
        s2, e2 = r.time(steps2, warm)
        res = r.result(s2, e2)
        res["timed_steps"], res["warmup_steps"] = steps2, warm
        print(f"[bench] {res}", file=sys.stderr, flush=True)
        secondary.append(res)
        del r
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu:
        from long_context_blockwise_amd import inputs

        wl0 = inputs.WORKLOADS[args.workload.split(":", 1)[-1]]
        host = inputs.Inputs(wl0, x_head.q.cpu(), [k.cpu() for k in x_head.ks], [v.cpu() for v in x_head.vs],
                             x_head.starts)
        del x_head
        torch.cuda.empty_cache()
        cpu = cpu_baseline(wl0.name, host)
    from long_context_blockwise_amd import inputs

    w = inputs.WORKLOADS[args.workload.split(":", 1)[-1]]
    model, affinity = host_cpu()
    line = {
        "metric": head["metric"],
        "value": head["value"],
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warm,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "fp32",
        "data": "synthetic",
        "config": {"workload": head["workload"], "mode": head["mode"], "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d_qk,
                   "chunk_len": w.chunk_len, "P": w.P, "Lq": w.Lq, "q_offset": w.q_offset,
                   "causal": w.causal, "tokens_per_s": head["tokens_per_s"],
                   "ms_per_step_median": head["ms_per_step_median"], "ms_per_step_min": head["ms_per_step_min"]},
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "run_info": {"gpu": props.name, "gcn_arch": getattr(props, "gcnArchName", None),
                     "cus": props.multi_processor_count, "sclk_mhz_sampled": clock.get("sclk_mhz"),
                     "sclk_sampled_during_timed_steps": clock_inside,
                     "sclk_max_mhz": 2400, "host_cpu": model, "host_affinity_cores": affinity,
                     "untimed_steps": est_steps + warm,
                     "torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
                     "source_digest": source_digest(), "git_rev": git_revision()},
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
