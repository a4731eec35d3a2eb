"""The workloads at full size, in the launch configuration bench.py
times (bench.WorkloadRun: staged ring for prefill shares, split-KV + merge
for decoding), checked against the oracle on sampled outputs the oracle
computes row by row: stratified query rows (one per tile plus tile and
chunk boundaries) for a subset of (batch, KV head) groups, every query head
of each group.  The local-window and packed-document workloads carry their
window, anchors and segment labels to both sides."""
import os
import sys

import numpy as np
import pytest
import torch

from parity import check, gather_sampled, sampled_reference

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from long_context_blockwise_amd import inputs  # noqa: E402

pytestmark = pytest.mark.gpu

CASES = {
    # workload: (row tile of the sample, KV heads, batches); every query head
    # of each sampled KV head.  The prefill shares take one row per 128-row
    # tile (the kernels' row tile) over all heads; the 1M-token share one per
    # 1024 rows (each of its rows sees up to 2^20 keys, ~0.9 s of oracle time
    # per row over its 32 heads); decoding all 16 rows of several groups.
    "tiny_ring_fp32": (1, [0], None),
    "prefill_bf16_h32_d128": (128, list(range(32)), None),
    "ring_1m_gqa32x8_d128": (1024, list(range(8)), None),
    "mla_h16_d512": (256, [0], None),
    "local_w4096_s4096_h32_d128": (128, list(range(32)), None),
    "docs4096_h32_d128": (128, list(range(32)), None),
    "decode_b4_gqa32x8_cache1m": (1, [0, 3, 7], [0, 1, 3]),
    "decode_b4_gqa32x8_cache1m_fp8": (1, [0, 3, 7], [0, 1, 3]),
    "decode_b4_gqa32x8_cache1m_bhsd": (1, [1, 6], [0, 2]),
    "decode_b4_gqa32x8_cache1m_fp8_bhsd": (1, [1, 6], [0, 2]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_workload_full_size(name):
    tile, kv_heads, batches = CASES[name]
    print(f"[workload] {name}", flush=True)
    run = bench.WorkloadRun(name)
    wl = run.wl
    run.step()
    run.step()  # second call reuses staging buffers and events
    torch.cuda.synchronize()
    if tile == 1:
        rows = list(range(wl.Lq))
    else:
        rows = inputs.sample_rows(wl.Lq, tile=tile, seed=3,
                                  extra=(wl.Lq - 64, wl.Lq - 65, 8191, 8192, 16383, 16384))
    q_seg, k_segs = inputs.segment_labels(wl)  # chunk index order, like run.x.chunks()
    ref = sampled_reference(run.x.q, run.x.chunks(), wl.q_offset, wl.causal, rows, kv_heads, batches,
                            window=wl.window, anchor=wl.anchor, q_seg=q_seg, k_segs=k_segs)
    G = wl.Hq // wl.Hkv
    got = np.concatenate([gather_sampled(run.out, rows, b, hk, G) for (b, hk) in ref])
    want = np.concatenate(list(ref.values()))
    e = check(got, want, wl.dtype, name)
    nb = len({b for (b, _) in ref})
    print(f"[workload] {name}: {len(rows)} rows x {len(ref) * G} (batch, query head) pairs "
          f"= {len(rows) * len(ref) * G} sampled output rows of {wl.B * wl.Lq * wl.Hq} "
          f"({nb} batches, {len(kv_heads)} KV heads); {e}", flush=True)
    del run
    torch.cuda.empty_cache()
