"""bench.py's accounting on the CPU: the visible (query, key) pairs it
counts for a workload (the algorithmic work behind TFLOP/s) equal the pairs
the oracle's attention sees.  With all queries zero every visible key gets
the same score, so the oracle's log-sum-exp of a row is ln(number of keys it
sees); the masked shapes use the same window, anchors and segment labels as
the timed call."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from long_context_blockwise_amd import inputs  # noqa: E402


def _oracle_pairs(wl, rows=None):
    x = inputs.make(wl, "cpu")
    q = torch.zeros_like(x.q)
    q_seg, k_segs = inputs.segment_labels(wl)
    _, lse = oracle.attention(q, x.chunks(), wl.q_offset, wl.causal, rows=rows, window=wl.window,
                              anchor=wl.anchor, q_seg=q_seg, k_segs=k_segs)
    counts = np.where(np.isfinite(lse), np.exp(lse), 0.0)  # [B, Hq, rows]
    return int(np.rint(counts[:, 0]).sum())


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("window,anchor,doc_mean", [(0, 0, 0), (10, 0, 0), (0, 16, 0), (10, 16, 0),
                                                    (0, 0, 20), (12, 8, 15)])
def test_visible_pairs_match_oracle(causal, window, anchor, doc_mean):
    wl = inputs.Workload("acct", B=2, Hq=1, Hkv=1, d_qk=64, d_v=64, dtype="fp32", chunk_len=64, P=3, Lq=70,
                         q_offset=100, causal=causal, std=1.0, seed=9, chunk_lens=(64, 48, 80), window=window,
                         anchor=anchor, doc_mean=doc_mean)
    assert bench.visible_pairs(wl) == _oracle_pairs(wl)
    rows = [0, 5, 33, 69]
    assert bench.visible_pairs(wl, rows) == _oracle_pairs(wl, rows)


def test_unmasked_counts_agree():
    """The closed form and the masked counter agree on unmasked shapes."""
    for name in ("prefill_bf16_h32_d128", "ring_1m_gqa32x8_d128", "decode_b4_gqa32x8_cache1m"):
        wl = inputs.WORKLOADS[name]
        assert bench.visible_pairs_fast(wl) * wl.B == bench.visible_pairs(wl)
        assert bench.visible_pairs_per_head(wl, range(0, wl.Lq, 97)) > 0


def test_bench_masked_workloads_counts():
    """The local-window and packed-document bench workloads count the pairs
    their definitions give (exact for the window: 4096 + 1 keys per row,
    plus the one future anchor A + S of rows in the first anchor block)."""
    wl = inputs.WORKLOADS["local_w4096_s4096_h32_d128"]
    assert bench.visible_pairs(wl) == 8192 * 4097 + 4096
    wl = inputs.WORKLOADS["docs4096_h32_d128"]
    assert 0 < bench.visible_pairs(wl) < bench.visible_pairs(inputs.WORKLOADS["prefill_bf16_h32_d128"])
