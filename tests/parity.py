"""Helpers for comparing the HIP path with the CPU oracle.

Tolerances.  The stated bar is max-abs <= 2e-2 and mean-abs <= 2e-3 for bf16
inputs and <= 1e-5 for fp32 inputs.  At long contexts |out| is ~1e-3, where
an all-zero output would meet the absolute bounds, so a relative L2 bound is
checked as well: <= 1e-2 for bf16 (the bf16 rounding of the probabilities
and of the output gives ~2-3e-3) and <= 1e-6 for fp32; the reference norm
must be non-zero for the check to mean anything.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

TOL = {
    "bf16": dict(max_abs=2e-2, mean_abs=2e-3, rel_l2=1e-2),
    "fp32": dict(max_abs=1e-5, mean_abs=1e-5, rel_l2=1e-6),
}


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    d = np.abs(got - ref)
    nref = float(np.linalg.norm(ref))
    return dict(max_abs=float(d.max()) if d.size else 0.0,
                mean_abs=float(d.mean()) if d.size else 0.0,
                rel_l2=float(np.linalg.norm(got - ref) / nref) if nref > 0 else float(np.linalg.norm(got)),
                ref_norm=nref, finite=bool(np.isfinite(got).all()))


def check(got, ref, dtype: str, what: str = "", rel_l2=True):
    e = errors(got, ref)
    tol = TOL[dtype]
    msg = f"{what}: {e} tol {tol}"
    assert e["finite"], msg
    assert e["max_abs"] <= tol["max_abs"], msg
    assert e["mean_abs"] <= tol["mean_abs"], msg
    if rel_l2 and e["ref_norm"] > 0:
        assert e["rel_l2"] <= tol["rel_l2"], msg
    return e


def to_host(chunks):
    """Chunks with their tensors on the host (8-bit chunks keep their exponents)."""
    return [tuple(t.cpu() if hasattr(t, "cpu") else t for t in c) for c in chunks]


def oracle_out(q, chunks, q_offset, causal, rows=None, scale=None, window=0):
    """Oracle output [B, n_rows, Hq, d_v] and lse for device tensors."""
    return oracle.attention(q.cpu(), to_host(chunks), q_offset, causal, scale=scale, rows=rows,
                            window=window)


def oracle_state(q, chunks, q_offset, causal, order=None, rows=None, window=0):
    """Oracle ring state (m, l, O) in the ABI layout [B, Lq, Hq](, d_v)."""
    st = oracle.ring(q.cpu(), to_host(chunks), order=order, q_offset=q_offset, causal=causal, rows=rows,
                     window=window)
    return (st.m.transpose(0, 2, 1), st.l.transpose(0, 2, 1), st.O.transpose(0, 2, 1, 3))


def group_slice(x, g0, G):
    """Query heads of KV group g0 (heads g0*G .. g0*G+G-1) of [B, S, Hq, d]."""
    return x[:, :, g0 * G:(g0 + 1) * G]


def kv_slice(chunks, hk):
    return [(k[:, :, hk:hk + 1], v[:, :, hk:hk + 1], s) for (k, v, s) in chunks]


def sampled_reference(q, chunks, q_offset, causal, rows, kv_heads, batches=None, window=0, anchor=0,
                      q_seg=None, k_segs=None):
    """Oracle values for the given rows, for the query heads of the given KV
    heads (and batches): returns {(b, hk): out [1, n_rows, G, d_v]}.  Slices
    are cut on the device and only they are copied to the host.  Window,
    anchors and segment labels (``q_seg [B, Lq]``, ``k_segs`` per chunk
    ``[B, len]``) mask as in the oracle's attention."""
    B, _, Hq, _ = q.shape
    Hkv = chunks[0][0].shape[2]
    G = Hq // Hkv
    res = {}
    for b in (range(B) if batches is None else batches):
        for hk in kv_heads:
            qs = q[b:b + 1, :, hk * G:(hk + 1) * G].cpu().contiguous()
            cs = []
            for c in chunks:
                k, v, s = c[0], c[1], c[2]
                cut = (k[b:b + 1, :, hk:hk + 1].cpu().contiguous(), v[b:b + 1, :, hk:hk + 1].cpu().contiguous(), s)
                if len(c) == 5:  # 8-bit chunk: exponents [B, Hkv, nblk] of the same (batch, head)
                    cut += (c[3][b:b + 1, hk:hk + 1].cpu().contiguous(), c[4][b:b + 1, hk:hk + 1].cpu().contiguous())
                cs.append(cut)
            qsb = None if q_seg is None else q_seg[b:b + 1].cpu().contiguous()
            ksb = None if k_segs is None else [t[b:b + 1].cpu().contiguous() for t in k_segs]
            out, _ = oracle.attention(qs, cs, q_offset, causal, rows=rows, window=window, anchor=anchor,
                                      q_seg=qsb, k_segs=ksb)
            res[(b, hk)] = out
    return res


def gather_sampled(out, rows, b, hk, G):
    return out[b:b + 1, rows][:, :, hk * G:(hk + 1) * G].float().cpu().numpy()
