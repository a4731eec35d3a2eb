"""Anchor tokens and segment labels on the GPU, forward and backward,
against the oracle's masks: anchors outside the window (extra tiles before
and after it), strides off the tile grid, two-sided windows, packed
documents and arbitrary labels, labels with anchors, split-KV decoding,
fp32, and the shapes that reject them."""
import numpy as np
import pytest
import torch

import long_context_blockwise_amd as ra
import oracle
from long_context_blockwise_amd import inputs
from parity import check, errors, to_host

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _wl(B=1, Hq=4, Hkv=2, d=128, dtype="bf16", lens=(256, 256), Lq=256, q_offset=0, causal=True, seed=41):
    std = 1.0 if dtype == "fp32" else 0.5
    return inputs.Workload("sparse_case", B=B, Hq=Hq, Hkv=Hkv, d_qk=d, d_v=d, dtype=dtype, chunk_len=lens[0],
                           P=len(lens), Lq=Lq, q_offset=q_offset, causal=causal, std=std, seed=seed,
                           chunk_lens=tuple(lens))


def _labels(x, kind, seed=5):
    """(q_seg, k_segs) on the device: packed documents or arbitrary labels."""
    wl = x.wl
    n = max(s + k.shape[1] for s, k in zip(x.starts, x.ks))
    n = max(n, wl.q_offset + wl.Lq)
    if kind == "packed":
        lab = inputs.packed_labels(wl.B, n, mean_doc=90, seed=seed)
    else:  # arbitrary small labels: no structure for the tile tests to use
        g = torch.Generator().manual_seed(seed)
        lab = torch.randint(0, 3, (wl.B, n), generator=g, dtype=torch.int32)
    lab = lab.to(DEV)
    q_seg = lab[:, wl.q_offset:wl.q_offset + wl.Lq].contiguous()
    k_segs = [lab[:, s:s + k.shape[1]].contiguous() for s, k in zip(x.starts, x.ks)]
    return q_seg, k_segs


def _fwd_check(x, causal, window, anchor, labels, flags, what, order=None):
    wl = x.wl
    order = list(range(len(x.ks))) if order is None else order
    chunks = x.chunks(order)
    q_seg = k_segs = None
    if labels:
        q_seg, k_all = _labels(x, labels)
        k_segs = [k_all[c] for c in order]
    out, _ = ra.ring_attn_fwd(x.q, chunks, causal, wl.q_offset, flags=flags, window=window, anchor=anchor,
                              q_seg=q_seg, k_segs=k_segs)
    torch.cuda.synchronize()
    ref, _ = oracle.attention(x.q.cpu(), to_host(chunks), wl.q_offset, causal, window=window, anchor=anchor,
                              q_seg=None if q_seg is None else q_seg.cpu(),
                              k_segs=None if k_segs is None else [k.cpu() for k in k_segs])
    dt = "fp32" if wl.dtype == "fp32" else "bf16"
    got = out.cpu().numpy() if dt == "fp32" else out.float().cpu().numpy()
    check(got, ref, dt, f"{what} W={window} S={anchor} labels={labels} flags={flags}")


PREFILL = [
    # d, lens, Lq, q_offset, causal, window, anchor, labels
    (128, (256, 256, 256), 256, 512, True, 32, 64, None),     # anchors before the window and one block ahead
    (128, (256, 256, 256), 256, 512, True, 0, 100, None),     # stride off the tile grid; causal, no window
    (128, (300, 200), 257, 43, False, 20, 50, None),          # two-sided window
    (64, (256, 256), 256, 256, True, 10, 48, None),
    (128, (256, 256, 256), 256, 512, True, 0, 0, "packed"),
    (64, (200, 300), 257, 100, True, 0, 0, "packed"),
    (128, (256, 256), 256, 256, True, 40, 0, "packed"),       # labels and a window
    (128, (192, 320), 200, 250, False, 0, 0, "arbitrary"),
    (128, (256, 256, 256), 256, 512, True, 16, 64, "packed"),  # labels and anchors
    (64, (128, 128, 128), 128, 256, True, 8, 32, "arbitrary"),
    (128, (300, 200), 257, 43, False, 20, 0, "arbitrary"),    # two-sided window, labels alone
]


@pytest.mark.parametrize("d,lens,Lq,q_off,causal,window,anchor,labels", PREFILL)
@pytest.mark.parametrize("flags", [0, 1], ids=["inplace", "staged"])
def test_sparse_prefill(d, lens, Lq, q_off, causal, window, anchor, labels, flags):
    x = inputs.make(_wl(B=2, d=d, lens=lens, Lq=Lq, q_offset=q_off, causal=causal), DEV)
    _fwd_check(x, causal, window, anchor, labels, flags | ra.RA_FLAG_NO_SPLIT_KV,
               f"d={d} {lens} Lq={Lq} off={q_off}", order=list(range(len(lens)))[::-1])


@pytest.mark.parametrize("Lq,q_off,window,anchor,labels", [(1, 1835, 64, 256, None), (16, 1820, 0, 500, None),
                                                          (4, 1832, 0, 0, "packed"), (7, 1000, 30, 128, "packed")])
def test_sparse_decode_split(Lq, q_off, window, anchor, labels):
    x = inputs.make(_wl(B=2, Hq=8, Hkv=2, lens=(512, 512, 512, 300), Lq=Lq, q_offset=q_off), DEV)
    _fwd_check(x, True, window, anchor, labels, ra.RA_FLAG_SPLIT_KV, f"decode Lq={Lq}")


@pytest.mark.parametrize("window,anchor,labels", [(20, 16, None), (0, 0, "packed"), (10, 30, "arbitrary")])
def test_sparse_fp32(window, anchor, labels):
    x = inputs.make(_wl(B=2, d=64, dtype="fp32", lens=(200, 200), Lq=200, q_offset=200), DEV)
    _fwd_check(x, True, window, anchor, labels, 0, "fp32")


def _check_grad(got, ref, what):
    got = got.float().cpu().numpy()
    e = errors(got, ref)
    peak = float(np.abs(ref).max()) if ref.size else 0.0
    msg = f"{what}: {e} peak {peak}"
    assert e["finite"], msg
    assert e["max_abs"] <= 2e-2 * peak + 1e-6, msg
    if e["ref_norm"] > 0:
        assert e["rel_l2"] <= 1e-2, msg


@pytest.mark.parametrize("d,window,anchor,labels", [(128, 32, 64, None), (64, 0, 100, None),
                                                    (128, 0, 0, "packed"), (128, 16, 64, "packed"),
                                                    (64, 8, 32, "arbitrary"), (128, 24, 0, "arbitrary")])
def test_sparse_backward(d, window, anchor, labels):
    x = inputs.make(_wl(B=1, d=d, lens=(256, 256, 256), Lq=256, q_offset=512), DEV)
    chunks = x.chunks()
    q_seg = k_segs = None
    if labels:
        q_seg, k_segs = _labels(x, labels)
    out, st = ra.ring_attn_fwd(x.q, chunks, True, 512, flags=ra.RA_FLAG_NO_SPLIT_KV, want_state=True, window=window,
                               anchor=anchor, q_seg=q_seg, k_segs=k_segs)
    dout = inputs.output_grad(x.wl, DEV)
    dq, grads = ra.ring_attn_bwd(x.q, chunks, out, dout, st, True, 512, window=window, anchor=anchor, q_seg=q_seg,
                                 k_segs=k_segs)
    torch.cuda.synchronize()
    dq_ref, dks, dvs = oracle.attention_bwd(x.q.cpu(), to_host(chunks), dout.cpu(), 512, True, window=window,
                                            anchor=anchor, q_seg=None if q_seg is None else q_seg.cpu(),
                                            k_segs=None if k_segs is None else [k.cpu() for k in k_segs])
    what = f"bwd d={d} W={window} S={anchor} labels={labels}"
    _check_grad(dq, dq_ref, what + " dQ")
    for c in range(3):
        _check_grad(grads[c][0], dks[c], f"{what} dK[{c}]")
        _check_grad(grads[c][1], dvs[c], f"{what} dV[{c}]")


def test_sparse_unsupported_shapes():
    x = inputs.make(_wl(Hq=16, Hkv=1, d=512, lens=(64,), Lq=32, q_offset=32), DEV)
    with pytest.raises(ra.RingAttnError) as e:
        ra.ring_attn_fwd(x.q, x.chunks(), True, 32, anchor=16)
    assert e.value.code == ra.RA_ERR_UNSUPPORTED


def test_sparse_backward_unseen_chunks():
    """Packed documents whose rows see no key of chunks 0 and 1: those
    chunks' dK/dV are written as exact zeros (over NaN-filled buffers), and
    with ACCUMULATE left bitwise as they were; chunk 2 matches the oracle in
    both modes."""
    x = inputs.make(_wl(B=1, d=128, lens=(256, 256, 256), Lq=256, q_offset=512), DEV)
    chunks = x.chunks()
    pos = torch.arange(768, dtype=torch.int32)
    lab = ((pos >= 512).int() + (pos >= 640).int()).unsqueeze(0).to(DEV)
    q_seg = lab[:, 512:].contiguous()
    k_segs = [lab[:, s:s + 256].contiguous() for s in (0, 256, 512)]
    out, st = ra.ring_attn_fwd(x.q, chunks, True, 512, flags=ra.RA_FLAG_NO_SPLIT_KV, want_state=True, q_seg=q_seg,
                               k_segs=k_segs)
    dout = inputs.output_grad(x.wl, DEV)
    dq_ref, dks, dvs = oracle.attention_bwd(x.q.cpu(), to_host(chunks), dout.cpu(), 512, True, q_seg=q_seg.cpu(),
                                            k_segs=[k.cpu() for k in k_segs])
    nan = lambda t: torch.full(t.shape, float("nan"), device=DEV, dtype=torch.float32)
    dq = nan(x.q)
    grads = [(nan(c[0]), nan(c[1])) for c in chunks]
    ra.ring_attn_bwd(x.q, chunks, out, dout, st, True, 512, dq=dq, grads=grads, q_seg=q_seg, k_segs=k_segs)
    torch.cuda.synchronize()
    for c in (0, 1):
        assert torch.count_nonzero(grads[c][0]).item() == 0 and torch.count_nonzero(grads[c][1]).item() == 0, c
    _check_grad(dq, dq_ref, "unseen chunks dQ")
    _check_grad(grads[2][0], dks[2], "unseen chunks dK[2]")
    _check_grad(grads[2][1], dvs[2], "unseen chunks dV[2]")

    g = torch.Generator(device=DEV).manual_seed(9)
    base = lambda t: torch.randn(t.shape, device=DEV, dtype=torch.float32, generator=g)
    dq0 = base(x.q)
    g0 = [(base(c[0]), base(c[1])) for c in chunks]
    dq1 = dq0.clone()
    g1 = [(a.clone(), b.clone()) for a, b in g0]
    ra.ring_attn_bwd(x.q, chunks, out, dout, st, True, 512, flags=ra.RA_FLAG_ACCUMULATE, dq=dq1, grads=g1,
                     q_seg=q_seg, k_segs=k_segs)
    torch.cuda.synchronize()
    for c in (0, 1):
        assert torch.equal(g1[c][0], g0[c][0]) and torch.equal(g1[c][1], g0[c][1]), c
    _check_grad(dq1 - dq0, dq_ref, "accumulated dQ")
    _check_grad(g1[2][0] - g0[2][0], dks[2], "accumulated dK[2]")
    _check_grad(g1[2][1] - g0[2][1], dvs[2], "accumulated dV[2]")

    # the unseen chunks' workgroups return before touching their gradients:
    # -0.0 seeded there stays -0.0 bit for bit (a pass over masked rows would
    # add +0.0 and turn it into +0.0)
    negz = lambda t: torch.full(t.shape, -0.0, device=DEV, dtype=torch.float32)
    gz = [(negz(c[0]), negz(c[1])) for c in chunks]
    ra.ring_attn_bwd(x.q, chunks, out, dout, st, True, 512, flags=ra.RA_FLAG_ACCUMULATE, dq=dq0.clone(), grads=gz,
                     q_seg=q_seg, k_segs=k_segs)
    torch.cuda.synchronize()
    for c in (0, 1):
        for t in gz[c]:
            assert torch.equal(t.view(torch.int32), negz(t).view(torch.int32)), c
