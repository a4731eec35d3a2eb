"""ring_attn_fwd_noalloc (the entry point on the library's static per-GPU
scratch) against ring_attn_fwd with a caller workspace, through the C ABI:
the same kernels on the same inputs must give the same bits, and both the
oracle's result within the bf16 bounds.  Each case makes two calls in a row,
the second with a smaller input, so the second runs on the scratch the first
left behind."""
import numpy as np
import pytest
import torch

import long_context_blockwise_amd as ra
from long_context_blockwise_amd import inputs
from parity import check, oracle_out, oracle_state

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _wl(B, Hq, Hkv, d, lens, Lq, q_offset, causal=True, seed=31):
    return inputs.Workload("noalloc", B=B, Hq=Hq, Hkv=Hkv, d_qk=d, d_v=d, dtype="bf16", chunk_len=lens[0],
                           P=len(lens), Lq=Lq, q_offset=q_offset, causal=causal, std=0.5, seed=seed,
                           chunk_lens=tuple(lens))


def _both(x, flags, want_state, order=None):
    """(workspace call, no-alloc call) outputs and states on the same inputs."""
    wl = x.wl
    chunks = x.chunks(order)
    ws_bytes = ra.ring_attn_workspace_size(x.q, chunks, wl.causal, wl.q_offset, flags, want_state)
    assert 0 < ws_bytes <= ra.RA_NOALLOC_SCRATCH_BYTES, ws_bytes
    res = []
    for noalloc in (False, True):
        out = torch.full((wl.B, wl.Lq, wl.Hq, wl.d_v), float("nan"), device=DEV, dtype=torch.bfloat16)
        st = None
        if want_state:
            st = (torch.full((wl.B, wl.Lq, wl.Hq), float("nan"), device=DEV),
                  torch.full((wl.B, wl.Lq, wl.Hq), float("nan"), device=DEV),
                  torch.full((wl.B, wl.Lq, wl.Hq, wl.d_v), float("nan"), device=DEV))
        if noalloc:
            ra.ring_attn_fwd_noalloc(x.q, chunks, wl.causal, wl.q_offset, flags=flags, out=out, state=st)
        else:
            ra.ring_attn_fwd(x.q, chunks, wl.causal, wl.q_offset, flags=flags, out=out, state=st)
        torch.cuda.synchronize()
        res.append((out, st))
    return res


def _same(a, b, what):
    assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), what


@pytest.mark.parametrize("case", ["decode", "staged"])
def test_noalloc_matches_workspace_entry_point(case):
    if case == "decode":
        # split-KV partials in the scratch: 1M-context decode in miniature
        # (GQA 4, 16 new tokens at the end of the cache), then a smaller one
        shapes = [_wl(2, 8, 2, 128, (2048,) * 8, 16, 8 * 2048 - 16),
                  _wl(1, 4, 1, 128, (1024, 1024, 700), 5, 2748 - 5, seed=32)]
        flags, want_state, orders = 0, True, [None, None]
    else:
        # the staged ring: both staging buffers in the scratch (device 3 of 4),
        # then device 1 of 3 with shorter, ragged chunks
        shapes = [_wl(1, 8, 2, 128, (512,) * 4, 512, 3 * 512),
                  _wl(1, 4, 4, 64, (300, 300, 211), 300, 300, seed=33)]
        flags, want_state = ra.RA_FLAG_STAGE, False
        orders = [ra.ring_attn_ring_order(3, 4), ra.ring_attn_ring_order(1, 3)]
    for i, (wl, order) in enumerate(zip(shapes, orders)):
        x = inputs.make(wl, DEV)
        (o_ws, s_ws), (o_na, s_na) = _both(x, flags, want_state, order)
        _same(o_na, o_ws, f"{case} call {i}: out")
        if want_state:
            for a, b, n in zip(s_na, s_ws, "mlO"):
                _same(a, b, f"{case} call {i}: {n}")
        ref, _ = oracle_out(x.q, x.chunks(), wl.q_offset, wl.causal)
        check(o_na.float().cpu().numpy(), ref, "bf16", f"{case} call {i} vs oracle")
        if want_state:
            m, l, O = oracle_state(x.q, x.chunks(), wl.q_offset, wl.causal)
            check(s_na[0].cpu().numpy(), m, "bf16", f"{case} call {i}: m", rel_l2=False)
            np.testing.assert_allclose(s_na[1].cpu().numpy(), l, rtol=1e-2)


def test_noalloc_refuses_calls_beyond_its_scratch():
    """A staged ring whose staging buffers exceed the static scratch is
    refused with RA_ERR_WORKSPACE before anything runs; the entry point then
    works again."""
    wl = _wl(1, 8, 8, 128, (49152,) * 2, 16384, 49152)  # 2 x 2 x 96 MiB staging
    x = inputs.make(wl, DEV)
    chunks = x.chunks([1, 0])
    assert ra.ring_attn_workspace_size(x.q, chunks, True, wl.q_offset, ra.RA_FLAG_STAGE) > ra.RA_NOALLOC_SCRATCH_BYTES
    out = torch.zeros((1, wl.Lq, 8, 128), device=DEV, dtype=torch.bfloat16)
    with pytest.raises(ra.RingAttnError) as e:
        ra.ring_attn_fwd_noalloc(x.q, chunks, True, wl.q_offset, flags=ra.RA_FLAG_STAGE, out=out)
    assert e.value.code == ra.RA_ERR_WORKSPACE and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0  # nothing was enqueued
    small = inputs.make(_wl(1, 2, 1, 128, (256, 256), 64, 512 - 64), DEV)
    o2 = torch.empty((1, 64, 2, 128), device=DEV, dtype=torch.bfloat16)
    ra.ring_attn_fwd_noalloc(small.q, small.chunks([1, 0]), True, 512 - 64, flags=ra.RA_FLAG_STAGE, out=o2)
    torch.cuda.synchronize()
    ref, _ = oracle_out(small.q, small.chunks(), 512 - 64, True)
    check(o2.float().cpu().numpy(), ref, "bf16", "after the refusal")
