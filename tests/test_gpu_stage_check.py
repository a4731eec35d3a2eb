"""The staged ring (the stand-in for receiving KV chunks from the ring
neighbour) under perturbations of its timing: the side stream delayed
before every staging copy, the compute stream delayed before every launch,
and every staging buffer overwritten with NaN right after the step that
read it.  Correct ordering (a step reads its buffer only after the copy
into it, a copy refills a buffer only after the step that read it) gives
the same bits with each of them; a missing wait would read stale chunks or
NaN.  Page "Ring Attention：百万 Token 上下文的秘密", §3.2 通信-计算重叠."""
import pytest
import torch

import long_context_blockwise_amd as ra
from long_context_blockwise_amd import inputs
from parity import check, oracle_out

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "fp32")])
def test_staged_ring_under_perturbations(d, dtype):
    P, n = 6, 384
    dev = P - 1  # the last device: every chunk visible, buffers reused twice
    wl = inputs.Workload("stagecheck", B=1, Hq=8, Hkv=2, d_qk=d, d_v=d, dtype=dtype, chunk_len=n, P=P, Lq=n,
                         q_offset=dev * n, causal=True, std=0.5, seed=41)
    x = inputs.make(wl, DEV)
    order = ra.ring_attn_ring_order(dev, P)
    chunks = x.chunks(order)
    ctx = ra.RingAttnContext(0)
    outs = {}
    settings = {
        "plain": 0,
        "delay_copy": ra.RA_CHECK_DELAY_COPY,
        "delay_compute": ra.RA_CHECK_DELAY_COMPUTE,
        "poison": ra.RA_CHECK_POISON,
        "all": ra.RA_CHECK_DELAY_COPY | ra.RA_CHECK_DELAY_COMPUTE | ra.RA_CHECK_POISON,
    }
    for name, checks in settings.items():
        ctx.set_check(checks, 300)
        out = torch.full((1, n, 8, d), float("nan"), device=DEV, dtype=x.q.dtype)
        for _ in range(2):  # the second call reuses the buffers the first one poisoned
            ra.ring_attn_fwd(x.q, chunks, True, wl.q_offset, flags=ra.RA_FLAG_STAGE, out=out, ctx=ctx)
        torch.cuda.synchronize()
        outs[name] = out
    ctx.set_check(0, 0)
    ref, _ = oracle_out(x.q, x.chunks(), wl.q_offset, True)
    check(outs["plain"].float().cpu().numpy(), ref, dtype, "plain staged ring")
    for name, out in outs.items():
        assert torch.isfinite(out.float()).all(), name
        assert torch.equal(out, outs["plain"]), f"{name} changed the output"
