"""HIP graph capture of the C ABI calls: ring_attn_fwd in place, staged
through the library's side stream (events fork and join it), split-KV
decoding with its merge, and ring_attn_bwd.  A captured call is replayed
several times, with other eager work and synchronisation between the
replays, and every replay must reproduce the eager result bit for bit."""
import pytest
import torch

import long_context_blockwise_amd as ra
from long_context_blockwise_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REPLAYS = 3


def _wl(lens, Lq, q_offset, Hq=4, Hkv=2, d=128, seed=61):
    return inputs.Workload("graph_case", B=1, Hq=Hq, Hkv=Hkv, d_qk=d, d_v=d, dtype="bf16", chunk_len=lens[0],
                           P=len(lens), Lq=Lq, q_offset=q_offset, causal=True, std=0.5, seed=seed,
                           chunk_lens=tuple(lens))


def _capture(fn):
    """Warm fn up on a side stream (as torch recommends before capture), then capture it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        res = fn()
    return g, res


def _replay_and_check(g, captured, eager, disturb):
    for r in range(REPLAYS):
        disturb()  # other eager work between replays
        for t in captured:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (c, e) in enumerate(zip(captured, eager)):
            assert torch.equal(c, e), f"replay {r}: output {i} differs from the eager call"


@pytest.mark.parametrize("flags", [ra.RA_FLAG_NO_SPLIT_KV, ra.RA_FLAG_NO_SPLIT_KV | ra.RA_FLAG_STAGE],
                         ids=["inplace", "staged"])
def test_graph_forward(flags):
    lens = (256, 192, 256, 256)
    x = inputs.make(_wl(lens, Lq=256, q_offset=704), DEV)
    chunks = x.chunks([3, 2, 1, 0])

    def call():
        out, state = ra.ring_attn_fwd(x.q, chunks, True, 704, flags=flags, want_state=True)
        return (out,) + tuple(state)

    eager = call()
    torch.cuda.synchronize()
    g, captured = _capture(call)
    _replay_and_check(g, captured, eager, lambda: ra.ring_attn_fwd(x.q, chunks[:2], True, 704, flags=flags))


def test_graph_decode_split_and_merge():
    lens = (512, 512, 512, 300)
    x = inputs.make(_wl(lens, Lq=4, q_offset=sum(lens) - 4, Hq=8), DEV)
    chunks = x.chunks()

    def call():
        out, _ = ra.ring_attn_fwd(x.q, chunks, True, sum(lens) - 4, flags=ra.RA_FLAG_SPLIT_KV)
        return (out,)

    eager = call()
    torch.cuda.synchronize()
    g, captured = _capture(call)
    _replay_and_check(g, captured, eager, lambda: ra.ring_attn_fwd(x.q, chunks[:1], True, sum(lens) - 4))


def test_graph_backward():
    lens = (256, 256, 256)
    x = inputs.make(_wl(lens, Lq=256, q_offset=512), DEV)
    chunks = x.chunks()
    out, st = ra.ring_attn_fwd(x.q, chunks, True, 512, flags=ra.RA_FLAG_NO_SPLIT_KV, want_state=True)
    dout = inputs.output_grad(x.wl, DEV)

    def call():
        dq, grads = ra.ring_attn_bwd(x.q, chunks, out, dout, st, True, 512)
        return (dq,) + tuple(t for pair in grads for t in pair)

    eager = call()
    torch.cuda.synchronize()
    g, captured = _capture(call)
    _replay_and_check(g, captured, eager, lambda: ra.ring_attn_bwd(x.q, chunks[:1], out, dout, st, True, 512))
