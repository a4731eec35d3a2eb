"""Backward (dQ, dK, dV) on the GPU against the oracle's gradients of the
attention definition, through the C ABI: causal and non-causal, windows,
GQA, ragged chunks and tails, d = 64 and 128, rows that see no key; the
accumulate flag, per-chunk calls, determinism, and a two-device ring whose
dK/dV travel with their chunks; 512-wide heads at small sizes, and the
d = 512 workload at full size (dQ of sampled rows of one head against the
oracle, dK and dV through identities that hold at any size).

Tolerance: the kernels round P and dS to bf16 for the matrix cores (unit
roundoff 2^-8) and accumulate in fp32; like the forward output this gives a
relative L2 error of a few 1e-3.  Each gradient must have relative L2 error
<= 1e-2 and max-abs error <= 2e-2 of its largest reference magnitude."""
import numpy as np
import pytest
import torch

import long_context_blockwise_amd as ra
import oracle
from long_context_blockwise_amd import inputs
from parity import errors, to_host

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _wl(B=1, Hq=4, Hkv=2, d=128, lens=(256, 256), Lq=256, q_offset=0, causal=True, seed=21):
    return inputs.Workload("bwd_case", B=B, Hq=Hq, Hkv=Hkv, d_qk=d, d_v=d, dtype="bf16",
                           chunk_len=lens[0], P=len(lens), Lq=Lq, q_offset=q_offset, causal=causal,
                           std=0.5, seed=seed, chunk_lens=tuple(lens))


def check_grad(got, ref, what):
    got = got.float().cpu().numpy() if hasattr(got, "cpu") else got
    e = errors(got, ref)
    peak = float(np.abs(ref).max()) if ref.size else 0.0
    msg = f"{what}: {e} peak {peak}"
    assert e["finite"], msg
    assert e["max_abs"] <= 2e-2 * peak + 1e-6, msg
    if e["ref_norm"] > 0:
        assert e["rel_l2"] <= 1e-2, msg
    return e


def forward(x, causal, q_off, window, chunks=None):
    chunks = x.chunks() if chunks is None else chunks
    out, st = ra.ring_attn_fwd(x.q, chunks, causal, q_off, flags=ra.RA_FLAG_NO_SPLIT_KV, want_state=True,
                               window=window)
    return out, st


def run_case(x, causal, q_off, window, what, order=None):
    chunks = x.chunks(order)
    out, st = forward(x, causal, q_off, window, chunks)
    dout = inputs.output_grad(x.wl, DEV)
    dq, grads = ra.ring_attn_bwd(x.q, chunks, out, dout, st, causal, q_off, window=window)
    torch.cuda.synchronize()
    dq_ref, dks, dvs = oracle.attention_bwd(x.q.cpu(), to_host(chunks), dout.cpu(), q_off, causal, window=window)
    check_grad(dq, dq_ref, what + " dQ")
    for c, ((gk, gv), rk, rv) in enumerate(zip(grads, dks, dvs)):
        check_grad(gk, rk, f"{what} dK[{c}]")
        check_grad(gv, rv, f"{what} dV[{c}]")
    return out, st, dout, dq, grads


CASES = [
    # B, d, Hq, Hkv, lens, Lq, q_offset, causal, window
    (1, 128, 4, 2, (256, 256, 256), 256, 512, True, 0),   # query chunk = last chunk
    (2, 128, 4, 4, (192, 320), 200, 250, True, 0),        # ragged, offset mid-chunk
    (1, 64, 8, 2, (64, 100, 37), 129, 72, True, 0),       # tails of 1 row / odd keys
    (1, 128, 2, 1, (300,), 257, 43, False, 0),
    (1, 128, 16, 1, (128, 128), 127, 129, True, 0),       # GQA 16, tile boundary +1
    (2, 64, 4, 2, (256, 256), 256, 256, True, 0),
    (1, 128, 4, 2, (256, 256, 256), 256, 512, True, 100),  # causal window across a chunk edge
    (1, 128, 4, 2, (200, 170), 180, 100, False, 40),      # two-sided window
    (1, 64, 2, 2, (77, 130), 300, 0, False, 65),          # rows past every window: no key
    (1, 128, 4, 4, (256,), 255, 0, True, 0),              # diagonal at position 0
    # 512-wide heads: four waves split the head dimension
    (1, 512, 4, 1, (96, 160), 100, 150, True, 0),         # GQA 4, ragged, offset mid-chunk
    (1, 512, 2, 1, (64, 33), 65, 0, True, 0),             # diagonal at position 0, 1-row tails
    (1, 512, 16, 1, (64, 64), 40, 90, True, 30),          # GQA 16, causal window
    (2, 512, 2, 2, (70,), 50, 10, False, 0),              # non-causal, two sequences
    (1, 512, 2, 2, (77, 50), 200, 0, False, 40),          # two-sided window; rows past every key see none
]


@pytest.mark.parametrize("B,d,Hq,Hkv,lens,Lq,q_off,causal,window", CASES)
def test_bwd_matches_oracle(B, d, Hq, Hkv, lens, Lq, q_off, causal, window):
    x = inputs.make(_wl(B=B, Hq=Hq, Hkv=Hkv, d=d, lens=lens, Lq=Lq, q_offset=q_off, causal=causal), DEV)
    order = list(range(len(lens)))[::-1]
    run_case(x, causal, q_off, window, f"B{B} d{d} Hq{Hq}/{Hkv} {lens} Lq{Lq} off{q_off} c{causal} w{window}",
             order)


@pytest.mark.parametrize("d", [128, 512])
def test_bwd_accumulate_chunkwise_and_deterministic(d):
    """Per-chunk calls adding into dq equal the all-chunk call; ACCUMULATE on
    the same inputs doubles every gradient (exactly for dK/dV, which one
    launch per chunk writes; dq of chunks of different lengths is summed
    over several launches, so its additions round in another order);
    repeated calls are bitwise equal."""
    x = inputs.make(_wl(d=d, lens=(256, 192, 256), Lq=256, q_offset=448, causal=True), DEV)
    chunks = x.chunks()
    out, st = forward(x, True, 448, 0)
    dout = inputs.output_grad(x.wl, DEV)
    dq, grads = ra.ring_attn_bwd(x.q, chunks, out, dout, st, True, 448)
    dq2, grads2 = ra.ring_attn_bwd(x.q, chunks, out, dout, st, True, 448)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and all(torch.equal(a, b) for p, q in zip(grads, grads2) for a, b in zip(p, q))
    ra.ring_attn_bwd(x.q, chunks, out, dout, st, True, 448, flags=ra.RA_FLAG_ACCUMULATE, dq=dq2, grads=grads2)
    torch.cuda.synchronize()
    e = errors(dq2.cpu().numpy(), 2 * dq.cpu().numpy())
    assert e["rel_l2"] <= 1e-6, e
    assert all(torch.equal(b, 2 * a) for p, q in zip(grads, grads2) for a, b in zip(p, q))
    # one chunk per call (a ring step each), dq summed with ACCUMULATE
    dq_acc = torch.zeros_like(dq)
    for c in (2, 0, 1):
        _, [(gk, gv)] = ra.ring_attn_bwd(x.q, [chunks[c]], out, dout, st, True, 448, flags=ra.RA_FLAG_ACCUMULATE,
                                       dq=dq_acc, grads=[tuple(torch.zeros_like(t) for t in grads[c])])
        torch.cuda.synchronize()
        assert torch.equal(gk, grads[c][0]) and torch.equal(gv, grads[c][1])
    e = errors(dq_acc.cpu().numpy(), dq.cpu().numpy())
    assert e["rel_l2"] <= 1e-6, e


def test_bwd_two_device_ring():
    """Two devices of a causal ring, each holding one query chunk: each runs
    its forward over the chunks in ring order, then its backward, adding its
    share into the dK/dV buffers that travel with each KV chunk.  The
    gathered dQ and the travelled dK/dV equal the oracle's gradients of
    attention over the whole sequence."""
    L, H, d = 192, 4, 128
    wl = _wl(B=1, Hq=H, Hkv=2, d=d, lens=(L, L), Lq=2 * L, q_offset=0, causal=True, seed=33)
    x = inputs.make(wl, DEV)
    dout_all = inputs.output_grad(wl, DEV)
    chunks = x.chunks()
    grads = [(torch.zeros(c[0].shape, device=DEV), torch.zeros(c[1].shape, device=DEV)) for c in chunks]
    dqs = []
    for dev in range(2):
        q = x.q[:, dev * L:(dev + 1) * L].contiguous()
        g = dout_all[:, dev * L:(dev + 1) * L].contiguous()
        order = ra.ring_attn_ring_order(dev, 2)
        ring = [chunks[c] for c in order]
        out, st = ra.ring_attn_fwd(q, ring, True, dev * L, flags=ra.RA_FLAG_NO_SPLIT_KV, want_state=True)
        dq, _ = ra.ring_attn_bwd(q, ring, out, g, st, True, dev * L, flags=ra.RA_FLAG_ACCUMULATE,
                                 dq=torch.zeros(q.shape, device=DEV), grads=[grads[c] for c in order])
        dqs.append(dq)
    torch.cuda.synchronize()
    dq_ref, dks, dvs = oracle.attention_bwd(x.q.cpu(), to_host(chunks), dout_all.cpu(), 0, True)
    check_grad(torch.cat(dqs, 1), dq_ref, "ring dQ")
    for c in range(2):
        check_grad(grads[c][0], dks[c], f"ring dK[{c}]")
        check_grad(grads[c][1], dvs[c], f"ring dV[{c}]")


def test_bwd_empty_and_skipped_chunks():
    """A chunk no row can see gets zero gradients (or keeps what it had under
    ACCUMULATE); an empty query block gives zero dK/dV."""
    x = inputs.make(_wl(lens=(128, 128, 128), Lq=64, q_offset=100, causal=True), DEV)
    chunks = x.chunks()
    out, st = forward(x, True, 100, 0)
    dout = inputs.output_grad(x.wl, DEV)
    _, grads = ra.ring_attn_bwd(x.q, chunks, out, dout, st, True, 100)
    torch.cuda.synchronize()
    assert float(grads[2][0].abs().max()) == 0.0 and float(grads[2][1].abs().max()) == 0.0
    assert float(grads[0][0].abs().max()) > 0.0
    keep = [(torch.full_like(a, 3.0), torch.full_like(b, 3.0)) for a, b in grads]
    ra.ring_attn_bwd(x.q, chunks, out, dout, st, True, 100, flags=ra.RA_FLAG_ACCUMULATE,
                     dq=torch.zeros_like(x.q, dtype=torch.float32), grads=keep)
    torch.cuda.synchronize()
    assert bool((keep[2][0] == 3.0).all()) and bool((keep[2][1] == 3.0).all())
    # an empty query block: nothing sees the keys
    q0 = x.q[:, :0]
    m0 = torch.zeros((1, 0, 4), device=DEV)
    _, g0 = ra.ring_attn_bwd(q0, chunks, q0, q0, (m0, m0), True, 100)
    torch.cuda.synchronize()
    assert all(float(t.abs().max()) == 0.0 for pair in g0 for t in pair)


def test_bwd_full_size_head_slice():
    """The bench's backward at full size (32 heads, d = 128, 4 x 8192 chunks,
    query chunk 3, causal, chunks in ring order): every dQ, dK, dV element of
    one head against the oracle run on that head alone."""
    wl = inputs.WORKLOADS["prefill_bf16_h32_d128"]
    x = inputs.make(wl, DEV)
    order = ra.ring_attn_ring_order(wl.q_offset // wl.chunk_len, wl.P)
    chunks = x.chunks(order)
    out, st = ra.ring_attn_fwd(x.q, chunks, True, wl.q_offset, flags=ra.RA_FLAG_NO_SPLIT_KV, want_state=True)
    dout = inputs.output_grad(wl, DEV)
    dq, grads = ra.ring_attn_bwd(x.q, chunks, out, dout, st, True, wl.q_offset)
    torch.cuda.synchronize()
    h = 13
    qh = x.q[:, :, h:h + 1].cpu().contiguous()
    ch = [(k[:, :, h:h + 1].cpu().contiguous(), v[:, :, h:h + 1].cpu().contiguous(), s) for (k, v, s) in chunks]
    dq_ref, dks, dvs = oracle.attention_bwd(qh, ch, dout[:, :, h:h + 1].cpu().contiguous(), wl.q_offset, True)
    check_grad(dq[:, :, h:h + 1], dq_ref, f"full-size dQ head {h}")
    for c in range(len(chunks)):
        check_grad(grads[c][0][:, :, h:h + 1], dks[c], f"full-size dK[{c}] head {h}")
        check_grad(grads[c][1][:, :, h:h + 1], dvs[c], f"full-size dV[{c}] head {h}")


def test_bwd_full_size_d512():
    """The d = 512 workload's backward at full size (16 query heads on one KV
    head, 8 x 16384 keys, query chunk 7, causal).  dQ of sampled rows of one
    query head against the oracle run on those rows alone (a row's dQ needs
    only its own softmax).  dK and dV through identities of the definition:
    the dS of a row sums to 0 over the keys it sees, so the dK of all keys
    sum to 0; its P sums to 1, so the dV of all keys sum to the dO of all
    rows of the group."""
    wl = inputs.WORKLOADS["mla_h16_d512"]
    x = inputs.make(wl, DEV)
    order = ra.ring_attn_ring_order(wl.q_offset // wl.chunk_len, wl.P)
    chunks = x.chunks(order)
    out, st = ra.ring_attn_fwd(x.q, chunks, True, wl.q_offset, flags=ra.RA_FLAG_NO_SPLIT_KV, want_state=True)
    dout = inputs.output_grad(wl, DEV)
    dq, grads = ra.ring_attn_bwd(x.q, chunks, out, dout, st, True, wl.q_offset)
    torch.cuda.synchronize()
    h = 5
    rows = inputs.sample_rows(wl.Lq, tile=2048, seed=7, extra=(0, 31, 32, wl.Lq - 33, wl.Lq - 1))
    print(f"[bwd d512] {len(rows)} sampled rows of head {h}", flush=True)
    # (bf16 bits as uint16 arrays, converted once for all the per-row calls)
    ch = [(k.cpu().view(torch.int16).numpy().view(np.uint16), v.cpu().view(torch.int16).numpy().view(np.uint16), st_)
          for (k, v, st_) in chunks]
    got = dq[0, rows, h].cpu().numpy()
    want = []
    for t in rows:
        qt = x.q[:, t:t + 1, h:h + 1].cpu().contiguous()
        gt = dout[:, t:t + 1, h:h + 1].cpu().contiguous()
        dq_ref, _, _ = oracle.attention_bwd(qt, ch, gt, wl.q_offset + t, True)
        want.append(dq_ref[0, 0, 0])
    check_grad(got, np.stack(want), "full-size d512 dQ (sampled rows)")
    dk_sum = sum(g[0].double().sum(dim=(0, 1)) for g in grads)  # [Hkv, d]
    dk_abs = sum(g[0].double().abs().sum(dim=(0, 1)) for g in grads)
    rel = float(dk_sum.norm() / dk_abs.norm())
    assert rel <= 1e-2, f"sum of dK over all keys: {rel} of the summed magnitudes"
    dv_sum = sum(g[1].double().sum(dim=(0, 1)) for g in grads)
    do_sum = dout.double().sum(dim=(0, 1)).reshape(wl.Hkv, wl.Hq // wl.Hkv, -1).sum(dim=1)
    e = errors(dv_sum.cpu().numpy(), do_sum.cpu().numpy())
    assert e["rel_l2"] <= 1e-2, f"sum of dV over all keys against the sum of dO: {e}"
    print(f"[bwd d512] dK sum {rel:.2e}, dV sum {e}", flush=True)
