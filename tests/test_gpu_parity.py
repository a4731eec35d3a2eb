"""HIP path vs the CPU oracle, element by element, at sizes the oracle runs in
seconds (several tiles, ragged tails, boundary offsets), through the C ABI."""
import numpy as np
import pytest
import torch

import long_context_blockwise_amd as ra
from long_context_blockwise_amd import inputs
from parity import check, oracle_out, oracle_state, errors

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def wl_of(name="t", B=1, Hq=4, Hkv=2, d=128, dtype="bf16", lens=(256, 256), Lq=256, q_offset=0,
          causal=True, std=0.5, seed=7):
    return inputs.Workload(name, B=B, Hq=Hq, Hkv=Hkv, d_qk=d, d_v=d, dtype=dtype,
                           chunk_len=lens[0], P=len(lens), Lq=Lq, q_offset=q_offset,
                           causal=causal, std=std, seed=seed, chunk_lens=tuple(lens))


def run(x, order=None, flags=0, want_state=False, causal=None):
    wl = x.wl
    causal = wl.causal if causal is None else causal
    out, st = ra.ring_attn_fwd(x.q, x.chunks(order), causal=causal, q_offset=wl.q_offset,
                               flags=flags, want_state=want_state)
    torch.cuda.synchronize()
    return out, st


def test_tiny_ring_fp32_every_device():
    """1 head, d=64, fp32, 4 chunks of 256, non-causal: every device of the
    4-device ring (its query chunk against the chunks in its ring order)."""
    base = inputs.WORKLOADS["tiny_ring_fp32"]
    for dev in range(4):
        wl = base.scaled(q_offset=dev * 256)
        x = inputs.make(wl, DEV)
        # query chunk `dev` of the sequence: draw a distinct query per device
        x.q = inputs.draw((1, 256, 1, 64), 1.0, torch.float32, DEV, wl.seed + 10 * dev, 0)
        ref, _ = oracle_out(x.q, x.chunks(), wl.q_offset, False)
        order = ra.ring_attn_ring_order(dev, 4)
        for flags in (0, ra.RA_FLAG_STAGE):
            out, _ = run(x, order, flags)
            check(out.cpu().numpy(), ref, "fp32", f"device {dev} flags {flags}")


SWEEP = [
    # d, Hq, Hkv, lens, Lq, q_offset, causal
    (128, 4, 2, (256, 256, 256), 256, 512, True),     # query chunk = last chunk
    (128, 4, 4, (192, 320), 200, 250, True),          # ragged, offset mid-chunk
    (128, 8, 2, (64, 100, 37), 129, 72, True),        # tails of 1 row / odd keys
    (128, 2, 1, (300,), 257, 43, False),
    (128, 16, 1, (128, 128), 127, 129, True),         # GQA 16, tile boundary +1
    (128, 4, 4, (256,), 255, 0, True),                # diagonal at position 0
    (64, 4, 2, (256, 256), 256, 256, True),
    (64, 2, 2, (77, 130), 300, 0, True),              # some rows see few keys
    (512, 16, 1, (96, 64), 128, 96, True),            # MLA-style: 16 heads, one 512-wide KV head
    (512, 4, 1, (50,), 33, 20, False),
]


@pytest.mark.parametrize("d,Hq,Hkv,lens,Lq,q_off,causal", SWEEP)
@pytest.mark.parametrize("flags", [0, 1], ids=["inplace", "staged"])
def test_bf16_sweep(d, Hq, Hkv, lens, Lq, q_off, causal, flags):
    wl = wl_of(B=2 if d < 512 else 1, Hq=Hq, Hkv=Hkv, d=d, lens=lens, Lq=Lq, q_offset=q_off,
               causal=causal, std=0.5 if d < 512 else 4 / 512 ** 0.5)
    x = inputs.make(wl, DEV)
    ref, _ = oracle_out(x.q, x.chunks(), q_off, causal)
    order = list(range(len(lens)))[::-1]
    out, _ = run(x, order, flags | ra.RA_FLAG_NO_SPLIT_KV)
    check(out.float().cpu().numpy(), ref, "bf16", f"d={d} lens={lens} Lq={Lq} off={q_off}")


@pytest.mark.parametrize("d", [64, 128, 512])
def test_peaky_logits_rescale(d):
    """Large logits (query x20) move the softmax reference often and from
    chunk to chunk; chunk order increasing and decreasing in max."""
    wl = wl_of(B=1, Hq=2, Hkv=1, d=d, lens=(128, 128, 128), Lq=128, q_offset=384, causal=True,
               std=0.5 if d < 512 else 4 / 512 ** 0.5)
    x = inputs.make(wl, DEV)
    x.q = (x.q.float() * 20).to(torch.bfloat16)
    ref, _ = oracle_out(x.q, x.chunks(), wl.q_offset, True)
    for order in ([0, 1, 2], [2, 1, 0]):
        out, _ = run(x, order, ra.RA_FLAG_NO_SPLIT_KV)
        check(out.float().cpu().numpy(), ref, "bf16", f"peaky d={d} order={order}")


@pytest.mark.parametrize("Lq,G,B", [(1, 1, 1), (1, 4, 2), (4, 4, 1), (16, 4, 4), (16, 1, 2), (7, 8, 1),
                                    (16, 16, 1)])
def test_decode_split_kv(Lq, G, B):
    """Incremental decoding: Lq new tokens at cache_idx attend causally to a
    cache whose last Lq slots are their own keys; split-KV partials + merge."""
    lens = (512, 512, 512, 300)
    cache = sum(lens)
    d = 128
    wl = wl_of(B=B, Hq=2 * G, Hkv=2, d=d, lens=lens, Lq=Lq, q_offset=cache - Lq, causal=True)
    x = inputs.make(wl, DEV)
    ref, _ = oracle_out(x.q, x.chunks(), wl.q_offset, True)
    out, _ = run(x)  # Lq <= 16: split-KV by default
    check(out.float().cpu().numpy(), ref, "bf16", f"decode Lq={Lq} G={G}")
    out2, _ = run(x, flags=ra.RA_FLAG_NO_SPLIT_KV)
    check(out2.float().cpu().numpy(), ref, "bf16", "decode via ring schedule")


@pytest.mark.parametrize("dtype,d,Hq,Hkv", [("bf16", 128, 16, 8), ("fp32", 64, 8, 8)])
def test_decode_split_kv_many_chunks(dtype, d, Hq, Hkv):
    """Split-KV decoding over 129 chunks: launches of 64 chunks, a launch of
    one ragged last chunk, and a merge of 129 partial states per row (split
    over thread groups)."""
    lens = (128,) * 128 + (100,)
    cache = sum(lens)
    Lq = 4
    wl = wl_of(B=2, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, lens=lens, Lq=Lq, q_offset=cache - Lq, causal=True,
               std=0.5 if dtype == "bf16" else 1.0)
    x = inputs.make(wl, DEV)
    ref, _ = oracle_out(x.q, x.chunks(), wl.q_offset, True)
    out, _ = run(x, flags=ra.RA_FLAG_SPLIT_KV)
    got = out.float().cpu().numpy() if dtype == "bf16" else out.cpu().numpy()
    check(got, ref, dtype, f"decode {dtype} over {len(lens)} chunks")


def test_decode_fp32_and_d512_split():
    wl = wl_of(B=1, Hq=16, Hkv=1, d=512, lens=(256, 256), Lq=8, q_offset=504, causal=True,
               std=4 / 512 ** 0.5)
    x = inputs.make(wl, DEV)
    ref, _ = oracle_out(x.q, x.chunks(), wl.q_offset, True)
    out, _ = run(x, flags=ra.RA_FLAG_SPLIT_KV)
    check(out.float().cpu().numpy(), ref, "bf16", "d512 split")
    wl = wl_of(B=2, Hq=4, Hkv=2, d=64, dtype="fp32", lens=(200, 200), Lq=5, q_offset=395, std=1.0)
    x = inputs.make(wl, DEV)
    ref, _ = oracle_out(x.q, x.chunks(), wl.q_offset, True)
    out, _ = run(x, flags=ra.RA_FLAG_SPLIT_KV)
    check(out.cpu().numpy(), ref, "fp32", "fp32 split")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp32", 128), ("bf16", 512)])
def test_state_outputs(dtype, d):
    """Exported (m, l, O) equal the oracle's running state after all chunks
    (m = running max in natural units, l and O relative to it)."""
    std = 1.0 if dtype == "fp32" else (0.5 if d < 512 else 4 / 512 ** 0.5)
    wl = wl_of(B=1, Hq=4, Hkv=2 if d < 512 else 1, d=d, dtype=dtype, lens=(128, 160), Lq=96,
               q_offset=200, causal=True, std=std)
    x = inputs.make(wl, DEV)
    m_ref, l_ref, O_ref = oracle_state(x.q, x.chunks(), wl.q_offset, True)
    for flags in (ra.RA_FLAG_NO_SPLIT_KV, ra.RA_FLAG_STAGE):
        _, (m, l, O) = run(x, flags=flags, want_state=True)
        m, l, O = m.cpu().numpy(), l.cpu().numpy(), O.cpu().numpy()
        # m is the exact running max of bf16-input logits (fp32 accumulation)
        tol_m = 1e-5 if dtype == "fp32" else 2e-3
        assert np.abs(m - m_ref).max() <= tol_m * (1 + np.abs(m_ref).max())
        # compare l and O relative to the same max
        scale = np.exp(m_ref - m)
        rel = np.abs(l * scale - l_ref) / l_ref
        assert rel.max() <= (1e-5 if dtype == "fp32" else 1e-2), rel.max()
        check(O / l[..., None], O_ref / l_ref[..., None], dtype, f"O/l flags={flags}")


def test_resume_and_merge():
    """State after chunks [0, k) continued with ACCUMULATE over [k, P), and
    two independent partial states merged with ring_attn_merge, both equal
    one pass over all chunks (the merge is the fusion layer's global
    normalisation)."""
    wl = wl_of(B=2, Hq=4, Hkv=2, d=128, lens=(128, 96, 160, 64), Lq=100, q_offset=450, causal=True)
    x = inputs.make(wl, DEV)
    ref, _ = oracle_out(x.q, x.chunks(), wl.q_offset, True)
    ch = x.chunks()
    _, st = ra.ring_attn_fwd(x.q, ch[:2], True, wl.q_offset, want_state=True, want_out=False,
                             flags=ra.RA_FLAG_NO_SPLIT_KV)
    out, st2 = ra.ring_attn_fwd(x.q, ch[2:], True, wl.q_offset, state=st,
                                flags=ra.RA_FLAG_ACCUMULATE | ra.RA_FLAG_STAGE)
    torch.cuda.synchronize()
    check(out.float().cpu().numpy(), ref, "bf16", "resume")
    _, a = ra.ring_attn_fwd(x.q, ch[:2], True, wl.q_offset, want_state=True, want_out=False,
                            flags=ra.RA_FLAG_NO_SPLIT_KV)
    _, b = ra.ring_attn_fwd(x.q, ch[2:], True, wl.q_offset, want_state=True, want_out=False,
                            flags=ra.RA_FLAG_NO_SPLIT_KV)
    B, Lq, Hq, dv = out.shape
    m = torch.stack([a[0].reshape(-1), b[0].reshape(-1)])
    l = torch.stack([a[1].reshape(-1), b[1].reshape(-1)])
    O = torch.stack([a[2].reshape(-1, dv), b[2].reshape(-1, dv)])
    merged, _ = ra.ring_attn_merge(m, l, O, torch.bfloat16)
    torch.cuda.synchronize()
    check(merged.reshape(B, Lq, Hq, dv).float().cpu().numpy(), ref, "bf16", "merge")


# few parts (flat kernel) and many (parts split over thread groups merged
# through LDS: 64 key ranges at d=128 as split-KV decoding makes them, a
# ragged share of 37 parts over 8 groups at d=64 with two rows per workgroup,
# 16 parts over 2 groups at d=512, 9 parts at d=256), rows not a multiple of
# the rows per workgroup
@pytest.mark.parametrize("n,rows,dv", [(5, 300, 128), (64, 301, 128), (37, 203, 64), (16, 77, 512),
                                       (9, 50, 256), (65, 130, 96)])
def test_merge_matches_oracle_merge(n, rows, dv):
    import oracle

    rng = np.random.default_rng(3 + n)
    m = rng.standard_normal((n, rows)) * 3
    m[1, :50] = -np.inf  # parts that saw no key
    m[:, 7] = -np.inf    # a row no part saw
    l = np.where(np.isinf(m), 0.0, rng.uniform(0.5, 5, (n, rows)))
    O = np.where(np.isinf(m)[..., None], 0.0, rng.standard_normal((n, rows, dv)))
    dev = lambda a: torch.tensor(a, dtype=torch.float32, device=DEV).contiguous()
    m32, l32, O32 = (a.astype(np.float32).astype(np.float64) for a in (m, l, O))
    out, (mm, ll, OO) = ra.ring_attn_merge(dev(m32), dev(l32), dev(O32), torch.float32, want_state=True)
    torch.cuda.synchronize()
    acc = None
    for i in range(n):
        s = oracle.State(1, 1, rows, dv)
        s.m[0, 0], s.l[0, 0], s.O[0, 0] = m32[i], l32[i], O32[i]
        acc = s if acc is None else oracle.merge(acc, s)
    ref_out, _ = oracle.finalize(acc)
    got = out.cpu().numpy()
    check(got, ref_out[0, :, 0], "fp32", "merge out")
    assert np.isneginf(mm.cpu().numpy()[7]) and ll.cpu().numpy()[7] == 0 and np.all(got[7] == 0)
    # the merged state: m exactly (a maximum), l and O relative to it
    fin = ~np.isneginf(acc.m[0, 0])
    assert np.array_equal(np.isneginf(mm.cpu().numpy()), ~fin)
    np.testing.assert_allclose(mm.cpu().numpy()[fin], acc.m[0, 0][fin], rtol=0, atol=1e-6)
    np.testing.assert_allclose(ll.cpu().numpy(), acc.l[0, 0], rtol=1e-5, atol=0)
    np.testing.assert_allclose(OO.cpu().numpy(), acc.O[0, 0], rtol=1e-5, atol=1e-5 * np.abs(acc.O).max())


def test_order_invariance_and_determinism():
    wl = wl_of(B=1, Hq=8, Hkv=2, d=128, lens=(256,) * 4, Lq=256, q_offset=768, causal=True)
    x = inputs.make(wl, DEV)
    ref, _ = oracle_out(x.q, x.chunks(), wl.q_offset, True)
    outs = []
    for order in ([3, 2, 1, 0], [0, 1, 2, 3], [2, 0, 3, 1]):
        o, _ = run(x, order, ra.RA_FLAG_STAGE)
        outs.append(o.float().cpu().numpy())
        check(outs[-1], ref, "bf16", f"order {order}")
    for o in outs[1:]:
        # different orders round differently; each output is rounded to bf16
        e = errors(o, outs[0])
        assert e["max_abs"] <= 2e-3 and e["rel_l2"] <= 1e-2, e
    again, _ = run(x, [3, 2, 1, 0], ra.RA_FLAG_STAGE)
    assert np.array_equal(again.float().cpu().numpy(), outs[0]), "same order must be bit-identical"
    # in place: one launch keeps the state in registers across chunks; staged:
    # the fp32 state goes through HBM between chunks -- equal within rounding
    inplace, _ = run(x, [3, 2, 1, 0], ra.RA_FLAG_NO_SPLIT_KV)
    e = errors(inplace.float().cpu().numpy(), outs[0])
    assert e["max_abs"] <= 2e-3 and e["rel_l2"] <= 1e-2, e
    again, _ = run(x, [3, 2, 1, 0], ra.RA_FLAG_NO_SPLIT_KV)
    assert torch.equal(again, inplace), "same order must be bit-identical"


def test_future_chunks_and_empty_inputs():
    wl = wl_of(B=1, Hq=2, Hkv=2, d=128, lens=(128, 128), Lq=64, q_offset=0, causal=True)
    x = inputs.make(wl, DEV)
    # rows 0..63 see only chunk 0; chunk 1 is entirely in the future (skipped)
    ref, _ = oracle_out(x.q, x.chunks(), 0, True)
    out, _ = run(x, [1, 0], ra.RA_FLAG_STAGE)
    check(out.float().cpu().numpy(), ref, "bf16", "future chunk skipped")
    # every chunk in the future: zero output, empty state
    fut = [(k, v, s + 1000) for (k, v, s) in x.chunks()]
    out, (m, l, O) = ra.ring_attn_fwd(x.q, fut, True, 0, want_state=True)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(m)) and torch.all(l == 0) and torch.all(O == 0)
    for flags in (ra.RA_FLAG_SPLIT_KV, ra.RA_FLAG_STAGE):
        out, _ = ra.ring_attn_fwd(x.q[:, :4], fut, True, 0, flags=flags)
        torch.cuda.synchronize()
        assert torch.all(out == 0)
    # empty chunk in the list and Lq = 0
    e = (x.ks[0][:, :0], x.vs[0][:, :0], 5000)
    out, _ = ra.ring_attn_fwd(x.q, x.chunks() + [e], True, 0, flags=ra.RA_FLAG_STAGE)
    torch.cuda.synchronize()
    check(out.float().cpu().numpy(), ref, "bf16", "empty chunk")
    out, _ = ra.ring_attn_fwd(x.q[:, :0], x.chunks(), True, 0)
    assert out.shape[1] == 0


def test_strided_layouts():
    """BHSD-strided query/output and KV chunks sliced out of one long cache."""
    wl = wl_of(B=2, Hq=4, Hkv=2, d=128, lens=(192, 192), Lq=128, q_offset=256, causal=True)
    x = inputs.make(wl, DEV)
    ref, _ = oracle_out(x.q, x.chunks(), wl.q_offset, True)
    q_bhsd = x.q.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)  # strides of BHSD
    K = torch.cat(x.ks, dim=1)
    V = torch.cat(x.vs, dim=1)
    chunks = [(K[:, :192], V[:, :192], 0), (K[:, 192:], V[:, 192:], 192)]  # batch stride 384*H*d
    out = torch.empty(2, 4, 128, 128, device=DEV, dtype=torch.bfloat16).permute(0, 2, 1, 3)
    for flags in (ra.RA_FLAG_NO_SPLIT_KV, ra.RA_FLAG_STAGE):
        ra.ring_attn_fwd(q_bhsd, chunks, True, wl.q_offset, out=out, flags=flags)
        torch.cuda.synchronize()
        check(out.float().cpu().numpy(), ref, "bf16", f"strided flags={flags}")


def test_nonfinite_reported_not_hidden():
    """Invalid arguments fail before any work; the context stays usable."""
    wl = wl_of(B=1, Hq=2, Hkv=2, d=128, lens=(64,), Lq=64)
    x = inputs.make(wl, DEV)
    with pytest.raises(ra.RingAttnError):
        ra.ring_attn_fwd(x.q, [(x.ks[0], x.vs[0], 0), (x.ks[0], x.vs[0], 32)], True, 0)
    out, _ = run(x)
    ref, _ = oracle_out(x.q, x.chunks(), 0, True)
    check(out.float().cpu().numpy(), ref, "bf16", "after an error")
