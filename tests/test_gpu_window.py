"""Local attention windows on the GPU, compared with the oracle's masked
attention: every kernel (bf16 d=64/128/512 in place and staged, split-KV
decoding, the 8-bit KV cache, fp32), causal and two-sided windows, widths on
and next to the 64/128-key tile boundaries, windows that cross chunk edges
and rows whose window misses every key."""
import numpy as np
import pytest
import torch

import long_context_blockwise_amd as ra
from long_context_blockwise_amd import inputs
from parity import check, oracle_out, oracle_state

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _wl(B=1, Hq=4, Hkv=2, d=128, dtype="bf16", lens=(256, 256), Lq=256, q_offset=0, causal=True,
        std=None, seed=11, kv_dtype=None):
    if std is None:
        std = 1.0 if dtype == "fp32" else (0.5 if d < 512 else 4 / 512 ** 0.5)
    kw = dict(kv_dtype=kv_dtype) if kv_dtype else {}
    return inputs.Workload("window_case", B=B, Hq=Hq, Hkv=Hkv, d_qk=d, d_v=d, dtype=dtype,
                           chunk_len=lens[0], P=len(lens), Lq=Lq, q_offset=q_offset, causal=causal,
                           std=std, seed=seed, chunk_lens=tuple(lens), **kw)


def _run_check(x, causal, window, flags, what, order=None):
    wl = x.wl
    chunks = x.chunks(order)
    out, _ = ra.ring_attn_fwd(x.q, chunks, causal, wl.q_offset, flags=flags, window=window)
    torch.cuda.synchronize()
    ref, _ = oracle_out(x.q, chunks, wl.q_offset, causal, window=window)
    dt = "fp32" if wl.dtype == "fp32" else "bf16"
    got = out.cpu().numpy() if dt == "fp32" else out.float().cpu().numpy()
    check(got, ref, dt, f"{what} W={window} flags={flags}")
    return got, ref


PREFILL = [
    # d, Hq, Hkv, lens, Lq, q_offset, causal, window
    (128, 4, 2, (256, 256, 256), 256, 512, True, 64),     # window = one 64-key tile
    (128, 4, 2, (256, 256, 256), 256, 512, True, 63),
    (128, 4, 2, (256, 256, 256), 256, 512, True, 65),
    (128, 4, 2, (256, 256, 256), 256, 512, True, 127),
    (128, 4, 2, (256, 256, 256), 256, 512, True, 128),
    (128, 4, 2, (256, 256, 256), 256, 512, True, 300),    # crosses a chunk edge
    (128, 8, 2, (64, 100, 37), 129, 72, True, 1),          # ragged chunks, two keys per row
    (128, 4, 4, (192, 320), 200, 250, True, 90),
    (128, 2, 1, (300, 200), 257, 43, False, 40),           # two-sided, query block inside the keys
    (128, 2, 1, (300, 200), 257, 43, False, 129),
    (128, 4, 4, (256,), 255, 0, True, 10),                 # diagonal at position 0
    (64, 4, 2, (256, 256), 256, 256, True, 100),
    (64, 2, 2, (77, 130), 300, 0, False, 65),              # rows past the last key: some see none
    (512, 16, 1, (96, 64), 128, 96, True, 50),             # 512-wide heads
    (512, 4, 1, (50, 80), 33, 20, False, 17),
]


@pytest.mark.parametrize("d,Hq,Hkv,lens,Lq,q_off,causal,window", PREFILL)
@pytest.mark.parametrize("flags", [0, 1], ids=["inplace", "staged"])
def test_window_prefill(d, Hq, Hkv, lens, Lq, q_off, causal, window, flags):
    x = inputs.make(_wl(B=2 if d < 512 else 1, Hq=Hq, Hkv=Hkv, d=d, lens=lens, Lq=Lq, q_offset=q_off,
                        causal=causal), DEV)
    order = list(range(len(lens)))[::-1]
    _run_check(x, causal, window, flags | ra.RA_FLAG_NO_SPLIT_KV, f"d={d} lens={lens} Lq={Lq} off={q_off}",
               order)


def test_window_wider_than_context_is_full_attention():
    """A window that reaches past every key gives the unwindowed output."""
    x = inputs.make(_wl(lens=(200, 300), Lq=160, q_offset=340, causal=True), DEV)
    full, _ = ra.ring_attn_fwd(x.q, x.chunks(), True, 340, flags=ra.RA_FLAG_NO_SPLIT_KV)
    wide, _ = ra.ring_attn_fwd(x.q, x.chunks(), True, 340, flags=ra.RA_FLAG_NO_SPLIT_KV, window=10 ** 6)
    torch.cuda.synchronize()
    assert torch.equal(full, wide)


def test_window_skips_chunks_outside():
    """Chunks entirely outside every row's window are classified skipped and
    the output is the same as without them."""
    lens = (512, 512, 512)
    x = inputs.make(_wl(lens=lens, Lq=128, q_offset=1124, causal=True), DEV)
    cls = ra.ring_attn_plan(128, 1124, True, [0, 512, 1024], list(lens), window=200)
    assert cls[0] == ra.RA_CHUNK_SKIP and cls[1] != ra.RA_CHUNK_SKIP
    got, _ = _run_check(x, True, 200, ra.RA_FLAG_NO_SPLIT_KV, "skip")
    only, _ = ra.ring_attn_fwd(x.q, x.chunks()[1:], True, 1124, flags=ra.RA_FLAG_NO_SPLIT_KV,
                               window=200)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(only.float().cpu().numpy(), got)


DECODE = [
    # B, Hq, Hkv, lens, Lq, q_offset, window
    (1, 8, 2, (512, 512, 512, 300), 1, 1835, 64),
    (2, 8, 2, (512, 512, 512, 300), 4, 1832, 127),
    (1, 32, 2, (512, 512, 512, 300), 16, 1820, 700),      # window across a chunk edge
    (1, 4, 4, (2048,), 7, 2041, 1),
]


@pytest.mark.parametrize("B,Hq,Hkv,lens,Lq,q_off,window", DECODE)
def test_window_decode_split(B, Hq, Hkv, lens, Lq, q_off, window):
    x = inputs.make(_wl(B=B, Hq=Hq, Hkv=Hkv, lens=lens, Lq=Lq, q_offset=q_off), DEV)
    _run_check(x, True, window, ra.RA_FLAG_SPLIT_KV, f"decode Lq={Lq}")
    _run_check(x, True, window, ra.RA_FLAG_NO_SPLIT_KV, f"decode via ring schedule Lq={Lq}")


@pytest.mark.parametrize("Lq,q_off,causal,window", [(1, 4095, True, 64), (16, 4080, True, 1000),
                                                    (5, 2000, False, 130), (3, 100, True, 3)])
def test_window_fp8_kv(Lq, q_off, causal, window):
    x = inputs.make(_wl(B=2, Hq=16, Hkv=4, lens=(1000, 3096), Lq=Lq, q_offset=q_off, causal=causal,
                        kv_dtype="fp8"), DEV)
    _run_check(x, causal, window, 0, f"fp8 Lq={Lq}")


@pytest.mark.parametrize("Lq,q_off,causal,window,flags", [
    (256, 256, True, 100, 0), (256, 256, True, 100, 1), (256, 100, False, 33, 0),
    (5, 395, True, 20, ra.RA_FLAG_SPLIT_KV)])
def test_window_fp32(Lq, q_off, causal, window, flags):
    x = inputs.make(_wl(B=2, Hq=4, Hkv=2, d=64, dtype="fp32", lens=(200, 200), Lq=Lq, q_offset=q_off,
                        causal=causal), DEV)
    _run_check(x, causal, window, flags, f"fp32 Lq={Lq}")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp32", 64)])
def test_window_state_outputs(dtype, d):
    """Exported (m, l, O) under a window equal the oracle's windowed ring
    state; rows whose window misses every key have m = -inf, l = 0, O = 0."""
    # non-causal, keys 0..287, queries 250..345: rows past 287+W see no key
    W = 30
    x = inputs.make(_wl(B=1, Hq=4, Hkv=2, d=d, dtype=dtype, lens=(128, 160), Lq=96, q_offset=250,
                        causal=False), DEV)
    m_ref, l_ref, O_ref = oracle_state(x.q, x.chunks(), 250, False, window=W)
    dead = l_ref == 0
    assert dead.any() and not dead.all()
    for flags in (ra.RA_FLAG_NO_SPLIT_KV, ra.RA_FLAG_STAGE):
        _, (m, l, O) = ra.ring_attn_fwd(x.q, x.chunks(), False, 250, flags=flags, want_state=True,
                                        window=W)
        torch.cuda.synchronize()
        m, l, O = m.cpu().numpy(), l.cpu().numpy(), O.cpu().numpy()
        assert np.all(np.isneginf(m[dead])) and np.all(l[dead] == 0) and np.all(O[dead] == 0)
        live = ~dead
        tol_m = 1e-5 if dtype == "fp32" else 2e-3
        assert np.abs(m[live] - m_ref[live]).max() <= tol_m * (1 + np.abs(m_ref[live]).max())
        scale = np.exp(m_ref[live] - m[live])
        rel = np.abs(l[live] * scale - l_ref[live]) / l_ref[live]
        assert rel.max() <= (1e-5 if dtype == "fp32" else 1e-2), rel.max()
        check(O[live] / l[live][..., None], O_ref[live] / l_ref[live][..., None], dtype, f"O/l flags={flags}")
