"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and its host-only logic (ring order, chunk classes,
workspace sizing, argument validation) behaves as documented.  No kernel is
launched here."""
import ctypes
import os
import re

import pytest

import long_context_blockwise_amd as ra
from long_context_blockwise_amd import ring_attn as rb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ring_attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rb.LIB_PATH):
        from long_context_blockwise_amd import build

        build.build()
    return rb.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ring_attn_\w+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert header_functions() == sorted(ra.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_version(lib):
    assert "gfx950" in ra.ring_attn_version()


@pytest.mark.parametrize("P", [1, 2, 4, 7, 32])
def test_ring_order_receives_from_previous_device(lib, P):
    for i in range(P):
        order = ra.ring_attn_ring_order(i, P)
        assert order[0] == i
        assert sorted(order) == list(range(P))
        # step s+1 holds the chunk device i-1 held at step s
        for s in range(P - 1):
            prev = ra.ring_attn_ring_order((i - 1) % P, P)
            assert order[s + 1] == prev[s]


def test_ring_order_rejects_bad_args(lib):
    with pytest.raises(ra.RingAttnError):
        ra.ring_attn_ring_order(4, 4)
    with pytest.raises(ra.RingAttnError):
        ra.ring_attn_ring_order(0, 0)


def _brute_class(Lq, q_off, causal, start, n, window=0, anchor=0):
    if n == 0 or Lq == 0:
        return ra.RA_CHUNK_SKIP

    def seen(qp, kp):
        if anchor > 0:
            A = qp // anchor * anchor
            if kp in (A - 1, A, A + anchor):
                return True
        if causal and kp > qp:
            return False
        return window <= 0 or abs(kp - qp) <= window

    vis = [[seen(q_off + r, start + j) for j in range(n)] for r in range(Lq)]
    if not any(any(row) for row in vis):
        return ra.RA_CHUNK_SKIP
    # FULL: no mask needed, i.e. every pair visible by the causal and window rules alone
    base = [[(not causal or start + j <= q_off + r) and (window <= 0 or abs(start + j - q_off - r) <= window)
             for j in range(n)] for r in range(Lq)]
    if all(all(row) for row in base):
        return ra.RA_CHUNK_FULL
    return ra.RA_CHUNK_DIAG


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", [0, 1, 3, 7, 40])
@pytest.mark.parametrize("anchor", [0, 1, 4, 7])
def test_plan_matches_brute_force(lib, causal, window, anchor):
    starts = [0, 5, 9, 20, 21, 30]
    lens = [5, 4, 11, 1, 9, 0]
    for Lq in (1, 3, 8):
        for q_off in (0, 4, 5, 8, 9, 19, 20, 29, 35):
            got = ra.ring_attn_plan(Lq, q_off, causal, starts, lens, window=window, anchor=anchor)
            want = [_brute_class(Lq, q_off, causal, s, n, window, anchor) for s, n in zip(starts, lens)]
            assert got == want, (Lq, q_off, window, anchor)


def test_plan_of_the_prefill_share():
    # query chunk 3 of 4 x 8192, causal: 0..2 unmasked, 3 on the diagonal
    cls = ra.ring_attn_plan(8192, 3 * 8192, True, [0, 8192, 16384, 24576], [8192] * 4)
    assert cls == [ra.RA_CHUNK_FULL] * 3 + [ra.RA_CHUNK_DIAG]
    # decode: 16 tokens at cache_idx 1048560 against 64 x 16384
    cls = ra.ring_attn_plan(16, 1048560, True, [16384 * i for i in range(64)], [16384] * 64)
    assert cls == [ra.RA_CHUNK_FULL] * 63 + [ra.RA_CHUNK_DIAG]


def _desc(B=1, Hq=4, Hkv=2, d=128, dtype=ra.RA_BF16):
    x = rb.ra_desc()
    x.B, x.Hq, x.Hkv, x.d_qk, x.d_v, x.dtype = B, Hq, Hkv, d, d, dtype
    return x


def _chunks(lens, start=0):
    arr = (rb.ra_kv_chunk * len(lens))()
    s = start
    for i, n in enumerate(lens):
        arr[i].k = arr[i].v = 1 << 12
        arr[i].start, arr[i].len = s, n
        s += n
    return arr


def _ws(lib, d, Lq, arr, P, causal, q_off, flags, want_state):
    n = ctypes.c_size_t()
    rc = lib.ring_attn_workspace_size(ctypes.byref(d), Lq, arr, P, causal, q_off, flags, want_state,
                                      ctypes.byref(n))
    return rc, n.value


def test_workspace_size(lib):
    d = _desc(B=2, Hq=4, Hkv=2, d=128)
    arr = _chunks([64, 64, 64])
    # in place, one launch, caller keeps no state: nothing needed
    assert _ws(lib, d, 64, arr, 3, 0, 0, 0, 0) == (0, 0)
    # staged: two buffers of K+V of the largest received chunk, plus the running state
    rc, n = _ws(lib, d, 64, arr, 3, 0, 0, ra.RA_FLAG_STAGE, 0)
    stage = 2 * 64 * 2 * 128 * 2 * 2  # B * len * Hkv * (dk + dv) * 2 bytes
    state = 2 * 64 * 4 * (128 + 2) * 4
    assert rc == 0 and n == 2 * stage + state
    rc, n2 = _ws(lib, d, 64, arr, 3, 0, 0, ra.RA_FLAG_STAGE, 1)
    assert rc == 0 and n2 == 2 * stage
    # split-KV (decode): partial states
    rc, n3 = _ws(lib, d, 4, arr, 3, 0, 0, 0, 1)
    assert rc == 0 and n3 > 0 and n3 % (2 * 4 * 4 * (128 + 2) * 4) == 0


@pytest.mark.parametrize("mutate,code", [
    (lambda d: setattr(d, "Hkv", 3), rb.RA_ERR_INVALID_ARG),
    (lambda d: setattr(d, "B", 0), rb.RA_ERR_INVALID_ARG),
    (lambda d: setattr(d, "dtype", 7), rb.RA_ERR_INVALID_ARG),
    (lambda d: setattr(d, "d_qk", 96), rb.RA_ERR_UNSUPPORTED),
    (lambda d: (setattr(d, "d_qk", 256), setattr(d, "d_v", 256)), rb.RA_ERR_UNSUPPORTED),
    (lambda d: setattr(d, "scale", -1.0), rb.RA_ERR_INVALID_ARG),
    (lambda d: d.q_strides.__setitem__(1, 3), rb.RA_ERR_INVALID_ARG),
])
def test_descriptor_validation(lib, mutate, code):
    d = _desc()
    mutate(d)
    rc, _ = _ws(lib, d, 16, _chunks([32]), 1, 0, 0, 0, 0)
    assert rc == code
    assert lib.ring_attn_last_error()


def test_fp32_head_sizes(lib):
    assert _ws(lib, _desc(d=64, dtype=ra.RA_F32), 8, _chunks([8]), 1, 0, 0, 0, 1)[0] == 0
    assert _ws(lib, _desc(d=512, dtype=ra.RA_F32), 8, _chunks([8]), 1, 0, 0, 0, 1)[0] == rb.RA_ERR_UNSUPPORTED


def test_chunk_validation(lib):
    d = _desc()
    arr = _chunks([32, 32])
    arr[1].start = 16  # overlaps chunk 0
    assert _ws(lib, d, 8, arr, 2, 0, 0, 0, 0)[0] == rb.RA_ERR_INVALID_ARG
    arr = _chunks([32])
    arr[0].len = -1
    assert _ws(lib, d, 8, arr, 1, 0, 0, 0, 0)[0] == rb.RA_ERR_INVALID_ARG
    assert _ws(lib, d, 8, _chunks([8]), 1, 0, -1, 0, 0)[0] == rb.RA_ERR_INVALID_ARG
    assert _ws(lib, d, 8, _chunks([8]), 1, 0, 0, 0x40, 0)[0] == rb.RA_ERR_INVALID_ARG
    both = ra.RA_FLAG_SPLIT_KV | ra.RA_FLAG_STAGE
    assert _ws(lib, d, 8, _chunks([8]), 1, 0, 0, both, 0)[0] == rb.RA_ERR_INVALID_ARG


def test_fwd_rejects_null_context_before_enqueueing(lib):
    d = _desc()
    rc = lib.ring_attn_fwd(None, ctypes.byref(d), 1 << 12, 8, _chunks([8]), 1, 0, 0, 0, 1 << 12,
                           None, None, None, None, 0, None)
    assert rc == rb.RA_ERR_INVALID_ARG


def test_merge_validation(lib):
    assert lib.ring_attn_merge(0, 4, 128, 1 << 12, 1 << 12, 1 << 12, None, None, None, 1 << 12, 0,
                               None) == rb.RA_ERR_INVALID_ARG
    assert lib.ring_attn_merge(1, 4, 6, 1 << 12, 1 << 12, 1 << 12, None, None, None, 1 << 12, 0,
                               None) == rb.RA_ERR_INVALID_ARG
    # only some of m, l, O
    assert lib.ring_attn_merge(1, 4, 8, 1 << 12, 1 << 12, 1 << 12, 1 << 12, None, None, None, 0,
                               None) == rb.RA_ERR_INVALID_ARG


def test_context_needs_a_device(lib):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    h = ctypes.c_void_p()
    assert lib.ring_attn_ctx_create(0, ctypes.byref(h)) == rb.RA_ERR_HIP


def test_struct_layouts_match_the_header():
    assert ctypes.sizeof(rb.ra_desc) == 8 * 4 + 15 * 8
    assert rb.ra_desc.window.offset == 8 * 4 + 12 * 8
    assert rb.ra_desc.anchor.offset == 8 * 4 + 13 * 8 and rb.ra_desc.q_seg.offset == 8 * 4 + 14 * 8
    assert ctypes.sizeof(rb.ra_kv_chunk) == 7 * 8 and rb.ra_kv_chunk.k_seg.offset == 48
    assert rb.ra_desc.kv_dtype.offset == 7 * 4
    assert rb.ra_kv_chunk.k_exp.offset == 32 and rb.ra_kv_chunk.v_exp.offset == 40


def test_fp8_kv_validation(lib):
    def fp8_desc(**kw):
        d = _desc(**kw)
        d.kv_dtype = rb.RA_FP8_E4M3
        return d

    def fp8_chunks(lens, start=0):
        arr = _chunks(lens, start)
        for i in range(len(lens)):
            arr[i].k_exp = arr[i].v_exp = 1 << 12
        return arr

    d, arr = fp8_desc(), fp8_chunks([256, 100])
    # decode-sized and longer query blocks both take the split-KV schedule: partial states
    for Lq in (4, 64):
        rc, n = _ws(lib, d, Lq, arr, 2, 1, 300, 0, 1)
        assert rc == 0 and n > 0 and n % (2 * Lq * 4 * (128 + 2) * 4) == 0
    # the 8-bit cache is read in place by split-KV only
    for flags in (ra.RA_FLAG_STAGE, ra.RA_FLAG_NO_SPLIT_KV):
        assert _ws(lib, d, 4, arr, 2, 1, 300, flags, 1)[0] == rb.RA_ERR_UNSUPPORTED
    # both exponent arrays are required for chunks with keys
    arr[1].v_exp = None
    assert _ws(lib, d, 4, arr, 2, 1, 300, 0, 1)[0] == rb.RA_ERR_INVALID_ARG
    empty = fp8_chunks([256, 0])
    empty[1].k_exp = empty[1].v_exp = None
    assert _ws(lib, d, 4, empty, 2, 1, 300, 0, 1)[0] == 0
    # built for bf16 queries with d = 128
    assert _ws(lib, fp8_desc(d=64), 4, fp8_chunks([64]), 1, 0, 0, 0, 1)[0] == rb.RA_ERR_UNSUPPORTED
    assert _ws(lib, fp8_desc(dtype=ra.RA_F32), 4, fp8_chunks([64]), 1, 0, 0, 0, 1)[0] == rb.RA_ERR_UNSUPPORTED
    # unknown kv dtypes; 8-bit strides are whole 16-byte units
    bad = fp8_desc()
    bad.kv_dtype = 9
    assert _ws(lib, bad, 4, fp8_chunks([64]), 1, 0, 0, 0, 1)[0] == rb.RA_ERR_INVALID_ARG
    st = fp8_desc()
    st.k_strides[:] = (64 * 2 * 136, 2 * 136, 136)
    assert _ws(lib, st, 4, fp8_chunks([64]), 1, 0, 0, 0, 1)[0] == rb.RA_ERR_INVALID_ARG
    st.k_strides[:] = (64 * 2 * 144, 2 * 144, 144)
    assert _ws(lib, st, 4, fp8_chunks([64]), 1, 0, 0, 0, 1)[0] == 0


def test_kv_stride_limits(lib):
    """Only the k/v token stride is limited (a key tile is addressed with
    32-bit offsets): a head-major cache of 2^24 elements per sequence passes,
    a token stride of 2^24 does not."""
    d = _desc(B=2, Hq=4, Hkv=2, d=128)
    arr = _chunks([1 << 16])
    d.k_strides[:] = d.v_strides[:] = (2 * (1 << 16) * 128, 128, (1 << 16) * 128)  # batch stride 2^24
    assert _ws(lib, d, 16, arr, 1, 1, (1 << 16) - 16, 0, 1)[0] == 0
    d.k_strides[:] = (2 * (1 << 24), 1 << 24, 128)
    assert _ws(lib, d, 16, arr, 1, 1, (1 << 16) - 16, 0, 1)[0] == rb.RA_ERR_UNSUPPORTED


def test_bwd_workspace_and_validation(lib):
    """Backward: workspace = the rows' (lse, D) pairs; what is not built is
    rejected; bad arguments are rejected before anything touches the device
    (a dummy context is safe because validation comes first)."""
    n = ctypes.c_size_t()
    assert lib.ring_attn_bwd_workspace_size(ctypes.byref(_desc(B=2, Hq=4, d=128)), 100, ctypes.byref(n)) == 0
    assert n.value == 2 * 4 * 100 * 8  # 6400, already a multiple of 256
    assert lib.ring_attn_bwd_workspace_size(ctypes.byref(_desc(B=1, Hq=3, Hkv=3, d=64)), 5, ctypes.byref(n)) == 0
    assert n.value == 256
    assert lib.ring_attn_bwd_workspace_size(ctypes.byref(_desc(B=1, Hq=16, Hkv=1, d=512)), 8, ctypes.byref(n)) == 0
    assert n.value == 16 * 8 * 8  # 1024, a multiple of 256
    for bad in (_desc(dtype=ra.RA_F32), _desc(d=256), _desc(d=512, dtype=ra.RA_F32)):
        assert lib.ring_attn_bwd_workspace_size(ctypes.byref(bad), 8, ctypes.byref(n)) == rb.RA_ERR_UNSUPPORTED
    f8 = _desc()
    f8.kv_dtype = rb.RA_FP8_E4M3
    assert lib.ring_attn_bwd_workspace_size(ctypes.byref(f8), 8, ctypes.byref(n)) == rb.RA_ERR_UNSUPPORTED

    ctx = ctypes.create_string_buffer(256)  # never dereferenced on these paths
    d, arr = _desc(B=1, Hq=4, Hkv=2, d=128), _chunks([64, 64])
    grads = (rb.ra_kv_grad * 2)()
    for i in range(2):
        grads[i].dk = grads[i].dv = 1 << 16
    buf = 1 << 20  # 16-byte aligned stand-in device addresses

    def bwd(flags=0, P=2, g=grads, dq=buf, ws=buf, ws_bytes=1 << 20, c=ctx, q_off=64, chunks=arr):
        return lib.ring_attn_bwd(c, ctypes.byref(d), buf, 64, chunks, P, 1, q_off, flags, buf, buf, buf, buf, dq, g,
                                 ws, ws_bytes, None)

    assert bwd(c=None) == rb.RA_ERR_INVALID_ARG
    assert bwd(flags=ra.RA_FLAG_STAGE) == rb.RA_ERR_INVALID_ARG
    assert bwd(flags=ra.RA_FLAG_SPLIT_KV) == rb.RA_ERR_INVALID_ARG
    assert bwd(P=65) == rb.RA_ERR_INVALID_ARG
    assert bwd(g=None) == rb.RA_ERR_INVALID_ARG
    assert bwd(dq=None) == rb.RA_ERR_INVALID_ARG
    assert bwd(dq=buf + 4) == rb.RA_ERR_INVALID_ARG
    assert bwd(ws=None) == rb.RA_ERR_WORKSPACE
    assert bwd(ws_bytes=100) == rb.RA_ERR_WORKSPACE
    assert bwd(ws=buf + 16) == rb.RA_ERR_WORKSPACE
    # positions are checked as in the forward: q_offset and chunk starts >= 0, chunks disjoint
    assert bwd(q_off=-1) == rb.RA_ERR_INVALID_ARG
    assert bwd(chunks=_chunks([64, 64], start=-64)) == rb.RA_ERR_INVALID_ARG
    overlap = _chunks([64, 64])
    overlap[1].start = 32
    assert bwd(chunks=overlap) == rb.RA_ERR_INVALID_ARG
    grads[1].dv = None
    assert bwd() == rb.RA_ERR_INVALID_ARG
    assert ctypes.sizeof(rb.ra_kv_grad) == 16



def test_ctx_check_validation(lib):
    """The staged-ring checks take only known bits and a bounded spin."""
    ctx = ctypes.create_string_buffer(256)  # its check fields are written, nothing else
    assert lib.ring_attn_ctx_set_check(None, 0, 0) == rb.RA_ERR_INVALID_ARG
    assert lib.ring_attn_ctx_set_check(ctx, 8, 0) == rb.RA_ERR_INVALID_ARG
    assert lib.ring_attn_ctx_set_check(ctx, 7, rb.RA_CHECK_MAX_SPIN_US + 1) == rb.RA_ERR_INVALID_ARG
    assert lib.ring_attn_ctx_set_check(ctx, 7, rb.RA_CHECK_MAX_SPIN_US) == 0
    assert lib.ring_attn_ctx_set_check(ctx, 0, 0) == 0


def test_anchor_and_label_validation(lib):
    """Anchors and labels: negative strides are rejected; d = 512 and the
    8-bit cache are not built for them; labels come for the queries and
    every non-empty chunk or not at all."""
    arr = _chunks([64, 64])
    d = _desc()
    d.anchor = -1
    assert _ws(lib, d, 8, arr, 2, 1, 64, 0, 0)[0] == rb.RA_ERR_INVALID_ARG
    for bad in (_desc(d=512, Hkv=1),):
        bad.anchor = 16
        assert _ws(lib, bad, 8, _chunks([64]), 1, 1, 64, 0, 0)[0] == rb.RA_ERR_UNSUPPORTED
    f8 = _desc()
    f8.kv_dtype = rb.RA_FP8_E4M3
    f8.q_seg = 1 << 12
    assert _ws(lib, f8, 8, _chunks([64]), 1, 1, 64, 0, 0)[0] == rb.RA_ERR_UNSUPPORTED
    ok = _desc()
    ok.anchor = 4096
    assert _ws(lib, ok, 8, arr, 2, 1, 64, 0, 0)[0] == 0
    # labels on the queries only, or on a chunk only: rejected before any device work
    ctx = ctypes.create_string_buffer(256)
    lab = _desc()
    lab.q_seg = 1 << 12

    def fwd(desc, chunks):
        return lib.ring_attn_fwd(ctx, ctypes.byref(desc), 1 << 20, 8, chunks, 2, 1, 64, 0, 1 << 20, None, None,
                                 None, None, 0, None)
    assert fwd(lab, _chunks([64, 64])) == rb.RA_ERR_INVALID_ARG
    one = _chunks([64, 64])
    one[0].k_seg = 1 << 12
    assert fwd(_desc(), one) == rb.RA_ERR_INVALID_ARG
    mis = _chunks([64, 64])
    mis[0].k_seg, mis[1].k_seg = 1 << 12, (1 << 12) + 2
    assert fwd(lab, mis) == rb.RA_ERR_INVALID_ARG
    # label scans index keys and rows with 32-bit integers and may step 2^16
    # entries past the end: a chunk or query chunk of 2^31 - 2^16 or more is refused
    lim = (1 << 31) - (1 << 16)
    for n in (lim, 1 << 31):
        big = _chunks([64, n])
        big[0].k_seg, big[1].k_seg = 1 << 12, 1 << 13
        assert fwd(lab, big) == rb.RA_ERR_UNSUPPORTED
        assert lib.ring_attn_fwd(ctx, ctypes.byref(lab), 1 << 20, n, _labelled([64, 64]), 2, 1, 0, 0, 1 << 20,
                                 None, None, None, None, 0, None) == rb.RA_ERR_UNSUPPORTED
    # one key fewer passes the label checks (and stops at the missing workspace)
    ok = _chunks([64, lim - 1])
    ok[0].k_seg, ok[1].k_seg = 1 << 12, 1 << 13
    assert fwd(lab, ok) == rb.RA_ERR_WORKSPACE


def _labelled(lens):
    arr = _chunks(lens)
    for i in range(len(lens)):
        arr[i].k_seg = (1 << 12) + 64 * i
    return arr
