"""Double-precision CPU oracle for ring attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library in
``long_context_blockwise_amd``) never imports, links or calls it, and the two
share no code: the only module both sides use is the seeded input generator
``long_context_blockwise_amd.inputs``, which holds none of the method's
arithmetic.

The arithmetic lives in ``oracle.c`` (plain C, double precision, OpenMP over
query rows); this module compiles it with gcc on first use and marshals numpy
arrays through ctypes.  See ``oracle.c`` for the passages of the pages that
each routine follows:

* :func:`attention` -- softmax(Q K^T * scale) V from the definition (page
  "从百毫秒到百万Token：长上下文推理优化的工程实践", section
  "注意力机制的数学本质与瓶颈"), over the union of all KV chunks (page
  "Ring Attention：百万 Token 上下文的秘密", §2.3 数学正确性).
* :func:`ring_step` / :func:`ring` -- the per-chunk online-softmax recurrence
  one ring device runs (same page, §2.2 环形通信 and §3.1 Flash Ring Attention).
* :func:`merge` / :func:`finalize` -- combining partial (m, l, O) states and
  normalising them (page "从百毫秒到百万Token", section "系统架构设计",
  注意力融合层).
* :func:`attention_bwd` -- dQ, dK, dV of sum(dO * attention(...)): the
  derivative of the definition above, for the training use the pages
  describe (page "Ring Attention：百万 Token 上下文的秘密", §5.1 训练效率).

Inputs are numpy arrays of float64, float32, or bfloat16 carried as raw
``uint16`` bit patterns (pass ``dtype="bf16"``); torch CPU tensors of those
dtypes are accepted too.  Everything is upcast exactly and computed in double.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "liboracle.so")

_F64, _F32, _BF16 = 0, 1, 2
_lib = None
_lock = threading.Lock()


def build(force: bool = False, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile ``oracle.c`` into a shared library with gcc and return its path."""
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
           "-Wextra", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def load_library(path: str) -> ctypes.CDLL:
    """Load an oracle shared library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
    lib.oracle_threads.restype = i32
    lib.oracle_attention.restype = i32
    lib.oracle_attention.argtypes = [i32, i32, i32, i32, i32, i32, vp, i64, i64,
                                     i32, vp, vp, vp, vp, vp, dbl, i64, vp, vp, vp]
    lib.oracle_ring_step.restype = i32
    lib.oracle_ring_step.argtypes = [i32, i32, i32, i32, i32, i32, vp, i64, i64,
                                     vp, vp, i64, i64, vp, dbl, i64, vp, vp, vp, vp]
    lib.oracle_state_init.restype = None
    lib.oracle_state_init.argtypes = [i64, i32, vp, vp, vp]
    lib.oracle_merge.restype = None
    lib.oracle_merge.argtypes = [i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_finalize.restype = None
    lib.oracle_finalize.argtypes = [i64, i32, vp, vp, vp, vp, vp]
    lib.oracle_dequant_fp8.restype = i32
    lib.oracle_dequant_fp8.argtypes = [i32, i64, i32, i32, i32, vp, vp, vp]
    lib.oracle_attention_bwd.restype = i32
    lib.oracle_attention_bwd.argtypes = [i32, i32, i32, i32, i32, i32, vp, i64, i64, i32, vp, vp,
                                         vp, vp, vp, dbl, vp, vp, vp, vp]
    return lib


def _get_lib():
    global _lib
    with _lock:
        if _lib is None:
            _lib = load_library(build())
        return _lib


def threads() -> int:
    """Number of OpenMP threads the oracle runs on."""
    return int(_get_lib().oracle_threads())


# --------------------------------------------------------------------------- #
# array marshalling
# --------------------------------------------------------------------------- #
def _to_numpy(x, dtype):
    """Return (contiguous numpy array, element-type code) for an input tensor."""
    if hasattr(x, "detach"):  # torch tensor
        import torch

        x = x.detach().cpu().contiguous()
        if x.dtype == torch.bfloat16:
            return np.ascontiguousarray(x.view(torch.int16).numpy().view(np.uint16)), _BF16
        if x.dtype == torch.float32:
            return np.ascontiguousarray(x.numpy()), _F32
        if x.dtype == torch.float64:
            return np.ascontiguousarray(x.numpy()), _F64
        raise TypeError(f"unsupported torch dtype {x.dtype}")
    x = np.asarray(x)
    if dtype == "bf16" or x.dtype == np.uint16:
        return np.ascontiguousarray(x, dtype=np.uint16), _BF16
    if x.dtype == np.float32:
        return np.ascontiguousarray(x), _F32
    if x.dtype == np.float64:
        return np.ascontiguousarray(x), _F64
    raise TypeError(f"unsupported numpy dtype {x.dtype}")


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _u8(x):
    """Raw bytes of an 8-bit tensor/array as a contiguous uint8 numpy array."""
    if hasattr(x, "detach"):
        import torch

        x = x.detach().cpu().contiguous()
        if x.dtype != torch.uint8:
            x = x.view(torch.uint8)
        return np.ascontiguousarray(x.numpy())
    return np.ascontiguousarray(np.asarray(x).view(np.uint8))


KV_SCALE_BLOCK = 64  # tokens per shared exponent of an 8-bit KV cache


def dequant_fp8(codes, exps, block: int = KV_SCALE_BLOCK) -> np.ndarray:
    """Decode an 8-bit (OCP FP8 E4M3) KV tensor ``codes [B, len, H, d]`` whose
    blocks of ``block`` tokens per (batch, head) share the power-of-two scale
    2^(e-127) in ``exps [B, H, ceil(len/block)]``; returns float64."""
    c = _u8(codes)
    e = _u8(exps)
    if c.ndim != 4 or e.ndim != 3:
        raise ValueError("codes must be [B, len, H, d] and exps [B, H, nblk]")
    B, n, H, d = (int(x) for x in c.shape)
    if e.shape != (B, H, (n + block - 1) // block):
        raise ValueError(f"exps shape {e.shape} does not match codes {c.shape}")
    out = np.zeros(c.shape, dtype=np.float64)
    if _get_lib().oracle_dequant_fp8(B, n, H, d, block, _ptr(c), _ptr(e), _ptr(out)) != 0:
        raise ValueError("oracle_dequant_fp8 failed")
    return out


def _decoded(chunk):
    """(k, v, start) of a chunk; 8-bit chunks (k, v, start, k_exp, v_exp) are decoded."""
    if len(chunk) == 5:
        k, v, start, ke, ve = chunk
        return dequant_fp8(k, ke), dequant_fp8(v, ve), start
    return chunk


def _chunk_arrays(chunks, dtype, code):
    ks, vs, starts, lens = [], [], [], []
    for (k, v, start) in (_decoded(c) for c in chunks):
        ka, kc = _to_numpy(k, dtype)
        va, vc = _to_numpy(v, dtype)
        if kc != code or vc != code:
            raise TypeError("q, k and v must share one element type")
        if ka.shape[1] != va.shape[1]:
            raise ValueError("k and v of a chunk must have the same length")
        ks.append(ka)
        vs.append(va)
        starts.append(int(start))
        lens.append(int(ka.shape[1]))
    return ks, vs, starts, lens


class _Problem:
    """Shapes and marshalled arrays shared by the entry points."""

    def __init__(self, q, chunks, dtype, rows):
        self.q, self.code = _to_numpy(q, dtype)
        if any(len(c) == 5 for c in chunks):  # decoded 8-bit KV: compute in float64
            q64 = q.detach().cpu().double().numpy() if hasattr(q, "detach") else np.asarray(q, np.float64)
            self.q, self.code = np.ascontiguousarray(q64), _F64
        if self.q.ndim != 4:
            raise ValueError("q must be [B, Lq, Hq, d_qk]")
        self.B, self.Lq, self.Hq, self.dqk = (int(s) for s in self.q.shape)
        self.ks, self.vs, self.starts, self.lens = _chunk_arrays(chunks, dtype, self.code)
        if self.ks:
            self.Hkv = int(self.ks[0].shape[2])
            self.dv = int(self.vs[0].shape[3])
        else:
            self.Hkv, self.dv = None, None
        if rows is None:
            rows = np.arange(self.Lq, dtype=np.int64)
        self.rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        self.nr = int(self.rows.shape[0])


class _Mask(ctypes.Structure):
    _fields_ = [("causal", ctypes.c_int), ("window", ctypes.c_int64), ("anchor", ctypes.c_int64),
                ("q_seg", ctypes.c_void_p), ("k_seg", ctypes.c_void_p)]


def _mask(p, causal, window, anchor, q_seg, k_segs):
    """The C mask of a call, plus the arrays it points into (kept alive by the caller)."""
    m = _Mask(int(bool(causal)), int(window), int(anchor), None, None)
    keep = []
    if (q_seg is None) != (k_segs is None):
        raise ValueError("q_seg and k_segs go together")
    if q_seg is not None:
        qs = np.ascontiguousarray(np.asarray(q_seg.cpu() if hasattr(q_seg, "cpu") else q_seg, dtype=np.int32))
        if qs.shape != (p.B, p.Lq) or len(k_segs) != len(p.ks):
            raise ValueError("q_seg must be [B, Lq] and k_segs one [B, len] array per chunk")
        ks = [np.ascontiguousarray(np.asarray(x.cpu() if hasattr(x, "cpu") else x, dtype=np.int32))
              for x in k_segs]
        for a, n in zip(ks, p.lens):
            if a.shape != (p.B, n):
                raise ValueError("each k_segs entry must be [B, len]")
        arr = (ctypes.c_void_p * max(len(ks), 1))(*[_ptr(a) for a in ks])
        m.q_seg, m.k_seg = _ptr(qs), ctypes.cast(arr, ctypes.c_void_p).value
        keep = [qs, ks, arr]
    return m, keep


def _scale(scale, dqk):
    return 1.0 / math.sqrt(dqk) if scale is None else float(scale)


# --------------------------------------------------------------------------- #
# entry points
# --------------------------------------------------------------------------- #
def attention(q, chunks, q_offset=0, causal=False, scale=None, rows=None,
              dtype=None, Hkv=None, dv=None, window=0, anchor=0, q_seg=None, k_segs=None):
    """Plain attention of the query rows ``rows`` against all keys of ``chunks``.

    ``chunks`` is a list of ``(k, v, start)``: k ``[B, len, Hkv, d_qk]``, v
    ``[B, len, Hkv, d_v]`` holding the keys at absolute positions
    ``start .. start+len-1``.  Query row r sits at position ``q_offset + r``.
    ``window > 0`` limits a query at p to keys at distance <= window (keys
    p - window .. p when causal).  ``anchor = S > 0`` also shows it the keys
    at a - 1, a and a + S, a = S * (p // S).  ``q_seg [B, Lq]`` with
    ``k_segs`` (one ``[B, len]`` per chunk) are segment labels: a query sees
    only keys with its label.  Returns ``(out [B, n_rows, Hq, d_v], lse
    [B, Hq, n_rows])`` in float64; a row that sees no key gets out = 0 and
    lse = -inf.
    """
    lib = _get_lib()
    p = _Problem(q, chunks, dtype, rows)
    Hkv = p.Hkv if p.Hkv is not None else Hkv
    dv = p.dv if p.dv is not None else dv
    if Hkv is None or dv is None:
        raise ValueError("with no chunks, pass Hkv and dv")
    out = np.zeros((p.B, p.nr, p.Hq, dv), dtype=np.float64)
    lse = np.zeros((p.B, p.Hq, p.nr), dtype=np.float64)
    n = len(p.ks)
    kp = (ctypes.c_void_p * max(n, 1))(*[_ptr(a) for a in p.ks])
    vp = (ctypes.c_void_p * max(n, 1))(*[_ptr(a) for a in p.vs])
    st = np.asarray(p.starts if n else [0], dtype=np.int64)
    ln = np.asarray(p.lens if n else [0], dtype=np.int64)
    mk, _keep = _mask(p, causal, window, anchor, q_seg, k_segs)
    rc = lib.oracle_attention(p.B, p.Hq, Hkv, p.dqk, dv, p.code, _ptr(p.q), p.Lq,
                              int(q_offset), n, kp, vp, _ptr(st), _ptr(ln),
                              ctypes.byref(mk), _scale(scale, p.dqk), p.nr,
                              _ptr(p.rows), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_attention failed ({rc})")
    return out, lse


def attention_bwd(q, chunks, dout, q_offset=0, causal=False, scale=None, dtype=None, window=0, anchor=0,
                  q_seg=None, k_segs=None):
    """Gradients of ``sum(dout * attention(q, chunks, ...))``: returns
    ``(dq [B, Lq, Hq, d_qk], [dk_c [B, len_c, Hkv, d_qk]], [dv_c [B, len_c, Hkv, d_v]])``
    in float64.  ``dout [B, Lq, Hq, d_v]`` has q's element type; masking
    (causal, window, q_offset) is as in :func:`attention`."""
    lib = _get_lib()
    p = _Problem(q, chunks, dtype, None)
    if not p.ks:
        raise ValueError("attention_bwd needs at least one chunk")
    do, code = _to_numpy(dout, dtype)
    if code != p.code or do.shape != (p.B, p.Lq, p.Hq, p.dv):
        raise ValueError("dout must have q's element type and shape [B, Lq, Hq, d_v]")
    dq = np.zeros((p.B, p.Lq, p.Hq, p.dqk), dtype=np.float64)
    dks = [np.zeros(k.shape, dtype=np.float64) for k in p.ks]
    dvs = [np.zeros(v.shape, dtype=np.float64) for v in p.vs]
    n = len(p.ks)
    kp = (ctypes.c_void_p * n)(*[_ptr(a) for a in p.ks])
    vp = (ctypes.c_void_p * n)(*[_ptr(a) for a in p.vs])
    dkp = (ctypes.c_void_p * n)(*[_ptr(a) for a in dks])
    dvp = (ctypes.c_void_p * n)(*[_ptr(a) for a in dvs])
    st = np.asarray(p.starts, dtype=np.int64)
    ln = np.asarray(p.lens, dtype=np.int64)
    mk, _keep = _mask(p, causal, window, anchor, q_seg, k_segs)
    rc = lib.oracle_attention_bwd(p.B, p.Hq, p.Hkv, p.dqk, p.dv, p.code, _ptr(p.q), p.Lq,
                                  int(q_offset), n, kp, vp, _ptr(st), _ptr(ln), ctypes.byref(mk),
                                  _scale(scale, p.dqk), _ptr(do), _ptr(dq), dkp, dvp)
    if rc != 0:
        raise ValueError(f"oracle_attention_bwd failed ({rc})")
    return dq, dks, dvs


class State:
    """Running softmax state of one device: m, l ``[B, Hq, n_rows]`` and O
    ``[B, Hq, n_rows, d_v]`` (unnormalised), all float64."""

    def __init__(self, B, Hq, nr, dv):
        self.m = np.empty((B, Hq, nr), dtype=np.float64)
        self.l = np.empty((B, Hq, nr), dtype=np.float64)
        self.O = np.empty((B, Hq, nr, dv), dtype=np.float64)
        _get_lib().oracle_state_init(B * Hq * nr, dv, _ptr(self.m), _ptr(self.l),
                                     _ptr(self.O))

    def copy(self):
        s = State.__new__(State)
        s.m, s.l, s.O = self.m.copy(), self.l.copy(), self.O.copy()
        return s


def ring_step(state: State, q, chunk, q_offset=0, causal=False, scale=None,
              rows=None, dtype=None, window=0, anchor=0, q_seg=None, k_seg=None) -> State:
    """Fold one KV chunk ``(k, v, start)`` into ``state`` in place."""
    lib = _get_lib()
    p = _Problem(q, [chunk], dtype, rows)
    if state.O.shape != (p.B, p.Hq, p.nr, p.dv):
        raise ValueError("state shape does not match the problem")
    mk, _keep = _mask(p, causal, window, anchor, q_seg, None if k_seg is None else [k_seg])
    rc = lib.oracle_ring_step(p.B, p.Hq, p.Hkv, p.dqk, p.dv, p.code, _ptr(p.q),
                              p.Lq, int(q_offset), _ptr(p.ks[0]), _ptr(p.vs[0]),
                              p.starts[0], p.lens[0], ctypes.byref(mk),
                              _scale(scale, p.dqk), p.nr, _ptr(p.rows),
                              _ptr(state.m), _ptr(state.l), _ptr(state.O))
    if rc != 0:
        raise ValueError(f"oracle_ring_step failed ({rc})")
    return state


def ring(q, chunks, order=None, q_offset=0, causal=False, scale=None, rows=None,
         dtype=None, window=0, anchor=0, q_seg=None, k_segs=None) -> State:
    """One device's share of the ring: fold the chunks in ``order`` (default:
    list order) into a fresh state and return it."""
    qa, _ = _to_numpy(q, dtype)
    B, Lq, Hq, _ = qa.shape
    nr = Lq if rows is None else len(rows)
    dv = int(chunks[0][1].shape[3])
    st = State(B, Hq, nr, dv)
    for c in (range(len(chunks)) if order is None else order):
        ring_step(st, q, chunks[c], q_offset, causal, scale, rows, dtype, window, anchor, q_seg,
                  None if k_segs is None else k_segs[c])
    return st


def merge(a: State, b: State) -> State:
    """Combine two partial states over disjoint key sets."""
    if a.O.shape != b.O.shape:
        raise ValueError("states must have the same shape")
    out = State.__new__(State)
    out.m, out.l, out.O = np.empty_like(a.m), np.empty_like(a.l), np.empty_like(a.O)
    n, dv = a.m.size, a.O.shape[-1]
    _get_lib().oracle_merge(n, dv, _ptr(a.m), _ptr(a.l), _ptr(a.O), _ptr(b.m),
                            _ptr(b.l), _ptr(b.O), _ptr(out.m), _ptr(out.l),
                            _ptr(out.O))
    return out


def finalize(state: State):
    """Return ``(out [B, n_rows, Hq, d_v], lse [B, Hq, n_rows])`` of a state."""
    B, Hq, nr, dv = state.O.shape
    out = np.empty((B, Hq, nr, dv), dtype=np.float64)
    lse = np.empty((B, Hq, nr), dtype=np.float64)
    _get_lib().oracle_finalize(B * Hq * nr, dv, _ptr(state.m), _ptr(state.l),
                               _ptr(state.O), _ptr(out), _ptr(lse))
    return np.ascontiguousarray(out.transpose(0, 2, 1, 3)), lse
