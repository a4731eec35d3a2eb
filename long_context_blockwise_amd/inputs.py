"""Seeded synthetic inputs for ring-attention workloads.

This module is shared by the HIP path (benchmark, GPU tests) and by the CPU
oracle's tests.  It holds none of the method's arithmetic: it only describes
workload shapes and draws seeded random tensors.  Every tensor is drawn in
float32 from N(0, 1) with a torch generator seeded per (workload seed, tensor,
chunk), multiplied by the workload's scale, and rounded to the workload dtype
(round-to-nearest-even for bfloat16).  The same bits are handed to both sides:
GPU tests copy the generated device tensors to the host for the oracle.

Workloads (one device's share of the ring, shapes from the pages' settings):

* ``tiny_ring_fp32``: 1 batch, 1 head, d=64, fp32, a 1024-token sequence as 4
  chunks of 256; query chunk 0 against all 4 KV chunks, non-causal.
* ``prefill_bf16_h32_d128``: 32 heads, d=128, bf16, 32768 tokens as 4 chunks
  of 8192; query chunk 3 against chunks 0..3, causal; entries N(0,1)*0.5.
* ``ring_1m_gqa32x8_d128``: 32 query / 8 KV heads, d=128, bf16, 1,048,576
  tokens as 32 chunks of 32768; the last query chunk, causal; N(0,1)*0.5.
* ``mla_h16_d512``: 16 query heads sharing one 512-wide KV head, bf16, 131072
  tokens as 8 chunks of 16384; query chunk 7, causal; N(0,1)*4/sqrt(512).
* ``local_w4096_s4096_h32_d128``: the prefill share with a local window (a
  query at p sees keys p - 4096 .. p) and anchor tokens every 4096 positions.
* ``docs4096_h32_d128``: the prefill share over packed documents of seeded
  lengths uniform in 1 .. 8192 (mean 4096), with segment labels: a query
  sees the earlier keys of its own document.
* ``decode_b4_gqa32x8_cache1m``: 4 sequences, 32 query / 8 KV heads, d=128,
  bf16, a 1,048,576-token KV cache in 64 chunks of 16384; 16 new query tokens
  at cache_idx = 1,048,560 (their K/V are the cache's last 16 slots), causal.
* ``decode_b4_gqa32x8_cache1m_fp8``: the same decode with the KV cache held
  in 8 bits (OCP FP8 E4M3, one power-of-two scale per 64 tokens of a
  (batch, KV head)); queries stay bf16.
* ``decode_b4_gqa32x8_cache1m_bhsd``, ``decode_b4_gqa32x8_cache1m_fp8_bhsd``:
  the same two decodes with the cache stored head-major (the same values;
  memory order [B, Hkv, len, d], passed as BSHD with strides).

8-bit KV caches are drawn like the others and then quantised block by block
(input preparation, not the method): each block of 64 tokens x d values of
one (batch, KV head) gets the scale 2^e with the smallest e for which its
largest magnitude fits under 448, and the values divided by the scale are
rounded to E4M3 (round to nearest even).  Chunks of such workloads are
``(k, v, start, k_exp, v_exp)`` with k, v ``torch.float8_e4m3fn`` and the
biased exponents e + 127 as ``uint8 [B, Hkv, ceil(len/64)]``.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import List, Optional, Tuple

import torch

_TENSOR_Q, _TENSOR_K, _TENSOR_V, _TENSOR_DO = 0, 1, 2, 3


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d_qk: int
    d_v: int
    dtype: str  # "fp32" | "bf16"
    chunk_len: int  # tokens per KV chunk
    P: int  # number of KV chunks
    Lq: int  # query rows of this device
    q_offset: int  # absolute position of query row 0
    causal: bool
    std: float  # inputs are N(0,1) * std before rounding
    seed: int
    # explicit per-chunk lengths (ragged tails); None means all chunk_len
    chunk_lens: Optional[Tuple[int, ...]] = field(default=None)
    kv_dtype: Optional[str] = None  # None: same as dtype; "fp8": 8-bit KV cache
    window: int = 0     # local window half-width in tokens (0: none)
    anchor: int = 0     # anchor stride in tokens (0: none)
    doc_mean: int = 0   # packed documents of this mean length carry segment labels (0: none)
    kv_heads_major: bool = False  # K/V stored head-major ([B, Hkv, len, d] memory, BSHD strides)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    def lens(self) -> List[int]:
        return list(self.chunk_lens) if self.chunk_lens else [self.chunk_len] * self.P

    def starts(self) -> List[int]:
        s, out = 0, []
        for n in self.lens():
            out.append(s)
            s += n
        return out

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny_ring_fp32": Workload("tiny_ring_fp32", B=1, Hq=1, Hkv=1, d_qk=64, d_v=64,
                               dtype="fp32", chunk_len=256, P=4, Lq=256, q_offset=0,
                               causal=False, std=1.0, seed=1),
    "prefill_bf16_h32_d128": Workload("prefill_bf16_h32_d128", B=1, Hq=32, Hkv=32,
                                      d_qk=128, d_v=128, dtype="bf16", chunk_len=8192,
                                      P=4, Lq=8192, q_offset=3 * 8192, causal=True,
                                      std=0.5, seed=2),
    "ring_1m_gqa32x8_d128": Workload("ring_1m_gqa32x8_d128", B=1, Hq=32, Hkv=8,
                                     d_qk=128, d_v=128, dtype="bf16", chunk_len=32768,
                                     P=32, Lq=32768, q_offset=31 * 32768, causal=True,
                                     std=0.5, seed=3),
    "mla_h16_d512": Workload("mla_h16_d512", B=1, Hq=16, Hkv=1, d_qk=512, d_v=512,
                             dtype="bf16", chunk_len=16384, P=8, Lq=16384,
                             q_offset=7 * 16384, causal=True, std=4.0 / 512 ** 0.5,
                             seed=4),
    "local_w4096_s4096_h32_d128": Workload("local_w4096_s4096_h32_d128", B=1, Hq=32, Hkv=32,
                                           d_qk=128, d_v=128, dtype="bf16", chunk_len=8192,
                                           P=4, Lq=8192, q_offset=3 * 8192, causal=True,
                                           std=0.5, seed=2, window=4096, anchor=4096),
    "docs4096_h32_d128": Workload("docs4096_h32_d128", B=1, Hq=32, Hkv=32, d_qk=128, d_v=128,
                                  dtype="bf16", chunk_len=8192, P=4, Lq=8192, q_offset=3 * 8192,
                                  causal=True, std=0.5, seed=2, doc_mean=4096),
    "decode_b4_gqa32x8_cache1m": Workload("decode_b4_gqa32x8_cache1m", B=4, Hq=32,
                                          Hkv=8, d_qk=128, d_v=128, dtype="bf16",
                                          chunk_len=16384, P=64, Lq=16,
                                          q_offset=1048560, causal=True, std=0.5,
                                          seed=5),
    "decode_b4_gqa32x8_cache1m_fp8": Workload("decode_b4_gqa32x8_cache1m_fp8", B=4, Hq=32,
                                              Hkv=8, d_qk=128, d_v=128, dtype="bf16",
                                              chunk_len=16384, P=64, Lq=16,
                                              q_offset=1048560, causal=True, std=0.5,
                                              seed=5, kv_dtype="fp8"),
}
# the two decode caches stored head-major ([B, Hkv, len, d] in memory): each
# (sequence, KV head) reads one contiguous range instead of 128- or 256-byte
# rows at the stride of all heads
for _n in ("decode_b4_gqa32x8_cache1m", "decode_b4_gqa32x8_cache1m_fp8"):
    WORKLOADS[_n + "_bhsd"] = replace(WORKLOADS[_n], name=_n + "_bhsd", kv_heads_major=True)

KV_SCALE_BLOCK = 64  # tokens per shared exponent of an 8-bit KV cache
FP8_MAX = 448.0      # largest finite OCP FP8 E4M3 value


def quantize_fp8(x: torch.Tensor, block: int = KV_SCALE_BLOCK):
    """``x [B, n, H, d]`` -> (E4M3 codes as ``torch.float8_e4m3fn`` [B, n, H, d],
    biased exponents ``uint8 [B, H, ceil(n/block)]``)."""
    B, n, H, d = x.shape
    nb = (n + block - 1) // block
    xf = x.float()
    pad = torch.zeros((B, nb * block - n, H, d), dtype=xf.dtype, device=xf.device)
    blocks = torch.cat([xf, pad], 1).view(B, nb, block, H, d)
    amax = blocks.abs().amax(dim=(2, 4))  # [B, nb, H]
    e = torch.ceil(torch.log2(torch.clamp(amax, min=2.0 ** -100) / FP8_MAX))
    e = torch.clamp(e, -126, 127)
    scale = torch.pow(2.0, e)  # exact powers of two
    per_token = scale.repeat_interleave(block, dim=1)[:, :n].unsqueeze(-1)  # [B, n, H, 1]
    codes = (xf / per_token).to(torch.float8_e4m3fn)
    exps = (e + 127).to(torch.uint8).permute(0, 2, 1).contiguous()  # [B, H, nb]
    return codes, exps


def _generator(device, seed: int, tensor: int, chunk: int) -> torch.Generator:
    g = torch.Generator(device=device)
    # one independent stream per (workload seed, tensor, chunk)
    g.manual_seed((seed * 1_000_003 + tensor * 65_537 + chunk * 257 + 12_345) % (2**63))
    return g


def draw(shape, std: float, dtype, device, seed: int, tensor: int, chunk: int = 0):
    """N(0,1)*std in float32 from a seeded stream, rounded to ``dtype``."""
    g = _generator(device, seed, tensor, chunk)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


@dataclass
class Inputs:
    wl: Workload
    q: torch.Tensor  # [B, Lq, Hq, d_qk]
    ks: List[torch.Tensor]  # chunk c: [B, len_c, Hkv, d_qk]
    vs: List[torch.Tensor]  # chunk c: [B, len_c, Hkv, d_v]
    starts: List[int]
    k_exps: Optional[List[torch.Tensor]] = None  # 8-bit KV: [B, Hkv, ceil(len_c/64)]
    v_exps: Optional[List[torch.Tensor]] = None

    def chunks(self, order=None):
        """``[(k, v, start)]`` (8-bit KV: ``(k, v, start, k_exp, v_exp)``) in
        ``order`` (default: chunk index order)."""
        idx = range(len(self.ks)) if order is None else order
        if self.k_exps is not None:
            return [(self.ks[c], self.vs[c], self.starts[c], self.k_exps[c], self.v_exps[c]) for c in idx]
        return [(self.ks[c], self.vs[c], self.starts[c]) for c in idx]


def output_grad(wl: Workload, device="cpu", std: float = 1.0) -> torch.Tensor:
    """A seeded gradient of the attention output, ``[B, Lq, Hq, d_v]`` in the
    workload dtype (N(0,1)*std), for the backward pass."""
    return draw((wl.B, wl.Lq, wl.Hq, wl.d_v), std, wl.torch_dtype, device, wl.seed, _TENSOR_DO)


def packed_labels(B: int, n: int, mean_doc: int, seed: int, device="cpu") -> torch.Tensor:
    """Segment labels ``[B, n]`` (int32) of sequences packed from documents
    of seeded random lengths (uniform in 1 .. 2 * mean_doc): position t of
    batch b carries the index of its document."""
    g = torch.Generator().manual_seed(seed)
    out = torch.empty((B, n), dtype=torch.int32)
    for b in range(B):
        pos, doc = 0, 0
        while pos < n:
            L = int(torch.randint(1, 2 * mean_doc + 1, (1,), generator=g))
            out[b, pos:pos + L] = doc
            pos += L
            doc += 1
    return out.to(device)


def segment_labels(wl: Workload, device="cpu"):
    """``(q_seg [B, Lq], [k_seg_c [B, len_c] for each chunk c])`` of a
    workload with packed documents (``packed_labels`` over all its tokens),
    or ``(None, None)``."""
    if not wl.doc_mean:
        return None, None
    total = sum(wl.lens())
    lab = packed_labels(wl.B, max(total, wl.q_offset + wl.Lq), wl.doc_mean, wl.seed, device)
    q_seg = lab[:, wl.q_offset:wl.q_offset + wl.Lq].contiguous()
    k_segs = [lab[:, s:s + n].contiguous() for s, n in zip(wl.starts(), wl.lens())]
    return q_seg, k_segs


def make(wl: Workload, device="cpu", q_std: Optional[float] = None) -> Inputs:
    """Draw the query chunk and all KV chunks of a workload on ``device``."""
    dt = wl.torch_dtype
    q = draw((wl.B, wl.Lq, wl.Hq, wl.d_qk), wl.std if q_std is None else q_std, dt,
             device, wl.seed, _TENSOR_Q)
    ks, vs = [], []
    kes, ves = ([], []) if wl.kv_dtype == "fp8" else (None, None)
    for c, n in enumerate(wl.lens()):
        k = draw((wl.B, n, wl.Hkv, wl.d_qk), wl.std, dt, device, wl.seed, _TENSOR_K, c)
        v = draw((wl.B, n, wl.Hkv, wl.d_v), wl.std, dt, device, wl.seed, _TENSOR_V, c)
        if kes is not None:
            k, ke = quantize_fp8(k)
            v, ve = quantize_fp8(v)
            kes.append(ke)
            ves.append(ve)
        if wl.kv_heads_major:  # the same values, each head's tokens contiguous
            k = k.transpose(1, 2).contiguous().transpose(1, 2)
            v = v.transpose(1, 2).contiguous().transpose(1, 2)
        ks.append(k)
        vs.append(v)
    return Inputs(wl, q, ks, vs, wl.starts(), kes, ves)


def sample_rows(Lq: int, tile: int = 128, seed: int = 0, extra=()) -> List[int]:
    """A stratified row sample: one seeded random row per ``tile`` rows plus
    rows at tile and chunk boundaries (and ``extra``), sorted and unique."""
    g = torch.Generator().manual_seed(seed)
    rows = set()
    for t0 in range(0, Lq, tile):
        n = min(tile, Lq - t0)
        rows.add(t0 + int(torch.randint(n, (1,), generator=g)))
    for r in (0, 1, 15, 16, 31, 32, 63, 64, 127, 128, Lq // 2 - 1, Lq // 2, Lq - 2,
              Lq - 1, *extra):
        if 0 <= r < Lq:
            rows.add(int(r))
    return sorted(rows)
