"""bf16 queries against an 8-bit KV cache (OCP FP8 E4M3 codes with one
power-of-two scale per 64 tokens of a (batch, KV head)) on the GPU, compared
with the oracle's plain attention over the decoded cache.  Decoding is exact
in bf16, so the bf16 tolerances apply."""
import numpy as np
import pytest
import torch

import long_context_blockwise_amd as ra
from long_context_blockwise_amd import inputs
from parity import check, oracle_out, oracle_state

pytestmark = pytest.mark.gpu


def _inputs(B, Hq, Hkv, lens, Lq, q_offset, causal, seed, q_std=0.5):
    wl = inputs.Workload("fp8_case", B=B, Hq=Hq, Hkv=Hkv, d_qk=128, d_v=128, dtype="bf16",
                         chunk_len=lens[0], P=len(lens), Lq=Lq, q_offset=q_offset, causal=causal,
                         std=0.5, seed=seed, chunk_lens=tuple(lens), kv_dtype="fp8")
    return inputs.make(wl, "cuda", q_std=q_std)


CASES = [
    # B, Hq, Hkv, chunk lengths, Lq, q_offset, causal, query std
    (1, 8, 8, (256,), 1, 255, True, 0.5),            # one new token, one head per KV head
    (2, 32, 8, (1000, 4133), 16, 5117, True, 0.5),   # GQA 4, ragged chunks, the last 16 tokens
    (1, 16, 1, (3000,), 3, 1500, True, 0.5),         # 16 query heads on one KV head, future keys masked
    (3, 4, 2, (64, 64, 130), 7, 0, False, 0.5),      # several small chunks, non-causal
    (1, 8, 2, (2048,), 40, 2008, True, 0.5),         # a 40-row query block (split-KV is forced)
    (2, 8, 4, (700, 333), 5, 1028, True, 6.0),       # large logits: the reference max moves
]


@pytest.mark.parametrize("B,Hq,Hkv,lens,Lq,q_off,causal,q_std", CASES,
                         ids=[f"B{c[0]}_Hq{c[1]}_Hkv{c[2]}_L{'-'.join(map(str, c[3]))}_Lq{c[4]}" for c in CASES])
def test_fp8_decode_matches_oracle(B, Hq, Hkv, lens, Lq, q_off, causal, q_std):
    x = _inputs(B, Hq, Hkv, lens, Lq, q_off, causal, seed=7 + Lq, q_std=q_std)
    chunks = x.chunks()
    out, _ = ra.ring_attn_fwd(x.q, chunks, causal, q_off)
    torch.cuda.synchronize()
    ref, _ = oracle_out(x.q, chunks, q_off, causal)
    check(out.float().cpu().numpy(), ref, "bf16", f"fp8 B{B} Hq{Hq} Hkv{Hkv} {lens} Lq{Lq}")


def test_fp8_state_outputs():
    x = _inputs(2, 8, 2, (500, 260), 9, 751, True, seed=3)
    chunks = x.chunks()
    out, (m, l, O) = ra.ring_attn_fwd(x.q, chunks, True, 751, want_state=True)
    torch.cuda.synchronize()
    rm, rl, rO = oracle_state(x.q, chunks, 751, True)
    check(m.cpu().numpy(), rm, "bf16", "fp8 m", rel_l2=True)
    ratio = l.cpu().numpy() / rl
    assert np.all(np.abs(ratio - 1) < 1e-2), ratio
    check((O / l.unsqueeze(-1)).cpu().numpy(), rO / rl[..., None], "bf16", "fp8 O/l")


def test_fp8_is_half_the_bytes_of_bf16():
    x = _inputs(1, 8, 2, (1024,), 4, 1020, True, seed=5)
    k8, v8, _, ke, _ = x.chunks()[0]
    assert k8.element_size() == 1 and v8.element_size() == 1
    assert ke.shape == (1, 2, 16) and ke.dtype == torch.uint8


def test_fp8_prefill_schedule_is_rejected():
    x = _inputs(1, 8, 2, (256,), 32, 224, True, seed=9)
    with pytest.raises(ra.RingAttnError) as e:
        ra.ring_attn_fwd(x.q, x.chunks(), True, 224, flags=ra.RA_FLAG_STAGE)
    assert e.value.code == ra.RA_ERR_UNSUPPORTED
