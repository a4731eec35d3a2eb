"""The CPU oracle against its pins (no GPU needed)."""
import math

import numpy as np
import pytest

import oracle_pins
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(oracle_mod, pin):
    pin()


def _wrong_sum_of_chunk_softmaxes(q, chunks, scale):
    """The per-chunk-normalised sum, read literally from the equation printed
    on page "Ring Attention：百万 Token 上下文的秘密", §2.3: it normalises each
    chunk on its own and adds the results.  Not attention."""
    out = 0.0
    for (k, v, _) in chunks:
        s = np.einsum("brhd,bthd->bhrt", q, k) * scale
        w = np.exp(s - s.max(-1, keepdims=True))
        w /= w.sum(-1, keepdims=True)
        out = out + np.einsum("bhrt,bthd->brhd", w, v)
    return out


def _wrong_two_chunk_window(q, chunks, scale, i):
    """Page "RingAttention与RAG技术对比及实战应用", §2.1 sketch: query chunk i
    attends only to KV chunks i and i+1 with no running rescale."""
    ks = np.concatenate([c[0] for c in chunks[i:i + 2]], axis=1)
    vs = np.concatenate([c[1] for c in chunks[i:i + 2]], axis=1)
    s = np.einsum("brhd,bthd->bhrt", q, ks) * scale
    w = np.exp(s - s.max(-1, keepdims=True))
    w /= w.sum(-1, keepdims=True)
    return np.einsum("bhrt,bthd->brhd", w, vs)


def test_known_wrong_readings_disagree(oracle_mod):
    """Two readings of the pages that are not attention must not match the
    oracle (so the oracle did not adopt either)."""
    rng = np.random.default_rng(0)
    q = rng.standard_normal((1, 6, 2, 8))
    chunks = [(rng.standard_normal((1, 6, 2, 8)), rng.standard_normal((1, 6, 2, 8)), 6 * i)
              for i in range(4)]
    out, _ = oracle_mod.attention(q, chunks, 0, False)
    scale = 1 / math.sqrt(8)
    assert np.abs(_wrong_sum_of_chunk_softmaxes(q, chunks, scale) - out).max() > 0.1
    assert np.abs(_wrong_two_chunk_window(q, chunks, scale, 0) - out).max() > 0.05


def test_oracle_threads(oracle_mod):
    assert oracle_mod.threads() >= 1


def test_oracle_rejects_bad_shapes(oracle_mod):
    q = np.zeros((1, 2, 3, 4))
    k = np.zeros((1, 2, 2, 4))  # Hq=3 not a multiple of Hkv=2
    with pytest.raises(ValueError):
        oracle_mod.attention(q, [(k, k, 0)], 0, False)
    k = np.zeros((1, 2, 1, 4))
    with pytest.raises(ValueError):
        oracle_mod.attention(q, [(k, k, 0)], 0, False, rows=[5])
