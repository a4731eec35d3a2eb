"""Pins that tie the CPU oracle to facts fixed outside it.

Each ``pin_*`` function raises ``AssertionError`` when the oracle disagrees
with something the pages or the mathematics fix independently of the
oracle's own code:

* a library routine that computes the same definition
  (``torch.nn.functional.scaled_dot_product_attention`` in float64 with an
  explicit position mask);
* closed forms that need no softmax code at all (zero queries give the mean
  of the visible values, constant values give that constant, two keys give a
  logistic mix, the first causal row gives V_0, ...);
* the exact result, computed with 50-digit mpmath arithmetic on tiny inputs,
  including logits large enough to overflow a softmax without the max shift;
* invariants the pages assert: the ring result equals plain attention for
  every chunk count and every chunk order (page "Ring Attention：百万 Token
  上下文的秘密", §2.2 环形通信 and §2.3 数学正确性), partial states merge
  into the global softmax (page "从百毫秒到百万Token", 注意力融合层), and a
  query at cache_idx + t reproduces prefill row cache_idx + t (page
  "RingAttention推理优化：cache_idx参数使用...", 增量推理实战).

``tests/test_oracle_pins.py`` runs them; ``tests/test_oracle_mutants.py``
plants mistakes in copies of ``oracle.c`` and checks that each one makes at
least one pin fail.
"""
from __future__ import annotations

import itertools
import math

import mpmath
import numpy as np
import torch

import oracle

TOL = 1e-12


def _rand(rng, B, Lq, Hq, Hkv, dqk, dv, lens, std=1.0, vstd=1.0):
    q = rng.standard_normal((B, Lq, Hq, dqk)) * std
    chunks, s = [], 0
    for n in lens:
        k = rng.standard_normal((B, n, Hkv, dqk)) * std
        v = rng.standard_normal((B, n, Hkv, dv)) * vstd
        chunks.append((k, v, s))
        s += n
    return q, chunks


def _close(a, b, tol, what):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    err = np.where(both_inf, 0.0, np.abs(a - b))
    bad = ~(err <= tol * (1.0 + np.abs(b)))
    assert not bad.any(), f"{what}: max err {np.nanmax(err)} (tol {tol})"


def _positions(chunks):
    return np.concatenate([s + np.arange(k.shape[1]) for (k, _, s) in chunks])


# --------------------------------------------------------------------------- #
# library routine
# --------------------------------------------------------------------------- #
def _sdpa(q, chunks, q_offset, causal, scale):
    """float64 SDPA with an explicit boolean position mask (SDPA's own
    ``is_causal`` aligns the diagonal to the top-left corner, which is wrong
    for a query chunk at an offset, so it is not used)."""
    K = torch.from_numpy(np.concatenate([c[0] for c in chunks], axis=1))
    V = torch.from_numpy(np.concatenate([c[1] for c in chunks], axis=1))
    Q = torch.from_numpy(q)
    pos = torch.from_numpy(_positions(chunks))
    qpos = q_offset + torch.arange(q.shape[1])
    mask = torch.ones(q.shape[1], K.shape[1], dtype=torch.bool)
    if causal:
        mask = pos[None, :] <= qpos[:, None]
    out = torch.nn.functional.scaled_dot_product_attention(
        Q.permute(0, 2, 1, 3), K.permute(0, 2, 1, 3), V.permute(0, 2, 1, 3),
        attn_mask=mask, scale=scale, enable_gqa=True)
    return out.permute(0, 2, 1, 3).numpy()


def pin_library_sdpa():
    rng = np.random.default_rng(101)
    cases = [
        # B, Lq, Hq, Hkv, dqk, dv, lens, q_offset, causal
        (1, 7, 1, 1, 8, 8, [5, 9, 3], 0, False),
        (2, 6, 4, 2, 5, 3, [4, 4, 4], 9, True),
        (1, 9, 6, 3, 16, 16, [7, 1, 8, 2], 11, True),
        (2, 4, 8, 1, 12, 7, [6, 10], 15, True),
        (1, 5, 2, 2, 4, 9, [3, 3], 0, False),
        (1, 8, 4, 4, 6, 6, [8, 8, 8], 16, True),   # query chunk = last chunk
    ]
    for (B, Lq, Hq, Hkv, dqk, dv, lens, q_off, causal) in cases:
        q, chunks = _rand(rng, B, Lq, Hq, Hkv, dqk, dv, lens)
        scale = 1.0 / math.sqrt(dqk)
        out, _ = oracle.attention(q, chunks, q_off, causal)
        ref = _sdpa(q, chunks, q_off, causal, scale)
        _close(out, ref, 1e-12, f"sdpa {B,Lq,Hq,Hkv,dqk,dv,lens,q_off,causal}")
        # explicit repeat of KV heads (contiguous head groups) gives the same
        g = Hq // Hkv
        chunks_rep = [(np.repeat(k, g, axis=2), np.repeat(v, g, axis=2), s)
                      for (k, v, s) in chunks]
        out_rep, _ = oracle.attention(q, chunks_rep, q_off, causal)
        _close(out, out_rep, 1e-14, "gqa == repeated kv heads")


# --------------------------------------------------------------------------- #
# closed forms
# --------------------------------------------------------------------------- #
def pin_zero_query_mean():
    """Q = 0 makes every visible score 0: the output is the plain mean of the
    visible value rows and lse = log(#visible)."""
    rng = np.random.default_rng(7)
    B, Lq, Hq, Hkv, dqk, dv = 2, 6, 4, 2, 8, 5
    lens = [5, 3, 6]
    _, chunks = _rand(rng, B, Lq, Hq, Hkv, dqk, dv, lens)
    q = np.zeros((B, Lq, Hq, dqk))
    for causal, q_off in ((False, 0), (True, 4), (True, 8)):
        out, lse = oracle.attention(q, chunks, q_off, causal)
        V = np.concatenate([c[1] for c in chunks], axis=1)
        pos = _positions(chunks)
        for r in range(Lq):
            vis = pos <= q_off + r if causal else np.ones_like(pos, dtype=bool)
            n = int(vis.sum())
            for h in range(Hq):
                want = V[:, vis, h // (Hq // Hkv), :].mean(axis=1)
                _close(out[:, r, h, :], want, 1e-14, f"mean row {r} head {h}")
                _close(lse[:, h, r], np.full(B, math.log(n)), 1e-14, "lse log n")


def pin_constant_values():
    """Softmax weights sum to one: constant value rows give that constant."""
    rng = np.random.default_rng(8)
    B, Lq, Hq, Hkv, dqk, dv = 1, 5, 2, 1, 6, 4
    q, chunks = _rand(rng, B, Lq, Hq, Hkv, dqk, dv, [4, 7], std=2.0)
    c = np.array([0.5, -3.0, 7.25, 1e-3])
    chunks = [(k, np.broadcast_to(c, v.shape).copy(), s) for (k, v, s) in chunks]
    out, _ = oracle.attention(q, chunks, 3, True)
    _close(out, np.broadcast_to(c, out.shape), 1e-14, "constant values")


def pin_first_causal_row():
    """A causal query at position 0 sees key 0 only: output V_0 exactly."""
    rng = np.random.default_rng(9)
    q, chunks = _rand(rng, 2, 3, 4, 2, 8, 8, [4, 4], std=3.0)
    out, lse = oracle.attention(q, chunks, 0, True, rows=[0])
    V0 = chunks[0][1][:, 0, :, :]  # [B, Hkv, dv]
    for h in range(4):
        assert np.array_equal(out[:, 0, h, :], V0[:, h // 2, :]), "row 0 must equal V_0"
    # lse = the single score
    k0 = chunks[0][0][:, 0, :, :]
    for h in range(4):
        s = (q[:, 0, h, :] * k0[:, h // 2, :]).sum(-1) / math.sqrt(8)
        _close(lse[:, h, 0], s, 1e-14, "lse of one key")


def pin_two_keys_logistic():
    """With two visible keys the output is v1 + (v2 - v1) * sigmoid(s2 - s1),
    s_i = q.k_i / sqrt(d); the scale 1/sqrt(d) is fixed by the definition."""
    d = 4
    q = np.array([[[[2.0, 0.0, 1.0, 0.0]]]])  # [1,1,1,4]
    k = np.array([[[[1.0, 0.0, 0.0, 0.0]], [[0.0, 0.0, 3.0, 0.0]]]])  # [1,2,1,4]
    v = np.array([[[[1.0, 2.0]], [[-1.0, 5.0]]]])
    out, lse = oracle.attention(q, [(k, v, 0)], 0, False)
    s1, s2 = 2.0 / math.sqrt(d), 3.0 / math.sqrt(d)
    sig = 1.0 / (1.0 + math.exp(-(s2 - s1)))
    want = v[0, 0, 0] + (v[0, 1, 0] - v[0, 0, 0]) * sig
    _close(out[0, 0, 0], want, 1e-15, "two-key logistic")
    _close(lse[0, 0, 0], s1 + math.log1p(math.exp(s2 - s1)), 1e-15, "two-key lse")
    # explicit scale overrides the default
    out2, _ = oracle.attention(q, [(k, v, 0)], 0, False, scale=1.0)
    sig2 = 1.0 / (1.0 + math.exp(-(3.0 - 2.0)))
    _close(out2[0, 0, 0], v[0, 0, 0] + (v[0, 1, 0] - v[0, 0, 0]) * sig2, 1e-15,
           "explicit scale")


def pin_hardmax_limit():
    """Q = lambda * K_t with large lambda and orthonormal keys: all weight on
    key t, output V_t (to double precision)."""
    d = 8
    K = np.eye(d)[None, :, None, :]  # [1, 8, 1, 8]
    rng = np.random.default_rng(3)
    V = rng.standard_normal((1, d, 1, 5))
    for t in range(d):
        q = (60.0 * K[:, t, :, :])[:, None, :, :]  # score gap 60/sqrt(8)*... > 20
        out, _ = oracle.attention(q * math.sqrt(d), [(K[:, :4], V[:, :4], 0),
                                                     (K[:, 4:], V[:, 4:], 4)], 0, False)
        _close(out[0, 0, 0], V[0, t, 0], 1e-20 + 1e-15, f"hardmax key {t}")


def pin_empty_rows():
    """A row that sees no key (all chunks in its future) gives 0 and lse -inf;
    a chunk entirely in the future leaves the running state bit-identical."""
    rng = np.random.default_rng(12)
    q, chunks = _rand(rng, 1, 4, 2, 2, 4, 3, [4, 4])
    shifted = [(k, v, s + 100) for (k, v, s) in chunks]
    out, lse = oracle.attention(q, shifted, 0, True)
    assert np.all(out == 0.0) and np.all(np.isneginf(lse)), "empty rows"
    st = oracle.ring(q, chunks, q_offset=2, causal=True)
    before = st.copy()
    oracle.ring_step(st, q, (chunks[0][0], chunks[0][1], 50), 2, True)
    for a, b in ((st.m, before.m), (st.l, before.l), (st.O, before.O)):
        assert np.array_equal(a, b), "future chunk must not touch the state"


# --------------------------------------------------------------------------- #
# exact arithmetic on tiny inputs
# --------------------------------------------------------------------------- #
def _mp_attention(q, chunks, q_off, causal, scale):
    mpmath.mp.dps = 50
    B, Lq, Hq, dqk = q.shape
    Hkv, dv = chunks[0][0].shape[2], chunks[0][1].shape[3]
    K = np.concatenate([c[0] for c in chunks], axis=1)
    V = np.concatenate([c[1] for c in chunks], axis=1)
    pos = _positions(chunks)
    out = np.zeros((B, Lq, Hq, dv))
    lse = np.zeros((B, Hq, Lq))
    for b, r, h in itertools.product(range(B), range(Lq), range(Hq)):
        hk = h // (Hq // Hkv)
        vis = [t for t in range(K.shape[1]) if (not causal) or pos[t] <= q_off + r]
        if not vis:
            lse[b, h, r] = -math.inf
            continue
        s = {t: mpmath.fsum(mpmath.mpf(float(q[b, r, h, e])) * mpmath.mpf(float(K[b, t, hk, e]))
                            for e in range(dqk)) * mpmath.mpf(scale) for t in vis}
        w = {t: mpmath.exp(s[t]) for t in vis}  # exact: no shift needed
        z = mpmath.fsum(w.values())
        for e in range(dv):
            out[b, r, h, e] = float(mpmath.fsum(w[t] * mpmath.mpf(float(V[b, t, hk, e]))
                                                for t in vis) / z)
        lse[b, h, r] = float(mpmath.log(z))
    return out, lse


def pin_exact_mpmath():
    rng = np.random.default_rng(2024)
    cases = [
        (1, 3, 1, 1, 3, 2, [2, 3], 0, False, 1.0),
        (2, 2, 2, 1, 4, 3, [1, 4, 2], 5, True, 1.0),
        (1, 4, 4, 2, 2, 2, [3, 3], 2, True, 1.0),
        (1, 3, 2, 2, 4, 1, [4, 2], 3, True, 40.0),   # logits ~ 1e3: overflow w/o shift
        (1, 2, 1, 1, 1, 2, [6], 0, False, 60.0),
    ]
    for (B, Lq, Hq, Hkv, dqk, dv, lens, q_off, causal, std) in cases:
        q, chunks = _rand(rng, B, Lq, Hq, Hkv, dqk, dv, lens, std=std)
        scale = 1.0 / math.sqrt(dqk)
        out, lse = oracle.attention(q, chunks, q_off, causal)
        ref, ref_lse = _mp_attention(q, chunks, q_off, causal, scale)
        _close(out, ref, 1e-13, f"mpmath out {lens} std={std}")
        _close(lse, ref_lse, 1e-13, f"mpmath lse {lens} std={std}")
        st = oracle.ring(q, chunks, q_offset=q_off, causal=causal)
        rout, rlse = oracle.finalize(st)
        _close(rout, ref, 1e-12, f"mpmath ring out {lens} std={std}")
        _close(rlse, ref_lse, 1e-12, f"mpmath ring lse {lens} std={std}")


# --------------------------------------------------------------------------- #
# invariants the pages assert
# --------------------------------------------------------------------------- #
def _split(n, P, rng=None):
    """Split n keys into P chunks (ragged when P does not divide n)."""
    if rng is None:
        base, rem = divmod(n, P)
        return [base + (1 if i < rem else 0) for i in range(P)]
    cuts = sorted(rng.choice(np.arange(1, n), size=P - 1, replace=False))
    return list(np.diff([0, *cuts, n]))


def pin_ring_equals_full():
    """Ring output equals plain attention for every chunk count P and every
    order in which the chunks arrive."""
    rng = np.random.default_rng(5)
    N = 24
    B, Lq, Hq, Hkv, dqk, dv = 1, 5, 4, 2, 6, 4
    q = rng.standard_normal((B, Lq, Hq, dqk)) * 1.5
    Kall = rng.standard_normal((B, N, Hkv, dqk)) * 1.5
    Vall = rng.standard_normal((B, N, Hkv, dv))
    for causal, q_off in ((False, 0), (True, 7), (True, 19)):
        full, full_lse = oracle.attention(q, [(Kall, Vall, 0)], q_off, causal)
        for P in (1, 2, 3, 4, 5, 6, 8, 12, 24):
            lens = _split(N, P)
            starts = np.cumsum([0, *lens[:-1]])
            chunks = [(Kall[:, s:s + n], Vall[:, s:s + n], int(s)) for s, n in zip(starts, lens)]
            orders = (list(itertools.permutations(range(P))) if P <= 4 else
                      [list(range(P)), list(range(P))[::-1]] +
                      [list(rng.permutation(P)) for _ in range(4)])
            for order in orders:
                st = oracle.ring(q, chunks, order=order, q_offset=q_off, causal=causal)
                out, lse = oracle.finalize(st)
                _close(out, full, 1e-12, f"ring P={P} order={order} causal={causal}")
                _close(lse, full_lse, 1e-12, f"ring lse P={P}")
        # ragged random splits
        for _ in range(3):
            lens = _split(N, 5, rng)
            starts = np.cumsum([0, *lens[:-1]])
            chunks = [(Kall[:, s:s + n], Vall[:, s:s + n], int(s)) for s, n in zip(starts, lens)]
            st = oracle.ring(q, chunks, order=list(rng.permutation(5)), q_offset=q_off,
                             causal=causal)
            _close(oracle.finalize(st)[0], full, 1e-12, f"ragged ring {lens}")


def pin_merge_laws():
    """Partial states over disjoint key sets merge into the global softmax:
    merge is commutative, associative, has the empty state as identity, and
    state(chunks 0..k-1) merged with state(chunks k..P-1) equals state(all)."""
    rng = np.random.default_rng(6)
    q, chunks = _rand(rng, 2, 4, 2, 1, 5, 3, [3, 4, 5, 2], std=2.0)
    for q_off, causal in ((0, False), (6, True)):
        parts = [oracle.ring(q, [c], q_offset=q_off, causal=causal) for c in chunks]
        full, _ = oracle.attention(q, chunks, q_off, causal)
        ab, ba = oracle.merge(parts[0], parts[1]), oracle.merge(parts[1], parts[0])
        for x, y in ((ab.m, ba.m), (ab.l, ba.l), (ab.O, ba.O)):
            assert np.array_equal(x, y), "merge must be commutative"
        left = oracle.merge(oracle.merge(parts[0], parts[1]), parts[2])
        right = oracle.merge(parts[0], oracle.merge(parts[1], parts[2]))
        _close(oracle.finalize(left)[0], oracle.finalize(right)[0], 1e-14, "associative")
        empty = oracle.State(*parts[0].O.shape)
        idm = oracle.merge(parts[2], empty)
        for x, y in ((idm.m, parts[2].m), (idm.l, parts[2].l), (idm.O, parts[2].O)):
            assert np.array_equal(x, y), "empty state must be the identity"
        for k in range(1, len(chunks)):
            a = oracle.ring(q, chunks[:k], q_offset=q_off, causal=causal)
            b = oracle.ring(q, chunks[k:], q_offset=q_off, causal=causal)
            _close(oracle.finalize(oracle.merge(a, b))[0], full, 1e-13, f"split at {k}")
        tot = parts[0]
        for p in parts[1:]:
            tot = oracle.merge(tot, p)
        _close(oracle.finalize(tot)[0], full, 1e-13, "merge of per-chunk states")


def pin_causal_future_ignored():
    """Keys after a query's position do not influence it (token-level causal
    mask, diagonal included): perturbing them leaves the output bit-identical,
    perturbing the diagonal key changes it."""
    rng = np.random.default_rng(13)
    q, chunks = _rand(rng, 1, 6, 2, 2, 4, 4, [8, 8])
    q_off = 5  # rows at positions 5..10
    out, _ = oracle.attention(q, chunks, q_off, True)
    for r in range(6):
        p = q_off + r
        pert = []
        for (k, v, s) in chunks:
            k2, v2 = k.copy(), v.copy()
            sel = (s + np.arange(k.shape[1])) > p
            k2[:, sel] += 10.0
            v2[:, sel] -= 7.0
            pert.append((k2, v2, s))
        o2, _ = oracle.attention(q, pert, q_off, True, rows=[r])
        assert np.array_equal(o2[:, 0], out[:, r]), f"future keys changed row {r}"
        diag = []
        for (k, v, s) in chunks:
            v2 = v.copy()
            sel = (s + np.arange(k.shape[1])) == p
            v2[:, sel] += 1.0
            diag.append((k, v2, s))
        o3, _ = oracle.attention(q, diag, q_off, True, rows=[r])
        assert not np.allclose(o3[:, 0], out[:, r]), f"diagonal key ignored at row {r}"


def pin_rows_and_decode_positions():
    """Evaluating a subset of rows gives the same values as the full run; a
    query at cache_idx + t (incremental decode) equals prefill row
    cache_idx + t of the same sequence."""
    rng = np.random.default_rng(17)
    B, N, Hq, Hkv, d = 2, 40, 4, 2, 8
    Qfull = rng.standard_normal((B, N, Hq, d))
    K = rng.standard_normal((B, N, Hkv, d))
    V = rng.standard_normal((B, N, Hkv, d))
    chunks = [(K[:, :16], V[:, :16], 0), (K[:, 16:32], V[:, 16:32], 16),
              (K[:, 32:], V[:, 32:], 32)]
    full, full_lse = oracle.attention(Qfull, chunks, 0, True)
    rows = [0, 3, 17, 39]
    sub, sub_lse = oracle.attention(Qfull, chunks, 0, True, rows=rows)
    assert np.array_equal(sub, full[:, rows]) and np.array_equal(sub_lse, full_lse[:, :, rows])
    for cache_idx, Lq in ((37, 3), (21, 5), (0, 1)):
        qd = Qfull[:, cache_idx:cache_idx + Lq]
        dec, dec_lse = oracle.attention(qd, chunks, cache_idx, True)
        _close(dec, full[:, cache_idx:cache_idx + Lq], 1e-15, f"decode at {cache_idx}")
        _close(dec_lse, full_lse[:, :, cache_idx:cache_idx + Lq], 1e-15, "decode lse")


def pin_input_types():
    """bf16 and fp32 inputs are upcast exactly: the oracle on bf16 bit
    patterns equals the oracle on the same values in float64."""
    rng = np.random.default_rng(19)
    q, chunks = _rand(rng, 1, 4, 2, 1, 8, 8, [5, 6])
    to_bf16 = lambda a: torch.from_numpy(a).to(torch.bfloat16)
    qb = to_bf16(q)
    cb = [(to_bf16(k), to_bf16(v), s) for (k, v, s) in chunks]
    out_b, _ = oracle.attention(qb, cb, 2, True)
    c64 = [(k.double().numpy(), v.double().numpy(), s) for (k, v, s) in cb]
    out_64, _ = oracle.attention(qb.double().numpy(), c64, 2, True)
    assert np.array_equal(out_b, out_64), "bf16 upcast"
    qf = torch.from_numpy(q).float()
    cf = [(torch.from_numpy(k).float(), torch.from_numpy(v).float(), s) for (k, v, s) in chunks]
    out_f, _ = oracle.attention(qf, cf, 2, True)
    out_f64, _ = oracle.attention(qf.double().numpy(),
                                  [(k.double().numpy(), v.double().numpy(), s) for (k, v, s) in cf],
                                  2, True)
    assert np.array_equal(out_f, out_f64), "fp32 upcast"


def pin_fp8_decode_library():
    """8-bit KV decoding against torch's own OCP FP8 E4M3 conversion
    (``torch.float8_e4m3fn``), for all 256 codes at several block exponents,
    with every block of 64 tokens taking its own exponent."""
    import torch

    codes = torch.arange(256, dtype=torch.int64).to(torch.uint8)
    ref_codes = codes.view(torch.float8_e4m3fn).double()
    # [B=2, len=256 (4 blocks of 64), H=3, d=1]: token t of batch b, head h holds code (t + 37h + 11b) % 256
    B, n, H = 2, 256, 3
    t = torch.arange(n).view(1, n, 1, 1)
    h = torch.arange(H).view(1, 1, H, 1)
    b = torch.arange(B).view(B, 1, 1, 1)
    idx = (t + 37 * h + 11 * b) % 256
    c = codes[idx]
    exps = torch.tensor([[[127, 128, 120, 134], [1, 254, 127, 100], [140, 127, 126, 129]],
                         [[127, 127, 127, 127], [130, 90, 160, 127], [127, 2, 253, 127]]], dtype=torch.uint8)
    got = oracle.dequant_fp8(c, exps)
    scale = torch.pow(2.0, exps.double() - 127)  # [B, H, 4]
    ref = ref_codes[idx] * scale.permute(0, 2, 1).repeat_interleave(64, dim=1).unsqueeze(-1)
    r = ref.numpy()
    same = (got == r) | (np.isnan(got) & np.isnan(r))
    assert same.all(), ("fp8 decode", np.argwhere(~same)[:5])
    assert np.isnan(got).sum() == np.isnan(r).sum() > 0


def pin_fp8_attention_equals_decoded():
    """Attention over 8-bit chunks equals attention over the same chunks
    decoded by torch (ragged chunk lengths, GQA, causal offsets)."""
    import torch

    rng = np.random.default_rng(41)
    B, Hq, Hkv, d, Lq = 2, 4, 2, 8, 5
    q = torch.from_numpy(rng.normal(size=(B, Lq, Hq, d))).to(torch.bfloat16)
    chunks8, chunks64, start = [], [], 0
    for n in (70, 64, 3):
        nb = (n + 63) // 64
        k = torch.from_numpy(rng.normal(size=(B, n, Hkv, d)) * 3).to(torch.float8_e4m3fn)
        v = torch.from_numpy(rng.normal(size=(B, n, Hkv, d))).to(torch.float8_e4m3fn)
        ke = torch.from_numpy(rng.integers(122, 131, size=(B, Hkv, nb))).to(torch.uint8)
        ve = torch.from_numpy(rng.integers(122, 131, size=(B, Hkv, nb))).to(torch.uint8)
        def dec(x, e):
            s = torch.pow(2.0, e.double() - 127).permute(0, 2, 1).repeat_interleave(64, dim=1)[:, :x.shape[1]]
            return (x.double() * s.unsqueeze(-1)).numpy()
        chunks8.append((k, v, start, ke, ve))
        chunks64.append((dec(k, ke), dec(v, ve), start))
        start += n
    for causal, off in ((True, 130), (False, 0), (True, 66)):
        a, la = oracle.attention(q, chunks8, off, causal)
        b, lb = oracle.attention(q.double().numpy(), chunks64, off, causal)
        _close(a, b, 1e-13, f"fp8 attention causal={causal} off={off}")
        _close(la, lb, 1e-13, "fp8 lse")
    st = oracle.ring(q, chunks8, order=[2, 0, 1], q_offset=130, causal=True)
    o, _ = oracle.finalize(st)
    ref, _ = oracle.attention(q.double().numpy(), chunks64, 130, True)
    _close(o, ref, 1e-12, "fp8 ring")


# --------------------------------------------------------------------------- #
# local windows (page "Ring Attention：百万 Token 上下文的秘密", §4.3)
# --------------------------------------------------------------------------- #
def _window_mask(qpos, kpos, causal, window):
    m = np.ones((len(qpos), len(kpos)), dtype=bool)
    if causal:
        m &= kpos[None, :] <= qpos[:, None]
    if window > 0:
        m &= np.abs(kpos[None, :] - qpos[:, None]) <= window
    return m


def pin_window_library_sdpa():
    """Windowed attention against float64 SDPA with the window written as an
    explicit boolean mask over absolute positions (causal one-sided windows,
    two-sided windows without causal masking, GQA, ragged chunks, and rows
    whose window holds no key, which must give 0)."""
    rng = np.random.default_rng(202)
    cases = [
        # B, Lq, Hq, Hkv, d, lens, q_offset, causal, window
        (1, 9, 2, 1, 6, [5, 9, 3], 4, True, 3),
        (2, 7, 4, 2, 5, [8, 8, 8], 16, True, 1),
        (1, 6, 3, 3, 8, [4, 11], 0, False, 2),
        (1, 5, 2, 2, 4, [7, 7], 30, True, 4),     # query positions past every key: empty rows
        (2, 8, 4, 1, 7, [6, 1, 9], 10, False, 5),
        (1, 10, 2, 2, 6, [10, 10], 10, True, 9),  # query chunk = last chunk
    ]
    for (B, Lq, Hq, Hkv, d, lens, q_off, causal, w) in cases:
        q, chunks = _rand(rng, B, Lq, Hq, Hkv, d, d, lens)
        out, _ = oracle.attention(q, chunks, q_off, causal, window=w)
        qpos = q_off + np.arange(Lq)
        mask = _window_mask(qpos, _positions(chunks), causal, w)
        seen = mask.any(1)
        K = torch.from_numpy(np.concatenate([c[0] for c in chunks], axis=1)).permute(0, 2, 1, 3)
        V = torch.from_numpy(np.concatenate([c[1] for c in chunks], axis=1)).permute(0, 2, 1, 3)
        Q = torch.from_numpy(q).permute(0, 2, 1, 3)
        if seen.any():
            ref = torch.nn.functional.scaled_dot_product_attention(
                Q[:, :, seen], K, V, attn_mask=torch.from_numpy(mask[seen]), scale=1.0 / math.sqrt(d),
                enable_gqa=True).permute(0, 2, 1, 3).numpy()
            _close(out[:, seen], ref, 1e-12, f"window sdpa {lens} q_off={q_off} causal={causal} w={w}")
        assert np.all(out[:, ~seen] == 0.0), "rows with an empty window must be 0"


def pin_window_of_one_is_two_keys():
    """A causal window of 1 leaves each query its own key and the one before:
    the two-key logistic closed form."""
    d = 4
    q = np.array([[[[2.0, 0.0, 1.0, 0.0]]]])
    keys = np.array([[[[5.0, 1.0, 0.0, 2.0]], [[1.0, 0.0, 0.0, 0.0]], [[0.0, 0.0, 3.0, 0.0]]]])  # positions 0,1,2
    vals = np.array([[[[9.0, 9.0]], [[1.0, 2.0]], [[-1.0, 5.0]]]])
    out, _ = oracle.attention(q, [(keys, vals, 0)], 2, True, window=1)  # query at position 2
    s1, s2 = 2.0 / math.sqrt(d), 3.0 / math.sqrt(d)
    sig = 1.0 / (1.0 + math.exp(-(s2 - s1)))
    _close(out[0, 0, 0], vals[0, 1, 0] + (vals[0, 2, 0] - vals[0, 1, 0]) * sig, 1e-15, "window of one")


def pin_window_wider_than_keys_and_ring():
    """A window wider than the key span changes nothing; with a window the
    ring recurrence in any chunk order still equals windowed attention."""
    rng = np.random.default_rng(303)
    q, chunks = _rand(rng, 2, 6, 4, 2, 8, 8, [9, 4, 12])
    for causal in (True, False):
        a, _ = oracle.attention(q, chunks, 7, causal)
        b, _ = oracle.attention(q, chunks, 7, causal, window=100)
        _close(a, b, 0.0, f"wide window causal={causal}")
    for w, order in ((3, [2, 0, 1]), (6, [1, 2, 0]), (13, [0, 1, 2])):
        full, _ = oracle.attention(q, chunks, 7, True, window=w)
        st = oracle.ring(q, chunks, order=order, q_offset=7, causal=True, window=w)
        o, _ = oracle.finalize(st)
        _close(o, full, 1e-12, f"windowed ring w={w} order={order}")


# --------------------------------------------------------------------------- #
# backward: gradients of sum(dO * out)
# --------------------------------------------------------------------------- #
def _mask(q_off, Lq, chunks, causal, w):
    return _window_mask(q_off + np.arange(Lq), _positions(chunks), causal, w)


def pin_bwd_library_autograd():
    """dQ, dK, dV against float64 autograd through library SDPA with an
    explicit position mask: causal, windows, two-sided windows, GQA, ragged
    chunks, d_qk != d_v, and rows that see no key (dropped from the library
    call: they must get dQ = 0 and add nothing to dK, dV)."""
    rng = np.random.default_rng(404)
    cases = [
        # B, Lq, Hq, Hkv, dqk, dv, lens, q_offset, causal, window
        (1, 7, 2, 1, 6, 6, [5, 9, 3], 6, True, 0),
        (2, 6, 4, 2, 5, 3, [8, 8], 8, True, 0),
        (1, 5, 3, 3, 4, 4, [6, 2], 0, False, 0),
        (2, 8, 4, 1, 7, 7, [6, 1, 9], 5, True, 3),
        (1, 6, 2, 2, 5, 5, [7, 7], 3, False, 2),
        (1, 5, 2, 1, 4, 4, [6, 6], 20, False, 4),  # the last rows' windows hold no key
    ]
    for (B, Lq, Hq, Hkv, dqk, dv, lens, q_off, causal, w) in cases:
        q, chunks = _rand(rng, B, Lq, Hq, Hkv, dqk, dv, lens)
        do = rng.standard_normal((B, Lq, Hq, dv))
        dq, dks, dvs = oracle.attention_bwd(q, chunks, do, q_off, causal, window=w)
        mask = _mask(q_off, Lq, chunks, causal, w)
        seen = mask.any(1)
        Q = torch.from_numpy(q).requires_grad_()
        K = torch.from_numpy(np.concatenate([c[0] for c in chunks], axis=1)).requires_grad_()
        V = torch.from_numpy(np.concatenate([c[1] for c in chunks], axis=1)).requires_grad_()
        out = torch.nn.functional.scaled_dot_product_attention(
            Q[:, seen].permute(0, 2, 1, 3), K.permute(0, 2, 1, 3), V.permute(0, 2, 1, 3),
            attn_mask=torch.from_numpy(mask[seen]), scale=1.0 / math.sqrt(dqk), enable_gqa=True)
        (out.permute(0, 2, 1, 3) * torch.from_numpy(do[:, seen])).sum().backward()
        what = f"bwd autograd {lens} q_off={q_off} causal={causal} w={w}"
        _close(dq, Q.grad.numpy(), 1e-11, what + " dQ")
        _close(np.concatenate(dks, 1), K.grad.numpy(), 1e-11, what + " dK")
        _close(np.concatenate(dvs, 1), V.grad.numpy(), 1e-11, what + " dV")
        assert np.all(dq[:, ~seen] == 0.0), what + ": rows with no key must get dQ = 0"


def pin_bwd_finite_differences():
    """Every gradient element against central differences of the forward
    oracle's sum(dO * out): brute force, no derivative code involved."""
    rng = np.random.default_rng(505)
    for (Hq, Hkv, lens, q_off, causal, w) in ((2, 1, [2, 3], 2, True, 0), (2, 2, [3, 2], 1, False, 2),
                                              (2, 1, [4, 1], 3, True, 2)):
        q, chunks = _rand(rng, 1, 3, Hq, Hkv, 3, 2, lens)
        do = rng.standard_normal((1, 3, Hq, 2))
        dq, dks, dvs = oracle.attention_bwd(q, chunks, do, q_off, causal, window=w)

        def loss(qq, cc):
            out, _ = oracle.attention(qq, cc, q_off, causal, window=w)
            return float((out * do).sum())

        eps = 1e-6
        arrays = [("q", q, dq)] + [(f"k{c}", chunks[c][0], dks[c]) for c in range(len(chunks))] + \
                 [(f"v{c}", chunks[c][1], dvs[c]) for c in range(len(chunks))]
        for name, a, g in arrays:
            for idx in np.ndindex(a.shape):
                old = a[idx]
                a[idx] = old + eps
                lp = loss(q, chunks)
                a[idx] = old - eps
                lm = loss(q, chunks)
                a[idx] = old
                num = (lp - lm) / (2 * eps)
                assert abs(num - g[idx]) <= 1e-7 * (1 + abs(num)), \
                    f"bwd finite difference {name}{idx}: {num} vs {g[idx]} (lens {lens} causal={causal} w={w})"


def pin_bwd_invariants_and_closed_forms():
    """Softmax shift invariance: the dK of all keys of a (batch, KV head) sum
    to 0; the dV sum to the summed dO of the rows that see a key (each row's
    weights sum to 1).  Closed forms: constant values give dQ = dK = 0; a
    row seeing one key gets dQ = 0; two keys give the logistic derivative."""
    rng = np.random.default_rng(606)
    q, chunks = _rand(rng, 2, 9, 4, 2, 6, 5, [7, 4, 10])
    do = rng.standard_normal((2, 9, 4, 5))
    for causal, w, q_off in ((True, 0, 12), (False, 3, 4), (True, 2, 14), (False, 0, 0)):
        dq, dks, dvs = oracle.attention_bwd(q, chunks, do, q_off, causal, window=w)
        _close(np.concatenate(dks, 1).sum(1), np.zeros((2, 2, 6)), 1e-12, f"sum dK causal={causal} w={w}")
        seen = _mask(q_off, 9, chunks, causal, w).any(1)
        want = do[:, seen].reshape(2, -1, 2, 2, 5).sum(1).sum(2)  # rows, then the 2 heads of each group
        _close(np.concatenate(dvs, 1).sum(1), want, 1e-12, f"sum dV causal={causal} w={w}")
    # constant values: out does not depend on the scores
    const = [(k, np.broadcast_to(np.arange(5.0), v.shape).copy(), s) for (k, v, s) in chunks]
    dq, dks, _ = oracle.attention_bwd(q, const, do, 12, True)
    _close(dq, np.zeros_like(dq), 1e-12, "constant V: dQ")
    _close(np.concatenate(dks, 1), np.zeros((2, 21, 2, 6)), 1e-12, "constant V: dK")
    # causal row 0 at position 0 sees key 0 only
    dq, _, _ = oracle.attention_bwd(q, chunks, do, 0, True)
    _close(dq[:, 0], np.zeros((2, 4, 6)), 0.0, "single visible key: dQ")
    # window of one: keys t-1, t; out = v1 + (v2 - v1) sig(s2 - s1)
    d = 4
    qq = np.array([[[[2.0, 0.5, 1.0, -1.0]]]])
    keys = np.array([[[[5.0, 1.0, 0.0, 2.0]], [[1.0, 0.0, -2.0, 0.0]], [[0.0, 1.0, 3.0, 0.0]]]])
    vals = np.array([[[[9.0, 9.0]], [[1.0, 2.0]], [[-1.0, 5.0]]]])
    g = np.array([[[[0.7, -1.3]]]])
    dq, dks, dvs = oracle.attention_bwd(qq, [(keys, vals, 0)], g, 2, True, window=1)
    sc = 1.0 / math.sqrt(d)
    s1, s2 = sc * qq[0, 0, 0] @ keys[0, 1, 0], sc * qq[0, 0, 0] @ keys[0, 2, 0]
    sig = 1.0 / (1.0 + math.exp(-(s2 - s1)))
    c = float(g[0, 0, 0] @ (vals[0, 2, 0] - vals[0, 1, 0])) * sig * (1 - sig)
    _close(dq[0, 0, 0], c * sc * (keys[0, 2, 0] - keys[0, 1, 0]), 1e-14, "two keys: dQ")
    _close(dks[0][0, 2, 0], c * sc * qq[0, 0, 0], 1e-14, "two keys: dK of the later key")
    _close(dks[0][0, 1, 0], -c * sc * qq[0, 0, 0], 1e-14, "two keys: dK of the earlier key")
    _close(dvs[0][0, 1, 0], (1 - sig) * g[0, 0, 0], 1e-14, "two keys: dV of the earlier key")
    _close(dks[0][0, 0, 0], np.zeros(d), 0.0, "key outside the window: dK")


def pin_bwd_chunking_invariance():
    """Gradients do not depend on how the keys are cut into chunks or in
    which order the chunks are listed (the ring's equivalence, page "Ring
    Attention：百万 Token 上下文的秘密", §2.3)."""
    rng = np.random.default_rng(707)
    q, chunks = _rand(rng, 1, 6, 2, 1, 5, 5, [12])
    do = rng.standard_normal((1, 6, 2, 5))
    k, v, _ = chunks[0]
    dq0, dk0, dv0 = oracle.attention_bwd(q, chunks, do, 6, True, window=4)
    cut = [(k[:, :5], v[:, :5], 0), (k[:, 5:7], v[:, 5:7], 5), (k[:, 7:], v[:, 7:], 7)]
    perm = [cut[2], cut[0], cut[1]]
    dq1, dk1, dv1 = oracle.attention_bwd(q, perm, do, 6, True, window=4)
    _close(dq1, dq0, 1e-13, "chunked dQ")
    _close(np.concatenate([dk1[1], dk1[2], dk1[0]], 1), dk0[0], 1e-13, "chunked dK")
    _close(np.concatenate([dv1[1], dv1[2], dv1[0]], 1), dv0[0], 1e-13, "chunked dV")


# --------------------------------------------------------------------------- #
# anchor tokens and segments
# --------------------------------------------------------------------------- #
def _page_sparse_mask(n, w, S):
    """The sparse mask of page "Ring Attention：百万 Token 上下文的秘密", §4.3,
    over a whole sequence of n positions: query i sees the keys
    max(0, i - w) .. i, and the anchors A, A - 1 (if A > 0) and A + S (if it
    is a position), A being the start of i's stride-S block."""
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        m[i, max(0, i - w):i + 1] = True
        A = (i // S) * S
        m[i, A] = True
        if A > 0:
            m[i, A - 1] = True
        if A + S < n:
            m[i, A + S] = True
    return m


def _sdpa_masked(q, chunks, mask, d):
    K = torch.from_numpy(np.concatenate([c[0] for c in chunks], axis=1)).permute(0, 2, 1, 3)
    V = torch.from_numpy(np.concatenate([c[1] for c in chunks], axis=1)).permute(0, 2, 1, 3)
    Q = torch.from_numpy(q).permute(0, 2, 1, 3)
    return torch.nn.functional.scaled_dot_product_attention(
        Q, K, V, attn_mask=torch.from_numpy(mask), scale=1.0 / math.sqrt(d), enable_gqa=True).permute(0, 2, 1, 3).numpy()


def pin_anchor_library_sdpa():
    """Causal window plus anchor tokens against library SDPA under the
    page's sparse mask built over the whole sequence (the query chunk is a
    slice of it; ragged chunks, GQA, strides 3, 4, 8)."""
    rng = np.random.default_rng(808)
    for (B, Hq, Hkv, d, lens, q_off, Lq, w, S) in ((1, 2, 1, 6, [9, 7, 8], 10, 14, 2, 4),
                                                  (2, 4, 2, 5, [16, 16], 16, 16, 5, 8),
                                                  (1, 3, 3, 4, [5, 11, 4], 0, 20, 1, 3),
                                                  (1, 2, 2, 8, [24], 3, 17, 0, 8)):
        q, chunks = _rand(rng, B, Lq, Hq, Hkv, d, d, lens)
        n = sum(lens)
        page = _page_sparse_mask(n, w if w > 0 else n, S)
        rows = page[q_off:q_off + Lq]
        out, _ = oracle.attention(q, chunks, q_off, True, window=w, anchor=S)
        _close(out, _sdpa_masked(q, chunks, rows, d), 1e-12, f"anchors S={S} w={w} lens={lens}")


def pin_anchor_ring_and_two_sided():
    """With anchors the ring recurrence in any order still equals full
    attention; without causal masking anchors join a two-sided window (SDPA
    with the explicit mask); a window covering everything leaves anchors
    nothing to add."""
    rng = np.random.default_rng(909)
    q, chunks = _rand(rng, 1, 12, 2, 1, 6, 6, [10, 9, 13])
    full, _ = oracle.attention(q, chunks, 8, True, window=3, anchor=5)
    for order in ([2, 0, 1], [1, 2, 0]):
        st = oracle.ring(q, chunks, order=order, q_offset=8, causal=True, window=3, anchor=5)
        o, _ = oracle.finalize(st)
        _close(o, full, 1e-12, f"anchor ring order={order}")
    qpos, kpos = 8 + np.arange(12), _positions(chunks)
    m = np.abs(kpos[None, :] - qpos[:, None]) <= 2
    A = (qpos // 5) * 5
    for extra in (A - 1, A, A + 5):
        m |= kpos[None, :] == extra[:, None]
    out, _ = oracle.attention(q, chunks, 8, False, window=2, anchor=5)
    _close(out, _sdpa_masked(q, chunks, m, 6), 1e-12, "anchors with a two-sided window")
    a, _ = oracle.attention(q, chunks, 8, False, window=100, anchor=5)
    b, _ = oracle.attention(q, chunks, 8, False)
    _close(a, b, 0.0, "window over everything")


def pin_segments_packing():
    """Packed documents: attention over a sequence whose segment labels mark
    three documents equals each document's own attention computed alone
    (causal, and with a window); labels against library SDPA with the
    equality mask, including rows whose label no key carries."""
    rng = np.random.default_rng(1010)
    docs = [5, 7, 4]
    n = sum(docs)
    q, chunks = _rand(rng, 2, n, 4, 2, 6, 6, [6, 10])  # the chunks cut across documents
    lab = np.repeat(np.arange(len(docs)), docs).astype(np.int32)
    q_seg = np.tile(lab, (2, 1))
    k_segs = [q_seg[:, :6], q_seg[:, 6:]]
    K = np.concatenate([c[0] for c in chunks], axis=1)
    V = np.concatenate([c[1] for c in chunks], axis=1)
    for w in (0, 2):
        out, _ = oracle.attention(q, chunks, 0, True, window=w, q_seg=q_seg, k_segs=k_segs)
        s0 = 0
        for L in docs:
            alone, _ = oracle.attention(q[:, s0:s0 + L], [(K[:, s0:s0 + L], V[:, s0:s0 + L], 0)], 0, True, window=w)
            _close(out[:, s0:s0 + L], alone, 1e-13, f"packed document at {s0} w={w}")
            s0 += L
    # arbitrary labels, non-causal, one label carried by no key
    q2, ch2 = _rand(rng, 1, 9, 2, 2, 5, 5, [7, 8])
    qs = rng.integers(0, 3, size=(1, 9)).astype(np.int32)
    qs[0, 4] = 7
    ks = [rng.integers(0, 3, size=(1, 7)).astype(np.int32), rng.integers(0, 3, size=(1, 8)).astype(np.int32)]
    out, _ = oracle.attention(q2, ch2, 0, False, q_seg=qs, k_segs=ks)
    m = qs[0][:, None] == np.concatenate(ks, axis=1)[0][None, :]
    seen = m.any(1)
    _close(out[:, seen], _sdpa_masked(q2[:, seen], ch2, m[seen], 5), 1e-12, "segment labels")
    assert np.all(out[:, ~seen] == 0.0)


def pin_bwd_with_anchors_and_segments():
    """Gradients under anchors and segment labels against float64 autograd
    through library SDPA with the same explicit mask."""
    rng = np.random.default_rng(1111)
    q, chunks = _rand(rng, 1, 10, 2, 1, 5, 5, [8, 9])
    do = rng.standard_normal((1, 10, 2, 5))
    qs = np.array([[0] * 4 + [1] * 6], dtype=np.int32)
    ks = [np.array([[0] * 8], dtype=np.int32), np.array([[0] * 3 + [1] * 6], dtype=np.int32)]
    for kw, m in ((dict(window=2, anchor=4), None), (dict(q_seg=qs, k_segs=ks), None)):
        qpos, kpos = 7 + np.arange(10), _positions(chunks)
        if "anchor" in kw:
            m = (kpos[None, :] <= qpos[:, None]) & (kpos[None, :] >= qpos[:, None] - 2)
            A = (qpos // 4) * 4
            for extra in (A - 1, A, A + 4):
                m |= kpos[None, :] == extra[:, None]
        else:
            m = (kpos[None, :] <= qpos[:, None]) & (qs[0][:, None] == np.concatenate(ks, 1)[0][None, :])
        dq, dks, dvs = oracle.attention_bwd(q, chunks, do, 7, True, **kw)
        Q = torch.from_numpy(q).requires_grad_()
        K = torch.from_numpy(np.concatenate([c[0] for c in chunks], axis=1)).requires_grad_()
        V = torch.from_numpy(np.concatenate([c[1] for c in chunks], axis=1)).requires_grad_()
        out = torch.nn.functional.scaled_dot_product_attention(
            Q.permute(0, 2, 1, 3), K.permute(0, 2, 1, 3), V.permute(0, 2, 1, 3), attn_mask=torch.from_numpy(m),
            scale=1.0 / math.sqrt(5), enable_gqa=True)
        (out.permute(0, 2, 1, 3) * torch.from_numpy(do)).sum().backward()
        _close(dq, Q.grad.numpy(), 1e-11, f"bwd {list(kw)} dQ")
        _close(np.concatenate(dks, 1), K.grad.numpy(), 1e-11, f"bwd {list(kw)} dK")
        _close(np.concatenate(dvs, 1), V.grad.numpy(), 1e-11, f"bwd {list(kw)} dV")


ALL_PINS = [
    pin_library_sdpa,
    pin_zero_query_mean,
    pin_constant_values,
    pin_first_causal_row,
    pin_two_keys_logistic,
    pin_hardmax_limit,
    pin_empty_rows,
    pin_exact_mpmath,
    pin_ring_equals_full,
    pin_merge_laws,
    pin_causal_future_ignored,
    pin_rows_and_decode_positions,
    pin_input_types,
    pin_fp8_decode_library,
    pin_fp8_attention_equals_decoded,
    pin_window_library_sdpa,
    pin_window_of_one_is_two_keys,
    pin_window_wider_than_keys_and_ring,
    pin_bwd_library_autograd,
    pin_bwd_finite_differences,
    pin_bwd_invariants_and_closed_forms,
    pin_bwd_chunking_invariance,
    pin_anchor_library_sdpa,
    pin_anchor_ring_and_two_sided,
    pin_segments_packing,
    pin_bwd_with_anchors_and_segments,
]
