"""Plant plausible mistakes in copies of oracle.c and check the pins catch each.

Every mutant is a textual edit of the oracle's C source (a dropped term, a
wrong sign or index, an off-by-one mask, a misread of the pages), compiled to
its own library in a temporary directory.  The pin suite of
``oracle_pins.py`` runs against it; at least one pin must fail.  The real
oracle is never modified.
"""
import os

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (id, original text, replacement, how many occurrences to replace: 1 or "all")
MUTANTS = [
    ("no_rescale_of_O", "o[e] *= alpha;", "(void)alpha;", 1),
    ("no_rescale_of_l", "l[st] = alpha * l[st] + psum;", "l[st] = l[st] + psum;", 1),
    ("strict_causal_diagonal", "if (causal && kpos > qpos)", "if (causal && kpos >= qpos)", 1),
    ("window_excludes_its_edge", "kpos < qpos - window", "kpos <= qpos - window", 1),
    ("window_one_sided_without_causal", " || kpos > qpos + window", "", 1),
    ("window_ignored", "if (window > 0 && (", "if (0 && (", 1),
    ("interleaved_gqa_heads", "int hk = h / (Hq / Hkv);", "int hk = h % Hkv;", "all"),
    ("q_offset_floored_to_512_chunk", "int64_t qpos = q_offset + r;",
     "int64_t qpos = (q_offset / 512) * 512 + r;", "all"),
    ("scale_dropped", "return dot * scale;", "return dot;", 1),
    ("no_max_shift", "double w = exp(s[t] - mx);", "double w = exp(s[t]);", 1),
    ("lse_without_max", "*ls = mx + log(sum);", "*ls = log(sum);", 1),
    ("wrong_query_head", "int hk = h / (Hq / Hkv);\n    int64_t qb = (((int64_t)b * Lq + r) * Hq + h) * dqk;",
     "int hk = h / (Hq / Hkv);\n    int64_t qb = (((int64_t)b * Lq + r) * Hq + 0) * dqk;", 1),
    ("key_index_transposed", "int64_t kb = (((int64_t)b * lenc + j) * Hkv + hk) * dqk;",
     "int64_t kb = (((int64_t)b * lenc + (lenc - 1 - j)) * Hkv + hk) * dqk;", 1),
    ("value_of_wrong_chunk_key",
     "sum += w;\n                    int64_t vb = (((int64_t)b * len[c] + j) * Hkv + hk) * dv;",
     "sum += w;\n                    int64_t vb = (((int64_t)b * len[c] + (j ? j - 1 : 0)) * Hkv + hk) * dv;", 1),
    ("only_two_chunks_seen",
     "/* pass 1: scores of all visible keys and their maximum */\n            double mx = -INFINITY;\n            int64_t t = 0;\n            for (int c = 0; c < n_chunks; ++c)",
     "/* pass 1: scores of all visible keys and their maximum */\n            double mx = -INFINITY;\n            int64_t t = 0;\n            for (int c = 0; c < n_chunks && c < 2; ++c)", 1),
    ("merge_weight_sign", "double a2 = m2[i] == -INFINITY ? 0.0 : exp(m2[i] - mx);",
     "double a2 = m2[i] == -INFINITY ? 0.0 : exp(mx - m2[i]);", 1),
    ("merge_drops_second_l", "l[i] = a1 * l1[i] + a2 * l2[i];", "l[i] = a1 * l1[i] + l2[i];", 1),
    ("finalize_lse_without_m", "lse[i] = m[i] + log(l[i]);", "lse[i] = log(l[i]);", 1),
    ("ring_step_alpha_inverted", "double alpha = m[st] == -INFINITY ? 0.0 : exp(m[st] - m_new);",
     "double alpha = m[st] == -INFINITY ? 0.0 : exp(m_new - m[st]);", 1),
    ("ring_step_ignores_previous_max", "double m_new = m[st] > cmax ? m[st] : cmax;",
     "double m_new = cmax;", 1),
    ("empty_row_nan", "if (mx == -INFINITY) { /* no visible key: output 0 */",
     "if (0) { /* no visible key: output 0 */", 1),
    ("bf16_truncated_mantissa", "uint32_t bits = (uint32_t)((const uint16_t *)p)[idx] << 16;",
     "uint32_t bits = ((uint32_t)((const uint16_t *)p)[idx] << 16) & 0xFFFF0000u & ~0x10000u;", 1),
    ("fp8_fnuz_exponent_bias", "v = ldexp(8.0 + man, ex - 10);", "v = ldexp(8.0 + man, ex - 11);", 1),
    ("fp8_subnormal_as_normal", "v = ldexp((double)man, -9);", "v = ldexp(8.0 + man, -10);", 1),
    ("fp8_no_nan_code", "if (ex == 15 && man == 7)\n        return NAN;", "if (0)\n        return NAN;", 1),
    ("fp8_scale_bias", "double scale = ldexp(1.0, e - 127);", "double scale = ldexp(1.0, e - 128);", 1),
    ("fp8_scale_block_of_next_token", "exps[((int64_t)b * H + h) * nblk + t / block]",
     "exps[((int64_t)b * H + h) * nblk + (t + 1) / block]", 1),
    ("anchor_without_previous_key", "if (kpos == a - 1 || kpos == a || kpos == a + mk->anchor)",
     "if (kpos == a || kpos == a + mk->anchor)", 1),
    ("anchor_future_key_off_by_one", "if (kpos == a - 1 || kpos == a || kpos == a + mk->anchor)",
     "if (kpos == a - 1 || kpos == a || kpos == a + mk->anchor - 1)", 1),
    ("anchor_block_of_next_token", "int64_t a = qpos / mk->anchor * mk->anchor;",
     "int64_t a = (qpos + 1) / mk->anchor * mk->anchor;", 1),
    ("anchors_obey_causal", "if (kpos == a - 1 || kpos == a || kpos == a + mk->anchor)",
     "if ((kpos == a - 1 || kpos == a || kpos == a + mk->anchor) && kpos <= qpos)", 1),
    ("anchors_ignored", "if (mk->anchor > 0) {", "if (0) {", 1),
    ("segments_ignored", "if (mk->q_seg &&\n", "if (0 && mk->q_seg &&\n", 1),
    ("segment_label_of_next_key", "mk->k_seg[c][(int64_t)b * lenc + j])",
     "mk->k_seg[c][(int64_t)b * lenc + (j + 1) % lenc])", 1),
    ("bwd_D_unweighted", "D += exp(s[t] - ls) * acc;", "D += acc;", 1),
    ("bwd_dq_without_D", "double ds = exp(s[t] - ls) * (dp[t] - D);", "double ds = exp(s[t] - ls) * dp[t];", 1),
    ("bwd_dk_without_D", "double ds = p * (dpv - Dsum[row]);", "double ds = p * dpv;", 1),
    ("bwd_dv_from_dS", "gv[e] += p * elem(dout, dtype, ob + e);", "gv[e] += ds * elem(dout, dtype, ob + e);", 1),
    ("bwd_dk_unscaled", "gk[e] += scale * ds * elem(q, dtype, qb + e);", "gk[e] += ds * elem(q, dtype, qb + e);", 1),
    ("bwd_dq_sign", "g[e] += scale * ds * elem(k[c], dtype, kb + e);", "g[e] -= scale * ds * elem(k[c], dtype, kb + e);", 1),
    ("bwd_first_head_of_group_only", "for (int h = hk * G; h < (hk + 1) * G; ++h)", "for (int h = hk * G; h < hk * G + 1; ++h)", 1),
    ("bwd_dkdv_ignore_mask", "if (!visible(mk, Lq, len[c], b, r, c, j, q_offset + r, start[c] + j))\n                    continue;",
     "if (0)\n                    continue;", 1),
    ("bwd_unnormalised_weights", "double p = exp(score(q, k[c], dtype, Lq, len[c], Hq, Hkv, dqk, b, r, h, j, scale) - lse[row]);",
     "double p = exp(score(q, k[c], dtype, Lq, len[c], Hq, Hkv, dqk, b, r, h, j, scale) - lse[row] + 0.01);", 1),
    ("bwd_dv_of_wrong_row", "int64_t ob = (((int64_t)b * Lq + r) * Hq + h) * dv;\n                int64_t qb",
     "int64_t ob = (((int64_t)b * Lq + (r + 1) % Lq) * Hq + h) * dv;\n                int64_t qb", 1),
]


def _mutate(text, old, new, count):
    n = text.count(old)
    assert n >= 1, f"snippet not found: {old!r}"
    if count == 1:
        assert n == 1, f"snippet not unique ({n}x): {old!r}"
    return text.replace(old, new)


@pytest.mark.parametrize("mid,old,new,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, monkeypatch, mid, old, new, count):
    src = open(SRC).read()
    mutated = _mutate(src, old, new, count)
    msrc = tmp_path / "oracle_mut.c"
    msrc.write_text(mutated)
    lib_path = oracle.build(force=True, src=str(msrc), out=str(tmp_path / "liboracle_mut.so"))
    monkeypatch.setattr(oracle, "_lib", oracle.load_library(lib_path))
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, FloatingPointError) as e:
            failed.append(pin.__name__)
    assert failed, f"mutant {mid} passed every pin"
