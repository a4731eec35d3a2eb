/*
 * oracle.c - slow, plain, double-precision reference for ring attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library under
 * long_context_blockwise_amd/) links, loads or calls this file, and this file
 * shares no code, header, table or helper with it.  Only tests/, the smoke
 * check and the CPU-baseline leg of bench.py use it.
 *
 * What it computes, and where the pages define it:
 *
 *  - oracle_attention: scaled dot-product attention, softmax(Q K^T / sqrt(d)) V,
 *    evaluated row by row straight from the definition with a two-pass softmax.
 *      page "从百毫秒到百万Token：长上下文推理优化的工程实践", section
 *        "注意力机制的数学本质与瓶颈" (the definition);
 *      page "billion-token context window engineering" (blog.hotdry.top),
 *        section "核心挑战：注意力机制的二次复杂度困境" (same definition);
 *      page "Ring Attention：百万 Token 上下文的秘密", §2.3 数学正确性 (ring
 *        result equals plain attention over all key chunks).
 *    The key set of a query row is the union of all KV chunks; chunk c holds
 *    the keys at absolute positions start[c] .. start[c]+len[c]-1, as in the
 *    sequence sharding of §2.1 分块计算注意力 on the same page.
 *
 *  - oracle_ring_step: one step of the chunked online-softmax recurrence
 *    (running max m, denominator l, unnormalised output O) that one device
 *    performs per received KV chunk:
 *      page "Ring Attention：百万 Token 上下文的秘密", §3.1 Flash Ring
 *        Attention (per-chunk blockwise attention inside the ring loop) and
 *        §2.2 环形通信 (one chunk per ring step).
 *    The pages do not write the recurrence out; this is the standard
 *    flash/online-softmax update, the reading taken for §2.3's equation.
 *
 *  - oracle_merge / oracle_finalize: combining two partial states and turning
 *    a state into the output (O / l), the "global softmax normalisation of
 *    local outputs" of the attention fusion layer:
 *      page "从百毫秒到百万Token：长上下文推理优化的工程实践", section
 *        "系统架构设计", item 4 注意力融合层.
 *
 * Causal masking is token level with the diagonal included: a query at
 * absolute position p sees a key at position t iff t <= p.  A local window
 * w > 0 further limits it to keys at distance <= w: t >= p - w (and, without
 * causal masking, t <= p + w); w <= 0 means no window.  Sparse local
 * attention over the last w tokens is the window of page "Ring Attention：
 * 百万 Token 上下文的秘密", §4.3 稀疏注意力掩码 (query i sees keys
 * i - w .. i); page "billion-token context window engineering" describes
 * the sliding window as keys within a range before and after the query,
 * the reading taken without causal masking.
 *
 * Anchor tokens (stride S > 0): the same section's sparse mask also lets a
 * query at p see the keys at a - 1, a and a + S, a = S * floor(p / S), when
 * they exist, whatever the window and the causal rule say (its mask adds
 * them to the local window, the later one included).  Segments: with
 * per-token segment labels (the segment_ids that page "RingAttention推理
 * 优化：cache_idx参数使用..." passes for packed sequences), a query sees only
 * keys of its own label; the label test applies on top of everything else.
 *
 * The query row r
 * sits at absolute position q_offset + r (q_offset = chunk index * chunk
 * length in a prefill ring, or cache_idx in incremental decoding:
 *   page "RingAttention推理优化：cache_idx参数使用与千万级上下文高效推理实践",
 *   sections "cache_idx的工作原理" and "增量推理实战").
 * Grouped-query attention: query head h reads KV head h / (Hq / Hkv).
 *
 * Layouts (all contiguous, row-major):
 *   q       [B][Lq][Hq][dqk]
 *   k[c]    [B][len[c]][Hkv][dqk]     v[c]  [B][len[c]][Hkv][dv]
 *   rows    the query rows (indices into 0..Lq-1) to evaluate
 *   out     [B][n_rows][Hq][dv]       lse   [B][Hq][n_rows]
 *   m, l    [B][Hq][n_rows]           O     [B][Hq][n_rows][dv]
 * Element type of q/k/v: ORACLE_F64, ORACLE_F32, or ORACLE_BF16 (raw 16-bit
 * patterns, upcast exactly).  All arithmetic is double.
 *
 * Return value: 0 on success, -1 on an argument error, -2 if out of memory.
 *
 *  - oracle_dequant_fp8: 8-bit keys/values of a quantised KV cache turned
 *    back into numbers.  The pages recommend storing the KV cache in 8 bits
 *    (page "billion-token context window engineering", section on production
 *    parameters: 4/8-bit KV-cache quantisation for serving; page
 *    "RingAttention与RAG技术对比及实战应用", §2.3: FP8 deployment) without
 *    fixing a format.  The reading taken: OCP FP8 E4M3 codes (1 sign bit,
 *    4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is subnormal;
 *    S.1111.111 is NaN; no infinities; largest finite value 448), each block
 *    of 64 consecutive tokens of one (batch, KV head) sharing a power-of-two
 *    scale 2^(e - 127) given by an 8-bit biased exponent e (1 .. 254).
 *    The attention itself is then oracle_attention on the decoded values.
 *
 *  - oracle_attention_bwd: the gradients dQ, dK, dV of L = sum(dO * out),
 *    out = oracle_attention(...), for a given output gradient dO.  The pages
 *    use ring attention for training (page "Ring Attention：百万 Token
 *    上下文的秘密", §5.1 训练效率; page "billion-token context window
 *    engineering", training with ring attention and FSDP) but print no
 *    backward algorithm, so this is the derivative of the definition,
 *    written out.  With P = softmax(S) over the visible keys of a row and
 *    S = scale * q k^T:
 *        dV_j = sum_i P_ij dO_i                     (out is linear in V)
 *        dP_ij = dO_i . v_j
 *        dS_ij = P_ij (dP_ij - sum_t P_it dP_it)    (softmax Jacobian)
 *        dQ_i = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i
 *    with sums over visible (i, j) only, and every query head of a KV head's
 *    group adding into that head's dK and dV.  Rows that see no key get
 *    dQ = 0 and add nothing.  It runs as a per-row pass (softmax, dQ) and
 *    a per-key pass (dK, dV), so no two threads write one element.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F64 = 0, ORACLE_F32 = 1, ORACLE_BF16 = 2 };

/* Read element idx of an array of the given element type as a double. */
static double elem(const void *p, int dtype, int64_t idx)
{
    if (dtype == ORACLE_F64)
        return ((const double *)p)[idx];
    if (dtype == ORACLE_F32)
        return (double)((const float *)p)[idx];
    /* bfloat16: the upper 16 bits of an IEEE binary32 value */
    uint32_t bits = (uint32_t)((const uint16_t *)p)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static int check_shapes(int B, int Hq, int Hkv, int dqk, int dv, int dtype,
                        int64_t Lq, int n_chunks, const int64_t *len,
                        int64_t n_rows, const int64_t *rows)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || dqk <= 0 || dv <= 0 || Lq < 0 ||
        n_chunks < 0 || n_rows < 0)
        return -1;
    if (Hq % Hkv != 0)
        return -1;
    if (dtype != ORACLE_F64 && dtype != ORACLE_F32 && dtype != ORACLE_BF16)
        return -1;
    for (int c = 0; c < n_chunks; ++c)
        if (len[c] < 0)
            return -1;
    for (int64_t i = 0; i < n_rows; ++i)
        if (rows[i] < 0 || rows[i] >= Lq)
            return -1;
    return 0;
}

/* Score of query (b, r, h) against key j of chunk c, both upcast to double. */
static double score(const void *q, const void *kc, int dtype, int64_t Lq,
                    int64_t lenc, int Hq, int Hkv, int dqk, int b, int64_t r,
                    int h, int64_t j, double scale)
{
    int hk = h / (Hq / Hkv);
    int64_t qb = (((int64_t)b * Lq + r) * Hq + h) * dqk;
    int64_t kb = (((int64_t)b * lenc + j) * Hkv + hk) * dqk;
    double dot = 0.0;
    for (int e = 0; e < dqk; ++e)
        dot += elem(q, dtype, qb + e) * elem(kc, dtype, kb + e);
    return dot * scale;
}

/* The masks of one call.  q_seg [B][Lq] and k_seg[c] [B][len[c]] are
 * segment labels, or NULL for none. */
typedef struct oracle_mask {
    int causal;
    int64_t window;
    int64_t anchor;
    const int32_t *q_seg;
    const int32_t *const *k_seg;
} oracle_mask;

/* May query row r (batch b, position qpos) see key j of chunk c (position
 * kpos, chunk length lenc)? */
static int visible(const oracle_mask *mk, int64_t Lq, int64_t lenc, int b,
                   int64_t r, int c, int64_t j, int64_t qpos, int64_t kpos)
{
    int causal = mk->causal;
    int64_t window = mk->window;
    if (mk->q_seg &&
        mk->q_seg[(int64_t)b * Lq + r] != mk->k_seg[c][(int64_t)b * lenc + j])
        return 0;
    if (mk->anchor > 0) {
        int64_t a = qpos / mk->anchor * mk->anchor;
        if (kpos == a - 1 || kpos == a || kpos == a + mk->anchor)
            return 1;
    }
    if (causal && kpos > qpos)
        return 0;
    if (window > 0 && (kpos < qpos - window || kpos > qpos + window))
        return 0;
    return 1;
}

int oracle_attention(int B, int Hq, int Hkv, int dqk, int dv, int dtype,
                     const void *q, int64_t Lq, int64_t q_offset, int n_chunks,
                     const void *const *k, const void *const *v,
                     const int64_t *start, const int64_t *len,
                     const oracle_mask *mk, double scale, int64_t n_rows,
                     const int64_t *rows, double *out, double *lse)
{
    if (check_shapes(B, Hq, Hkv, dqk, dv, dtype, Lq, n_chunks, len, n_rows,
                     rows))
        return -1;
    int64_t nkeys = 0;
    for (int c = 0; c < n_chunks; ++c)
        nkeys += len[c];
    int64_t units = (int64_t)B * Hq * n_rows;
    int err = 0;

#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(nkeys ? nkeys : 1));
        double *acc = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!s || !acc) {
#pragma omp atomic write
            err = -2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < units; ++u) {
            if (!s || !acc)
                continue;
            int b = (int)(u / ((int64_t)Hq * n_rows));
            int h = (int)((u / n_rows) % Hq);
            int64_t i = u % n_rows;
            int64_t r = rows[i];
            int64_t qpos = q_offset + r;
            int hk = h / (Hq / Hkv);

            /* pass 1: scores of all visible keys and their maximum */
            double mx = -INFINITY;
            int64_t t = 0;
            for (int c = 0; c < n_chunks; ++c)
                for (int64_t j = 0; j < len[c]; ++j, ++t) {
                    if (!visible(mk, Lq, len[c], b, r, c, j, qpos, start[c] + j)) {
                        s[t] = -INFINITY;
                        continue;
                    }
                    s[t] = score(q, k[c], dtype, Lq, len[c], Hq, Hkv, dqk, b,
                                 r, h, j, scale);
                    if (s[t] > mx)
                        mx = s[t];
                }

            double *o = out + (((int64_t)b * n_rows + i) * Hq + h) * dv;
            double *ls = lse + ((int64_t)b * Hq + h) * n_rows + i;
            if (mx == -INFINITY) { /* no visible key: output 0 */
                for (int e = 0; e < dv; ++e)
                    o[e] = 0.0;
                *ls = -INFINITY;
                continue;
            }
            /* pass 2: weights exp(s - max), their sum, and the weighted sum of V */
            double sum = 0.0;
            for (int e = 0; e < dv; ++e)
                acc[e] = 0.0;
            t = 0;
            for (int c = 0; c < n_chunks; ++c)
                for (int64_t j = 0; j < len[c]; ++j, ++t) {
                    if (s[t] == -INFINITY)
                        continue;
                    double w = exp(s[t] - mx);
                    sum += w;
                    int64_t vb = (((int64_t)b * len[c] + j) * Hkv + hk) * dv;
                    for (int e = 0; e < dv; ++e)
                        acc[e] += w * elem(v[c], dtype, vb + e);
                }
            for (int e = 0; e < dv; ++e)
                o[e] = acc[e] / sum;
            *ls = mx + log(sum);
        }
        free(s);
        free(acc);
    }
    return err;
}

int oracle_ring_step(int B, int Hq, int Hkv, int dqk, int dv, int dtype,
                     const void *q, int64_t Lq, int64_t q_offset,
                     const void *kc, const void *vc, int64_t start,
                     int64_t len, const oracle_mask *mk, double scale,
                     int64_t n_rows, const int64_t *rows, double *m,
                     double *l, double *O)
{
    if (check_shapes(B, Hq, Hkv, dqk, dv, dtype, Lq, 1, &len, n_rows, rows))
        return -1;
    int64_t units = (int64_t)B * Hq * n_rows;
    int err = 0;

#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(len ? len : 1));
        if (!s) {
#pragma omp atomic write
            err = -2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < units; ++u) {
            if (!s)
                continue;
            int b = (int)(u / ((int64_t)Hq * n_rows));
            int h = (int)((u / n_rows) % Hq);
            int64_t i = u % n_rows;
            int64_t r = rows[i];
            int64_t qpos = q_offset + r;
            int hk = h / (Hq / Hkv);
            int64_t st = ((int64_t)b * Hq + h) * n_rows + i;

            /* largest score of this chunk's visible keys */
            double cmax = -INFINITY;
            for (int64_t j = 0; j < len; ++j) {
                if (!visible(mk, Lq, len, b, r, 0, j, qpos, start + j)) {
                    s[j] = -INFINITY;
                    continue;
                }
                s[j] = score(q, kc, dtype, Lq, len, Hq, Hkv, dqk, b, r, h, j,
                             scale);
                if (s[j] > cmax)
                    cmax = s[j];
            }
            if (cmax == -INFINITY) /* chunk invisible to this row */
                continue;

            /* new running max, and the factor that rescales the old state */
            double m_new = m[st] > cmax ? m[st] : cmax;
            double alpha = m[st] == -INFINITY ? 0.0 : exp(m[st] - m_new);
            double *o = O + st * dv;
            double psum = 0.0;
            for (int e = 0; e < dv; ++e)
                o[e] *= alpha;
            for (int64_t j = 0; j < len; ++j) {
                if (s[j] == -INFINITY)
                    continue;
                double p = exp(s[j] - m_new);
                psum += p;
                int64_t vb = (((int64_t)b * len + j) * Hkv + hk) * dv;
                for (int e = 0; e < dv; ++e)
                    o[e] += p * elem(vc, dtype, vb + e);
            }
            l[st] = alpha * l[st] + psum;
            m[st] = m_new;
        }
        free(s);
    }
    return err;
}

void oracle_state_init(int64_t n, int dv, double *m, double *l, double *O)
{
    for (int64_t i = 0; i < n; ++i) {
        m[i] = -INFINITY;
        l[i] = 0.0;
        for (int e = 0; e < dv; ++e)
            O[i * dv + e] = 0.0;
    }
}

void oracle_merge(int64_t n, int dv, const double *m1, const double *l1,
                  const double *O1, const double *m2, const double *l2,
                  const double *O2, double *m, double *l, double *O)
{
    for (int64_t i = 0; i < n; ++i) {
        double mx = m1[i] > m2[i] ? m1[i] : m2[i];
        if (mx == -INFINITY) { /* both partials saw no key */
            m[i] = -INFINITY;
            l[i] = 0.0;
            for (int e = 0; e < dv; ++e)
                O[i * dv + e] = 0.0;
            continue;
        }
        double a1 = m1[i] == -INFINITY ? 0.0 : exp(m1[i] - mx);
        double a2 = m2[i] == -INFINITY ? 0.0 : exp(m2[i] - mx);
        l[i] = a1 * l1[i] + a2 * l2[i];
        for (int e = 0; e < dv; ++e)
            O[i * dv + e] = a1 * O1[i * dv + e] + a2 * O2[i * dv + e];
        m[i] = mx;
    }
}

void oracle_finalize(int64_t n, int dv, const double *m, const double *l,
                     const double *O, double *out, double *lse)
{
    for (int64_t i = 0; i < n; ++i) {
        if (l[i] > 0.0) {
            for (int e = 0; e < dv; ++e)
                out[i * dv + e] = O[i * dv + e] / l[i];
            lse[i] = m[i] + log(l[i]);
        } else {
            for (int e = 0; e < dv; ++e)
                out[i * dv + e] = 0.0;
            lse[i] = -INFINITY;
        }
    }
}

/* Value of one OCP FP8 E4M3 code. */
static double fp8_e4m3_value(uint8_t code)
{
    int sign = code >> 7, ex = (code >> 3) & 15, man = code & 7;
    double v;
    if (ex == 15 && man == 7)
        return NAN;
    if (ex == 0)
        v = ldexp((double)man, -9); /* subnormal: man/8 * 2^(1-7) */
    else
        v = ldexp(8.0 + man, ex - 10); /* (1 + man/8) * 2^(ex-7) */
    return sign ? -v : v;
}

/* codes [B][len][H][d] with exponents [B][H][ceil(len/block)] -> out (double,
 * same layout as codes).  Returns -1 on bad arguments. */
int oracle_dequant_fp8(int B, int64_t len, int H, int d, int block,
                       const uint8_t *codes, const uint8_t *exps, double *out)
{
    if (B < 0 || len < 0 || H <= 0 || d <= 0 || block <= 0 || (len && (!codes || !exps || !out)))
        return -1;
    int64_t nblk = (len + block - 1) / block;
    for (int b = 0; b < B; ++b)
        for (int64_t t = 0; t < len; ++t)
            for (int h = 0; h < H; ++h) {
                int e = exps[((int64_t)b * H + h) * nblk + t / block];
                double scale = ldexp(1.0, e - 127);
                int64_t base = (((int64_t)b * len + t) * H + h) * d;
                for (int i = 0; i < d; ++i)
                    out[base + i] = fp8_e4m3_value(codes[base + i]) * scale;
            }
    return 0;
}

/* Gradients of L = sum(dout * attention(q, k, v)).  dout has q's element
 * type and layout [B][Lq][Hq][dv]; dq [B][Lq][Hq][dqk], dk[c]
 * [B][len[c]][Hkv][dqk] and dvv[c] [B][len[c]][Hkv][dv] are written (double).
 * Returns 0, -1 on an argument error, -2 if out of memory. */
int oracle_attention_bwd(int B, int Hq, int Hkv, int dqk, int dv, int dtype,
                         const void *q, int64_t Lq, int64_t q_offset,
                         int n_chunks, const void *const *k,
                         const void *const *v, const int64_t *start,
                         const int64_t *len, const oracle_mask *mk,
                         double scale, const void *dout, double *dq,
                         double *const *dk, double *const *dvv)
{
    if (check_shapes(B, Hq, Hkv, dqk, dv, dtype, Lq, n_chunks, len, 0, NULL))
        return -1;
    const int G = Hq / Hkv;
    int64_t nkeys = 0;
    for (int c = 0; c < n_chunks; ++c)
        nkeys += len[c];
    int64_t units = (int64_t)B * Hq * Lq;
    /* per row: log-sum-exp of its visible scores, and sum_t P_t dP_t */
    double *lse = (double *)malloc(sizeof(double) * (size_t)(units ? units : 1));
    double *Dsum = (double *)malloc(sizeof(double) * (size_t)(units ? units : 1));
    if (!lse || !Dsum) {
        free(lse);
        free(Dsum);
        return -2;
    }
    int err = 0;

    /* pass 1, per query row: softmax weights, D, and dQ */
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(nkeys ? nkeys : 1));
        double *dp = (double *)malloc(sizeof(double) * (size_t)(nkeys ? nkeys : 1));
        if (!s || !dp) {
#pragma omp atomic write
            err = -2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < units; ++u) {
            if (!s || !dp)
                continue;
            int b = (int)(u / ((int64_t)Hq * Lq));
            int h = (int)((u / Lq) % Hq);
            int64_t r = u % Lq;
            int64_t qpos = q_offset + r;
            int hk = h / G;
            int64_t row = ((int64_t)b * Hq + h) * Lq + r;
            double *g = dq + (((int64_t)b * Lq + r) * Hq + h) * dqk;
            int64_t ob = (((int64_t)b * Lq + r) * Hq + h) * dv;
            for (int e = 0; e < dqk; ++e)
                g[e] = 0.0;

            double mx = -INFINITY;
            int64_t t = 0;
            for (int c = 0; c < n_chunks; ++c)
                for (int64_t j = 0; j < len[c]; ++j, ++t) {
                    if (!visible(mk, Lq, len[c], b, r, c, j, qpos, start[c] + j)) {
                        s[t] = -INFINITY;
                        continue;
                    }
                    s[t] = score(q, k[c], dtype, Lq, len[c], Hq, Hkv, dqk, b, r, h, j, scale);
                    if (s[t] > mx)
                        mx = s[t];
                }
            if (mx == -INFINITY) { /* no visible key */
                lse[row] = -INFINITY;
                Dsum[row] = 0.0;
                continue;
            }
            double sum = 0.0;
            for (t = 0; t < nkeys; ++t)
                if (s[t] != -INFINITY)
                    sum += exp(s[t] - mx);
            double ls = mx + log(sum);
            lse[row] = ls;

            /* dP_t = dO . v_t and D = sum_t P_t dP_t */
            double D = 0.0;
            t = 0;
            for (int c = 0; c < n_chunks; ++c)
                for (int64_t j = 0; j < len[c]; ++j, ++t) {
                    if (s[t] == -INFINITY)
                        continue;
                    int64_t vb = (((int64_t)b * len[c] + j) * Hkv + hk) * dv;
                    double acc = 0.0;
                    for (int e = 0; e < dv; ++e)
                        acc += elem(dout, dtype, ob + e) * elem(v[c], dtype, vb + e);
                    dp[t] = acc;
                    D += exp(s[t] - ls) * acc;
                }
            Dsum[row] = D;

            /* dQ = scale sum_t P_t (dP_t - D) k_t */
            t = 0;
            for (int c = 0; c < n_chunks; ++c)
                for (int64_t j = 0; j < len[c]; ++j, ++t) {
                    if (s[t] == -INFINITY)
                        continue;
                    double ds = exp(s[t] - ls) * (dp[t] - D);
                    int64_t kb = (((int64_t)b * len[c] + j) * Hkv + hk) * dqk;
                    for (int e = 0; e < dqk; ++e)
                        g[e] += scale * ds * elem(k[c], dtype, kb + e);
                }
        }
        free(s);
        free(dp);
    }
    if (err) {
        free(lse);
        free(Dsum);
        return err;
    }

    /* pass 2, per key: dK and dV summed over every row of every query head
     * in the key's group */
    int64_t kunits = (int64_t)B * Hkv * nkeys;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t u = 0; u < kunits; ++u) {
        int b = (int)(u / ((int64_t)Hkv * nkeys));
        int hk = (int)((u / nkeys) % Hkv);
        int64_t t = u % nkeys;
        int c = 0;
        while (t >= len[c]) { /* chunk c and index j of global key t */
            t -= len[c];
            ++c;
        }
        int64_t j = t;
        int64_t kb = (((int64_t)b * len[c] + j) * Hkv + hk) * dqk;
        int64_t vb = (((int64_t)b * len[c] + j) * Hkv + hk) * dv;
        double *gk = dk[c] + kb, *gv = dvv[c] + vb;
        for (int e = 0; e < dqk; ++e)
            gk[e] = 0.0;
        for (int e = 0; e < dv; ++e)
            gv[e] = 0.0;
        for (int h = hk * G; h < (hk + 1) * G; ++h)
            for (int64_t r = 0; r < Lq; ++r) {
                if (!visible(mk, Lq, len[c], b, r, c, j, q_offset + r, start[c] + j))
                    continue;
                int64_t row = ((int64_t)b * Hq + h) * Lq + r;
                if (lse[row] == -INFINITY)
                    continue;
                double p = exp(score(q, k[c], dtype, Lq, len[c], Hq, Hkv, dqk, b, r, h, j, scale) - lse[row]);
                int64_t ob = (((int64_t)b * Lq + r) * Hq + h) * dv;
                int64_t qb = (((int64_t)b * Lq + r) * Hq + h) * dqk;
                double dpv = 0.0;
                for (int e = 0; e < dv; ++e)
                    dpv += elem(dout, dtype, ob + e) * elem(v[c], dtype, vb + e);
                double ds = p * (dpv - Dsum[row]);
                for (int e = 0; e < dqk; ++e)
                    gk[e] += scale * ds * elem(q, dtype, qb + e);
                for (int e = 0; e < dv; ++e)
                    gv[e] += p * elem(dout, dtype, ob + e);
            }
    }
    free(lse);
    free(Dsum);
    return 0;
}
