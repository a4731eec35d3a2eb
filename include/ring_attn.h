/*
 * ring_attn.h - C ABI of libringattn, one device's share of ring attention on
 * AMD Instinct MI355X (gfx950).
 *
 * What one device computes.  The sequence is cut into chunks; this device
 * holds one query chunk and attends it to every KV chunk as the chunks come
 * round the ring, one chunk per step, keeping a running softmax state
 * (running max m, denominator l, unnormalised output O) that is rescaled and
 * extended chunk after chunk, so that the final O / l equals
 * softmax(Q K^T * scale) V over all keys:
 *   - page "Ring Attention：百万 Token 上下文的秘密", §2.1 分块计算注意力
 *     (sequence sharding), §2.2 环形通信 (one KV chunk per ring step),
 *     §2.3 数学正确性 (the result equals plain attention), §3.1 Flash Ring
 *     Attention (blockwise attention per received chunk) and §3.2
 *     通信-计算重叠 (the next chunk is received while the current one is
 *     computed, into a second buffer);
 *   - page "从百毫秒到百万Token：长上下文推理优化的工程实践", section
 *     "注意力机制的数学本质与瓶颈" (the definition of attention) and
 *     "系统架构设计" item 注意力融合层 (partial outputs are normalised into
 *     one global softmax: ring_attn_merge);
 *   - page "RingAttention推理优化：cache_idx参数使用与千万级上下文高效推理实践",
 *     sections "cache_idx的工作原理" and "增量推理实战" (queries of an
 *     incremental step sit at cache_idx, cache_idx+1, ... of the cached
 *     sequence: the q_offset argument).
 *
 * Conventions shared by every call:
 *   - All tensor pointers are DEVICE pointers (HIP global memory on the
 *     context's device) unless stated otherwise; descriptor structs and
 *     arrays of them are HOST memory, read only during the call.
 *   - The caller owns every buffer.  The library never allocates or frees
 *     device memory in ring_attn_fwd / ring_attn_merge; scratch space comes
 *     from the caller's workspace (ring_attn_workspace_size).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is
 *     enqueued after prior work on `stream`; calls return without waiting
 *     for the GPU.  A context's side stream joins back into `stream` with
 *     events before ring_attn_fwd returns.
 *   - Return value: RA_OK (0) or a negative RA_ERR_* code.  Arguments are
 *     validated before anything is enqueued: on a validation error nothing
 *     runs.  ring_attn_last_error() describes the most recent failure of the
 *     calling thread.  Faults inside kernels surface on a later call or
 *     synchronisation, as usual for HIP.  NaN/Inf inputs are not checked;
 *     they propagate.
 *
 * Layouts.  Tensors are [B, S, H, d] ("BSHD", token-major as in the pages'
 * [batch, sequence, dim] convention); the head dimension d is contiguous and
 * the other three strides are given in ELEMENTS per tensor (all-zero strides
 * mean dense BSHD).  bf16 tensors need 16-byte aligned base pointers and
 * strides that are multiples of 8 elements; fp32 tensors need 16-byte
 * aligned pointers and strides that are multiples of 4 elements.  The token
 * strides of k and v must be below 2^24 elements (a key tile is addressed
 * with 32-bit offsets); any other order of the three strides works, e.g. a
 * head-major KV cache [B, H, S, d] passed as BSHD with strides
 * (H*S*d, d, S*d).
 * Softmax state buffers are dense fp32: m and l are [B, Lq, Hq], O is
 * [B, Lq, Hq, d_v]; m is in natural-log units of the scaled logits, l is
 * sum(exp(s - m)) and O is sum(exp(s - m) * v), so out = O / l and the
 * log-sum-exp is m + ln(l).  A row that has seen no key has m = -inf, l = 0,
 * O = 0 and gets out = 0.
 *
 * Grouped-query attention: query head h reads KV head h / (Hq / Hkv).
 * Causal masking is per token with the diagonal included: the query at
 * absolute position p sees the key at absolute position t iff t <= p.
 */
#ifndef RING_ATTN_H
#define RING_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define RA_OK 0
#define RA_ERR_INVALID_ARG (-1) /* null, negative or inconsistent argument */
#define RA_ERR_UNSUPPORTED (-2) /* dtype / head size / layout not built    */
#define RA_ERR_WORKSPACE (-3)   /* workspace missing or too small          */
#define RA_ERR_HIP (-4)         /* HIP runtime or launch failure           */

/* element types */
#define RA_F32 0
#define RA_BF16 1
/* 8-bit KV cache (ra_desc.kv_dtype only): OCP FP8 E4M3 codes (1 sign, 4
 * exponent bits with bias 7, 3 mantissa bits; no infinities; 0x7f/0xff are
 * NaN; largest finite 448).  Every RA_KV_SCALE_BLOCK consecutive tokens of
 * one (batch, KV head) share the scale 2^(e - 127), e an 8-bit biased
 * exponent in 1..254 (ra_kv_chunk.k_exp / v_exp): value = code x scale.
 * The pages recommend an 8-bit KV cache for serving without fixing a
 * format (page "billion-token context window engineering", production
 * parameters; page "RingAttention与RAG技术对比及实战应用", §2.3). */
#define RA_FP8_E4M3 2
#define RA_KV_SCALE_BLOCK 64

/* ring_attn_fwd flags */
#define RA_FLAG_STAGE 1u      /* ring stand-in: copy each received chunk into a
                                 double buffer on the side stream (see fwd) */
#define RA_FLAG_SPLIT_KV 2u   /* force the split-KV (decode) schedule        */
#define RA_FLAG_NO_SPLIT_KV 4u /* force the ring schedule                    */
#define RA_FLAG_ACCUMULATE 8u /* start from the state in m/l/O instead of an
                                 empty one (resume / continue a ring)        */

/* chunk classes reported by ring_attn_plan */
#define RA_CHUNK_SKIP 0 /* every key is after every query: not computed   */
#define RA_CHUNK_FULL 1 /* every key is visible to every query: no mask   */
#define RA_CHUNK_DIAG 2 /* some keys are masked for some queries          */

typedef struct ra_desc {
    int32_t B;     /* batch size                                    */
    int32_t Hq;    /* query heads                                   */
    int32_t Hkv;   /* key/value heads; Hq % Hkv == 0                */
    int32_t d_qk;  /* query/key head size                           */
    int32_t d_v;   /* value/output head size                        */
    int32_t dtype; /* RA_F32 or RA_BF16: q, out (and k, v)          */
    float scale;   /* logit scale; 0 selects 1/sqrt(d_qk)           */
    int32_t kv_dtype; /* element type of k and v: 0 (same as dtype) or
                         RA_FP8_E4M3 (with dtype RA_BF16)            */
    int64_t q_strides[3]; /* q   [B, Lq, Hq, d_qk]: (batch, token, head) */
    int64_t k_strides[3]; /* k   [B, len, Hkv, d_qk], every chunk        */
    int64_t v_strides[3]; /* v   [B, len, Hkv, d_v],  every chunk        */
    /* (all strides in elements: bytes for an 8-bit KV cache)             */
    int64_t o_strides[3]; /* out [B, Lq, Hq, d_v]                        */
    /* Local window: with window > 0 a query at position p sees only keys
     * at distance <= window: p - window .. p under causal masking, p -
     * window .. p + window without it (page "Ring Attention：百万 Token
     * 上下文的秘密", §4.3 稀疏注意力掩码: query i sees keys i - w .. i).
     * window <= 0: no window.  Tiles and chunks outside every window of a
     * workgroup are not read. */
    int64_t window;
    /* Anchor tokens: with anchor = S > 0 a query at position p also sees
     * the keys at A - 1, A and A + S, A = S * floor(p / S), when they
     * exist, whatever the window and the causal rule say (the same
     * section's sparse mask, whose anchor stride is 4096).  0: none. */
    int64_t anchor;
    /* Segment labels of the query rows, [B, Lq] int32 dense (device), or
     * NULL.  With labels (given for the queries and every chunk) a query
     * sees only keys with its own label: packed sequences, the
     * segment_ids of page "RingAttention推理优化：cache_idx参数使用...".
     * Anchors and labels are built for d = 64 and 128 (bf16 and fp32);
     * RA_ERR_UNSUPPORTED with d = 512 or an 8-bit KV cache. */
    const int32_t *q_seg;
} ra_desc;

typedef struct ra_kv_chunk {
    const void *k;  /* device pointer to the chunk's keys                  */
    const void *v;  /* device pointer to the chunk's values                */
    int64_t start;  /* absolute position of the chunk's first key          */
    int64_t len;    /* number of keys (ragged chunks allowed; 0 = empty)   */
    /* 8-bit KV cache only (else NULL): device pointers to the biased scale
     * exponents, dense [B, Hkv, ceil(len / RA_KV_SCALE_BLOCK)] uint8 */
    const uint8_t *k_exp;
    const uint8_t *v_exp;
    /* segment labels of the keys, [B, len] int32 dense (device), or NULL;
     * required exactly when ra_desc.q_seg is given */
    const int32_t *k_seg;
} ra_kv_chunk;

typedef struct ra_ctx ra_ctx;

/* Library version string (static storage). */
const char *ring_attn_version(void);

/* Message of the calling thread's most recent failure ("" if none). */
const char *ring_attn_last_error(void);

/* Create a context on HIP device `device`: it owns one side stream (default
 * priority) and the events that pace the double buffer.  No device memory.
 * RA_ERR_HIP if the device does not exist. */
int ring_attn_ctx_create(int device, ra_ctx **out);
int ring_attn_ctx_destroy(ra_ctx *ctx);

/* Perturbations of the staged ring (RA_FLAG_STAGE) for checking its
 * ordering -- page "Ring Attention：百万 Token 上下文的秘密", §3.2
 * 通信-计算重叠: a step reads a received chunk only after it has arrived,
 * and a buffer is refilled only after the step reading it has finished.
 * With them on, ring_attn_fwd delays the side stream before each staging
 * copy (DELAY_COPY) and the caller's stream before each launch
 * (DELAY_COMPUTE) with a one-wave spin of spin_us microseconds that always
 * ends, and overwrites each staging buffer with NaN right after the step
 * that read it (POISON, a fill kernel).  Correct ordering gives bit-identical
 * results with any of them.  They cost time and are meant for tests only.
 * RA_ERR_INVALID_ARG for unknown bits or spin_us > RA_CHECK_MAX_SPIN_US. */
#define RA_CHECK_DELAY_COPY 1u
#define RA_CHECK_DELAY_COMPUTE 2u
#define RA_CHECK_POISON 4u
#define RA_CHECK_MAX_SPIN_US 100000
int ring_attn_ctx_set_check(ra_ctx *ctx, uint32_t checks, uint32_t spin_us);

/* Order in which ring device `device_index` of `P` meets the KV chunks when
 * every step receives the chunk of the previous device (page "Ring
 * Attention：百万 Token 上下文的秘密", §3.1: receive from the left
 * neighbour, send to the right): its own chunk, then device_index-1,
 * device_index-2, ... modulo P.  Host only; writes P ints to `order`. */
int ring_attn_ring_order(int device_index, int P, int32_t *order);

/* Chunk classes of one ring device's schedule (page "RingAttention推理优化：
 * cache_idx参数使用与千万级上下文高效推理实践", section cache_idx的工作原理 and
 * its blockwise settings with causal_block_size=1: token-level causality on
 * absolute positions; page "Ring Attention：百万 Token 上下文的秘密", §4.3
 * 稀疏注意力掩码: local window plus anchor tokens).
 * For a query chunk of Lq rows at absolute positions
 * q_offset .. q_offset+Lq-1 (host only): cls[c] = RA_CHUNK_SKIP (no key
 * visible to any query) / FULL (every key visible to every query by the
 * causal and window rules alone: no mask is applied) / DIAG (masked per
 * element) for the chunk at starts[c] with lens[c] keys, under causal masking, the
 * local window and anchor tokens (as ra_desc.window and ra_desc.anchor;
 * <= 0 / 0: none).  A chunk holding an anchor of some query is never
 * skipped.  Segment labels are device data and not considered here: they
 * can only hide more keys.  Non-causal without a window: all FULL (empty
 * chunks: SKIP). */
int ring_attn_plan(int64_t Lq, int64_t q_offset, int causal, int64_t window,
                   int64_t anchor, int P, const int64_t *starts,
                   const int64_t *lens, int32_t *cls);

/* Bytes of device workspace ring_attn_fwd needs for these arguments
 * (host only; k/v pointers are not read).  0 is a valid answer. */
int ring_attn_workspace_size(const ra_desc *d, int64_t Lq,
                             const ra_kv_chunk *chunks, int P, int causal,
                             int64_t q_offset, uint32_t flags, int want_state,
                             size_t *bytes);

/* One device's share of ring attention (page "Ring Attention：百万 Token
 * 上下文的秘密": §2.2 环形通信 for the ring of KV chunks, §2.3 数学正确性 for
 * the exactness of the chunked result, §3.1 Flash Ring Attention for the
 * blockwise online-softmax computation of each step, §3.2 通信-计算重叠 for
 * the double-buffered receive that STAGE stands in for; page
 * "RingAttention推理优化：cache_idx参数使用与千万级上下文高效推理实践",
 * section cache_idx的工作原理, for q_offset = cache_idx in decoding).  Each
 * output row is softmax(q k^T * scale) v over the keys of all chunks the
 * row may see; the fp32 state (m, l, O) after the call is the running max,
 * denominator and unnormalised output of the online softmax.
 *
 *   q          [B, Lq, Hq, d_qk] query chunk (device)
 *   chunks     P KV chunks (host array of device pointers), processed in
 *              array order: pass them in ring order (ring_attn_ring_order)
 *              to mirror a ring; the result does not depend on the order
 *              beyond rounding.  Chunks must not overlap in position.
 *   causal     0/1; chunks whose keys all follow every query are skipped
 *   q_offset   absolute position of query row 0: (query chunk index) x
 *              (chunk length) in a prefill ring, or cache_idx in
 *              incremental decoding (no rounding to any chunk size)
 *   flags      RA_FLAG_*:
 *                STAGE: the first computed chunk is read in place (the
 *                  device's own chunk); every later chunk is first copied
 *                  into one of two workspace buffers on the context's side
 *                  stream, one step ahead of the compute stream, standing in
 *                  for the receive from the ring neighbour.  Requires chunks
 *                  whose (token, head) strides are dense.
 *                SPLIT_KV / NO_SPLIT_KV: choose the schedule.  By default
 *                  Lq <= 16 (incremental decoding) uses split-KV: the keys
 *                  are cut into many ranges computed in parallel, each
 *                  writing a partial state, then merged.  Otherwise chunks
 *                  are folded in order into one running state.
 *                ACCUMULATE: m_out/l_out/O_out hold a state to continue from.
 *   out        [B, Lq, Hq, d_v] in desc->dtype, or NULL
 *   m_out, l_out, O_out   fp32 state after the call, or all NULL
 *   workspace, ws_bytes   device scratch of ring_attn_workspace_size bytes
 *   stream     hipStream_t
 * At least one of out / (m_out, l_out, O_out) must be given.
 * Supported: bf16 with d_qk == d_v in {64, 128, 512}; fp32 with d_qk == d_v
 * in {64, 128}; an 8-bit KV cache (kv_dtype RA_FP8_E4M3) with bf16 queries,
 * d_qk == d_v == 128, on the split-KV schedule (incremental decoding, no
 * STAGE); RA_ERR_UNSUPPORTED otherwise.  RA_ERR_INVALID_ARG if an 8-bit
 * chunk with keys lacks k_exp or v_exp. */
int ring_attn_fwd(ra_ctx *ctx, const ra_desc *d, const void *q, int64_t Lq,
                  const ra_kv_chunk *chunks, int P, int causal,
                  int64_t q_offset, uint32_t flags, void *out, float *m_out,
                  float *l_out, float *O_out, void *workspace,
                  size_t ws_bytes, void *stream);

/* Bytes of the static device scratch behind ring_attn_fwd_noalloc (96 MiB
 * per GPU). */
#define RA_NOALLOC_SCRATCH_BYTES (96u << 20)

/* ring_attn_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  It allocates nothing: the
 * scratch ring_attn_fwd would take from `workspace` (staging buffers,
 * the carried state, split-KV partials) comes from a file-scope device
 * array of RA_NOALLOC_SCRATCH_BYTES, one per GPU, placed when the library
 * is loaded on that GPU and held until the process ends; its address is
 * looked up when a context is created on the device.  Arguments, results,
 * ownership of the caller's buffers and the errors are those of
 * ring_attn_fwd, plus RA_ERR_WORKSPACE (nothing enqueued) when the call
 * needs more scratch than RA_NOALLOC_SCRATCH_BYTES (ring_attn_workspace_size
 * tells how much), and RA_ERR_HIP when the scratch of ctx's device could
 * not be found.  Every call on one GPU shares that GPU's scratch and
 * leaves its contents behind (no call relies on it being zero): calls
 * whose device work overlaps -- on different streams without ordering
 * between them, or from several host threads -- race on it. */
int ring_attn_fwd_noalloc(ra_ctx *ctx, const ra_desc *d, const void *q,
                          int64_t Lq, const ra_kv_chunk *chunks, int P,
                          int causal, int64_t q_offset, uint32_t flags,
                          void *out, float *m_out, float *l_out,
                          float *O_out, void *stream);

/* Gradients of one KV chunk (fp32, dense [B, len, Hkv, d], device). */
typedef struct ra_kv_grad {
    float *dk; /* [B, len, Hkv, d_qk] */
    float *dv; /* [B, len, Hkv, d_v]  */
} ra_kv_grad;

/* Bytes of device workspace ring_attn_bwd needs (host only). */
int ring_attn_bwd_workspace_size(const ra_desc *d, int64_t Lq, size_t *bytes);

/* Gradients of one device's share of ring attention, for training with it
 * (page "Ring Attention：百万 Token 上下文的秘密", §5.1 训练效率, which uses
 * it to train; the pages give no backward algorithm, so this is the
 * derivative of softmax(Q K^T * scale) V over the visible keys).  With
 * P = softmax(S), dO the gradient of out and D = rowsum(dO * out):
 *   dV = P^T dO,  dS = P * (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q
 * summed over the query heads of each KV head's group.
 *
 *   q, chunks, P, causal, q_offset, d->window: as for ring_attn_fwd (the same
 *              masks; d->o_strides also describe dout)
 *   out        [B, Lq, Hq, d_v] bf16: the forward output
 *   dout       [B, Lq, Hq, d_v] bf16: the gradient of out
 *   m, l       [B, Lq, Hq] fp32: the forward state after all the key chunks
 *              the output attended (m_out and l_out of ring_attn_fwd)
 *   dq         [B, Lq, Hq, d_qk] fp32, dense (device)
 *   grads      P entries: dK and dV of chunk c go to grads[c] (entries of
 *              empty chunks are not touched)
 *   flags      0 or RA_FLAG_ACCUMULATE: add into dq, dk and dv instead of
 *              overwriting them (the dK/dV of a chunk travelling the ring
 *              collect each device's share this way)
 *   workspace, ws_bytes   ring_attn_bwd_workspace_size bytes, 256-aligned
 * The chunks given may be a subset of those the forward saw (one ring step
 * at a time, say): m and l carry the softmax normalisation over all of them.
 * Rows with l = 0 (no visible key) have zero gradients.  Supported: bf16
 * with d_qk == d_v in {64, 128, 512}, bf16 keys and values (at 512 without
 * anchor tokens or segment labels, as the forward); RA_ERR_UNSUPPORTED
 * otherwise.  The call is deterministic (no atomics). */
int ring_attn_bwd(ra_ctx *ctx, const ra_desc *d, const void *q, int64_t Lq,
                  const ra_kv_chunk *chunks, int P, int causal,
                  int64_t q_offset, uint32_t flags, const void *out,
                  const void *dout, const float *m, const float *l, float *dq,
                  const ra_kv_grad *grads, void *workspace, size_t ws_bytes,
                  void *stream);

/* Merge n_parts partial softmax states over disjoint key sets into one (the
 * fusion layer's global normalisation, page "从百毫秒到百万Token", 系统架构设计,
 * 注意力融合层):
 *   m = max_i m_i,  l = sum_i e^(m_i - m) l_i,  O = sum_i e^(m_i - m) O_i,
 * where a part with m_i = -inf has weight 0.
 *   m_parts, l_parts  [n_parts, rows] fp32 (device)
 *   O_parts           [n_parts, rows, d_v] fp32 (device)
 *   m, l, O           merged state (device, may alias nothing), or all NULL
 *   out               [rows, d_v] = O / l in out_dtype (RA_F32 / RA_BF16), or NULL
 * rows is any row count (e.g. B*Lq*Hq for fwd states).  n_parts >= 1. */
int ring_attn_merge(int n_parts, int64_t rows, int d_v, const float *m_parts,
                    const float *l_parts, const float *O_parts, float *m,
                    float *l, float *O, void *out, int out_dtype,
                    void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RING_ATTN_H */
