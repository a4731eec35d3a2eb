// ra_internal.h - argument blocks shared by the host runtime and the HIP
// kernels of libringattn.  Not part of the public ABI (include/ring_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

// KV chunks one kernel launch can walk (kernel arguments are at most 4 KiB).
constexpr int kMaxChunks = 64;
// Scale blocks of one 8-bit workgroup's key range (its exponents sit in LDS).
constexpr int kFp8MaxRangeBlocks = 4096;

struct ChunkArg {
    const void *k;
    const void *v;
    int64_t start;  // absolute position of key 0
    int64_t len;    // keys in the chunk
    const uint8_t *kexp, *vexp;  // 8-bit KV: biased scale exponents [B, Hkv, ceil(len/64)]
    const int32_t *kseg;         // segment labels of the keys [B, len], or null
};

// Arguments of the forward kernels (bf16 MFMA and fp32 paths).
//
// Query rows are "packed" per KV head: packed row p = g * Lq_pad + t is token
// t of query head hk * G + g.  Lq_pad == Lq packs the G heads densely
// (incremental decoding: G heads x a few tokens fill one tile); Lq_pad
// rounded up to the row tile keeps every tile inside one head (prefill).
struct FwdArgs {
    const void *q;
    void *out;                 // [B, Lq, Hq, d_v] in the input dtype, or null
    float *m, *l, *O;          // running state [B, Lq, Hq](, d_v), or null
    float *pm, *pl, *pO;       // split mode: partial states [slot][B, Lq, Hq](, d_v)
    int64_t q_sb, q_ss, q_sh;  // element strides (batch, token, head)
    int64_t k_sb, k_ss, k_sh;
    int64_t v_sb, v_ss, v_sh;
    int64_t o_sb, o_ss, o_sh;
    int64_t Lq, Lq_pad, q_offset;
    int64_t sub_len;           // split mode: keys per sub-range of a chunk
    int64_t window;            // local window (> 0), or 0: none
    int64_t anchor;            // anchor-token stride (> 0), or 0: none
    const int32_t *q_seg;      // segment labels of the query rows [B, Lq], or null
    int B, Hq, Hkv, G;
    int causal;
    int load_state;            // start from (m, l, O) instead of empty
    int store_state;           // write (m, l, O)
    int store_out;             // write out = O / l
    int split_mode;            // 0: fold all chunks; 1: one (chunk, sub-range) per workgroup
    int n_sub;                 // split mode: sub-ranges per chunk
    int part_base;             // split mode: partial slot of (chunk 0, sub 0)
    int n_rowtiles;            // row tiles per (batch, KV head)
    int n_chunks;
    float scale_log2;          // logit scale * log2(e)
    ChunkArg chunks[kMaxChunks];
};

// Arguments of the backward kernels.  The query rows, chunks, strides and
// masks are those of the forward (f); out and dout share f's o strides.
struct BwdArgs {
    FwdArgs f;
    const void *out, *dout;  // [B, Lq, Hq, d_v] in the input dtype
    const float *m, *l;      // forward state after all chunks [B, Lq, Hq]
    float *ld;               // workspace [B, Hq, Lq][2]: -(m + ln l) log2(e), -rowsum(dO * out)
    float *dq;               // [B, Lq, Hq, d_qk] fp32, dense
    float *dk, *dv;          // dK/dV kernel: the launch's chunk, [B, len, Hkv, d] fp32, dense
    int chunk;               // dK/dV kernel: index into f.chunks
    int accumulate;          // add into dq / dk / dv instead of overwriting them
    float scale;             // logit scale
};

struct MergeArgs {
    const float *pm, *pl, *pO;  // [n, rows](, d_v)
    float *m, *l, *O;           // merged state or null
    void *out;                  // [rows, d_v] or null
    int64_t rows;
    int n_parts;
    int d_v;
    int out_bf16;
};

// Launchers (defined next to their kernels).  They return hipSuccess or the
// launch error; bm_out reports the row tile the kernel uses.
int fwd_bf16_row_tile(int d, bool split_mode);
hipError_t launch_fwd_bf16(const FwdArgs &a, int d, bool split_mode, hipStream_t s);
// bf16 queries against an 8-bit (FP8 E4M3) KV cache, d = 128, split-KV only
int fwd_fp8kv_row_tile();
hipError_t launch_fwd_fp8kv(const FwdArgs &a, hipStream_t s);
int fwd_f32_row_tile(int d);
hipError_t launch_fwd_f32(const FwdArgs &a, int d, hipStream_t s);
hipError_t launch_merge(const MergeArgs &a, hipStream_t s);
// Checks of the staged ring's ordering: a bounded spin of one wave, and a
// NaN fill of a staging buffer (a kernel, so it can be captured in a graph).
hipError_t launch_spin(uint32_t microseconds, hipStream_t s);
hipError_t launch_fill_nan(void *p, size_t bytes, hipStream_t s);
// Backward, bf16 with d = 64 or 128: row statistics, dQ over the chunks of
// a.f (rows tiled like the forward, bwd_dq_row_tile rows per workgroup), and
// dK/dV of chunk a.chunk.
int bwd_dq_row_tile(int d);
hipError_t launch_bwd_pre(const BwdArgs &a, int d, hipStream_t s);
hipError_t launch_bwd_dq(const BwdArgs &a, int d, hipStream_t s);
hipError_t launch_bwd_dkdv(const BwdArgs &a, int d, hipStream_t s);

}  // namespace ra
