// ring_attn.cpp - host runtime behind include/ring_attn.h: argument checks,
// the chunk schedule of one ring device, the double-buffered chunk staging on
// a side stream, the split-KV decode schedule, and kernel launches.
//
// Ring step structure (page "Ring Attention：百万 Token 上下文的秘密", §3.1
// Flash Ring Attention and §3.2 通信-计算重叠): step s attends the resident
// query chunk to the KV chunk held in buffer s%2 while the chunk of step s+1
// is brought into the other buffer; a buffer is refilled only after the step
// that read it has finished.  Here the "receive" is a device-to-device copy
// on the context's side stream, paced by two events per buffer.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/ring_attn.h"
#include "ra_internal.h"

using ra::BwdArgs;
using ra::ChunkArg;
using ra::FwdArgs;
using ra::MergeArgs;

static_assert(sizeof(BwdArgs) <= 4096, "kernel arguments are limited to 4 KiB");

struct ra_ctx {
    int device;
    uint32_t check;        // RA_CHECK_* perturbations of the staged ring
    uint32_t check_us;     // their spin length
    hipStream_t side;
    hipEvent_t start;     // caller stream reached the call
    hipEvent_t ready[2];  // staging buffer b holds its chunk
    hipEvent_t freed[2];  // the step reading staging buffer b has finished
    hipEvent_t join;      // side stream's last copy
};

// Scratch of ring_attn_fwd_noalloc: a file-scope device array, one copy per
// GPU (the loader places it when the library's code object is loaded on the
// device, and it stays until the process ends).  Host code never passes the
// array's name to a kernel or a copy: that name is a host-side stand-in.  The
// device address of each GPU's copy is looked up once per device, with that
// device current, when a context is created there, and kept below.
static __device__ __align__(256) char scratch[RA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;

constexpr int kMaxScratchDevices = 64;
struct ScratchSlot {
    std::once_flag once;
    void *ptr = nullptr;           // device address of this GPU's copy of `scratch`
    hipError_t err = hipSuccess;   // result of the lookup
};
ScratchSlot g_scratch[kMaxScratchDevices];

// Look up this device's copy of `scratch` (the device must be current).
void scratch_lookup(int device) {
    if (device < 0 || device >= kMaxScratchDevices) return;
    ScratchSlot &sl = g_scratch[device];
    std::call_once(sl.once, [&sl] {
        void *p = nullptr;
        sl.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        sl.ptr = sl.err == hipSuccess ? p : nullptr;
    });
}

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(RA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Decode-sized query chunks take the split-KV schedule by default.
constexpr int64_t kSplitMaxLq = 16;
// Split-KV aims at this many workgroups (a few per compute unit).
constexpr int64_t kSplitTargetWorkgroups = 2048;

struct Strides {
    int64_t q[3], k[3], v[3], o[3];
};

int elem_size(int dtype) { return dtype == RA_BF16 ? 2 : 4; }

// 8-bit KV cache (bf16 queries, FP8 E4M3 keys/values with block exponents)
bool kv_fp8(const ra_desc *d) { return d->kv_dtype == RA_FP8_E4M3; }

// Query rows per workgroup of the kernel a schedule launches.
int row_tile(const ra_desc *d, bool split) {
    if (kv_fp8(d) && split) return ra::fwd_fp8kv_row_tile();
    return d->dtype == RA_BF16 ? ra::fwd_bf16_row_tile(d->d_qk, split) : ra::fwd_f32_row_tile(d->d_qk);
}

bool supported_head(int dtype, int d) {
    if (dtype == RA_BF16) return d == 64 || d == 128 || d == 512;
    if (dtype == RA_F32) return d == 64 || d == 128;
    return false;
}

int check_desc(const ra_desc *d, int64_t Lq, Strides *st) {
    if (!d) return fail(RA_ERR_INVALID_ARG, "desc is NULL");
    if (d->B < 1 || d->Hq < 1 || d->Hkv < 1 || d->d_qk < 1 || d->d_v < 1)
        return fail(RA_ERR_INVALID_ARG, "B, Hq, Hkv, d_qk, d_v must be >= 1");
    if (d->Hq % d->Hkv != 0) return fail(RA_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", d->Hq, d->Hkv);
    if (d->dtype != RA_F32 && d->dtype != RA_BF16) return fail(RA_ERR_INVALID_ARG, "dtype %d unknown", d->dtype);
    if (!(d->scale >= 0.f) || std::isinf(d->scale)) return fail(RA_ERR_INVALID_ARG, "scale must be finite and >= 0");
    if (Lq < 0) return fail(RA_ERR_INVALID_ARG, "Lq must be >= 0");
    if (d->d_qk != d->d_v || !supported_head(d->dtype, d->d_qk))
        return fail(RA_ERR_UNSUPPORTED, "head sizes d_qk=%d d_v=%d not built for dtype %d", d->d_qk, d->d_v, d->dtype);
    if (d->kv_dtype != 0 && d->kv_dtype != d->dtype && d->kv_dtype != RA_FP8_E4M3)
        return fail(RA_ERR_INVALID_ARG, "kv_dtype %d unknown", d->kv_dtype);
    if (kv_fp8(d) && (d->dtype != RA_BF16 || d->d_qk != 128))
        return fail(RA_ERR_UNSUPPORTED, "an 8-bit KV cache is built for bf16 queries with d = 128");
    if (d->anchor < 0) return fail(RA_ERR_INVALID_ARG, "anchor must be >= 0");
    if ((d->anchor > 0 || d->q_seg) && (kv_fp8(d) || (d->dtype == RA_BF16 && d->d_qk == 512)))
        return fail(RA_ERR_UNSUPPORTED, "anchor tokens and segment labels are built for d = 64, 128 (bf16, fp32)");
    if (d->q_seg && ((uintptr_t)d->q_seg & 3)) return fail(RA_ERR_INVALID_ARG, "q_seg must be 4-byte aligned");
    const int qalign = d->dtype == RA_BF16 ? 8 : 4;  // elements of 16-byte units
    const int kvalign = kv_fp8(d) ? 16 : qalign;
    auto fill = [&](const int64_t *in, int64_t *out, int64_t S, int64_t H, int64_t D, const char *name) -> int {
        const int align = name[0] == 'k' || name[0] == 'v' ? kvalign : qalign;
        if (in[0] == 0 && in[1] == 0 && in[2] == 0) {
            out[2] = D;
            out[1] = H * D;
            out[0] = S * H * D;
            return RA_OK;
        }
        for (int i = 0; i < 3; ++i) {
            if (in[i] <= 0 || in[i] % align != 0)
                return fail(RA_ERR_INVALID_ARG, "%s strides must be positive multiples of %d elements", name, align);
            out[i] = in[i];
        }
        return RA_OK;
    };
    int rc;
    // kernels address one key tile (<= 128 rows) with 32-bit byte offsets from
    // the token stride; batch and head offsets are 64-bit
    if (d->k_strides[1] >= ((int64_t)1 << 24) || d->v_strides[1] >= ((int64_t)1 << 24))
        return fail(RA_ERR_UNSUPPORTED, "k/v token strides must be below 2^24 elements");
    if ((rc = fill(d->q_strides, st->q, Lq, d->Hq, d->d_qk, "q"))) return rc;
    if ((rc = fill(d->o_strides, st->o, Lq, d->Hq, d->d_v, "out"))) return rc;
    // k/v: dense strides depend on each chunk's length; 0 in st->k[0] marks "dense"
    for (int i = 0; i < 3; ++i) st->k[i] = d->k_strides[i], st->v[i] = d->v_strides[i];
    if (!(st->k[0] == 0 && st->k[1] == 0 && st->k[2] == 0)) {
        int64_t tmp[3];
        if ((rc = fill(d->k_strides, tmp, 1, d->Hkv, d->d_qk, "k"))) return rc;
    }
    if (!(st->v[0] == 0 && st->v[1] == 0 && st->v[2] == 0)) {
        int64_t tmp[3];
        if ((rc = fill(d->v_strides, tmp, 1, d->Hkv, d->d_v, "v"))) return rc;
    }
    return RA_OK;
}

bool dense_kv(const int64_t *s) { return s[0] == 0 && s[1] == 0 && s[2] == 0; }

// Segment labels come for the queries and every non-empty chunk, or not at all.
int check_labels(const ra_desc *d, int64_t Lq, const ra_kv_chunk *chunks, int P) {
    // the label scans index keys and query rows with 32-bit integers, and a
    // pass may step up to 2^16 entries past the end before it stops
    const int64_t lim = ((int64_t)1 << 31) - ((int64_t)1 << 16);
    if (d->q_seg && Lq >= lim) return fail(RA_ERR_UNSUPPORTED, "with segment labels Lq must be below 2^31 - 2^16");
    for (int c = 0; c < P && chunks; ++c) {
        if (chunks[c].k_seg && chunks[c].len >= lim)
            return fail(RA_ERR_UNSUPPORTED,
                        "chunk %d: with segment labels a chunk must hold fewer than 2^31 - 2^16 keys", c);
        if (chunks[c].len <= 0) continue;
        const bool has = chunks[c].k_seg != nullptr;
        if (has != (d->q_seg != nullptr))
            return fail(RA_ERR_INVALID_ARG, "chunk %d: segment labels must be given for the queries and every chunk", c);
        if (has && ((uintptr_t)chunks[c].k_seg & 3)) return fail(RA_ERR_INVALID_ARG, "chunk %d: k_seg misaligned", c);
    }
    return RA_OK;
}

// k/v strides of one chunk (dense BSHD when the descriptor gives none)
void chunk_strides(const int64_t *given, int64_t len, int Hkv, int dd, int64_t *out) {
    if (dense_kv(given)) {
        out[2] = dd;
        out[1] = (int64_t)Hkv * dd;
        out[0] = len * Hkv * dd;
    } else {
        out[0] = given[0], out[1] = given[1], out[2] = given[2];
    }
}

// Do the keys start .. start+len-1 hold an anchor (stride S) of a query at
// q_offset .. q_offset+Lq-1?  Block m's anchors are mS - 1, mS and (m+1)S.
bool holds_anchor(int64_t Lq, int64_t q_offset, int64_t S, int64_t start, int64_t len) {
    if (S <= 0 || len <= 0 || Lq <= 0) return false;
    const int64_t m_lo = q_offset / S, m_hi = (q_offset + Lq - 1) / S, end = start + len - 1;
    // some m in [lo, hi] with start <= mS + off <= end (start - off and end - off are >= 0)
    auto any = [&](int64_t lo, int64_t hi, int64_t off) {
        return std::max(lo, (start - off + S - 1) / S) <= std::min(hi, (end - off) / S);
    };
    return any(m_lo, m_hi, -1) || any(m_lo, m_hi + 1, 0);
}

// Chunk class of keys start .. start+len-1 for queries q_offset .. q_offset+Lq-1.
int classify(int64_t Lq, int64_t q_offset, int causal, int64_t window, int64_t anchor, int64_t start, int64_t len) {
    if (len <= 0 || Lq <= 0) return RA_CHUNK_SKIP;
    if (holds_anchor(Lq, q_offset, anchor, start, len)) {
        const int c = classify(Lq, q_offset, causal, window, 0, start, len);
        return c == RA_CHUNK_SKIP ? RA_CHUNK_DIAG : c;
    }
    const int64_t first_q = q_offset, last_q = q_offset + Lq - 1, last_k = start + len - 1;
    const bool win = window > 0;
    // keys any query may see: [first_q - window, last_q (+ window)]
    if (causal && start > last_q) return RA_CHUNK_SKIP;
    if (win && (last_k < first_q - window || (!causal && start > last_q + window))) return RA_CHUNK_SKIP;
    // keys every query sees
    bool full = true;
    if (causal && last_k > first_q) full = false;
    if (win && (start < last_q - window || (!causal && last_k > first_q + window))) full = false;
    return full ? RA_CHUNK_FULL : RA_CHUNK_DIAG;
}

// Launches of the ring schedule: one chunk per launch when staged, else up to
// kMaxChunks chunks that can share one set of k/v strides.
std::vector<std::vector<int>> group_ring_launches(const ra_desc *d, const ra_kv_chunk *chunks,
                                                  const std::vector<int> &steps, bool stage) {
    std::vector<std::vector<int>> launches;
    if (stage) {
        for (int c : steps) launches.push_back({c});
    } else {
        const bool dense = dense_kv(d->k_strides) || dense_kv(d->v_strides);
        std::vector<int> cur;
        for (int c : steps) {
            const bool same = cur.empty() || !dense || chunks[c].len == chunks[cur[0]].len;
            if (cur.size() == (size_t)ra::kMaxChunks || !same) {
                launches.push_back(cur);
                cur.clear();
            }
            cur.push_back(c);
        }
        if (!cur.empty()) launches.push_back(cur);
    }
    if (launches.empty()) launches.push_back({});  // writes the (possibly accumulated) state / zero output
    return launches;
}

// Everything ring_attn_fwd decides before enqueueing work.
struct Plan {
    bool split = false;
    bool stage = false;
    std::vector<int> steps;  // indices of computed chunks, in array order
    int64_t sub_len = 0;     // split: keys per sub-range
    int n_sub_total = 0;     // split: partial slots from chunks
    int n_parts = 0;         // split: slots incl. an accumulated input state
    size_t stage_bytes = 0;  // one staging buffer (K + V)
    size_t state_bytes = 0;  // internal (m, l, O) when the caller keeps none
    size_t part_bytes = 0;
    size_t off_stage[2] = {0, 0}, off_state = 0, off_parts = 0, total = 0;
    int G = 1;
    int64_t rows = 0;  // B * Lq * Hq
};

// Positions of a call: q_offset >= 0, chunks with start, len >= 0, their
// k and v given, and disjoint in position (shared by the forward and the
// backward).
int check_positions(const ra_kv_chunk *chunks, int P, int64_t q_offset) {
    if (P < 0) return fail(RA_ERR_INVALID_ARG, "P must be >= 0");
    if (P > 0 && !chunks) return fail(RA_ERR_INVALID_ARG, "chunks is NULL");
    if (q_offset < 0) return fail(RA_ERR_INVALID_ARG, "q_offset must be >= 0");
    std::vector<std::pair<int64_t, int64_t>> iv;
    for (int c = 0; c < P; ++c) {
        if (chunks[c].len < 0 || chunks[c].start < 0)
            return fail(RA_ERR_INVALID_ARG, "chunk %d: start and len must be >= 0", c);
        if (chunks[c].len > 0 && (!chunks[c].k || !chunks[c].v))
            return fail(RA_ERR_INVALID_ARG, "chunk %d: k or v is NULL", c);
        if (chunks[c].len > 0) iv.push_back({chunks[c].start, chunks[c].start + chunks[c].len});
    }
    std::sort(iv.begin(), iv.end());
    for (size_t i = 1; i < iv.size(); ++i)
        if (iv[i].first < iv[i - 1].second) return fail(RA_ERR_INVALID_ARG, "KV chunks overlap in position");
    return RA_OK;
}

int make_plan(const ra_desc *d, int64_t Lq, const ra_kv_chunk *chunks, int P, int causal, int64_t q_offset,
              uint32_t flags, bool caller_state, Plan *pl) {
    if (flags & ~(RA_FLAG_STAGE | RA_FLAG_SPLIT_KV | RA_FLAG_NO_SPLIT_KV | RA_FLAG_ACCUMULATE))
        return fail(RA_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
    if ((flags & RA_FLAG_SPLIT_KV) && (flags & (RA_FLAG_NO_SPLIT_KV | RA_FLAG_STAGE)))
        return fail(RA_ERR_INVALID_ARG, "SPLIT_KV cannot be combined with NO_SPLIT_KV or STAGE");
    int rc = check_positions(chunks, P, q_offset);
    if (rc) return rc;

    pl->G = d->Hq / d->Hkv;
    pl->rows = (int64_t)d->B * Lq * d->Hq;
    pl->stage = (flags & RA_FLAG_STAGE) != 0;
    pl->split = !pl->stage && !(flags & RA_FLAG_NO_SPLIT_KV) &&
                ((flags & RA_FLAG_SPLIT_KV) || (Lq > 0 && Lq <= kSplitMaxLq) || kv_fp8(d));
    if (kv_fp8(d)) {  // the 8-bit cache is read in place by the split-KV schedule only
        if (!pl->split) return fail(RA_ERR_UNSUPPORTED, "an 8-bit KV cache needs the split-KV schedule (no STAGE / NO_SPLIT_KV)");
        for (int c = 0; c < P; ++c)
            if (chunks[c].len > 0 && (!chunks[c].k_exp || !chunks[c].v_exp))
                return fail(RA_ERR_INVALID_ARG, "chunk %d: an 8-bit KV chunk needs k_exp and v_exp", c);
    }
    for (int c = 0; c < P; ++c)
        if (classify(Lq, q_offset, causal, d->window, d->anchor, chunks[c].start, chunks[c].len) != RA_CHUNK_SKIP)
            pl->steps.push_back(c);

    const int es = elem_size(d->dtype);
    size_t off = 0;
    if (pl->stage) {
        if (!dense_kv(d->k_strides) && !(d->k_strides[1] == (int64_t)d->Hkv * d->d_qk && d->k_strides[2] == d->d_qk))
            return fail(RA_ERR_UNSUPPORTED, "STAGE needs token-dense k chunks");
        if (!dense_kv(d->v_strides) && !(d->v_strides[1] == (int64_t)d->Hkv * d->d_v && d->v_strides[2] == d->d_v))
            return fail(RA_ERR_UNSUPPORTED, "STAGE needs token-dense v chunks");
        int64_t maxlen = 0;
        for (size_t s = 1; s < pl->steps.size(); ++s) maxlen = std::max(maxlen, chunks[pl->steps[s]].len);
        pl->stage_bytes = (size_t)d->B * maxlen * d->Hkv * (size_t)(d->d_qk + d->d_v) * es;
        if (pl->stage_bytes) {
            pl->off_stage[0] = off;
            off += align_up(pl->stage_bytes);
            pl->off_stage[1] = off;
            off += align_up(pl->stage_bytes);
        }
    }
    if (pl->split) {
        // sub-ranges per chunk: enough workgroups to fill the GPU, whole key tiles
        const int bm = row_tile(d, true);
        const int64_t rowtiles = (pl->G * Lq + bm - 1) / bm;
        const int64_t base_wg = (int64_t)d->B * d->Hkv * rowtiles * (int64_t)std::max<size_t>(pl->steps.size(), 1);
        int64_t maxlen = 1;
        for (int c : pl->steps) maxlen = std::max(maxlen, chunks[c].len);
        int64_t n_sub = std::max<int64_t>(1, (kSplitTargetWorkgroups + base_wg - 1) / base_wg);
        int64_t sub_len = (maxlen + n_sub - 1) / n_sub;
        sub_len = std::max<int64_t>(256, (sub_len + 63) / 64 * 64);
        // the 8-bit kernel copies the scale exponents of its key range to LDS
        if (kv_fp8(d)) sub_len = std::min<int64_t>(sub_len, (int64_t)ra::kFp8MaxRangeBlocks * 64 - 256);
        pl->sub_len = sub_len;
        int total = 0;
        for (int c : pl->steps) total += (int)((chunks[c].len + sub_len - 1) / sub_len);
        pl->n_sub_total = total;
        pl->n_parts = total + ((flags & RA_FLAG_ACCUMULATE) ? 1 : 0);
        pl->part_bytes = (size_t)pl->n_parts * pl->rows * (size_t)(d->d_v + 2) * 4;
        pl->off_parts = off;
        off += align_up(pl->part_bytes);
    } else if (!caller_state && group_ring_launches(d, chunks, pl->steps, pl->stage).size() > 1) {
        pl->state_bytes = (size_t)pl->rows * (size_t)(d->d_v + 2) * 4;
        pl->off_state = off;
        off += align_up(pl->state_bytes);
    }
    pl->total = off;
    return RA_OK;
}

FwdArgs base_args(const ra_desc *d, const Strides &st, const void *q, int64_t Lq, int causal, int64_t q_offset,
                  void *out) {
    FwdArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = q;
    a.out = out;
    a.q_sb = st.q[0], a.q_ss = st.q[1], a.q_sh = st.q[2];
    a.o_sb = st.o[0], a.o_ss = st.o[1], a.o_sh = st.o[2];
    a.Lq = Lq;
    a.q_offset = q_offset;
    a.B = d->B, a.Hq = d->Hq, a.Hkv = d->Hkv, a.G = d->Hq / d->Hkv;
    a.causal = causal ? 1 : 0;
    a.window = d->window > 0 ? d->window : 0;
    a.anchor = d->anchor;
    a.q_seg = d->q_seg;
    const float scale = d->scale > 0.f ? d->scale : 1.f / std::sqrt((float)d->d_qk);
    a.scale_log2 = scale * 1.4426950408889634f;
    return a;
}

// Row tiling: prefill keeps each row tile inside one head; decode packs heads.
void set_rows(FwdArgs &a, const ra_desc *d, bool split) {
    const int bm = row_tile(d, split);
    if (split || a.Lq * a.G <= bm) {
        a.Lq_pad = a.Lq;  // packed
    } else {
        a.Lq_pad = (a.Lq + bm - 1) / bm * bm;
    }
    a.n_rowtiles = (int)(((int64_t)a.G * a.Lq_pad + bm - 1) / bm);
}

hipError_t launch_fwd(const FwdArgs &a, const ra_desc *d, bool split, hipStream_t s) {
    if (kv_fp8(d) && split) return ra::launch_fwd_fp8kv(a, s);
    return d->dtype == RA_BF16 ? ra::launch_fwd_bf16(a, d->d_qk, split, s) : ra::launch_fwd_f32(a, d->d_qk, s);
}

void set_chunk_strides(FwdArgs &a, const ra_desc *d, int64_t len) {
    int64_t ks[3], vs[3];
    chunk_strides(d->k_strides, len, d->Hkv, d->d_qk, ks);
    chunk_strides(d->v_strides, len, d->Hkv, d->d_v, vs);
    a.k_sb = ks[0], a.k_ss = ks[1], a.k_sh = ks[2];
    a.v_sb = vs[0], a.v_ss = vs[1], a.v_sh = vs[2];
}

struct DeviceGuard {
    int prev = -1;
    bool ok = true;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        if (prev != dev) ok = hipSetDevice(dev) == hipSuccess;
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

}  // namespace

extern "C" {

const char *ring_attn_version(void) { return "ringattn 0.4 (gfx950)"; }

const char *ring_attn_last_error(void) { return g_err.c_str(); }

int ring_attn_ctx_create(int device, ra_ctx **out) {
    if (!out) return fail(RA_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    int n = 0;
    hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceCount");
    if (device < 0 || device >= n) return fail(RA_ERR_HIP, "device %d does not exist (%d devices)", device, n);
    DeviceGuard guard(device);
    if (!guard.ok) return fail(RA_ERR_HIP, "hipSetDevice(%d) failed", device);
    ra_ctx *c = new ra_ctx();
    c->device = device;
    if ((e = hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking)) != hipSuccess) {
        delete c;
        return hip_fail(e, "hipStreamCreateWithFlags");
    }
    hipEvent_t *evs[] = {&c->start, &c->ready[0], &c->ready[1], &c->freed[0], &c->freed[1], &c->join};
    for (hipEvent_t *ev : evs) {
        if ((e = hipEventCreateWithFlags(ev, hipEventDisableTiming)) != hipSuccess) {
            (void)hipStreamDestroy(c->side);
            delete c;
            return hip_fail(e, "hipEventCreateWithFlags");
        }
    }
    // the static scratch of ring_attn_fwd_noalloc on this device (its failure
    // only disables that entry point, which reports it)
    scratch_lookup(device);
    *out = c;
    return RA_OK;
}

int ring_attn_ctx_set_check(ra_ctx *c, uint32_t checks, uint32_t spin_us) {
    if (!c) return fail(RA_ERR_INVALID_ARG, "ctx is NULL");
    if (checks & ~(uint32_t)(RA_CHECK_DELAY_COPY | RA_CHECK_DELAY_COMPUTE | RA_CHECK_POISON))
        return fail(RA_ERR_INVALID_ARG, "unknown check bits 0x%x", checks);
    if (spin_us > RA_CHECK_MAX_SPIN_US) return fail(RA_ERR_INVALID_ARG, "spin_us above %d", RA_CHECK_MAX_SPIN_US);
    c->check = checks;
    c->check_us = spin_us;
    return RA_OK;
}

int ring_attn_ctx_destroy(ra_ctx *c) {
    if (!c) return RA_OK;
    DeviceGuard guard(c->device);
    (void)hipStreamSynchronize(c->side);
    hipEvent_t evs[] = {c->start, c->ready[0], c->ready[1], c->freed[0], c->freed[1], c->join};
    for (hipEvent_t ev : evs) (void)hipEventDestroy(ev);
    (void)hipStreamDestroy(c->side);
    delete c;
    return RA_OK;
}

int ring_attn_ring_order(int device_index, int P, int32_t *order) {
    if (P < 1 || !order || device_index < 0 || device_index >= P)
        return fail(RA_ERR_INVALID_ARG, "need 0 <= device_index < P and an order array");
    for (int s = 0; s < P; ++s) order[s] = ((device_index - s) % P + P) % P;
    return RA_OK;
}

int ring_attn_plan(int64_t Lq, int64_t q_offset, int causal, int64_t window, int64_t anchor, int P,
                   const int64_t *starts, const int64_t *lens, int32_t *cls) {
    if (P < 0 || Lq < 0 || q_offset < 0 || anchor < 0) return fail(RA_ERR_INVALID_ARG, "negative argument");
    if (P > 0 && (!starts || !lens || !cls)) return fail(RA_ERR_INVALID_ARG, "NULL array");
    for (int c = 0; c < P; ++c) {
        if (starts[c] < 0 || lens[c] < 0) return fail(RA_ERR_INVALID_ARG, "chunk %d: negative start/len", c);
        cls[c] = classify(Lq, q_offset, causal, window, anchor, starts[c], lens[c]);
    }
    return RA_OK;
}

int ring_attn_workspace_size(const ra_desc *d, int64_t Lq, const ra_kv_chunk *chunks, int P, int causal,
                             int64_t q_offset, uint32_t flags, int want_state, size_t *bytes) {
    if (!bytes) return fail(RA_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = 0;
    Strides st;
    int rc = check_desc(d, Lq, &st);
    if (rc) return rc;
    // pointers are not needed for sizing: check positions only
    std::vector<ra_kv_chunk> cc(chunks, chunks + (P > 0 && chunks ? P : 0));
    for (auto &c : cc)
        if (c.len > 0) c.k = c.v = (const void *)1;
    Plan pl;
    if ((rc = make_plan(d, Lq, cc.data(), P, causal, q_offset, flags, want_state != 0, &pl))) return rc;
    *bytes = pl.total;
    return RA_OK;
}

}  // extern "C"

// The forward of ring_attn_fwd and ring_attn_fwd_noalloc: validation, the
// plan, then the launches, with `workspace` as scratch.  Enqueues nothing
// on error and allocates nothing.
static int fwd_impl(ra_ctx *ctx, const ra_desc *d, const void *q, int64_t Lq, const ra_kv_chunk *chunks, int P,
                    int causal, int64_t q_offset, uint32_t flags, void *out, float *m_out, float *l_out,
                    float *O_out, void *workspace, size_t ws_bytes, void *stream, bool noalloc) {
    if (!ctx) return fail(RA_ERR_INVALID_ARG, "ctx is NULL");
    Strides st;
    int rc = check_desc(d, Lq, &st);
    if (rc) return rc;
    if (Lq == 0) return RA_OK;  // nothing to compute or write
    const bool have_state = m_out || l_out || O_out;
    if (have_state && !(m_out && l_out && O_out))
        return fail(RA_ERR_INVALID_ARG, "m_out, l_out and O_out must be given together");
    if (!out && !have_state) return fail(RA_ERR_INVALID_ARG, "nothing to write: out and state are NULL");
    if ((flags & RA_FLAG_ACCUMULATE) && !have_state)
        return fail(RA_ERR_INVALID_ARG, "ACCUMULATE needs the state buffers");
    if (Lq > 0 && !q) return fail(RA_ERR_INVALID_ARG, "q is NULL");
    auto misaligned = [](const void *p) { return ((uintptr_t)p & 15) != 0; };
    if ((q && misaligned(q)) || (out && misaligned(out)) || (O_out && misaligned(O_out)))
        return fail(RA_ERR_INVALID_ARG, "q, out and O must be 16-byte aligned");
    for (int c = 0; c < P && chunks; ++c)
        if (chunks[c].len > 0 && (misaligned(chunks[c].k) || misaligned(chunks[c].v)))
            return fail(RA_ERR_INVALID_ARG, "chunk %d: k/v must be 16-byte aligned", c);
    if ((rc = check_labels(d, Lq, chunks, P))) return rc;
    Plan pl;
    if ((rc = make_plan(d, Lq, chunks, P, causal, q_offset, flags, have_state, &pl))) return rc;
    if (noalloc && pl.total > ws_bytes)
        return fail(RA_ERR_WORKSPACE,
                    "these arguments need %zu bytes of scratch; the static scratch of ring_attn_fwd_noalloc "
                    "holds %zu (use ring_attn_fwd with a workspace)", pl.total, ws_bytes);
    if (pl.total > 0 && (!workspace || ws_bytes < pl.total))
        return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", pl.total, ws_bytes);
    if (pl.total > 0 && ((uintptr_t)workspace % kAlign) != 0)
        return fail(RA_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
    // the merge writes the output densely (checked before anything is enqueued)
    if (pl.split && out && !(st.o[2] == d->d_v && st.o[1] == (int64_t)d->Hq * d->d_v && st.o[0] == Lq * d->Hq * d->d_v))
        return fail(RA_ERR_UNSUPPORTED, "split-KV needs a dense output");

    DeviceGuard guard(ctx->device);
    if (!guard.ok) return fail(RA_ERR_HIP, "hipSetDevice(%d) failed", ctx->device);
    hipStream_t s = (hipStream_t)stream;
    char *ws = (char *)workspace;
    hipError_t e;
    FwdArgs a = base_args(d, st, q, Lq, causal, q_offset, out);
    const bool accumulate = (flags & RA_FLAG_ACCUMULATE) != 0;

    // ------------------------------------------------------------ split-KV ----
    if (pl.split) {
        set_rows(a, d, true);
        a.split_mode = 1;
        a.sub_len = pl.sub_len;
        float *pm = (float *)(ws + pl.off_parts);
        float *pl_ = pm + (size_t)pl.n_parts * pl.rows;
        float *pO = pl_ + (size_t)pl.n_parts * pl.rows;
        a.pm = pm, a.pl = pl_, a.pO = pO;
        int slot = accumulate ? 1 : 0;
        if (accumulate) {  // the incoming state joins the merge as one more part
            if ((e = hipMemcpyAsync(pm, m_out, pl.rows * 4, hipMemcpyDeviceToDevice, s)) != hipSuccess ||
                (e = hipMemcpyAsync(pl_, l_out, pl.rows * 4, hipMemcpyDeviceToDevice, s)) != hipSuccess ||
                (e = hipMemcpyAsync(pO, O_out, pl.rows * d->d_v * 4, hipMemcpyDeviceToDevice, s)) != hipSuccess)
                return hip_fail(e, "copy of the incoming state");
        }
        // launches of up to kMaxChunks chunks with a common sub-range count
        size_t i = 0;
        while (i < pl.steps.size()) {
            // group chunks with the same dense strides and sub-range count
            const int64_t len0 = chunks[pl.steps[i]].len;
            const int nsub0 = (int)((len0 + pl.sub_len - 1) / pl.sub_len);
            size_t j = i;
            a.n_chunks = 0;
            while (j < pl.steps.size() && a.n_chunks < ra::kMaxChunks) {
                const ra_kv_chunk &ch = chunks[pl.steps[j]];
                const int nsub = (int)((ch.len + pl.sub_len - 1) / pl.sub_len);
                if (nsub != nsub0) break;
                if (dense_kv(d->k_strides) || dense_kv(d->v_strides))
                    if (ch.len != len0) break;  // dense strides depend on the length
                a.chunks[a.n_chunks++] = ChunkArg{ch.k, ch.v, ch.start, ch.len, ch.k_exp, ch.v_exp, ch.k_seg};
                ++j;
            }
            set_chunk_strides(a, d, len0);
            a.n_sub = nsub0;
            a.part_base = slot;
            if ((e = launch_fwd(a, d, true, s)) != hipSuccess) return hip_fail(e, "split-KV launch");
            slot += a.n_chunks * nsub0;
            i = j;
        }
        if (slot == 0) {
            // nothing visible and nothing accumulated: an empty state
            FwdArgs z = a;
            z.split_mode = 0;
            z.n_chunks = 0;
            z.m = m_out, z.l = l_out, z.O = O_out;
            z.store_state = have_state;
            z.store_out = out != nullptr;
            set_rows(z, d, false);
            if ((e = launch_fwd(z, d, false, s)) != hipSuccess) return hip_fail(e, "empty-state launch");
            return RA_OK;
        }
        MergeArgs mg;
        mg.pm = pm, mg.pl = pl_, mg.pO = pO;
        mg.m = m_out, mg.l = l_out, mg.O = O_out;
        mg.out = out;
        mg.rows = pl.rows;
        mg.n_parts = slot;
        mg.d_v = d->d_v;
        mg.out_bf16 = d->dtype == RA_BF16;
        if ((e = ra::launch_merge(mg, s)) != hipSuccess) return hip_fail(e, "merge launch");
        return RA_OK;
    }

    // ------------------------------------------------------------ ring --------
    set_rows(a, d, false);
    float *sm = m_out, *sl = l_out, *sO = O_out;
    if (!have_state && pl.state_bytes) {
        sm = (float *)(ws + pl.off_state);
        sl = sm + pl.rows;
        sO = sl + pl.rows;
    }
    a.m = sm, a.l = sl, a.O = sO;

    const std::vector<std::vector<int>> launches = group_ring_launches(d, chunks, pl.steps, pl.stage);
    const int nl = (int)launches.size();
    const int es = elem_size(d->dtype);
    auto stage_copy = [&](int step) -> hipError_t {
        // copy the chunk of launch `step` into staging buffer step % 2 on the side stream
        const ra_kv_chunk &ch = chunks[launches[step][0]];
        char *dst = ws + pl.off_stage[step & 1];
        if (ctx->check & RA_CHECK_DELAY_COPY) {
            const hipError_t r = ra::launch_spin(ctx->check_us, ctx->side);
            if (r != hipSuccess) return r;
        }
        int64_t ks[3], vs[3];
        chunk_strides(d->k_strides, ch.len, d->Hkv, d->d_qk, ks);
        chunk_strides(d->v_strides, ch.len, d->Hkv, d->d_v, vs);
        const size_t krow = (size_t)ch.len * d->Hkv * d->d_qk * es;
        const size_t vrow = (size_t)ch.len * d->Hkv * d->d_v * es;
        // one linear copy per tensor when its batches are contiguous, else a
        // strided (2D) copy of B rows
        auto copy = [&](char *to, const void *from, size_t row, int64_t stride) -> hipError_t {
            if ((size_t)stride * es == row || d->B == 1)
                return hipMemcpyAsync(to, from, (size_t)d->B * row, hipMemcpyDeviceToDevice, ctx->side);
            return hipMemcpy2DAsync(to, row, from, (size_t)stride * es, row, d->B, hipMemcpyDeviceToDevice,
                                    ctx->side);
        };
        hipError_t r = copy(dst, ch.k, krow, ks[0]);
        if (r != hipSuccess) return r;
        r = copy(dst + (size_t)d->B * krow, ch.v, vrow, vs[0]);
        if (r != hipSuccess) return r;
        return hipEventRecord(ctx->ready[step & 1], ctx->side);
    };

    if (pl.stage && nl > 1) {
        if ((e = hipEventRecord(ctx->start, s)) != hipSuccess) return hip_fail(e, "event record");
        if ((e = hipStreamWaitEvent(ctx->side, ctx->start, 0)) != hipSuccess) return hip_fail(e, "side wait");
        if ((e = stage_copy(1)) != hipSuccess) return hip_fail(e, "staging copy");
    }
    for (int li = 0; li < nl; ++li) {
        const std::vector<int> &L = launches[li];
        const bool staged = pl.stage && li > 0;
        if (pl.stage && li + 1 < nl && li >= 1) {
            // refill the buffer of step li-1 (now li+1) once step li-1 is done;
            // step 0 reads its chunk in place, so at li = 1 the buffer is unused
            // (and its event was not recorded by this call: waiting on it would
            // tie the side stream to earlier work, which graph capture rejects)
            if (li >= 2 && (e = hipStreamWaitEvent(ctx->side, ctx->freed[(li + 1) & 1], 0)) != hipSuccess)
                return hip_fail(e, "side wait");
            if ((e = stage_copy(li + 1)) != hipSuccess) return hip_fail(e, "staging copy");
        }
        a.n_chunks = (int)L.size();
        for (int i = 0; i < a.n_chunks; ++i) {
            const ra_kv_chunk &ch = chunks[L[i]];
            if (staged) {
                const char *base = ws + pl.off_stage[li & 1];
                const size_t kbytes = (size_t)d->B * ch.len * d->Hkv * d->d_qk * es;
                a.chunks[i] = ChunkArg{base, base + kbytes, ch.start, ch.len, nullptr, nullptr, ch.k_seg};
            } else {
                a.chunks[i] = ChunkArg{ch.k, ch.v, ch.start, ch.len, nullptr, nullptr, ch.k_seg};
            }
        }
        if (staged) {
            // staged copies are dense BSHD
            const int64_t len = chunks[L[0]].len;
            a.k_sb = len * d->Hkv * d->d_qk, a.k_ss = (int64_t)d->Hkv * d->d_qk, a.k_sh = d->d_qk;
            a.v_sb = len * d->Hkv * d->d_v, a.v_ss = (int64_t)d->Hkv * d->d_v, a.v_sh = d->d_v;
            if ((e = hipStreamWaitEvent(s, ctx->ready[li & 1], 0)) != hipSuccess) return hip_fail(e, "wait");
        } else {
            set_chunk_strides(a, d, L.empty() ? 0 : chunks[L[0]].len);
        }
        a.load_state = li > 0 || accumulate;
        a.store_state = li + 1 < nl || have_state;
        a.store_out = li + 1 == nl && out != nullptr;
        if ((a.load_state || a.store_state) && !a.m)
            return fail(RA_ERR_WORKSPACE, "internal state buffer missing");
        if ((ctx->check & RA_CHECK_DELAY_COMPUTE) && (e = ra::launch_spin(ctx->check_us, s)) != hipSuccess)
            return hip_fail(e, "check spin");
        if ((e = launch_fwd(a, d, false, s)) != hipSuccess) return hip_fail(e, "forward launch");
        // the step is done with its staging buffer: poison it before it may be refilled
        if (staged && (ctx->check & RA_CHECK_POISON) &&
            (e = ra::launch_fill_nan(ws + pl.off_stage[li & 1], pl.stage_bytes, s)) != hipSuccess)
            return hip_fail(e, "check fill");
        if (staged && li + 2 < nl)
            if ((e = hipEventRecord(ctx->freed[li & 1], s)) != hipSuccess) return hip_fail(e, "event record");
    }
    if (pl.stage && nl > 1) {
        if ((e = hipEventRecord(ctx->join, ctx->side)) != hipSuccess) return hip_fail(e, "event record");
        if ((e = hipStreamWaitEvent(s, ctx->join, 0)) != hipSuccess) return hip_fail(e, "join");
    }
    return RA_OK;
}

extern "C" {

int ring_attn_fwd(ra_ctx *ctx, const ra_desc *d, const void *q, int64_t Lq, const ra_kv_chunk *chunks, int P,
                  int causal, int64_t q_offset, uint32_t flags, void *out, float *m_out, float *l_out, float *O_out,
                  void *workspace, size_t ws_bytes, void *stream) {
    return fwd_impl(ctx, d, q, Lq, chunks, P, causal, q_offset, flags, out, m_out, l_out, O_out, workspace,
                    ws_bytes, stream, false);
}

int ring_attn_fwd_noalloc(ra_ctx *ctx, const ra_desc *d, const void *q, int64_t Lq, const ra_kv_chunk *chunks,
                          int P, int causal, int64_t q_offset, uint32_t flags, void *out, float *m_out,
                          float *l_out, float *O_out, void *stream) {
    if (!ctx) return fail(RA_ERR_INVALID_ARG, "ctx is NULL");
    if (ctx->device < 0 || ctx->device >= kMaxScratchDevices)
        return fail(RA_ERR_UNSUPPORTED, "the static scratch covers devices 0..%d", kMaxScratchDevices - 1);
    const ScratchSlot &sl = g_scratch[ctx->device];
    if (!sl.ptr)
        return fail(RA_ERR_HIP, "static scratch of device %d unavailable: %s", ctx->device,
                    hipGetErrorString(sl.err));
    return fwd_impl(ctx, d, q, Lq, chunks, P, causal, q_offset, flags, out, m_out, l_out, O_out, sl.ptr,
                    (size_t)RA_NOALLOC_SCRATCH_BYTES, stream, true);
}

// Row statistics of the backward: (lse2, D) per (b, h, t).
static size_t bwd_ld_bytes(const ra_desc *d, int64_t Lq) { return align_up((size_t)d->B * d->Hq * Lq * 8); }

static int check_bwd(const ra_desc *d, int64_t Lq, Strides *st) {
    int rc = check_desc(d, Lq, st);
    if (rc) return rc;
    if (d->dtype != RA_BF16 || (d->d_qk != 64 && d->d_qk != 128 && d->d_qk != 512))
        return fail(RA_ERR_UNSUPPORTED, "the backward is built for bf16 with d_qk = d_v in {64, 128, 512}");
    if (kv_fp8(d)) return fail(RA_ERR_UNSUPPORTED, "the backward takes bf16 keys and values");
    // 32-row tiles of q and dout are addressed with 32-bit offsets from a 64-bit base
    if (st->q[1] >= ((int64_t)1 << 24) || st->o[1] >= ((int64_t)1 << 24))
        return fail(RA_ERR_UNSUPPORTED, "q/out token strides must be below 2^24 elements");
    return RA_OK;
}

int ring_attn_bwd_workspace_size(const ra_desc *d, int64_t Lq, size_t *bytes) {
    if (!bytes) return fail(RA_ERR_INVALID_ARG, "bytes is NULL");
    Strides st;
    int rc = check_bwd(d, Lq, &st);
    if (rc) return rc;
    *bytes = bwd_ld_bytes(d, Lq);
    return RA_OK;
}

int ring_attn_bwd(ra_ctx *ctx, const ra_desc *d, const void *q, int64_t Lq, const ra_kv_chunk *chunks, int P,
                  int causal, int64_t q_offset, uint32_t flags, const void *out, const void *dout, const float *m,
                  const float *l, float *dq, const ra_kv_grad *grads, void *workspace, size_t ws_bytes,
                  void *stream) {
    if (!ctx) return fail(RA_ERR_INVALID_ARG, "ctx is NULL");
    Strides st;
    int rc = check_bwd(d, Lq, &st);
    if (rc) return rc;
    if (P < 0 || P > ra::kMaxChunks) return fail(RA_ERR_INVALID_ARG, "P must be in 0..%d", ra::kMaxChunks);
    if (P > 0 && (!chunks || !grads)) return fail(RA_ERR_INVALID_ARG, "chunks and grads must be given");
    if ((flags & ~RA_FLAG_ACCUMULATE) != 0) return fail(RA_ERR_INVALID_ARG, "the backward takes only ACCUMULATE");
    if ((rc = check_positions(chunks, P, q_offset))) return rc;
    if (P > 0 && (rc = check_labels(d, Lq, chunks, P))) return rc;
    const bool accumulate = (flags & RA_FLAG_ACCUMULATE) != 0;
    auto misaligned = [](const void *p) { return ((uintptr_t)p & 15) != 0; };
    for (int c = 0; c < P; ++c) {
        if (chunks[c].len == 0) continue;
        if (!chunks[c].k || !chunks[c].v || !grads[c].dk || !grads[c].dv)
            return fail(RA_ERR_INVALID_ARG, "chunk %d: k, v, dk and dv must be given", c);
        if (misaligned(chunks[c].k) || misaligned(chunks[c].v) || misaligned(grads[c].dk) ||
            misaligned(grads[c].dv))
            return fail(RA_ERR_INVALID_ARG, "chunk %d: k, v, dk and dv must be 16-byte aligned", c);
    }
    if (Lq > 0) {
        if (!q || !out || !dout || !m || !l || !dq)
            return fail(RA_ERR_INVALID_ARG, "q, out, dout, m, l and dq must be given");
        if (misaligned(q) || misaligned(out) || misaligned(dout) || misaligned(dq))
            return fail(RA_ERR_INVALID_ARG, "q, out, dout and dq must be 16-byte aligned");
    }
    const size_t need = Lq > 0 ? bwd_ld_bytes(d, Lq) : 0;
    if (need > 0 && (!workspace || ws_bytes < need))
        return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
    if (need > 0 && ((uintptr_t)workspace % kAlign) != 0)
        return fail(RA_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);

    DeviceGuard guard(ctx->device);
    if (!guard.ok) return fail(RA_ERR_HIP, "hipSetDevice(%d) failed", ctx->device);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    BwdArgs A;
    std::memset(&A, 0, sizeof A);
    A.f = base_args(d, st, q, Lq, causal, q_offset, nullptr);
    A.out = out, A.dout = dout, A.m = m, A.l = l;
    A.ld = (float *)workspace;
    A.dq = dq;
    A.scale = d->scale > 0.f ? d->scale : 1.f / std::sqrt((float)d->d_qk);
    const int bm = ra::bwd_dq_row_tile(d->d_qk);
    A.f.Lq_pad = A.f.Lq * A.f.G <= bm ? A.f.Lq : (A.f.Lq + bm - 1) / bm * bm;
    A.f.n_rowtiles = (int)(((int64_t)A.f.G * A.f.Lq_pad + bm - 1) / bm);

    if (Lq > 0) {
        if ((e = ra::launch_bwd_pre(A, d->d_qk, s)) != hipSuccess) return hip_fail(e, "backward row statistics");
        // dQ: chunks that share k/v strides go in one launch; later launches add
        std::vector<int> steps;
        for (int c = 0; c < P; ++c)
            if (classify(Lq, q_offset, causal, d->window, d->anchor, chunks[c].start, chunks[c].len) != RA_CHUNK_SKIP)
                steps.push_back(c);
        std::vector<std::vector<int>> launches = group_ring_launches(d, chunks, steps, false);
        bool first = true;
        for (const std::vector<int> &grp : launches) {
            A.accumulate = accumulate || !first;
            A.f.n_chunks = (int)grp.size();
            for (size_t i = 0; i < grp.size(); ++i) {
                const ra_kv_chunk &c = chunks[grp[i]];
                A.f.chunks[i] = ChunkArg{c.k, c.v, c.start, c.len, nullptr, nullptr, c.k_seg};
            }
            if (!grp.empty()) set_chunk_strides(A.f, d, chunks[grp[0]].len);
            // with no chunk to walk, the launch writes dQ = 0 (or leaves the sum)
            if ((e = ra::launch_bwd_dq(A, d->d_qk, s)) != hipSuccess) return hip_fail(e, "backward dQ launch");
            first = false;
        }
    }
    // dK, dV of every chunk (zero, or unchanged when accumulating, where no row sees it)
    A.accumulate = accumulate;
    A.f.n_chunks = 1;
    A.chunk = 0;
    for (int c = 0; c < P; ++c) {
        if (chunks[c].len == 0) continue;
        A.f.chunks[0] =
            ChunkArg{chunks[c].k, chunks[c].v, chunks[c].start, chunks[c].len, nullptr, nullptr, chunks[c].k_seg};
        set_chunk_strides(A.f, d, chunks[c].len);
        A.dk = grads[c].dk, A.dv = grads[c].dv;
        if ((e = ra::launch_bwd_dkdv(A, d->d_qk, s)) != hipSuccess) return hip_fail(e, "backward dK/dV launch");
    }
    return RA_OK;
}

int ring_attn_merge(int n_parts, int64_t rows, int d_v, const float *m_parts, const float *l_parts,
                    const float *O_parts, float *m, float *l, float *O, void *out, int out_dtype, void *stream) {
    if (n_parts < 1 || rows < 0 || d_v < 4 || d_v % 4 != 0)
        return fail(RA_ERR_INVALID_ARG, "need n_parts >= 1, rows >= 0 and d_v a positive multiple of 4");
    if (rows > 0 && (!m_parts || !l_parts || !O_parts)) return fail(RA_ERR_INVALID_ARG, "partials are NULL");
    const bool st = m || l || O;
    if (st && !(m && l && O)) return fail(RA_ERR_INVALID_ARG, "m, l and O must be given together");
    if (!st && !out) return fail(RA_ERR_INVALID_ARG, "nothing to write");
    if (out_dtype != RA_F32 && out_dtype != RA_BF16) return fail(RA_ERR_INVALID_ARG, "out_dtype unknown");
    if (((uintptr_t)O_parts & 15) || ((uintptr_t)O & 15) || ((uintptr_t)out & 7))
        return fail(RA_ERR_INVALID_ARG, "O buffers must be 16-byte aligned, out 8-byte aligned");
    if (rows == 0) return RA_OK;
    MergeArgs a;
    a.pm = m_parts, a.pl = l_parts, a.pO = O_parts;
    a.m = m, a.l = l, a.O = O;
    a.out = out;
    a.rows = rows;
    a.n_parts = n_parts;
    a.d_v = d_v;
    a.out_bf16 = out_dtype == RA_BF16;
    hipError_t e = ra::launch_merge(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
    return RA_OK;
}

}  // extern "C"
