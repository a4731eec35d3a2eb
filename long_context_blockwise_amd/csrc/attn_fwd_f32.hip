// attn_fwd_f32.hip - the same blockwise ring-step attention for fp32 inputs,
// computed with true fp32 products and sums on the vector ALUs (no reduced
// precision anywhere, for callers that need fp32 accuracy).
//
// Each query row is owned by 16 consecutive threads: TPR = d/64 threads per
// 64-wide slice of d times KS = 16/TPR key groups.  A thread holds 64 of the
// row's query and output elements in registers and takes 32/KS of the keys of
// every tile, with a running softmax state of its own; the key groups of a
// row (lanes of one wave) merge their states at the end with lane shuffles.
// K/V tiles of 32 keys are staged in LDS and read by all threads.  The running
// softmax state follows the same online update as the bf16 path (page "Ring
// Attention：百万 Token 上下文的秘密", §3.1 Flash Ring Attention: blockwise
// attention per received KV chunk; §2.3: the state after all chunks equals
// plain attention), in base 2 with an exact rescale on every new maximum.
#include "ra_internal.h"

namespace ra {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;
constexpr int kThreads = 256;
constexpr int kKeys = 32;     // keys per LDS tile
constexpr int kRowLanes = 16;  // threads per query row

template <int D>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(const FwdArgs a) {
    constexpr int TPR = D / 64;               // threads per 64-wide slice set of a row
    constexpr int KS = kRowLanes / TPR;       // key groups per row
    constexpr int kSub = kKeys / KS;          // keys of a tile per thread
    constexpr int RB = kThreads / kRowLanes;  // rows per workgroup
    __shared__ __attribute__((aligned(16))) float Ks[kKeys][D];
    __shared__ __attribute__((aligned(16))) float Vs[kKeys][D];
    __shared__ int Ls[kKeys];  // segment labels of the tile's keys (0 without labels)

    const int tid = threadIdx.x;
    const int part = tid % TPR;               // which 64-wide slice of d
    const int kg = (tid / TPR) % KS;          // which keys of each tile
    const int nsplit = a.split_mode ? a.n_chunks * a.n_sub : 1;
    int lid = blockIdx.x;
    const int rt = lid % a.n_rowtiles;
    lid /= a.n_rowtiles;
    const int split = lid % nsplit;
    lid /= nsplit;
    const int hk = lid % a.Hkv;
    const int b = lid / a.Hkv;

    const int64_t Lq = a.Lq, Lq_pad = a.Lq_pad;
    const int64_t prow = (int64_t)rt * RB + tid / kRowLanes;
    const int gq = (int)(prow / Lq_pad);
    const int64_t t = prow % Lq_pad;
    const bool row_ok = gq < a.G && t < Lq;
    const int h = hk * a.G + gq;
    const int64_t qpos = a.q_offset + t;
    // first and last query positions among this workgroup's rows (for skipping keys)
    int64_t pos_lo, pos_hi;
    {
        const int64_t pa = (int64_t)rt * RB;
        int64_t pb = pa + RB;
        const int64_t pend = (int64_t)a.G * Lq_pad;
        pb = (pb < pend ? pb : pend) - 1;
        int64_t thi = (pa / Lq_pad == pb / Lq_pad) ? pb % Lq_pad : Lq - 1;
        thi = thi < Lq - 1 ? thi : Lq - 1;
        pos_hi = a.q_offset + thi;
        pos_lo = a.q_offset + ((pa / Lq_pad == pb / Lq_pad) ? pa % Lq_pad : 0);
    }

    float q[64], o[64];
    const float *qp = (const float *)a.q + b * a.q_sb + t * a.q_ss + h * a.q_sh + 64 * part;
#pragma unroll
    for (int e = 0; e < 64; e += 4) {
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (row_ok) v = *(const f32x4 *)(qp + e);
        q[e] = v[0], q[e + 1] = v[1], q[e + 2] = v[2], q[e + 3] = v[3];
        o[e] = o[e + 1] = o[e + 2] = o[e + 3] = 0.f;
    }
    float m = kNegInf, l = 0.f;
    const int64_t srow = ((int64_t)b * Lq + t) * a.Hq + h;
    if (a.load_state && row_ok && kg == 0) {  // one key group carries the prior state
        m = a.m[srow] * kLog2e;
        l = a.l[srow];
        const float *op = a.O + srow * D + 64 * part;
#pragma unroll
        for (int e = 0; e < 64; ++e) o[e] = op[e];
    }
    const float c2 = a.scale_log2;
    const int ql = a.q_seg && row_ok ? a.q_seg[(int64_t)b * Lq + t] : 0;
    const int64_t anc = a.anchor > 0 ? qpos / a.anchor * a.anchor : 0;  // the row's anchor block

    int c_begin = 0, c_end = a.n_chunks, sub = 0;
    if (a.split_mode) {
        c_begin = split / a.n_sub;
        sub = split % a.n_sub;
        c_end = c_begin + 1;
    }
    for (int c = c_begin; c < c_end; ++c) {
        const ChunkArg ch = a.chunks[c];
        int64_t kbeg = 0, kend = ch.len;
        if (a.split_mode) {
            kbeg = sub * a.sub_len;
            kend = kbeg + a.sub_len < ch.len ? kbeg + a.sub_len : ch.len;
        }
        int64_t kstop = kend;
        if (a.causal || a.window > 0) {
            const int64_t vis = pos_hi - ch.start + 1 + (a.causal ? 0 : a.window);
            kstop = vis < kstop ? vis : kstop;
        }
        if (a.window > 0 && a.anchor <= 0) {  // start at the tile of the first key the first row may see
            const int64_t lo = pos_lo - a.window - ch.start;
            if (lo > kbeg) kbeg += (lo - kbeg) / kKeys * kKeys;
        }
        if (a.anchor > 0) kstop = kend;  // anchors may lie anywhere: walk every key
        const float *kbase = (const float *)ch.k + b * a.k_sb + hk * a.k_sh;
        const float *vbase = (const float *)ch.v + b * a.v_sb + hk * a.v_sh;
        for (int64_t k0 = kbeg; k0 < kstop; k0 += kKeys) {
            __syncthreads();
            for (int u = tid; u < kKeys * D / 4; u += kThreads) {
                const int row = u / (D / 4), col = (u % (D / 4)) * 4;
                f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
                if (k0 + row < kend) {
                    kv = *(const f32x4 *)(kbase + (k0 + row) * a.k_ss + col);
                    vv = *(const f32x4 *)(vbase + (k0 + row) * a.v_ss + col);
                }
                *(f32x4 *)&Ks[row][col] = kv;
                *(f32x4 *)&Vs[row][col] = vv;
            }
            if (tid < kKeys)
                Ls[tid] = ch.kseg && k0 + tid < kend ? ch.kseg[(int64_t)b * ch.len + k0 + tid] : 0;
            __syncthreads();
            {
                const int j0 = kg * kSub;
                float s[kSub];
                float smax = kNegInf;
#pragma unroll
                for (int j = 0; j < kSub; ++j) {
                    float acc = 0.f;
#pragma unroll
                    for (int e = 0; e < 64; ++e) acc = __builtin_fmaf(q[e], Ks[j0 + j][64 * part + e], acc);
                    if constexpr (TPR > 1) {
#pragma unroll
                        for (int x = 1; x < TPR; x <<= 1) acc += __shfl_xor(acc, x);
                    }
                    const int64_t key = k0 + j0 + j;
                    const int64_t kpos = ch.start + key;
                    const bool anchor = a.anchor > 0 && (kpos == anc - 1 || kpos == anc || kpos == anc + a.anchor);
                    const bool vis = key < kend && Ls[j0 + j] == ql &&
                                     (anchor || ((!a.causal || kpos <= qpos) &&
                                                 (a.window <= 0 || (kpos >= qpos - a.window &&
                                                                    (a.causal || kpos <= qpos + a.window)))));
                    s[j] = vis ? acc * c2 : kNegInf;
                    smax = fmaxf(smax, s[j]);
                }
                if (smax == kNegInf) continue;  // nothing visible in these keys (skips to the next tile)
                const float mn = fmaxf(m, smax);
                const float alpha = m == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m - mn);
                l *= alpha;
#pragma unroll
                for (int e = 0; e < 64; ++e) o[e] *= alpha;
#pragma unroll
                for (int j = 0; j < kSub; ++j) {
                    const float p = __builtin_amdgcn_exp2f(s[j] - mn);
                    l += p;
#pragma unroll
                    for (int e = 0; e < 64; ++e) o[e] = __builtin_fmaf(p, Vs[j0 + j][64 * part + e], o[e]);
                }
                m = mn;
            }
        }
    }

    // merge the key groups' states: lanes tid ^ (TPR << i) hold the same
    // row and slice with other keys
#pragma unroll
    for (int x = TPR; x < kRowLanes; x <<= 1) {
        const float m2 = __shfl_xor(m, x), l2 = __shfl_xor(l, x);
        const float mn = fmaxf(m, m2);
        const float a1 = m == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m - mn);
        const float a2 = m2 == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m2 - mn);
        l = a1 * l + a2 * l2;
#pragma unroll
        for (int e = 0; e < 64; ++e) o[e] = a1 * o[e] + a2 * __shfl_xor(o[e], x);
        m = mn;
    }
    if (!row_ok || kg != 0) return;
    if (a.split_mode || a.store_state) {
        const int64_t slot_rows = (int64_t)a.B * Lq * a.Hq;
        float *mp = a.split_mode ? a.pm + (a.part_base + split) * slot_rows : a.m;
        float *lp = a.split_mode ? a.pl + (a.part_base + split) * slot_rows : a.l;
        float *Op = a.split_mode ? a.pO + (a.part_base + split) * slot_rows * D : a.O;
        if (part == 0) {
            mp[srow] = m == kNegInf ? kNegInf : m * kLn2;
            lp[srow] = l;
        }
        float *op = Op + srow * D + 64 * part;
#pragma unroll
        for (int e = 0; e < 64; e += 4) *(f32x4 *)(op + e) = f32x4{o[e], o[e + 1], o[e + 2], o[e + 3]};
    }
    if (!a.split_mode && a.store_out) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        float *op = (float *)a.out + b * a.o_sb + t * a.o_ss + h * a.o_sh + 64 * part;
#pragma unroll
        for (int e = 0; e < 64; e += 4)
            *(f32x4 *)(op + e) = f32x4{o[e] * inv, o[e + 1] * inv, o[e + 2] * inv, o[e + 3] * inv};
    }
}

template <int D>
hipError_t launch(const FwdArgs &a, hipStream_t s) {
    const int nsplit = a.split_mode ? a.n_chunks * a.n_sub : 1;
    const int64_t grid = (int64_t)a.B * a.Hkv * nsplit * a.n_rowtiles;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(fwd_f32_kernel<D>, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

int fwd_f32_row_tile(int d) { return d == 64 || d == 128 ? kThreads / kRowLanes : 0; }

hipError_t launch_fwd_f32(const FwdArgs &a, int d, hipStream_t s) {
    switch (d) {
    case 64: return launch<64>(a, s);
    case 128: return launch<128>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ra
