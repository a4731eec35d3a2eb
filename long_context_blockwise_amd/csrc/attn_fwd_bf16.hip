// attn_fwd_bf16.hip - blockwise attention of a resident query chunk against
// KV chunks, bf16 inputs, fp32 accumulation, on CDNA4 (gfx950) MFMA.
//
// One workgroup owns a tile of query rows and walks the keys of its chunks in
// tiles of BN keys, keeping the running softmax state of each row (running
// max m, denominator l, unnormalised output O) in registers: the per-chunk
// blockwise ("flash") attention of page "Ring Attention：百万 Token 上下文的秘密",
// §3.1 Flash Ring Attention, with the query block resident and K/V tiles
// staged in on-chip memory (LDS here).  The state after a chunk is exactly
// what the next ring step continues from (§2.3 数学正确性 of the same page).
//
// Data movement.  K and V tiles go from HBM straight into LDS with
// buffer_load ... lds (no registers, no VALU); the buffer descriptor covers
// only the valid keys, so a ragged tail is zero-filled by the hardware.  Both
// tiles stay row-major ([key][d]) with the 16-byte units of row r stored at
// unit ^ swz(r), which makes the two read patterns below bank-conflict free.
// Tiles are double buffered: tile t+1 is requested before tile t is computed.
//
// Matrix cores.  Scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_bf16: keys are M (A operand, ds_read_b128 from LDS),
// the wave's 32 query rows are N (B operand, registers for the whole launch).
// In the 32x32 result lane l owns query row l%32 and 16 of the 32 keys (the
// rest sit in lane l^32), so each per-row softmax step is lane-local plus one
// exchange with the partner lane.  The probabilities in that layout are
// already the B operand of O^T = V^T P^T; the V^T A operand is read from the
// row-major V tile with ds_read_b64_tr_b16 (4x4 transposes within each 16
// lanes), in the key order the result layout dictates.
//
// Online softmax (base 2): with c = scale*log2(e), p = exp2(s*c - m_ref).  The
// reference m_ref only moves when a tile maximum exceeds it by more than 8
// (a factor 256), so the O/l rescale is rare; p <= 256 is harmless in fp32 and
// bf16, and the result is identical in exact arithmetic.  The true running
// max is tracked alongside and the state is renormalised to it at the end, so
// the exported m is the running maximum.
#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;
// The softmax reference moves when a tile max exceeds it by more than this
// (log2 units): p = exp2(s*c - m_ref) <= 2^8.
constexpr float kRescaleThreshold = 8.0f;
// gfx9 buffer descriptor word 3 for raw (untyped) dword access
constexpr int kBufferFlags = 0x00020000;

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Maximum of x over lanes l and l^32 (the two lanes that share a query row).
// (v_permlane32_swap with both operands equal is folded by the compiler to a
// single result, losing the other half, so the exchange uses ds_bpermute.)
__device__ inline float max_pair(float x) { return fmaxf(x, __shfl_xor(x, 32)); }

// Workgroup ids are handed to the 8 XCDs round robin; renumber them so that
// each XCD runs a contiguous range of logical tiles (tiles that share K/V then
// share that XCD's L2).
__device__ inline int xcd_remap(int bid, int n) {
    const int q = n >> 3, r = n & 7;
    const int x = bid & 7, s = bid >> 3;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + s;
}

// Swizzle of the 16-byte units of LDS row r (key r of a tile): unit u is
// stored at u ^ swz(r).  Eight consecutive rows read at one unit (K fragment
// reads) land on 8 distinct units, and the 4 rows x 2 units of one transposed
// V read do too.
__device__ inline int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

__device__ inline bf16x8 to_bf16x8(const u32x4 &u) { return __builtin_bit_cast(bf16x8, u); }

__device__ inline unsigned pack_bf16(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

__device__ inline bf16x8 lds_read_b128(const char *smem, int byte) {
    return *reinterpret_cast<const bf16x8 *>(smem + byte);
}

// Two transposed 4-key reads make one V^T A-operand fragment.
__device__ inline bf16x8 lds_read_vt(const char *smem, int byte0, int byte1) {
    const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(smem + byte0));
    const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(smem + byte1));
    const s16x8 xy = __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, xy);
}

template <int D, int BN, int NW, int KSPLIT>
struct Cfg {
    static constexpr int NT = NW * 64;           // threads
    static constexpr int ROWW = NW / KSPLIT;     // waves along rows
    static constexpr int BM = 32 * ROWW;         // query rows per workgroup
    static constexpr int KW = BN / KSPLIT;       // keys per wave per tile
    static constexpr int KB = KW / 32;           // 32-key blocks per wave
    static constexpr int DS = D / 16;            // reduction steps of S^T
    static constexpr int DB = D / 32;            // 32-wide blocks of O^T
    static constexpr int ROWB = D * 2;           // bytes per K/V row in LDS
    static constexpr int UPR = D / 8;            // 16-byte units per row
    static constexpr int TILE = BN * ROWB;       // bytes of one K (or V) tile
    static constexpr int BUF = 2 * TILE;         // K + V
    static constexpr int LDS = 2 * BUF;          // double buffered
    static constexpr int LOADS = TILE / 1024;    // 1 KiB wave loads per K (or V) tile
    static constexpr int LOADS_PER_WAVE = LOADS / NW;
    static_assert(KW % 32 == 0, "each wave needs whole 32-key blocks");
    static_assert(D % 64 == 0, "head size must be a multiple of 64");
    static_assert(LOADS % NW == 0, "tile loads must split evenly over the waves");
    static_assert(KSPLIT == 1 || (KSPLIT - 1) * ROWW * 64 * (16 * DB + 2) * 4 <= LDS,
                  "merge scratch must fit in LDS");
};

template <int D, int BN, int NW, int KSPLIT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1, D <= 128 ? 2 : 1)))
void fwd_bf16_kernel(const FwdArgs a) {
    using C = Cfg<D, BN, NW, KSPLIT>;
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int wr = w % C::ROWW, wk = w / C::ROWW;
    const int l32 = lane & 31, g = lane >> 5;

    // ---- which tile of which (batch, KV head, key range) -------------------
    const int nsplit = a.split_mode ? a.n_chunks * a.n_sub : 1;
    int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int rt = lid % a.n_rowtiles;
    lid /= a.n_rowtiles;
    const int split = lid % nsplit;
    lid /= nsplit;
    const int hk = lid % a.Hkv;
    const int b = lid / a.Hkv;

    const int64_t Lq = a.Lq, Lq_pad = a.Lq_pad;
    const int64_t prow_end = (int64_t)a.G * Lq_pad;
    int64_t p0;
    if (Lq_pad % C::BM == 0) {  // one head per tile; heaviest (latest) rows first
        const int64_t ntt = Lq_pad / C::BM;
        const int gq = rt % a.G;
        const int64_t tt = ntt - 1 - rt / a.G;
        p0 = gq * Lq_pad + tt * C::BM;
    } else {
        p0 = (int64_t)rt * C::BM;
    }

    // token range (for causal skipping) of a run of packed rows
    auto t_range = [&](int64_t pa, int64_t pb, int64_t &lo, int64_t &hi) {
        pb = pb < prow_end ? pb : prow_end;
        --pb;
        if (pa / Lq_pad == pb / Lq_pad) {
            lo = pa % Lq_pad;
            hi = pb % Lq_pad;
            hi = hi < Lq - 1 ? hi : Lq - 1;
        } else {
            lo = 0;
            hi = Lq - 1;
        }
    };
    int64_t wg_tlo, wg_thi, wv_tlo, wv_thi;
    t_range(p0, p0 + C::BM, wg_tlo, wg_thi);
    t_range(p0 + 32 * wr, p0 + 32 * wr + 32, wv_tlo, wv_thi);

    // this lane's query row
    const int64_t prow = p0 + 32 * wr + l32;
    const int gq = (int)(prow / Lq_pad);
    const int64_t t = prow % Lq_pad;
    const bool row_ok = prow < prow_end && t < Lq;
    const int h = hk * a.G + gq;
    const int64_t qpos = a.q_offset + t;

    // ---- resident query fragments (B operand of S^T = K Q^T) ---------------
    bf16x8 qf[C::DS];
    {
        const uint16_t *qp = (const uint16_t *)a.q + b * a.q_sb + t * a.q_ss + h * a.q_sh + 8 * g;
#pragma unroll
        for (int ds = 0; ds < C::DS; ++ds) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row_ok) v = *(const u32x4 *)(qp + 16 * ds);
            qf[ds] = to_bf16x8(v);
        }
    }

    // ---- running state --------------------------------------------------------
    f32x16 oacc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    float m_run = kNegInf, m_true = kNegInf, lsum = 0.f;
    const int64_t srow = ((int64_t)b * Lq + t) * a.Hq + h;  // state row index
    if (a.load_state && row_ok && wk == 0) {
        const float m0 = a.m[srow];
        m_run = m_true = m0 * kLog2e;
        lsum = g == 0 ? a.l[srow] : 0.f;
        const float *op = a.O + srow * D + 4 * g;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const f32x4 v = *(const f32x4 *)(op + 32 * db + 8 * i4);
#pragma unroll
                for (int j = 0; j < 4; ++j) oacc[db][4 * i4 + j] = v[j];
            }
    }
    const float c2 = a.scale_log2;

    // ---- per-lane LDS addresses (bytes, buffer 0) ------------------------------
    // K fragment (kb, ds): row wk*KW + 32kb + l32, unit 2ds+g -> stored at
    // (2ds+g) ^ swz(l32&7); for ds = 4a + x that is 8a + ((2x+g) ^ sw).
    int kaddr[4];
    {
        const int sw = swz(l32 & 7);
        const int rowb = (wk * C::KW + l32) * C::ROWB;
#pragma unroll
        for (int x = 0; x < 4; ++x) kaddr[x] = rowb + (((2 * x + g) ^ sw) << 4);
    }
    // V^T fragment (ks, db): lane = 16*G + 4k + q provides V[key][d] with
    // key = wk*KW + 16ks + 4(G>>1) + 8hh + k and d = 32db + 16(G&1) + 4q.
    int vaddr[2];
    {
        const int G = lane >> 4, k = (lane >> 2) & 3, q = lane & 3;
        const int gi = G & 1, gk = G >> 1;
        const int s = 2 * k + gk;  // swz of the row (row & 7 == 4gk + k)
        const int c = 2 * gi + (q >> 1);
        const int f = s >> 2;
        const int A = (wk * C::KW + 4 * gk + k) * C::ROWB + ((c ^ (s & 3)) << 4) + ((q & 1) << 3);
        vaddr[0] = A + 64 * f;        // even d-blocks: + 128 * (db / 2)
        vaddr[1] = A + 64 * (1 - f);  // odd d-blocks
    }

    // ---- K/V tile loads: HBM -> LDS, no registers --------------------------------
    auto load_tile = [&](const uint16_t *kbase, const uint16_t *vbase, int64_t k0, int64_t kend, int buf) {
        const int nvalid = (int)(kend - k0 < BN ? kend - k0 : BN);
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(kbase + k0 * a.k_ss), (short)0, (int)(nvalid * a.k_ss * 2), kBufferFlags);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(vbase + k0 * a.v_ss), (short)0, (int)(nvalid * a.v_ss * 2), kBufferFlags);
        char *kt = smem + buf * C::BUF;
        char *vt = kt + C::TILE;
#pragma unroll
        for (int j = 0; j < C::LOADS_PER_WAVE; ++j) {
            const int inst = j * NW + w;
            const int pos = inst * 64 + lane;
            const int r = pos / C::UPR, u = (pos % C::UPR) ^ swz(r);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)(kt + inst * 1024), 16,
                                                     (unsigned)(r * a.k_ss * 2 + u * 16), 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(vt + inst * 1024), 16,
                                                     (unsigned)(r * a.v_ss * 2 + u * 16), 0, 0, 0);
        }
    };
    auto wait_tile = [&]() {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };

    // ---- one KV tile for this wave ----------------------------------------------
    auto compute_tile = [&](int buf, int64_t k0, int64_t kend, int64_t cstart, bool masked) {
        const char *kt = smem + buf * C::BUF;
        const char *vt = kt + C::TILE;
        f32x16 sacc[C::KB];
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
        for (int ds = 0; ds < C::DS; ++ds)
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb) {
                const bf16x8 kf = lds_read_b128(kt, kaddr[ds & 3] + 128 * (ds >> 2) + 32 * kb * C::ROWB);
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ds], sacc[kb], 0, 0, 0);
            }
        if (masked) {
            // key index of element i: 8*(i/4) + 4*g + i%4 within its 32-key block
            const int64_t klim = a.causal ? qpos - cstart : (int64_t)1 << 62;
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int64_t key = k0 + wk * C::KW + 32 * kb + 8 * (i >> 2) + 4 * g + (i & 3);
                    if (key >= kend || key > klim) sacc[kb][i] = kNegInf;
                }
        }
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
        mx = max_pair(mx);
        const float mt = mx * c2;
        m_true = fmaxf(m_true, mt);
        const bool need = mt > m_run + kRescaleThreshold;
        if (__builtin_amdgcn_ballot_w64(need)) {
            const float alpha = need ? exp2_fast(m_run - mt) : 1.f;
            m_run = need ? mt : m_run;
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        }
        const float mref = m_run == kNegInf ? 0.f : m_run;
        bf16x8 pf[2 * C::KB];
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                u32x4 pk;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float e0 = exp2_fast(__builtin_fmaf(sacc[kb][8 * hh + 2 * j], c2, -mref));
                    const float e1 = exp2_fast(__builtin_fmaf(sacc[kb][8 * hh + 2 * j + 1], c2, -mref));
                    lsum += e0 + e1;
                    pk[j] = pack_bf16(e0, e1);
                }
                pf[2 * kb + hh] = to_bf16x8(pk);
            }
#pragma unroll
        for (int ks = 0; ks < 2 * C::KB; ++ks)
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
                const int base = vaddr[db & 1] + 128 * (db >> 1) + 16 * ks * C::ROWB;
                const bf16x8 vf = lds_read_vt(vt, base, base + 8 * C::ROWB);
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], oacc[db], 0, 0, 0);
            }
    };

    // ---- walk the chunks --------------------------------------------------------
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
        if (a.causal) {
            const int64_t vis = a.q_offset + wg_thi - ch.start + 1;  // keys < vis can be visible
            kstop = vis < kstop ? vis : kstop;
        }
        if (kstop <= kbeg) continue;  // uniform across the workgroup
        const int ntiles = (int)((kstop - kbeg + BN - 1) / BN);
        const uint16_t *kbase = (const uint16_t *)ch.k + b * a.k_sb + hk * a.k_sh;
        const uint16_t *vbase = (const uint16_t *)ch.v + b * a.v_sb + hk * a.v_sh;

        __syncthreads();  // the previous chunk's last tile is no longer read
        load_tile(kbase, vbase, kbeg, kend, 0);
        wait_tile();
        for (int it = 0; it < ntiles; ++it) {
            const int64_t k0 = kbeg + (int64_t)it * BN;
            if (it + 1 < ntiles) load_tile(kbase, vbase, k0 + BN, kend, (it + 1) & 1);
            // this wave's keys k0 + wk*KW .. + KW-1
            const int64_t wk0 = k0 + wk * C::KW;
            const bool skip = a.causal && ch.start + wk0 > a.q_offset + wv_thi;
            const bool full = wk0 + C::KW <= kend &&
                              (!a.causal || ch.start + wk0 + C::KW - 1 <= a.q_offset + wv_tlo);
            if (!skip) compute_tile(it & 1, k0, kend, ch.start, !full);
            wait_tile();
        }
    }

    // ---- epilogue: combine key-split waves, renormalise, write ------------------
    if (m_true != kNegInf) {
        const float alpha = exp2_fast(m_run - m_true);
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }
    if constexpr (KSPLIT > 1) {
        // waves wk > 0 hand their (m, l, O) to wave wk == 0 of the same rows
        __syncthreads();
        float *scr = reinterpret_cast<float *>(smem);
        constexpr int STRIDE = 16 * C::DB + 2;
        if (wk > 0) {
            float *p = scr + ((wr * (KSPLIT - 1) + (wk - 1)) * STRIDE) * 64 + lane;
            p[0] = m_true;
            p[64] = lsum;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) p[(2 + 16 * db + i) * 64] = oacc[db][i];
        }
        __syncthreads();
        if (wk == 0) {
#pragma unroll 1
            for (int o = 0; o < KSPLIT - 1; ++o) {
                const float *p = scr + ((wr * (KSPLIT - 1) + o) * STRIDE) * 64 + lane;
                const float m1 = p[0], l1 = p[64];
                const float mn = fmaxf(m_true, m1);
                if (mn == kNegInf) continue;
                const float a0 = m_true == kNegInf ? 0.f : exp2_fast(m_true - mn);
                const float a1 = m1 == kNegInf ? 0.f : exp2_fast(m1 - mn);
                lsum = a0 * lsum + a1 * l1;
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        oacc[db][i] = a0 * oacc[db][i] + a1 * p[(2 + 16 * db + i) * 64];
                m_true = mn;
            }
        }
        if (wk > 0) return;
    }
    const float ltot = lsum + __shfl_xor(lsum, 32);
    if (!row_ok) return;

    if (a.split_mode || a.store_state) {
        const int64_t slot_rows = (int64_t)a.B * Lq * a.Hq;
        float *mp = a.split_mode ? a.pm + (a.part_base + split) * slot_rows : a.m;
        float *lp = a.split_mode ? a.pl + (a.part_base + split) * slot_rows : a.l;
        float *Op = a.split_mode ? a.pO + (a.part_base + split) * slot_rows * D : a.O;
        if (g == 0) {
            mp[srow] = m_true == kNegInf ? kNegInf : m_true * kLn2;
            lp[srow] = ltot;
        }
        float *op = Op + srow * D + 4 * g;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                f32x4 v;
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = oacc[db][4 * i4 + j];
                *(f32x4 *)(op + 32 * db + 8 * i4) = v;
            }
    }
    if (!a.split_mode && a.store_out) {
        const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
        uint16_t *op = (uint16_t *)a.out + b * a.o_sb + t * a.o_ss + h * a.o_sh + 4 * g;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                u32x2 v;
                v[0] = pack_bf16(oacc[db][4 * i4] * inv, oacc[db][4 * i4 + 1] * inv);
                v[1] = pack_bf16(oacc[db][4 * i4 + 2] * inv, oacc[db][4 * i4 + 3] * inv);
                *(u32x2 *)(op + 32 * db + 8 * i4) = v;
            }
    }
}

template <int D, int BN, int NW, int KSPLIT>
hipError_t launch(const FwdArgs &a, hipStream_t s) {
    using C = Cfg<D, BN, NW, KSPLIT>;
    const int nsplit = a.split_mode ? a.n_chunks * a.n_sub : 1;
    const int64_t grid = (int64_t)a.B * a.Hkv * nsplit * a.n_rowtiles;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, BN, NW, KSPLIT>), dim3((unsigned)grid), dim3(C::NT), 0, s, a);
    return hipGetLastError();
}

}  // namespace

// Tile shapes per head size: (keys per tile, waves, key split of a tile).
// Prefill: 4 waves x 32 rows = 128 rows per workgroup.  Split (decode): the
// 64 packed rows of a KV head's query group, two waves per 32 rows, each
// taking half of every key tile.
int fwd_bf16_row_tile(int d, bool split_mode) {
    if (d == 64) return Cfg<64, 64, 4, 1>::BM;
    if (d == 128) return split_mode ? Cfg<128, 64, 4, 2>::BM : Cfg<128, 64, 4, 1>::BM;
    if (d == 512) return Cfg<512, 32, 4, 1>::BM;
    return 0;
}

hipError_t launch_fwd_bf16(const FwdArgs &a, int d, bool split_mode, hipStream_t s) {
    switch (d) {
    case 64: return launch<64, 64, 4, 1>(a, s);
    case 128: return split_mode ? launch<128, 64, 4, 2>(a, s) : launch<128, 64, 4, 1>(a, s);
    case 512: return launch<512, 32, 4, 1>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ra
