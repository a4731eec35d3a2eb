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
// Tile buffers are separate LDS arrays, each named statically where it is
// used, so the compiler can tell reads of one buffer from the in-flight loads
// into another and does not stall the reads on them.
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
//
// Scheduling.  Tile t+1 is requested (HBM -> LDS) before tile t is computed;
// two workgroups share a CU, so while one wave of a SIMD turns scores into
// probabilities the other can feed the matrix cores.  Within a wave the
// probabilities of keys 16(k+1) .. 16(k+1)+15 are computed between the O^T
// MFMAs of keys 16k .. 16k+15, so the wave's own VALU work overlaps them.  For split-KV decoding
// KSPLIT waves share each row block, each over its part of every key tile,
// and merge their states through LDS at the end.
#include "tile_common.h"

// Tuning knobs (compile-time) of the d=128 query-chunk kernel: key tile and
// stage count.
#ifndef RA_TUNE_BN128
#define RA_TUNE_BN128 64
#endif
#ifndef RA_TUNE_NS
#define RA_TUNE_NS 2
#endif
// Interleave the probabilities of the next 16 keys with the O^T MFMAs of the
// current 16 (1), or compute all probabilities before the MFMAs (0); and the
// VALU instructions placed after each MFMA when interleaving.
#ifndef RA_TUNE_FUSE
#define RA_TUNE_FUSE 1
#endif
#ifndef RA_TUNE_FUSE_VALU
#define RA_TUNE_FUSE_VALU 7
#endif
// Scores of the d <= 128 kernel come out of the MFMAs already in log2 units
// and relative to the softmax reference (queries pre-scaled, the reference
// folded into the accumulator's start), so p = exp2(s) (1), or p = exp2(s*c -
// m_ref) with one FMA per score (0).
#ifndef RA_TUNE_BIAS
#define RA_TUNE_BIAS 1
#endif
// keep the bias block live across tiles (a splat the compiler would rebuild
// with 15 moves per tile)
#ifndef RA_TUNE_KEEPREF
#define RA_TUNE_KEEPREF 1
#endif
#ifndef RA_TUNE_BIASPIN
#define RA_TUNE_BIASPIN 1
#endif


namespace ra {
namespace {

// Starting state: empty, or (m, l, O) from the caller, for output dimensions
// dv0 .. dv0 + 32*NDB - 1 of rows with d_v = DV.  O^T element i of block db in
// lane l is d = dv0 + 32db + 8(i/4) + 4g + i%4; lane pairs split l.
template <int DV, int NDB>
__device__ inline void load_state(const FwdArgs &a, const LaneRow &r, int g, bool owner, int dv0,
                                  f32x16 (&o)[NDB], float &m_run, float &m_true, float &lsum) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
    m_run = m_true = kNegInf;
    lsum = 0.f;
    if (!(a.load_state && r.ok && owner)) return;
    m_run = m_true = a.m[r.srow] * kLog2e;
    lsum = g == 0 ? a.l[r.srow] : 0.f;
    const float *op = a.O + r.srow * DV + dv0 + 4 * g;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const f32x4 v = *(const f32x4 *)(op + 32 * db + 8 * i4);
#pragma unroll
            for (int j = 0; j < 4; ++j) o[db][4 * i4 + j] = v[j];
        }
}

// New tile maximum: update the true max, and move the reference (rescaling O
// and l) when the tile max exceeds it by more than the threshold.
template <class C, int NDB>
__device__ inline void update_max(const f32x16 (&s)[C::KB], float c2, float &m_run, float &m_true, float &lsum,
                                  f32x16 (&o)[NDB]) {
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = max_pair(mx);
    const float mt = mx * c2;
    m_true = fmaxf(m_true, mt);
    const bool need = mt > m_run + kRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(need)) {
        const float alpha = need ? exp2_fast(m_run - mt) : 1.f;
        m_run = need ? mt : m_run;
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    }
}

// update_max for an O accumulator the matrix cores keep in AGPRs: the rare
// rescale multiplies each register where it lives (read, multiply, write
// back), so the compiler has no reason to keep a VGPR copy of O across the
// loop.  VALU instructions cannot read AGPRs directly, hence the asm.  The
// s_nops keep the gfx950 wait states between the last MFMA write of O and the
// first read here, and between the last write here and the next MFMA that
// reads O; both are far apart in the kernel already.
template <class C, int NDB>
__device__ inline void update_max_agpr(const f32x16 (&s)[C::KB], float c2, float &m_run, float &m_true, float &lsum,
                                       f32x16 (&o)[NDB]) {
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = max_pair(mx);
    const float mt = mx * c2;
    m_true = fmaxf(m_true, mt);
    const bool need = mt > m_run + kRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(need)) {
        const float alpha = need ? exp2_fast(m_run - mt) : 1.f;
        m_run = need ? mt : m_run;
        lsum *= alpha;
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float x = o[db][i], t;
                asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                             : "+a"(x), "=&v"(t)
                             : "v"(alpha));
                o[db][i] = x;
            }
        asm volatile("s_nop 7" ::: "memory");
    }
}

// p = exp2(s*c - m_ref) as bf16 B operands of O^T += V^T P^T; adds the fp32 p to lsum.
template <class C>
__device__ inline void probabilities(const f32x16 (&s)[C::KB], float c2, float m_run, float &lsum,
                                     bf16x8 (&pf)[2 * C::KB]) {
    const float mref = m_run == kNegInf ? 0.f : m_run;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            u32x4 pk;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float e0 = exp2_fast(__builtin_fmaf(s[kb][8 * hh + 2 * j], c2, -mref));
                const float e1 = exp2_fast(__builtin_fmaf(s[kb][8 * hh + 2 * j + 1], c2, -mref));
                lsum += e0 + e1;
                pk[j] = pack_bf16(e0, e1);
            }
            pf[2 * kb + hh] = to_bf16x8(pk);
        }
}

// Waves raise their issue priority while they feed the matrix cores.
__device__ inline void prio_mfma() {
    if constexpr (RA_TUNE_SETPRIO) __builtin_amdgcn_s_setprio(1);
}
__device__ inline void prio_valu() {
    if constexpr (RA_TUNE_SETPRIO) __builtin_amdgcn_s_setprio(0);
}

// Probabilities of reduction step ks (16 keys) as one bf16 B operand of
// O^T += V^T P^T; adds the fp32 p to lsum.
template <class C>
__device__ inline bf16x8 prob_step(const f32x16 (&s)[C::KB], int ks, float c2, float mref, float &lsum) {
    const int kb = ks / 2, hh = ks % 2;
    u32x4 pk;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float e0 = exp2_fast(__builtin_fmaf(s[kb][8 * hh + 2 * j], c2, -mref));
        const float e1 = exp2_fast(__builtin_fmaf(s[kb][8 * hh + 2 * j + 1], c2, -mref));
        lsum += e0 + e1;
        pk[j] = pack_bf16(e0, e1);
    }
    return to_bf16x8(pk);
}

// probabilities + accumulate_pv with the VALU work of step ks+1 placed
// between the MFMAs of step ks: the matrix cores run an MFMA while the same
// wave issues the exponentials of the next step, so one wave keeps both
// pipes busy instead of alternating between them.
template <class C, int NDB>
__device__ inline void softmax_pv(const f32x16 (&s)[C::KB], float c2, float m_run, float &lsum, const char *vt,
                                  const int (&vaddr)[2][C::NVD], f32x16 (&o)[NDB]) {
    const float mref = m_run == kNegInf ? 0.f : m_run;
    constexpr int NK = 2 * C::KB;
    bf16x8 fr[2][NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) fr[0][db] = vfrag<C>(vt, vaddr, 0, db);
    bf16x8 p = prob_step<C>(s, 0, c2, mref, lsum);
    __builtin_amdgcn_sched_barrier(0);
    prio_mfma();
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
        if (ks + 1 < NK) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) fr[(ks + 1) & 1][db] = vfrag<C>(vt, vaddr, ks + 1, db);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] = mfma(fr[ks & 1][db], p, o[db]);
        if (ks + 1 < NK) {
            p = prob_step<C>(s, ks + 1, c2, mref, lsum);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
                __builtin_amdgcn_sched_group_barrier(0x002, RA_TUNE_FUSE_VALU, 0);  // VALU
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    prio_valu();
}

// Final state of a lane's row: renormalise to the true max, then write the
// state (or a split partial) and/or the normalised output.
template <int NDB>
__device__ inline void renormalise(float m_run, float m_true, float &lsum, f32x16 (&o)[NDB]) {
    if (m_true == kNegInf) return;
    const float alpha = exp2_fast(m_run - m_true);
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
}

// ---------------------------------------------------------------------------
// Biased scores.  The queries are multiplied by c = scale*log2(e) once, when
// they are loaded (rounded to bf16: a relative change below 2^-9 per
// element), and every score chain of a tile starts from the accumulator
// value -m_ref instead of 0, so the MFMAs deliver s = c q.k - m_ref and the
// probability is exp2(s) with no vector work per score beyond the exp.  The
// reference starts at 0 and moves only when a tile maximum exceeds it by more
// than the threshold (up) or the running maximum falls more than 64 below it
// (down, so that probabilities keep their precision); the true maximum is
// tracked as before and the state is renormalised to it at the end.
// ---------------------------------------------------------------------------
constexpr float kRefFloor = 64.f;  // log2 units below the reference that move it down

template <int NDS>
__device__ inline void load_q_scaled(const FwdArgs &a, const WorkTile &wt, const LaneRow &r, int g, int d0, float c,
                                     bf16x8 (&qf)[NDS]) {
    load_q(a, wt, r, g, d0, qf);
    scale_q(qf, c);
}

// Starting state for biased scores: a loaded state keeps its maximum as the
// reference, so O is first read by the first P V product, which hides its
// load behind the first tile's scores (RA_TUNE_KEEPREF 0: the reference is 0
// unless the loaded maximum lies outside [-kRefFloor, threshold] (log2
// units), and a loaded O and l are rescaled to it).  No state: reference 0.
template <int DV, int NDB>
__device__ inline void load_state_biased(const FwdArgs &a, const LaneRow &r, int g, bool owner, int dv0,
                                         f32x16 (&o)[NDB], float &m_run, float &m_true, float &lsum) {
    load_state<DV, NDB>(a, r, g, owner, dv0, o, m_run, m_true, lsum);
    if (m_true == kNegInf) {
        m_run = 0.f;
        return;
    }
    // keep the loaded maximum as reference (always with RA_TUNE_KEEPREF: O is
    // then first touched by the first P V product, which hides its load)
    if (RA_TUNE_KEEPREF || m_true < -kRefFloor || m_true > kRescaleThreshold) return;
    const float alpha = exp2_fast(m_true);
    m_run = 0.f;
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
}

template <class C>
__device__ inline f32x16 bias_block(float m_run) {
    f32x16 b;
#pragma unroll
    for (int i = 0; i < 16; ++i) b[i] = -m_run;
    return b;
}

// update_max for biased scores: the tile maximum is max(s) + m_ref.  When
// the reference moves, O and l are rescaled, this tile's scores shifted and
// the bias block rebuilt.
template <class C, int NDB>
__device__ inline void update_max_biased(f32x16 (&s)[C::KB], float &m_run, float &m_true, float &lsum,
                                         f32x16 (&o)[NDB], f32x16 &bias) {
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = max_pair(mx);
    const float mt = mx + m_run;
    m_true = fmaxf(m_true, mt);
    const bool up = mt > m_run + kRescaleThreshold;
    const bool down = m_true != kNegInf && m_true < m_run - kRefFloor;
    if (__builtin_amdgcn_ballot_w64(up || down)) {
        const float ref = up ? mt : (down ? m_true : m_run);
        const float alpha = exp2_fast(m_run - ref);
        const float shift = ref - m_run;
        m_run = ref;
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kb][i] -= shift;
        bias = bias_block<C>(m_run);
    }
}

// prob_step / softmax_pv / probabilities for biased scores: p = exp2(s).
template <class C>
__device__ inline bf16x8 prob_step_biased(const f32x16 (&s)[C::KB], int ks, float &lsum) {
    const int kb = ks / 2, hh = ks % 2;
    u32x4 pk;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float e0 = exp2_fast(s[kb][8 * hh + 2 * j]);
        const float e1 = exp2_fast(s[kb][8 * hh + 2 * j + 1]);
        lsum += e0 + e1;
        pk[j] = pack_bf16(e0, e1);
    }
    return to_bf16x8(pk);
}

template <class C, int NDB>
__device__ inline void softmax_pv_biased(const f32x16 (&s)[C::KB], float &lsum, const char *vt,
                                         const int (&vaddr)[2][C::NVD], f32x16 (&o)[NDB]) {
    constexpr int NK = 2 * C::KB;
    bf16x8 fr[2][NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) fr[0][db] = vfrag<C>(vt, vaddr, 0, db);
    bf16x8 p = prob_step_biased<C>(s, 0, lsum);
    __builtin_amdgcn_sched_barrier(0);
    prio_mfma();
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
        if (ks + 1 < NK) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) fr[(ks + 1) & 1][db] = vfrag<C>(vt, vaddr, ks + 1, db);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] = mfma(fr[ks & 1][db], p, o[db]);
        if (ks + 1 < NK) {
            p = prob_step_biased<C>(s, ks + 1, lsum);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
                __builtin_amdgcn_sched_group_barrier(0x002, RA_TUNE_FUSE_VALU, 0);  // VALU
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    prio_valu();
}

template <class C>
__device__ inline void probabilities_biased(const f32x16 (&s)[C::KB], float &lsum, bf16x8 (&pf)[2 * C::KB]) {
#pragma unroll
    for (int ks = 0; ks < 2 * C::KB; ++ks) pf[ks] = prob_step_biased<C>(s, ks, lsum);
}

// Final (or partial) results of output dimensions dv0 .. dv0 + 32*NDB - 1 of
// rows with d_v = DV: the state (or a split partial) and/or the normalised
// output; m and l are written by the lanes with write_ml.
template <int DV, int NDB>
__device__ inline void write_results(const FwdArgs &a, const WorkTile &wt, const LaneRow &r, int g, int dv0,
                                     bool write_ml, const f32x16 (&o)[NDB], float m_true, float ltot) {
    if (!r.ok) return;
    if (a.split_mode || a.store_state) {
        const int64_t slot_rows = (int64_t)a.B * a.Lq * a.Hq;
        float *mp = a.split_mode ? a.pm + (a.part_base + wt.split) * slot_rows : a.m;
        float *lp = a.split_mode ? a.pl + (a.part_base + wt.split) * slot_rows : a.l;
        float *Op = a.split_mode ? a.pO + (a.part_base + wt.split) * slot_rows * DV : a.O;
        if (g == 0 && write_ml) {
            mp[r.srow] = m_true == kNegInf ? kNegInf : m_true * kLn2;
            lp[r.srow] = ltot;
        }
        float *op = Op + r.srow * DV + dv0 + 4 * g;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                f32x4 v;
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = o[db][4 * i4 + j];
                *(f32x4 *)(op + 32 * db + 8 * i4) = v;
            }
    }
    if (!a.split_mode && a.store_out) {
        const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
        uint16_t *op = (uint16_t *)a.out + wt.b * a.o_sb + r.t * a.o_ss + r.h * a.o_sh + dv0 + 4 * g;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                u32x2 v;
                v[0] = pack_bf16(o[db][4 * i4] * inv, o[db][4 * i4 + 1] * inv);
                v[1] = pack_bf16(o[db][4 * i4 + 2] * inv, o[db][4 * i4 + 3] * inv);
                *(u32x2 *)(op + 32 * db + 8 * i4) = v;
            }
    }
}

// ---------------------------------------------------------------------------
// The attention kernel: one tile at a time (query-chunk prefill and split-KV decoding)
// ---------------------------------------------------------------------------
// EXT instantiations add anchor tokens (EXT bit 1) and segment labels
// (EXT bit 2): up to five extra tiles hold anchors outside the window's range,
// and with labels each stage also holds 64 key labels per wave (after the K
// tile).
template <int D, int BN, int NW, int KSPLIT, int NS, int EXT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(const FwdArgs a) {
    using C = Cfg<D, BN, NW, KSPLIT>;
    constexpr bool ANC = (EXT & 1) != 0, LAB = (EXT & 2) != 0;
    constexpr int LPT = 2 * C::LOADS_PER_WAVE + (LAB ? 1 : 0);
    constexpr int LABB = LAB ? NW * 256 : 0;  // bytes of key labels per stage
    RA_STAGE_ARRAYS(NS, C::TILE + LABB)
    static_assert(!LAB || C::KW <= 64, "a wave's labels are 64 dwords");
    // merge scratch of the key-split waves: slot s spans tile buffers 2s, 2s+1
    static_assert(KSPLIT == 1 || (C::ROWW * (KSPLIT - 1) <= 2 && (16 * C::DB + 2) * 64 * 4 <= 2 * C::TILE),
                  "merge scratch must fit in the tile buffers");

    const int lane = threadIdx.x & 63, w = wave_index();
    const int wr = w % C::ROWW, wk = w / C::ROWW;
    const int l32 = lane & 31, g = lane >> 5;
    const WorkTile wt = work_tile<C>(a);
    int64_t wv_tlo, wv_thi;
    token_range(a, wt.p0 + 32 * wr, wt.p0 + 32 * wr + 32, wv_tlo, wv_thi);
    const LaneRow row = lane_row(a, wt, wt.p0 + 32 * wr + l32);

    // With labels a workgroup may find no visible key in any chunk of the
    // launch (packed documents): the queries and the state are then read only
    // when the first chunk with tiles comes (live), and an untouched state
    // that stays in place is not written back.  (With anchors alone the early
    // loads hide latency that the deferred ones would expose.)
    bf16x8 qf[C::DS];
    f32x16 oacc[C::DB];
    float m_run, m_true, lsum;
    bool live = !LAB;
    const float c2 = a.scale_log2;
    f32x16 bias;  // -m_run in every element (biased scores)
    auto start = [&]() {
        if constexpr (RA_TUNE_BIAS) {
            load_q_scaled(a, wt, row, g, 0, c2, qf);
            load_state_biased<D>(a, row, g, wk == 0, 0, oacc, m_run, m_true, lsum);
            bias = bias_block<C>(m_run);
        } else {
            load_q(a, wt, row, g, 0, qf);
            load_state<D>(a, row, g, wk == 0, 0, oacc, m_run, m_true, lsum);
        }
    };
    if constexpr (!LAB) start();
    int kaddr[C::NKA];
    k_addrs<C>(wk * C::KW, l32, g, kaddr);
    int vaddr[2][C::NVD];
    v_addrs<C>(wk * C::KW, lane, vaddr);
    int ql = 0, lab_L = 0;  // the row's segment label; the wave's common one
    bool lab_uniform = true;
    int lab_lo = 0, lab_hi = 0;  // the labels of the workgroup's rows lie in [lab_lo, lab_hi]
    __shared__ int red[LAB ? 2 * NW : 1];
    if constexpr (LAB) {
        if (a.q_seg && row.ok) ql = a.q_seg[wt.b * a.Lq + row.t];
        wave_label(ql, row.ok, lab_L, lab_uniform);
        if (a.q_seg)  // uniform
            wg_min_max<NW>(row.ok ? ql : 2147483647, row.ok ? ql : -2147483647 - 1, red, w, lane, lab_lo, lab_hi);
    }

    int c_begin = 0, c_end = a.n_chunks, sub = 0;
    if (a.split_mode) {
        c_begin = wt.split / a.n_sub;
        sub = wt.split % a.n_sub;
        c_end = c_begin + 1;
    }
    for (int c = c_begin; c < c_end; ++c) {
        // (without EXT the plain range: the same code as a kernel without
        // anchors, which the compiler schedules with fewer waits)
        TileRange tr;
        int64_t kbeg, kend;
        int ntiles;
        if constexpr (ANC || LAB) {
            int64_t kf = 0, kl = INT64_MAX;  // keys that can carry a label of the rows
            if (LAB && a.q_seg && a.chunks[c].kseg) {  // uniform
                int64_t k0 = a.split_mode ? sub * a.sub_len : 0;
                const int64_t len = a.chunks[c].len;
                int64_t k1 = a.split_mode && k0 + a.sub_len < len ? k0 + a.sub_len : len;
                if (!ANC || a.anchor == 0) {  // uniform: then only keys in the rows' causal/window range are seen
                    int64_t rb, re;
                    int rn;
                    if (!chunk_range(a, wt, c, sub, rb, re, rn, BN)) continue;
                    const int64_t rend = rb + (int64_t)rn * BN;
                    k0 = rb > k0 ? rb : k0;
                    k1 = rend < k1 ? rend : k1;
                }
                label_key_span<NW>(a.chunks[c].kseg + wt.b * len, k0, k1, lab_lo, lab_hi, red, w, lane, kf, kl);
                if (kl < kf) continue;  // no key of the chunk carries a label of the rows
            }
            if (!chunk_tiles<ANC, LAB>(a, wt, c, sub, BN, tr, kf, kl)) continue;  // uniform
            kbeg = tr.kbeg, kend = tr.kend, ntiles = tr.ntot;
            if (ntiles == 0) continue;
            if (LAB && !live) {  // uniform
                live = true;
                start();
            }
        } else {
            if (!chunk_range(a, wt, c, sub, kbeg, kend, ntiles, BN)) continue;  // uniform
        }
        const ChunkArg ch = a.chunks[c];
        const VisRange vis = visible_range(a, row, ch.start, kbeg, kend);
        // tile tests as integer bounds (tiles are evenly spaced unless anchor
        // tiles follow the main range)
        TileSpan span{0, 0, 0, 0};
        if constexpr (!ANC) span = tile_span(a, ch.start, kbeg, kend, BN, wk * C::KW, C::KW, wv_tlo, wv_thi, ntiles);
        Anchors an{kNoKey, kNoKey, kNoKey};
        if constexpr (ANC) an = row_anchors(a, row.qpos, ch.start, tr.kbase, kbeg, kend);
        const int32_t *kseg = LAB && ch.kseg ? ch.kseg + wt.b * ch.len : nullptr;
        const uint16_t *kbase = (const uint16_t *)ch.k + wt.b * a.k_sb + wt.hk * a.k_sh;
        const uint16_t *vbase = (const uint16_t *)ch.v + wt.b * a.v_sb + wt.hk * a.v_sh;
        auto tile_start = [&](int t) -> int64_t {
            if constexpr (ANC) return tr.start(t, BN);
            else return kbeg + (int64_t)t * BN;  // (with labels alone: main tiles only)
        };
        auto issue = [&](auto u, int t) {
            const int64_t k0 = tile_start(t);
            load_tile<C>(kbase, a.k_ss, k0, kend, kst(u), w, lane);
            load_tile<C>(vbase, a.v_ss, k0, kend, vst(u), w, lane);
            if constexpr (LAB) load_labels(kseg, k0 + wk * C::KW, kend, kst(u) + C::TILE + 256 * w, lane);
        };
        auto wait_for = [&](int need, int last) {
            const int after = last - need;
            wait_tiles_in_flight<LPT>(after < 0 ? 0 : after);
        };

        tile_barrier();  // the previous chunk's tiles are no longer read
        const int pre = ntiles < NS - 1 ? ntiles : NS - 1;
        for_tiles<NS>(pre, [&](auto u, int t) { issue(u, t); });
        wait_for(0, pre - 1);
        for_tiles<NS>(ntiles, [&](auto u, int it) {
            constexpr int U = decltype(u)::value;
            if (it + NS - 1 < ntiles) issue(ic<(U + NS - 1) % NS>{}, it + NS - 1);
            // this wave's keys k0 + wk*KW .. + KW-1
            const int64_t k0 = tile_start(it);
            const int64_t wk0 = k0 + wk * C::KW;
            bool skip, full;
            if constexpr (ANC) {
                skip = keys_unseen(a, ch.start, wk0, C::KW, wv_tlo, wv_thi);
                full = keys_all_seen(a, ch.start, wk0, C::KW, kend, wv_tlo, wv_thi);
            } else {
                skip = span.unseen(it);
                full = span.all_seen(it);
            }
            const char *lab = kst(u) + C::TILE + 256 * w;
            if constexpr (ANC) {
                if (skip && tile_has_anchor(a, ch.start, wk0, C::KW, wv_tlo, wv_thi)) skip = false;
            }
            const bool range_full = full;
            if (!skip) {
                // the key labels are read before the scores, whose MFMAs hide
                // the read; a tile whose keys carry no label of the wave's
                // rows is dropped after them
                int lk = 0;
                if constexpr (LAB) lk = reinterpret_cast<const int *>(lab)[lane];
                prio_mfma();
                f32x16 s[C::KB];
                if constexpr (RA_TUNE_BIAS) {
                    scores_biased<C>(kst(u), kaddr, qf, bias, s);
                    if constexpr (RA_TUNE_BIASPIN) asm volatile("" : "+v"(bias));
                } else {
                    scores<C>(kst(u), kaddr, qf, s);
                }
                prio_valu();
                LabelTest lt{true, false, false, true};
                if constexpr (LAB) {
                    lt = label_test(lk, C::KW, kend - wk0, lane, ql, row.ok, lab_L, lab_uniform);
                    full = full && lt.all;
                }
                if (!lt.none) {  // uniform
                    if (!full) {
                        if constexpr (LAB) {
                            if (lt.per_lane) {  // uniform
                                if (!range_full) mask_scores_ext<C, false>(s, vis, an, (int)(wk0 - kbeg), g, lab, ql);
                                if (!lt.all) mask_lane(s, lt.hit);
                            } else {
                                mask_scores_ext<C, true>(s, vis, an, (int)(wk0 - kbeg), g, lab, ql);
                            }
                        } else if constexpr (ANC) {
                            mask_scores_ext<C, false>(s, vis, an, (int)(wk0 - kbeg), g, lab, ql);
                        } else {
                            mask_scores<C>(s, vis, (int)(wk0 - kbeg), g);
                        }
                    }
                    if constexpr (RA_TUNE_BIAS) {
                        update_max_biased<C>(s, m_run, m_true, lsum, oacc, bias);
                        if constexpr (RA_TUNE_FUSE) {
                            softmax_pv_biased<C>(s, lsum, vst(u), vaddr, oacc);
                        } else {
                            bf16x8 pf[2 * C::KB];
                            probabilities_biased<C>(s, lsum, pf);
                            prio_mfma();
                            accumulate_pv<C>(vst(u), vaddr, pf, oacc);
                            prio_valu();
                        }
                    } else {
                        update_max<C>(s, c2, m_run, m_true, lsum, oacc);
                        if constexpr (RA_TUNE_FUSE) {
                            softmax_pv<C>(s, c2, m_run, lsum, vst(u), vaddr, oacc);
                        } else {
                            bf16x8 pf[2 * C::KB];
                            probabilities<C>(s, c2, m_run, lsum, pf);
                            prio_mfma();
                            accumulate_pv<C>(vst(u), vaddr, pf, oacc);
                            prio_valu();
                        }
                    }
                }
            }
            // (after the last tile too, where nothing is in flight: every path
            // round the loop then ends with a wait the compiler can see, and it
            // adds no wait for the next tile's loads before this tile's reads)
            wait_for(it + 1, it + NS - 1 < ntiles ? it + NS - 1 : ntiles - 1);
        });
    }

    if (!live) {  // uniform
        if (a.load_state && a.store_state && !a.store_out && !a.split_mode) return;  // the state is the result
        if constexpr (RA_TUNE_BIAS) load_state_biased<D>(a, row, g, wk == 0, 0, oacc, m_run, m_true, lsum);
        else load_state<D>(a, row, g, wk == 0, 0, oacc, m_run, m_true, lsum);
    }
    renormalise(m_run, m_true, lsum, oacc);
    if constexpr (KSPLIT > 1) {
        // waves wk > 0 hand their (m, l, O) to wave wk == 0 of the same rows.
        // Value idx of a lane in slot sl is float idx*64 + lane of the slot,
        // which spans tile buffers 2sl and 2sl+1.
        __syncthreads();
        constexpr int TF = C::TILE / 4;  // floats per tile buffer
        auto at = [&](int sl, int idx) -> float & {
            const int f = idx * 64 + lane;
            const int bi = 2 * sl + f / TF;
            char *buf = bi < 2 ? kv0 + bi * C::TILE : kv1 + (bi - 2) * C::TILE;
            return reinterpret_cast<float *>(buf)[f % TF];
        };
        if (wk > 0) {
            const int sl = wr * (KSPLIT - 1) + (wk - 1);
            at(sl, 0) = m_true;
            at(sl, 1) = lsum;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) at(sl, 2 + 16 * db + i) = oacc[db][i];
        }
        __syncthreads();
        if (wk > 0) return;
#pragma unroll 1
        for (int o = 0; o < KSPLIT - 1; ++o) {
            const int sl = wr * (KSPLIT - 1) + o;
            const float m1 = at(sl, 0), l1 = at(sl, 1);
            const float mn = fmaxf(m_true, m1);
            if (mn == kNegInf) continue;
            const float a0 = m_true == kNegInf ? 0.f : exp2_fast(m_true - mn);
            const float a1 = m1 == kNegInf ? 0.f : exp2_fast(m1 - mn);
            lsum = a0 * lsum + a1 * l1;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[db][i] = a0 * oacc[db][i] + a1 * at(sl, 2 + 16 * db + i);
            m_true = mn;
        }
    }
    const float ltot = lsum + __shfl_xor(lsum, 32);
    write_results<D>(a, wt, row, g, 0, true, oacc, m_true, ltot);
}

// ---------------------------------------------------------------------------
// Wide heads (d = 512): one wave per SIMD holding 32 query rows with the whole
// head dimension -- Q as 32 B operands (128 VGPRs), O^T as 16 accumulator
// blocks of 32x32 (256 AGPRs) -- so no wave needs another's partial scores
// and every K/V fragment read from LDS feeds 32 rows.  Four waves (128 rows)
// share each 32-key K/V tile.
//
// With one wave per SIMD nothing else fills the matrix cores while a wave
// turns scores into probabilities, so the wave overlaps them itself: K runs
// one tile ahead of V, and iteration j computes the scores of tile j+1 and
// then the O^T MFMAs of tile j with the softmax of tile j+1 interleaved
// between them.  The rare O rescale follows the MFMAs of tile j.  Every tile
// of the workgroup's range is computed: keys a row may not see are masked to
// zero probability (a branch around a tile would join two copies of O, which
// the compiler would then copy out of the AGPRs on every tile).
// ---------------------------------------------------------------------------
namespace wide {
using C = Cfg<512, 32, 4, 1>;
static_assert(C::KB == 1, "one 32-key block per tile");

// S^T = K Q^T of one 32-key tile over the whole head, in VGPRs.  Written as
// inline asm so that the scores stay out of the AGPRs, which O fills (the
// builtin's accumulator takes the AGPR form in this kernel, and there are no
// 16 AGPRs to spare).  Consecutive MFMAs accumulate into the same registers,
// which the hardware chains back to back.  The compiler sees no MFMA inside
// asm and inserts no wait states for one: the s_nop in front of each covers a
// vector write of a source register just before it (2 wait states), the
// s_nops after the last one those before a VALU instruction may read the
// result.
__device__ inline void scores(const char *kt, const int (&kaddr)[C::NKA], const bf16x8 (&qf)[C::DS], f32x16 &s) {
    constexpr int N = C::DS;
    constexpr int PF = C::PF;
    bf16x8 fr[PF];
#pragma unroll
    for (int n = 0; n < PF; ++n) fr[n] = kfrag<C>(kt, kaddr, n, 0);
#pragma unroll
    for (int n = 0; n < N; ++n) {
        if (n == 0)
            asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(fr[0]), "v"(qf[0]));
        else if (n < N - 1)
            asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(fr[n % PF]), "v"(qf[n]));
        else
            asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 4"
                         : "+v"(s)
                         : "v"(fr[n % PF]), "v"(qf[n]));
        if (n + PF < N) fr[n % PF] = kfrag<C>(kt, kaddr, n + PF, 0);
    }
}

// O^T += V^T P^T of tile j (pf, vt) with the softmax of tile j+1 (its
// masked scores s1) interleaved: row maximum, new reference and the
// probabilities pn.  Returns the rescale factor alpha of O, which the caller
// applies after these MFMAs.  Program order is kept exactly (a scheduling
// barrier after every step): each step issues one MFMA, the LDS reads of the
// fragment PF steps ahead, and a few vector instructions of the softmax, so
// the reads are in flight while the MFMAs run and the vector work fills the
// issue slots between them.
template <int... Ns>
__device__ inline void pv_softmax_steps(std::integer_sequence<int, Ns...>, const char *vt,
                                        const int (&vaddr)[2][C::NVD], const bf16x8 (&pf)[2], f32x16 (&o)[C::DB],
                                        const f32x16 &s1, float c2, float &m_run, float &m_true, float &lsum,
                                        bf16x8 (&pn)[2], float &alpha) {
    constexpr int N = 2 * C::DB;  // 32 MFMAs: step n is (ks = n / DB, db = n % DB)
    constexpr int PF = C::PF;
    bf16x8 fr[PF];
#pragma unroll
    for (int n = 0; n < PF; ++n) fr[n] = vfrag<C>(vt, vaddr, n / C::DB, n % C::DB);
    float mx = kNegInf, mref = 0.f, ls = 0.f;
    float e[16];
    u32x4 pk[2];
    __builtin_amdgcn_sched_barrier(0);
    auto step = [&](auto nn) {
        constexpr int n = decltype(nn)::value;
        o[n % C::DB] = mfma(fr[n % PF], pf[n / C::DB], o[n % C::DB]);
        if constexpr (n + PF < N) fr[n % PF] = vfrag<C>(vt, vaddr, (n + PF) / C::DB, (n + PF) % C::DB);
        if constexpr (n < 5) {  // row maximum of the tile: 16 scores in the lane ...
            constexpr int i0 = 3 * n;
            if constexpr (i0 + 2 < 16) mx = fmaxf(fmaxf(mx, s1[i0]), fmaxf(s1[i0 + 1], s1[i0 + 2]));
            else mx = fmaxf(mx, s1[15]);
        } else if constexpr (n == 5) {  // ... and its partner lane
            mx = max_pair(fmaxf(mx, s1[15]));
        } else if constexpr (n == 6) {  // new reference (moves rarely) and the rescale factor of O and l
            const float mt = mx * c2;
            m_true = fmaxf(m_true, mt);
            const bool need = mt > m_run + kRescaleThreshold;
            alpha = need ? exp2_fast(m_run - mt) : 1.f;
            m_run = need ? mt : m_run;
            mref = m_run == kNegInf ? 0.f : m_run;
        } else if constexpr (n >= 7 && n < 23) {  // one probability per step
            e[n - 7] = exp2_fast(__builtin_fmaf(s1[n - 7], c2, -mref));
        } else if constexpr (n >= 23 && n < 31) {  // bf16 pairs and their sum
            constexpr int k = n - 23;
            ls += e[2 * k] + e[2 * k + 1];
            pk[k / 4][k % 4] = pack_bf16(e[2 * k], e[2 * k + 1]);
        } else if constexpr (n == 31) {
            lsum = lsum * alpha + ls;
            pn[0] = to_bf16x8(pk[0]);
            pn[1] = to_bf16x8(pk[1]);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    (step(ic<Ns>{}), ...);
}

__device__ inline void pv_softmax(const char *vt, const int (&vaddr)[2][C::NVD], const bf16x8 (&pf)[2],
                                  f32x16 (&o)[C::DB], const f32x16 &s1, float c2, float &m_run, float &m_true,
                                  float &lsum, bf16x8 (&pn)[2], float &alpha) {
    static_assert(2 * C::DB == 32, "the softmax steps are laid out for 32 MFMAs");
    pv_softmax_steps(std::make_integer_sequence<int, 2 * C::DB>{}, vt, vaddr, pf, o, s1, c2, m_run, m_true, lsum,
                     pn, alpha);
}

// O *= alpha where the matrix cores keep it (AGPRs), for the rows that need it.
__device__ inline void rescale_o(f32x16 (&o)[C::DB], float alpha) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float x = o[db][i], t;
            asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                         : "+a"(x), "=&v"(t)
                         : "v"(alpha));
            o[db][i] = x;
        }
    asm volatile("s_nop 7" ::: "memory");
}
}  // namespace wide

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_bf16_wide_kernel(const FwdArgs a) {
    using C = wide::C;
    constexpr int D = 512, BN = 32;
    constexpr int LPT = C::LOADS_PER_WAVE;  // loads of one K (or V) tile per wave
    // V (two reads per fragment) in the low 64 KiB, where the ds_read offset
    // field reaches every byte without an address add (the compiler lays the
    // arrays out in the order of their names)
    __shared__ __attribute__((aligned(1024))) char lds_a_v0[C::TILE];
    __shared__ __attribute__((aligned(1024))) char lds_a_v1[C::TILE];
    __shared__ __attribute__((aligned(1024))) char lds_b_k0[C::TILE];
    __shared__ __attribute__((aligned(1024))) char lds_b_k1[C::TILE];
    auto kbuf = [&](auto u) -> char * {
        if constexpr (decltype(u)::value % 2 == 0) return lds_b_k0;
        else return lds_b_k1;
    };
    auto vbuf = [&](auto u) -> char * {
        if constexpr (decltype(u)::value % 2 == 0) return lds_a_v0;
        else return lds_a_v1;
    };

    const int lane = threadIdx.x & 63, w = wave_index();
    const int l32 = lane & 31, g = lane >> 5;
    const WorkTile wt = work_tile<C>(a);
    int64_t wv_tlo, wv_thi;
    token_range(a, wt.p0 + 32 * w, wt.p0 + 32 * w + 32, wv_tlo, wv_thi);
    const LaneRow row = lane_row(a, wt, wt.p0 + 32 * w + l32);

    bf16x8 qf[C::DS];
    load_q(a, wt, row, g, 0, qf);
    f32x16 oacc[C::DB];
    float m_run, m_true, lsum;
    load_state<D>(a, row, g, true, 0, oacc, m_run, m_true, lsum);
    const float c2 = a.scale_log2;
    int kaddr[C::NKA];
    k_addrs<C>(0, l32, g, kaddr);
    int vaddr[2][C::NVD];
    v_addrs<C>(0, lane, vaddr);

    int c_begin = 0, c_end = a.n_chunks, sub = 0;
    if (a.split_mode) {
        c_begin = wt.split / a.n_sub;
        sub = wt.split % a.n_sub;
        c_end = c_begin + 1;
    }
    for (int c = c_begin; c < c_end; ++c) {
        int64_t kbeg, kend;
        int ntiles;
        if (!chunk_range(a, wt, c, sub, kbeg, kend, ntiles, BN)) continue;  // uniform
        const ChunkArg ch = a.chunks[c];
        const VisRange vis = visible_range(a, row, ch.start, kbeg, kend);
        const uint16_t *kbase = (const uint16_t *)ch.k + wt.b * a.k_sb + wt.hk * a.k_sh;
        const uint16_t *vbase = (const uint16_t *)ch.v + wt.b * a.v_sb + wt.hk * a.v_sh;
        // tiles past the end load nothing and zero-fill their buffer, so every
        // iteration issues the same loads
        auto tile_k0 = [&](int t) {
            const int64_t k0 = kbeg + (int64_t)t * BN;
            return k0 < kend ? k0 : kend;
        };
        auto load_k = [&](auto u, int t) { load_tile<C>(kbase, a.k_ss, tile_k0(t), kend, kbuf(u), w, lane); };
        auto load_v = [&](auto u, int t) { load_tile<C>(vbase, a.v_ss, tile_k0(t), kend, vbuf(u), w, lane); };
        auto full_of = [&](int t) {
            return keys_all_seen(a, ch.start, kbeg + (int64_t)t * BN, BN, kend, wv_tlo, wv_thi);
        };

        // prologue: K and V of tile 0, K of tile 1; the softmax of tile 0
        tile_barrier();  // the previous chunk's tiles are no longer read
        load_k(ic<0>{}, 0);
        load_v(ic<0>{}, 0);
        load_k(ic<1>{}, 1);
        wait_tiles_in_flight<LPT>(0);
        f32x16 s1;
        wide::scores(kbuf(ic<0>{}), kaddr, qf, s1);
        if (!full_of(0)) mask_scores<C>(*reinterpret_cast<f32x16(*)[1]>(&s1), vis, 0, g);
        {
            f32x16 st[1] = {s1};
            update_max_agpr<C>(st, c2, m_run, m_true, lsum, oacc);
        }
        bf16x8 pf[2];
        {
            f32x16 st[1] = {s1};
            probabilities<C>(st, c2, m_run, lsum, pf);
        }
        // iteration j: loads of K(j+2) and V(j+1); scores of tile j+1; O^T of
        // tile j with the softmax of tile j+1 between its MFMAs
        for_tiles<2>(ntiles - 1, [&](auto u, int j) {
            constexpr int U = decltype(u)::value;
            load_k(ic<U>{}, j + 2);
            load_v(ic<U ^ 1>{}, j + 1);
            wide::scores(kbuf(ic<U ^ 1>{}), kaddr, qf, s1);
            if (!full_of(j + 1)) mask_scores<C>(*reinterpret_cast<f32x16(*)[1]>(&s1), vis, (j + 1) * BN, g);
            bf16x8 pn[2];
            float alpha;
            wide::pv_softmax(vbuf(ic<U>{}), vaddr, pf, oacc, s1, c2, m_run, m_true, lsum, pn, alpha);
            if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) wide::rescale_o(oacc, alpha);
            pf[0] = pn[0];
            pf[1] = pn[1];
            wait_tiles_in_flight<LPT>(0);  // K(j+2), V(j+1)
        });
        // the last tile's O^T (its V buffer chosen at run time: no loads are
        // in flight any more, and two code paths would join two copies of O)
        accumulate_pv<C>((ntiles - 1) % 2 == 0 ? lds_a_v0 : lds_a_v1, vaddr, pf, oacc);
    }

    renormalise(m_run, m_true, lsum, oacc);
    const float ltot = lsum + __shfl_xor(lsum, 32);
    write_results<D>(a, wt, row, g, 0, true, oacc, m_true, ltot);
}

// ---------------------------------------------------------------------------
// bf16 queries against an 8-bit KV cache (OCP FP8 E4M3 codes, one
// power-of-two scale per 64 tokens of a (batch, KV head)), d = 128, split-KV
// decoding.  Tiles of 128 keys go HBM -> LDS as raw bytes (16 KiB for K and
// for V), so the cache is read at half the bytes of bf16.  Fragments are
// widened to bf16 in registers with v_cvt_scalef32_pk_bf16_fp8, whose scale
// operand applies the block's power of two exactly, and then feed the same
// bf16 MFMAs, softmax and merge as the bf16 kernels.
//  * LDS rows are keys (128 bytes = 8 units of 16 bytes); unit u of row r is
//    stored at u ^ swz8(r), swz8(r) = 2((r>>1)&3) + ((r>>3)&1), which keeps
//    both read patterns below free of bank conflicts.
//  * K: one ds_read_b128 gives a lane 16 consecutive dimensions of its key,
//    i.e. the A fragments of two MFMAs.  The contraction order is permuted to
//    match: MFMA 2c+h takes dimensions 32c + 16g + 8h + j in lane group g,
//    and the query fragments are loaded in that order.
//  * V^T: one ds_read_b64_tr_b8 gives each lane 8 keys of one dimension.  In
//    a group of 16 lanes, lane i receives byte i%8 of the 8-byte rows that
//    lanes 2k + i/8 address (k = 0..7); lanes address the keys in the order
//    of the probability fragments (keys 4g..4g+3, 8+4g..8+4g+3 of each 16).
// ---------------------------------------------------------------------------
namespace fp8kv {
constexpr int D = 128;           // head size
constexpr int BN = 128;          // keys per tile
constexpr int ROWB = D;          // bytes per key row in LDS
constexpr int TILE = BN * ROWB;  // bytes of one K (or V) tile
constexpr int NW = 4;            // waves: 2 row blocks x 2 key halves
constexpr int LOADS_PER_WAVE = TILE / 1024 / NW;
constexpr int BLOCK = 64;        // tokens per scale exponent (= keys per wave per tile)
constexpr int kMaxRangeBlocks = kFp8MaxRangeBlocks;  // scale blocks of one workgroup's key range
using C = Cfg<D, BN, NW, 2>;     // row/key geometry: 64 rows, 64 keys per wave, KB = 2
static_assert(C::KW == BLOCK, "each wave's keys of a tile share one scale block");

// Swizzle of the 16-byte units of 128-byte row r: a bijection on the eight
// rows of one parity within 16 (the K reads: 16 rows at one unit), and rows
// {0,2,8,10} (+1, +4) land in distinct unit pairs (the V^T reads: two 16-lane
// groups on units u and u^1 of the same rows), so both read patterns are free
// of bank conflicts.
__device__ inline int swz8(int r) { return (((r >> 3) & 1) << 2) | (((r >> 1) & 1) << 1) | ((r >> 2) & 1); }

// Scale 2^(e-127) of a biased exponent e in 1..254, as a float.
__device__ inline float exp_scale(unsigned e) { return __builtin_bit_cast(float, e << 23); }

// 8 E4M3 codes (bytes of w) -> 8 bf16 values times the power-of-two scale.
__device__ inline bf16x8 widen(u32x2 w, float scale) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[0], scale, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[0], scale, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[1], scale, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[1], scale, true);
    const bf16x4 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
    const bf16x4 cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
    return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ inline void load_tile(const uint8_t *base, int64_t stride, int64_t k0, int64_t kend, char *dst, int w,
                                 int lane) {
    const unsigned stride_b = (unsigned)stride;
    const unsigned nvalid = (unsigned)(kend - k0 < BN ? kend - k0 : BN);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(base + k0 * stride), (short)0, (int)(nvalid * stride_b), kBufferFlags);
#pragma unroll
    for (int j = 0; j < LOADS_PER_WAVE; ++j) {
        const int inst = j * NW + w;
        const int pos = inst * 64 + lane;
        const int r = pos / (ROWB / 16), u = (pos % (ROWB / 16)) ^ swz8(r);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(dst + inst * 1024), 16,
                                                 (unsigned)r * stride_b + (unsigned)(u * 16), 0, 0, 0);
    }
}
}  // namespace fp8kv

template <int NS>
__global__ __launch_bounds__(fp8kv::NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_fp8kv_kernel(const FwdArgs a) {
    using namespace fp8kv;
    constexpr int LPT = 2 * LOADS_PER_WAVE;
    RA_STAGE_ARRAYS(NS, TILE)
    // the scale exponents of the workgroup's key range, copied once per chunk
    // (per-tile loads into registers would be waited for behind the next
    // tile's prefetch)
    __shared__ unsigned char exk[kMaxRangeBlocks], exv[kMaxRangeBlocks];

    const int lane = threadIdx.x & 63, w = wave_index();
    const int wr = w % C::ROWW, wk = w / C::ROWW;
    const int l32 = lane & 31, g = lane >> 5;
    const WorkTile wt = work_tile<C>(a);
    int64_t wv_tlo, wv_thi;
    token_range(a, wt.p0 + 32 * wr, wt.p0 + 32 * wr + 32, wv_tlo, wv_thi);
    const LaneRow row = lane_row(a, wt, wt.p0 + 32 * wr + l32);

    // query fragments in the permuted contraction order: qf[2c+h] holds
    // dimensions 32c + 16g + 8h .. +8
    bf16x8 qf[C::DS];
    {
        const uint16_t *qp = (const uint16_t *)a.q + wt.b * a.q_sb + row.t * a.q_ss + row.h * a.q_sh + 16 * g;
#pragma unroll
        for (int ds = 0; ds < C::DS; ++ds) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row.ok) v = *(const u32x4 *)(qp + 32 * (ds / 2) + 8 * (ds % 2));
            qf[ds] = to_bf16x8(v);
        }
    }
    const float c2 = a.scale_log2;
    // biased scores, as in the bf16 kernel: s = c q.k - m_ref out of the MFMAs
    scale_q(qf, c2);
    f32x16 oacc[C::DB];
    float m_run, m_true, lsum;
    load_state_biased<D>(a, row, g, wk == 0, 0, oacc, m_run, m_true, lsum);
    f32x16 bias = bias_block<C>(m_run);

    // per-lane LDS byte addresses (tile-relative)
    int kaddr[D / 32];  // K: row wk*64 + l32, units 2c + g
    {
        const int r = wk * C::KW + l32;
#pragma unroll
        for (int c = 0; c < D / 32; ++c) kaddr[c] = r * ROWB + 16 * ((2 * c + g) ^ swz8(l32));
    }
    int vaddr[C::DB];  // V^T provider row wk*64 + keyofs, unit 2db + (G&1), half p&1
    {
        const int G = lane >> 4, p = lane & 15, kk = p >> 1;
        const int keyofs = kk < 4 ? 4 * (G >> 1) + kk : 8 + 4 * (G >> 1) + (kk - 4);
        const int r = wk * C::KW + keyofs;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
            vaddr[db] = r * ROWB + 16 * ((2 * db + (G & 1)) ^ swz8(keyofs)) + 8 * (p & 1);
    }

    int c_begin = 0, c_end = a.n_chunks, sub = 0;
    if (a.split_mode) {
        c_begin = wt.split / a.n_sub;
        sub = wt.split % a.n_sub;
        c_end = c_begin + 1;
    }
    for (int c = c_begin; c < c_end; ++c) {
        int64_t kbeg, kend;
        int ntiles;
        if (!chunk_range(a, wt, c, sub, kbeg, kend, ntiles, BN)) continue;  // uniform
        const ChunkArg ch = a.chunks[c];
        const VisRange vis = visible_range(a, row, ch.start, kbeg, kend);
        const uint8_t *kbase = (const uint8_t *)ch.k + wt.b * a.k_sb + wt.hk * a.k_sh;
        const uint8_t *vbase = (const uint8_t *)ch.v + wt.b * a.v_sb + wt.hk * a.v_sh;
        const int64_t nblk = (ch.len + BLOCK - 1) / BLOCK;
        const uint8_t *kexp = ch.kexp + ((int64_t)wt.b * a.Hkv + wt.hk) * nblk;
        const uint8_t *vexp = ch.vexp + ((int64_t)wt.b * a.Hkv + wt.hk) * nblk;
        auto issue = [&](auto u, int t) {
            const int64_t k0 = kbeg + (int64_t)t * BN;
            load_tile(kbase, a.k_ss, k0, kend, kst(u), w, lane);
            load_tile(vbase, a.v_ss, k0, kend, vst(u), w, lane);
        };
        auto wait_for = [&](int need, int last) {
            const int after = last - need;
            wait_tiles_in_flight<LPT>(after < 0 ? 0 : after);
        };

        tile_barrier();  // the previous chunk's tiles and exponents are no longer read
        const int64_t b0 = kbeg / BLOCK;  // exponents of blocks b0 .. b0 + nb - 1
        {
            const int64_t b1 = (kbeg + (int64_t)ntiles * BN + BLOCK - 1) / BLOCK;
            int nb = (int)((b1 < nblk ? b1 : nblk) - b0);  // <= kMaxRangeBlocks (host caps the range)
            nb = nb < kMaxRangeBlocks ? nb : kMaxRangeBlocks;
            for (int i = (int)threadIdx.x; i < nb; i += NW * 64) {
                exk[i] = kexp[b0 + i];
                exv[i] = vexp[b0 + i];
            }
        }
        const int pre = ntiles < NS - 1 ? ntiles : NS - 1;
        for_tiles<NS>(pre, [&](auto u, int t) { issue(u, t); });
        wait_for(0, pre - 1);
        for_tiles<NS>(ntiles, [&](auto u, int it) {
            constexpr int U = decltype(u)::value;
            if (it + NS - 1 < ntiles) issue(ic<(U + NS - 1) % NS>{}, it + NS - 1);
            const int64_t k0 = kbeg + (int64_t)it * BN;
            const int64_t wk0 = k0 + wk * C::KW;  // this wave's 64 keys: one scale block
            const bool skip = wk0 >= kend || keys_unseen(a, ch.start, wk0, C::KW, wv_tlo, wv_thi);
            const bool full = keys_all_seen(a, ch.start, wk0, C::KW, kend, wv_tlo, wv_thi);
            if (!skip) {
                const int bi = (int)(wk0 / BLOCK - b0);
                const float ks = exp_scale(exk[bi]), vs = exp_scale(exv[bi]);
                const char *kt = kst(u);
                const char *vt = vst(u);
                // every K code of the wave's tile is read from LDS before the
                // first score MFMA, and every V^T code before the softmax, so
                // the LDS latency is paid once per tile rather than per MFMA
                u32x4 rk[C::KB][D / 32];
#pragma unroll
                for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
                    for (int cc = 0; cc < D / 32; ++cc)
                        rk[kb][cc] = *reinterpret_cast<const u32x4 *>(kt + kaddr[cc] + kb * 32 * ROWB);
                f32x16 s[C::KB];
#pragma unroll
                for (int kb = 0; kb < C::KB; ++kb) {
                    s[kb] = bias;
#pragma unroll
                    for (int cc = 0; cc < D / 32; ++cc) {
                        s[kb] = mfma(widen(u32x2{rk[kb][cc][0], rk[kb][cc][1]}, ks), qf[2 * cc], s[kb]);
                        s[kb] = mfma(widen(u32x2{rk[kb][cc][2], rk[kb][cc][3]}, ks), qf[2 * cc + 1], s[kb]);
                    }
                }
                u32x2 rv[2 * C::KB][C::DB];
#pragma unroll
                for (int kss = 0; kss < 2 * C::KB; ++kss)
#pragma unroll
                    for (int db = 0; db < C::DB; ++db)
                        rv[kss][db] = __builtin_bit_cast(
                            u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                                       (__attribute__((address_space(3))) i32x2 *)(vt + vaddr[db] + kss * 16 * ROWB)));
                if (!full) mask_scores<C>(s, vis, (int)(wk0 - kbeg), g);
                update_max_biased<C>(s, m_run, m_true, lsum, oacc, bias);
                bf16x8 pf[2 * C::KB];
                probabilities_biased<C>(s, lsum, pf);
#pragma unroll
                for (int kss = 0; kss < 2 * C::KB; ++kss)
#pragma unroll
                    for (int db = 0; db < C::DB; ++db) oacc[db] = mfma(widen(rv[kss][db], vs), pf[kss], oacc[db]);
            }
            // (after the last tile too, where nothing is in flight: every path
            // round the loop then ends with a wait the compiler can see, and it
            // adds no wait for the next tile's loads before this tile's reads)
            wait_for(it + 1, it + NS - 1 < ntiles ? it + NS - 1 : ntiles - 1);
        });
    }

    renormalise(m_run, m_true, lsum, oacc);
    // the key-half waves (wk = 1) hand their state to wave wk = 0 of the same rows
    __syncthreads();
    float *slot = reinterpret_cast<float *>(wr == 0 ? kv0 : kv1);  // (16 DB + 2) x 64 floats
    if (wk == 1) {
        slot[lane] = m_true;
        slot[64 + lane] = lsum;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) slot[(2 + 16 * db + i) * 64 + lane] = oacc[db][i];
    }
    __syncthreads();
    if (wk == 1) return;
    {
        const float m1 = slot[lane], l1 = slot[64 + lane];
        const float mn = fmaxf(m_true, m1);
        if (mn != kNegInf) {
            const float a0 = m_true == kNegInf ? 0.f : exp2_fast(m_true - mn);
            const float a1 = m1 == kNegInf ? 0.f : exp2_fast(m1 - mn);
            lsum = a0 * lsum + a1 * l1;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[db][i] = a0 * oacc[db][i] + a1 * slot[(2 + 16 * db + i) * 64 + lane];
            m_true = mn;
        }
    }
    const float ltot = lsum + __shfl_xor(lsum, 32);
    write_results<D>(a, wt, row, g, 0, true, oacc, m_true, ltot);
}

template <class C, class K>
hipError_t launch(K kernel, const FwdArgs &a, hipStream_t s) {
    const int nsplit = a.split_mode ? a.n_chunks * a.n_sub : 1;
    const int64_t grid = (int64_t)a.B * a.Hkv * nsplit * a.n_rowtiles;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(C::NT), 0, s, a);
    return hipGetLastError();
}

}  // namespace

// Tile shapes per head size.  Query-chunk prefill: 4 waves x 32 rows = 128
// rows per workgroup, 64-key tiles (d <= 128), two stages.  Split (decoding):
// the packed rows of a KV head's query group; at d=128 two waves per 32 rows,
// each taking half of every key tile.  d=512: 2 row blocks x 2 halves of the
// head dimensions = 64 rows per workgroup, 32-key tiles.
int fwd_bf16_row_tile(int d, bool split_mode) {
    if (d == 64) return Cfg<64, 64, 4, 1>::BM;
    if (d == 128) return split_mode ? Cfg<128, 64, 4, 2>::BM : Cfg<128, RA_TUNE_BN128, 4, 1>::BM;
    if (d == 512) return wide::C::BM;
    return 0;
}

int fwd_fp8kv_row_tile() { return fp8kv::C::BM; }

hipError_t launch_fwd_fp8kv(const FwdArgs &a, hipStream_t s) {
    return launch<fp8kv::C>(fwd_fp8kv_kernel<2>, a, s);
}

// The kernel for the call's masks: plain, with anchors, with labels (and anchors).
template <int D, int BN, int NW, int KS, int NS>
hipError_t launch_masked(const FwdArgs &a, hipStream_t s) {
    using C = Cfg<D, BN, NW, KS>;
    if (a.q_seg && a.anchor > 0) return launch<C>(fwd_bf16_kernel<D, BN, NW, KS, NS, 3>, a, s);
    if (a.q_seg) return launch<C>(fwd_bf16_kernel<D, BN, NW, KS, NS, 2>, a, s);
    if (a.anchor > 0) return launch<C>(fwd_bf16_kernel<D, BN, NW, KS, NS, 1>, a, s);
    return launch<C>(fwd_bf16_kernel<D, BN, NW, KS, NS, 0>, a, s);
}

hipError_t launch_fwd_bf16(const FwdArgs &a, int d, bool split_mode, hipStream_t s) {
    switch (d) {  // anchors / labels: d = 64, 128 only
    case 64: return launch_masked<64, 64, 4, 1, 2>(a, s);
    case 128:
        if (split_mode) return launch_masked<128, 64, 4, 2, 2>(a, s);
        return launch_masked<128, RA_TUNE_BN128, 4, 1, RA_TUNE_NS>(a, s);
    case 512: return launch<wide::C>(fwd_bf16_wide_kernel, a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ra
