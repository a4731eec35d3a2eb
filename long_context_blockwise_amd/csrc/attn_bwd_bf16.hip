// attn_bwd_bf16.hip - gradients of blockwise attention (dQ, dK, dV) for bf16
// inputs on CDNA4 (gfx950) MFMA, fp32 accumulation.
//
// For L = sum(dO * out), out = softmax(S) V with S = scale * Q K^T over the
// visible keys, and P = exp(S - lse) the forward's probabilities:
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),   D = rowsum(dO * out),
//     dQ = scale * dS K,   dK = scale * dS^T Q,
// with every query head of a KV group adding into that KV head's dK and dV.
// This is what training with ring attention needs per ring step (page "Ring
// Attention：百万 Token 上下文的秘密", §5.1 训练效率): dQ stays with the
// device's query chunk, dK and dV travel with the KV chunk they belong to.
//
// Three kernels.  bwd_pre turns the forward's final state into the per-row
// log-sum-exp (log2 units) and computes D; it stores both negated, as the
// starting values of the score chains: with one operand of S pre-scaled by
// scale*log2(e), the chain of S that starts from -lse2 ends at the exponent of
// P (P = exp2 of it), and the chain of dP that starts from -D ends at dP - D,
// so no vector work per score remains besides the exp and one multiply for
// dS.  bwd_dq keeps a tile of query rows
// resident and walks the key tiles like the forward kernel: with S^T = K Q^T
// in the lane-per-row layout, P^T needs only the lane's own lse, dP^T = V dO^T
// reads V exactly as the forward reads K, and dS^T is the B operand of
// dQ^T += K^T dS^T (K read transposed, as the forward reads V).  bwd_dkdv
// keeps 32 keys per wave resident (their K and V fragments in registers, their
// dK^T and dV^T accumulators in the matrix-core result layout) and walks the
// query rows that can see them in tiles of 32: S = Q K^T puts the keys on the
// lanes, so P and dS are directly the B operands of dV^T += dO^T P and
// dK^T += Q^T dS, whose A operands are transposed reads of the Q and dO tiles.
// Neither kernel needs atomics, and both are deterministic.
#include "tile_common.h"

namespace ra {
namespace {

constexpr float kPosInf = __builtin_inff();

// ---------------------------------------------------------------------------
// Row statistics: 16 lanes per row
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const BwdArgs A) {
    const FwdArgs &a = A.f;
    constexpr int EPL = D / 16;  // elements per lane
    const int64_t rows = (int64_t)a.B * a.Lq * a.Hq;
    const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;  // (b * Lq + t) * Hq + h
    const int sub = threadIdx.x & 15;
    float acc = 0.f;
    int64_t b = 0, t = 0;
    int h = 0;
    if (row < rows) {
        h = (int)(row % a.Hq);
        t = (row / a.Hq) % a.Lq;
        b = row / ((int64_t)a.Hq * a.Lq);
        const int64_t off = b * a.o_sb + t * a.o_ss + h * a.o_sh + sub * EPL;
        const uint16_t *o = (const uint16_t *)A.out + off;
        const uint16_t *g = (const uint16_t *)A.dout + off;
        uint16_t ov[EPL], gv[EPL];
        if constexpr (EPL % 8 == 0) {
#pragma unroll
            for (int k = 0; k < EPL / 8; ++k) {
                *(u32x4 *)(ov + 8 * k) = *(const u32x4 *)(o + 8 * k);
                *(u32x4 *)(gv + 8 * k) = *(const u32x4 *)(g + 8 * k);
            }
        } else {
            *(u32x2 *)ov = *(const u32x2 *)o;
            *(u32x2 *)gv = *(const u32x2 *)g;
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            acc = __builtin_fmaf(__builtin_bit_cast(float, (unsigned)ov[e] << 16),
                                 __builtin_bit_cast(float, (unsigned)gv[e] << 16), acc);
    }
#pragma unroll
    for (int x = 8; x >= 1; x >>= 1) acc += __shfl_xor(acc, x);
    if (row < rows && sub == 0) {
        const float l = A.l[row];
        const int64_t idx = ((b * a.Hq + h) * a.Lq + t) * 2;
        A.ld[idx] = l > 0.f ? -(A.m[row] + logf(l)) * kLog2e : -kPosInf;  // -lse2 (rows that see no key: P = 0)
        A.ld[idx + 1] = -acc;                                                // -D
    }
}

// ---------------------------------------------------------------------------
// dQ: query rows resident, key tiles streamed (the forward's structure)
// ---------------------------------------------------------------------------
// EXT bit 1: anchor tokens (one wave per SIMD, for the registers of the
// anchor tiles); EXT bit 2: segment labels.
template <int D, int BN, int NW, int NS, int EXT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu((EXT & 1) ? 1 : 2, (EXT & 1) ? 1 : 2)))
void bwd_dq_kernel(const BwdArgs A) {
    constexpr bool ANC = (EXT & 1) != 0, LAB = (EXT & 2) != 0;
    const FwdArgs &a = A.f;
    using C = Cfg<D, BN, NW, 1>;
    constexpr int LPT = 2 * C::LOADS_PER_WAVE + (LAB ? 1 : 0);
    constexpr int LABB = LAB ? NW * 256 : 0;  // bytes of key labels per stage (after the K tile)
    RA_STAGE_ARRAYS(NS, C::TILE + LABB)
    static_assert(!LAB || C::KW <= 64, "a wave's labels are 64 dwords");

    const int lane = threadIdx.x & 63, w = wave_index();
    const int l32 = lane & 31, g = lane >> 5;
    const WorkTile wt = work_tile<C>(a);
    int64_t wv_tlo, wv_thi;
    token_range(a, wt.p0 + 32 * w, wt.p0 + 32 * w + 32, wv_tlo, wv_thi);
    const LaneRow row = lane_row(a, wt, wt.p0 + 32 * w + l32);

    // resident B operands: the row's queries and output gradients
    bf16x8 qf[C::DS], gf[C::DS];
    load_q(a, wt, row, g, 0, qf);
    {
        const uint16_t *gp = (const uint16_t *)A.dout + wt.b * a.o_sb + row.t * a.o_ss + row.h * a.o_sh + 8 * g;
#pragma unroll
        for (int ds = 0; ds < C::DS; ++ds) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row.ok) v = *(const u32x4 *)(gp + 16 * ds);
            gf[ds] = to_bf16x8(v);
        }
    }
    // -lse2 and -D of the row (rows past Lq get P = 0).  (Starting the score
    // chains from them, as the dK/dV kernel does, would take 16 registers per
    // splat, which this kernel does not have at two waves per SIMD.)
    float nl = -kPosInf, nd = 0.f;
    if (row.ok) {
        const int64_t idx = (((int64_t)wt.b * a.Hq + row.h) * a.Lq + row.t) * 2;
        nl = A.ld[idx];
        nd = A.ld[idx + 1];
    }
    const float c2 = a.scale_log2;
    f32x16 acc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
    int kaddr[C::NKA];
    k_addrs<C>(0, l32, g, kaddr);
    int vaddr[2][C::NVD];
    v_addrs<C>(0, lane, vaddr);
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

    for (int c = 0; c < a.n_chunks; ++c) {
        TileRange tr;  // (without EXT the plain range, as in the forward kernel)
        int64_t kbeg, kend;
        int ntiles;
        if constexpr (ANC || LAB) {
            int64_t kf = 0, kl = INT64_MAX;  // keys that can carry a label of the rows
            if (LAB && a.q_seg && a.chunks[c].kseg) {  // uniform
                const int64_t len = a.chunks[c].len;
                int64_t k0 = 0, k1 = len;
                if (!ANC || a.anchor == 0) {  // uniform: then only keys in the rows' causal/window range are seen
                    int64_t rb, re;
                    int rn;
                    if (!chunk_range(a, wt, c, 0, rb, re, rn, BN)) continue;
                    const int64_t rend = rb + (int64_t)rn * BN;
                    k0 = rb;
                    k1 = rend < len ? rend : len;
                }
                label_key_span<NW>(a.chunks[c].kseg + wt.b * len, k0, k1, lab_lo, lab_hi, red, w, lane, kf, kl);
                if (kl < kf) continue;  // no key of the chunk carries a label of the rows
            }
            if (!chunk_tiles<ANC, LAB>(a, wt, c, 0, BN, tr, kf, kl)) continue;  // uniform
            kbeg = tr.kbeg, kend = tr.kend, ntiles = tr.ntot;
            if (ntiles == 0) continue;
        } else {
            if (!chunk_range(a, wt, c, 0, kbeg, kend, ntiles, BN)) continue;  // uniform
        }
        const ChunkArg ch = a.chunks[c];
        const VisRange vis = visible_range(a, row, ch.start, kbeg, kend);
        Anchors an{kNoKey, kNoKey, kNoKey};
        if constexpr (ANC) an = row_anchors(a, row.qpos, ch.start, tr.kbase, kbeg, kend);
        const int32_t *kseg = LAB && ch.kseg ? ch.kseg + wt.b * ch.len : nullptr;
        const uint16_t *kbase = (const uint16_t *)ch.k + wt.b * a.k_sb + wt.hk * a.k_sh;
        const uint16_t *vbase = (const uint16_t *)ch.v + wt.b * a.v_sb + wt.hk * a.v_sh;
        auto tile_start = [&](int t) -> int64_t {
            if constexpr (ANC) return tr.start(t, BN);
            else return kbeg + (int64_t)t * BN;
        };
        auto issue = [&](auto u, int t) {
            const int64_t k0 = tile_start(t);
            load_tile<C>(kbase, a.k_ss, k0, kend, kst(u), w, lane);
            load_tile<C>(vbase, a.v_ss, k0, kend, vst(u), w, lane);
            if constexpr (LAB) load_labels(kseg, k0, kend, kst(u) + C::TILE + 256 * w, lane);
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
            const int64_t k0 = tile_start(it);
            bool skip = keys_unseen(a, ch.start, k0, BN, wv_tlo, wv_thi);
            bool full = keys_all_seen(a, ch.start, k0, BN, kend, wv_tlo, wv_thi);
            const char *lab = kst(u) + C::TILE + 256 * w;
            const bool range_full = full;
            LabelTest lt{true, false, false, true};
            if constexpr (ANC) {
                if (skip && tile_has_anchor(a, ch.start, k0, BN, wv_tlo, wv_thi)) skip = false;
            }
            if constexpr (LAB) {
                lt = label_tile(lab, BN, kend - k0, lane, ql, row.ok, lab_L, lab_uniform);
                skip = skip || lt.none;
                full = full && lt.all;
            }
            if (!skip) {
                f32x16 s[C::KB], dp[C::KB];
                scores<C>(kst(u), kaddr, qf, s);   // S^T = K Q^T
                scores<C>(vst(u), kaddr, gf, dp);  // dP^T = V dO^T
                if (!full) {
                    if constexpr (LAB) {
                        if (lt.per_lane) {  // uniform
                            if (!range_full) mask_scores_ext<C, false>(s, vis, an, (int)(k0 - kbeg), g, lab, ql);
                            if (!lt.all) mask_lane(s, lt.hit);
                        } else {
                            mask_scores_ext<C>(s, vis, an, (int)(k0 - kbeg), g, lab, ql);
                        }
                    } else if constexpr (ANC) {
                        mask_scores_ext<C, false>(s, vis, an, (int)(k0 - kbeg), g, lab, ql);
                    } else {
                        mask_scores<C>(s, vis, (int)(k0 - kbeg), g);
                    }
                }
                // dS^T = P^T (dP^T - D), packed as the B operands of dQ^T += K^T dS^T
                bf16x8 pf[2 * C::KB];
#pragma unroll
                for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        u32x4 pk;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int i0 = 8 * hh + 2 * j, i1 = i0 + 1;
                            const float p0 = exp2_fast(__builtin_fmaf(s[kb][i0], c2, nl));
                            const float p1 = exp2_fast(__builtin_fmaf(s[kb][i1], c2, nl));
                            pk[j] = pack_bf16(p0 * (dp[kb][i0] + nd), p1 * (dp[kb][i1] + nd));
                        }
                        pf[2 * kb + hh] = to_bf16x8(pk);
                    }
                accumulate_pv<C>(kst(u), vaddr, pf, acc);
            }
            // (after the last tile too, where nothing is in flight: every path
            // round the loop then ends with a wait the compiler can see, and it
            // adds no wait for the next tile's loads before this tile's reads)
            wait_for(it + 1, it + NS - 1 < ntiles ? it + NS - 1 : ntiles - 1);
        });
    }

    if (!row.ok) return;
    // dQ element i of block db in lane l is d = 32db + 8(i/4) + 4g + i%4; with
    // ACCUMULATE every old value is loaded before any store
    float *dq = A.dq + row.srow * D + 4 * g;
    f32x4 old[C::DB][4];
    if (A.accumulate) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) old[db][i4] = *(const f32x4 *)(dq + 32 * db + 8 * i4);
    }
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            f32x4 v;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = A.scale * acc[db][4 * i4 + j];
            if (A.accumulate) v += old[db][i4];
            *(f32x4 *)(dq + 32 * db + 8 * i4) = v;
        }
}

// ---------------------------------------------------------------------------
// dK, dV: keys resident (32 per wave), query-row tiles of 32 * RB streamed
// ---------------------------------------------------------------------------
constexpr int kKvWaves = 4;
constexpr int kKvKeys = 32 * kKvWaves;  // keys per workgroup
#ifndef RA_TUNE_KV_VALU
#define RA_TUNE_KV_VALU 3  // VALU instructions placed after each dV/dK MFMA
#endif
#ifndef RA_TUNE_KV_NS
#define RA_TUNE_KV_NS 2  // LDS stages of the dK/dV kernel
#endif
#ifndef RA_TUNE_KV_RB
#define RA_TUNE_KV_RB 2
#endif

#ifndef RA_TUNE_KV_PF
#define RA_TUNE_KV_PF 4  // Q and dO fragments read ahead of the S and dP MFMAs
#endif
#ifndef RA_TUNE_KV_ASM
#define RA_TUNE_KV_ASM 1  // S and dP chains as inline asm (VGPR results, K and V fragments in AGPRs)
#endif

// S = Q (cK)^T - lse2 and dP = dO V^T - D of an RB-block row tile; s and dp
// hold the chains' starting values.  MFMA n reduces step ds = n / 2RB of
// block rb = (n/2) % RB, S for even n and dP for odd n; PF fragments of the
// Q and dO tiles are read ahead.  As inline asm the results stay in VGPRs,
// where the vector work reads them, and the resident K and V fragments in
// AGPRs (the builtin would put every accumulator of this kernel in AGPRs and
// copy the scores out).  The compiler does not see an MFMA inside asm, so it
// inserts none of the wait states around one: the s_nop in front of each MFMA
// gives the 2 that a vector write of a source register needs before the matrix
// core reads it (the compiler may copy a K or V fragment into its AGPRs just
// before), and the s_nops after the last one those before a vector
// instruction may touch a result.
template <class C, int RB>
__device__ inline void kv_scores(const char *qt, const char *gt, const int (&kaddr)[C::NKA],
                                 const bf16x8 (&kf)[C::DS], const bf16x8 (&vf)[C::DS], f32x16 (&s)[RB],
                                 f32x16 (&dp)[RB]) {
    constexpr int N = 2 * RB * C::DS;
    constexpr int PF = RA_TUNE_KV_PF;
    auto frag = [&](int n) { return kfrag<C>((n & 1) ? gt : qt, kaddr, n / (2 * RB), (n / 2) % RB); };
    bf16x8 fr[PF];
#pragma unroll
    for (int n = 0; n < PF; ++n) fr[n] = frag(n);
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const int ds = n / (2 * RB), rb = (n / 2) % RB;
        if constexpr (RA_TUNE_KV_ASM) {
            if (n & 1)
                asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(dp[rb]) : "v"(fr[n % PF]), "a"(vf[ds]));
            else
                asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s[rb]) : "v"(fr[n % PF]), "a"(kf[ds]));
        } else {
            if (n & 1) dp[rb] = mfma(fr[n % PF], vf[ds], dp[rb]);
            else s[rb] = mfma(fr[n % PF], kf[ds], s[rb]);
        }
        if (n + PF < N) fr[n % PF] = frag(n + PF);
        if (n % PF == PF - 1) __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (RA_TUNE_KV_ASM) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" ::: "memory");
}

// A tile is RB blocks of 32 query rows.  Stage u holds the Q tile (row-major,
// swizzled), then each wave's copy of the rows' -lse2 and -D (256 bytes per
// 32 rows per wave: the 32 values of -lse2, then the 32 of -D), then the dO tile: RA_STAGE_ARRAYS(NS, TILE + 1024 RB)
// gives 2 TILE + 2048 RB bytes a stage.  The RB row blocks are independent
// chains of matrix-core work, which lets one wave overlap the softmax of one
// block with the products of another.
template <int D, int RB, int NS, bool EXT>
__global__ __launch_bounds__(kKvWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(const BwdArgs A) {
    const FwdArgs &a = A.f;
    constexpr int RT = 32 * RB;              // query rows per tile
    using C = Cfg<D, RT, kKvWaves, 1>;       // RT-row tiles: TILE bytes each for Q and dO; KB = RB
    constexpr int LDW = 256 * RB;            // bytes of (-lse2, -D) per wave (row labels: half that)
    // EXT: each wave's copy of the rows' segment labels follows the dO tile
    constexpr int LPT = 2 * C::LOADS_PER_WAVE + RB + (EXT ? 1 : 0);
    static_assert(!EXT || RT <= 64, "a wave's row labels are 64 dwords");
    RA_STAGE_ARRAYS(NS, C::TILE + 1024 * RB)
    auto qtile = [&](auto u) { return kst(u); };
    auto ldtile = [&](auto u) { return kst(u) + C::TILE; };
    auto gtile = [&](auto u) { return vst(u); };

    const int lane = threadIdx.x & 63, w = wave_index();
    const int l32 = lane & 31, g = lane >> 5;
    const ChunkArg ch = a.chunks[A.chunk];
    const int64_t len = ch.len;
    const int nkt = (int)((len + kKvKeys - 1) / kKvKeys);
    int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int kt = lid % nkt;  // earliest keys (most rows under causal masking) first
    lid /= nkt;
    const int hk = lid % a.Hkv;
    const int b = lid / a.Hkv;
    const int64_t kt0 = (int64_t)kt * kKvKeys;
    const int64_t wk0 = kt0 + 32 * w;       // this wave's first key
    const int64_t key = wk0 + l32;          // this lane's key
    const bool key_ok = key < len;
    auto kpos_of = [&](int64_t k) { return ch.start + k; };

    // resident B operands: K^T and V^T fragments of the lane's key (with EXT
    // read once the workgroup is known to have rows to visit)
    bf16x8 kf[C::DS], vf[C::DS], kfa[C::DS], vfa[C::DS];
    auto load_kv = [&]() {
        const uint16_t *kp = (const uint16_t *)ch.k + b * a.k_sb + key * a.k_ss + hk * a.k_sh + 8 * g;
        const uint16_t *vp = (const uint16_t *)ch.v + b * a.v_sb + key * a.v_ss + hk * a.v_sh + 8 * g;
#pragma unroll
        for (int ds = 0; ds < C::DS; ++ds) {
            u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
            if (key_ok) {
                x = *(const u32x4 *)(kp + 16 * ds);
                y = *(const u32x4 *)(vp + 16 * ds);
            }
            kf[ds] = to_bf16x8(x);
            vf[ds] = to_bf16x8(y);
        }
        scale_q(kf, a.scale_log2);  // S comes out in log2 units
        if constexpr (RA_TUNE_KV_ASM) {
            // moved into AGPRs once: the asm operands then read them there
#pragma unroll
            for (int ds = 0; ds < C::DS; ++ds) {
                asm volatile("" : "=a"(kfa[ds]) : "0"(kf[ds]));
                asm volatile("" : "=a"(vfa[ds]) : "0"(vf[ds]));
            }
        }
    };
    if constexpr (!EXT) load_kv();
    f32x16 dk[C::DB], dv[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dk[db][i] = dv[db][i] = 0.f;

    // query rows that can see any key of the workgroup
    const int64_t kp_lo = ch.start + kt0;
    const int64_t kp_hi = ch.start + (kt0 + kKvKeys < len ? kt0 + kKvKeys : len) - 1;
    int64_t t_lo = 0, t_hi = a.Lq - 1;
    if (a.causal) t_lo = kp_lo - a.q_offset > t_lo ? kp_lo - a.q_offset : t_lo;
    if (a.window > 0) {
        const int64_t hi = kp_hi + a.window - a.q_offset;
        t_hi = hi < t_hi ? hi : t_hi;
        if (!a.causal) {
            const int64_t lo = kp_lo - a.window - a.q_offset;
            t_lo = lo > t_lo ? lo : t_lo;
        }
    }
    // anchors: a key at a block start m anchors rows [m - S, m + S) (as A and
    // as A + S), the key before it rows [m, m + S) (as A - 1)
    int64_t ar_lo = 1, ar_hi = 0;  // the lane's anchored rows [lo, hi) (positions)
    int64_t u_lo = 0, u_hi = -1;   // rows anchored by any key of the workgroup (tokens)
    if constexpr (EXT) {
        if (a.anchor > 0) {
            const int64_t S = a.anchor;
            if (key_ok && kpos_of(key) % S == 0) ar_lo = kpos_of(key) - S, ar_hi = kpos_of(key) + S;
            if (key_ok && (kpos_of(key) + 1) % S == 0) {
                const int64_t lo = kpos_of(key) + 1, hi = lo + S;
                ar_lo = ar_lo < ar_hi && ar_lo < lo ? ar_lo : lo;
                ar_hi = ar_hi > hi ? ar_hi : hi;
            }
            const int64_t m0 = (kp_lo + S - 1) / S * S, y0 = (kp_lo + 1 + S - 1) / S * S;
            int64_t blo = INT64_MAX, bhi = INT64_MIN;
            if (m0 <= kp_hi) blo = m0 - S, bhi = kp_hi / S * S + S;
            if (y0 <= kp_hi + 1) {
                blo = y0 < blo ? y0 : blo;
                const int64_t yl = (kp_hi + 1) / S * S + S;
                bhi = yl > bhi ? yl : bhi;
            }
            if (blo < bhi) {
                u_lo = blo - a.q_offset > 0 ? blo - a.q_offset : 0;
                u_hi = bhi - 1 - a.q_offset < a.Lq - 1 ? bhi - 1 - a.q_offset : a.Lq - 1;
            }
        }
    }
    int kl = 0, lab_L = 0;  // the key's segment label; the wave's common one
    bool lab_uniform = true;
    __shared__ int red[EXT ? 2 * kKvWaves : 1];
    if constexpr (EXT) {
        if (ch.kseg && key_ok) kl = ch.kseg[b * len + key];
        wave_label(kl, key_ok, lab_L, lab_uniform);
        if (a.q_seg && ch.kseg) {  // uniform: only rows with a label of the workgroup's keys see them
            int klo, khi;
            wg_min_max<kKvWaves>(key_ok ? kl : 2147483647, key_ok ? kl : -2147483647 - 1, red, w, lane, klo, khi);
            // (only the rows of the window's range and the anchored rows are scanned)
            int64_t r0 = t_lo, r1 = t_hi + 1;
            if (u_lo <= u_hi) {
                r0 = u_lo < r0 ? u_lo : r0;
                r1 = u_hi + 1 > r1 ? u_hi + 1 : r1;
            }
            if (r1 < r0) r1 = r0;
            int64_t rf, rl;
            label_key_span<kKvWaves>(a.q_seg + b * a.Lq, r0, r1, klo, khi, red, w, lane, rf, rl);
            t_lo = rf > t_lo ? rf : t_lo;
            t_hi = rl < t_hi ? rl : t_hi;
            if (u_lo <= u_hi) {
                u_lo = rf > u_lo ? rf : u_lo;
                u_hi = rl < u_hi ? rl : u_hi;
            }
        }
    }
    // row segments: the window's rows, then the anchored rows not next to them
    // (without EXT the single range, in the code of a kernel without anchors).
    // An empty range (no row sees the keys, or no row carries their labels)
    // stays empty: rounding its start down to the tile grid must not revive it.
    const bool no_rows = t_hi < t_lo;
    t_lo = t_lo / RT * RT;
    int n1 = no_rows ? 0 : (int)((t_hi - t_lo) / RT + 1);
    int64_t s2 = 0;
    int n2 = 0;
    if (EXT && u_lo <= u_hi) {
        const int64_t ulo = u_lo / RT * RT;
        if (n1 == 0) {
            t_lo = ulo, n1 = (int)((u_hi - ulo) / RT + 1);
        } else if (ulo <= t_hi + 1 && u_hi + 1 >= t_lo) {  // overlapping or adjacent: one segment
            const int64_t lo = ulo < t_lo ? ulo : t_lo, hi = u_hi > t_hi ? u_hi : t_hi;
            t_lo = lo, n1 = (int)((hi - lo) / RT + 1);
        } else {
            s2 = ulo, n2 = (int)((u_hi - ulo) / RT + 1);
        }
    }
    const int nseg = n1 + n2;
    const int ntiles = nseg * a.G;
    if constexpr (EXT) {
        // no row sees the workgroup's keys (packed documents): their gradients
        // are zero, which ACCUMULATE leaves as they are
        if (ntiles == 0 && A.accumulate) return;  // uniform
        if (ntiles > 0) load_kv();
    }

    int kaddr[C::NKA];
    k_addrs<C>(0, l32, g, kaddr);
    int vaddr[2][C::NVD];
    v_addrs<C>(0, lane, vaddr);
    const int64_t kpos = ch.start + key;

    // tile -> (query head, first row): the group's heads outer, the row
    // segments inner.  Two cursors walk the tiles, one for the tile computed
    // and one for the tile loaded NS-1 ahead, so no tile needs a division.
    struct Cursor {
        int gq, j;
    };
    auto tile_at = [&](const Cursor &c, int &h, int64_t &t0) {
        h = hk * a.G + c.gq;
        if constexpr (EXT) t0 = c.j < n1 ? t_lo + RT * (int64_t)c.j : s2 + RT * (int64_t)(c.j - n1);
        else t0 = t_lo + RT * (int64_t)c.j;
    };
    auto advance = [&](Cursor &c) {
        if (++c.j == nseg) c.j = 0, ++c.gq;
    };
    Cursor cur{0, 0}, nxt{0, 0};
    auto issue = [&](auto u) {
        int h;
        int64_t t0;
        tile_at(nxt, h, t0);
        advance(nxt);
        const uint16_t *qb = (const uint16_t *)a.q + b * a.q_sb + h * a.q_sh;
        const uint16_t *gb = (const uint16_t *)A.dout + b * a.o_sb + h * a.o_sh;
        load_tile<C>(qb, a.q_ss, t0, a.Lq, qtile(u), w, lane);
        load_tile<C>(gb, a.o_ss, t0, a.Lq, gtile(u), w, lane);
        // (-lse2, -D) of rows t0 .. t0+RT-1 into the wave's own copy, one
        // dword per lane per 32 rows, split by kind: block rb holds -lse2 of
        // its 32 rows, then their -D (lanes 0-31 read the first of each pair,
        // lanes 32-63 the second)
        const int64_t nrows = a.Lq - t0 < RT ? a.Lq - t0 : RT;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(A.ld + (((int64_t)b * a.Hq + h) * a.Lq + t0) * 2), (short)0, (int)(nrows * 8), kBufferFlags);
        const unsigned pair = (unsigned)(8 * l32 + 4 * g);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(ldtile(u) + LDW * w + 256 * rb), 4,
                                                     (unsigned)(256 * rb) + pair, 0, 0, 0);
        if constexpr (EXT)  // the rows' segment labels (RT <= 64: one dword per lane)
            load_labels(a.q_seg ? a.q_seg + b * a.Lq : nullptr, t0, a.Lq, gtile(u) + C::TILE + 256 * w, lane);
    };
    auto wait_for = [&](int need, int last) {
        const int after = last - need;
        wait_tiles_in_flight<LPT>(after < 0 ? 0 : after);
    };

    const int pre = ntiles < NS - 1 ? ntiles : NS - 1;
    for_tiles<NS>(pre, [&](auto u, int) { issue(u); });
    wait_for(0, pre - 1);
    for_tiles<NS>(ntiles, [&](auto u, int it) {
        constexpr int U = decltype(u)::value;
        if (it + NS - 1 < ntiles) issue(ic<(U + NS - 1) % NS>{});
        int h;
        int64_t t0;
        tile_at(cur, h, t0);
        advance(cur);
        const int64_t thi = t0 + RT - 1 < a.Lq - 1 ? t0 + RT - 1 : a.Lq - 1;
        bool skip = wk0 >= len || keys_unseen(a, ch.start, wk0, 32, t0, thi);
        bool full = t0 + RT - 1 < a.Lq && keys_all_seen(a, ch.start, wk0, 32, len, t0, thi);
        const bool range_full = full;
        LabelTest lbt{true, false, false, true};
        const char *rlab = gtile(u) + C::TILE + 256 * w;  // EXT: labels of the tile's rows
        if constexpr (EXT) {
            // anchored rows of a lane's key inside the tile
            const bool anch = ar_lo < ar_hi && ar_lo <= a.q_offset + thi && ar_hi > a.q_offset + t0;
            if (skip && wk0 < len && __builtin_amdgcn_ballot_w64(anch) != 0) skip = false;
            lbt = label_tile(rlab, RT, a.Lq - t0, lane, kl, key_ok, lab_L, lab_uniform);
            skip = skip || lbt.none;
            full = full && lbt.all;
        }
        if (!skip) {
            const char *qt = qtile(u), *gt = gtile(u), *lt = ldtile(u) + LDW * w;
            // S = Q (cK)^T - lse2 and dP = dO V^T - D per 32-row block: rows on
            // M, this wave's keys on N.  Element i of block rb is row
            // 32rb + 8(i/4) + 4g + i%4; its chains start from that row's -lse2
            // and -D.
            f32x16 s[RB], dp[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4 x = __builtin_bit_cast(f32x4, lds_read_b128(lt, 256 * rb + 32 * j + 16 * g));
                    const f32x4 y = __builtin_bit_cast(f32x4, lds_read_b128(lt, 256 * rb + 128 + 32 * j + 16 * g));
#pragma unroll
                    for (int e = 0; e < 4; ++e) s[rb][4 * j + e] = x[e], dp[rb][4 * j + e] = y[e];
                }
            if constexpr (RA_TUNE_KV_ASM) kv_scores<C, RB>(qt, gt, kaddr, kfa, vfa, s, dp);
            else kv_scores<C, RB>(qt, gt, kaddr, kf, vf, s, dp);
            // element i of block rb is row t0 + 32rb + 4g + ro(i), ro(i) = 8(i/4) + i%4, of the lane's key
            if (!full) {
                const int64_t big = 1 << 30;
                const int64_t base = a.q_offset + t0 + 4 * g - kpos;  // qpos - kpos at rb = 0, ro = 0
                int64_t lo = -big, hi = a.Lq - t0 - 4 * g;
                if (a.causal) lo = -base;
                if (a.window > 0) {
                    hi = a.window - base + 1 < hi ? a.window - base + 1 : hi;
                    if (!a.causal) lo = -a.window - base;
                }
                if (!key_ok) lo = big;
                lo = lo < -big ? -big : (lo > big ? big : lo);
                hi = hi < -big ? -big : (hi > big ? big : hi);
                const int lo32 = (int)lo, hi32 = (int)hi;
                if constexpr (EXT) {
                    // anchored rows and labels
                    const int64_t p0 = a.q_offset + t0 + 4 * g;  // position at ro = 0
                    int64_t alo = ar_lo - p0, ahi = ar_hi - p0;
                    if (!key_ok || ar_lo >= ar_hi) alo = big, ahi = big;
                    alo = alo < -big ? -big : (alo > big ? big : alo);
                    ahi = ahi < -big ? -big : (ahi > big ? big : ahi);
                    const int alo32 = (int)alo, ahi32 = (int)ahi;
                    if (lbt.per_lane) {  // uniform: the tile's rows carry one label
                        if (!range_full) {
#pragma unroll
                            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                                for (int i = 0; i < 16; ++i) {
                                    const int ro = 32 * rb + 8 * (i >> 2) + (i & 3);
                                    const bool in = (ro >= lo32 && ro < hi32) || (ro >= alo32 && ro < ahi32);
                                    if (!in) s[rb][i] = kNegInf;
                                }
                        }
                        if (!lbt.all) mask_lane(s, lbt.hit);
                    } else {
#pragma unroll
                        for (int rb = 0; rb < RB; ++rb) {
                            int rl[16];
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const i32x4 x = *(const i32x4 *)(rlab + 4 * (32 * rb + 8 * j + 4 * g));
#pragma unroll
                                for (int e = 0; e < 4; ++e) rl[4 * j + e] = x[e];
                            }
#pragma unroll
                            for (int i = 0; i < 16; ++i) {
                                const int ro = 32 * rb + 8 * (i >> 2) + (i & 3);
                                const bool in = (ro >= lo32 && ro < hi32) || (ro >= alo32 && ro < ahi32);
                                if (!in || rl[i] != kl) s[rb][i] = kNegInf;
                            }
                        }
                    }
                } else {
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int ro = 32 * rb + 8 * (i >> 2) + (i & 3);
                            if (ro < lo32 || ro >= hi32) s[rb][i] = kNegInf;
                        }
                }
            }
            // P = exp2(S c - lse2) and dS = P (dP - D) of k-step ks (rows 16ks .. 16ks+15),
            // packed as B operands
            auto p_ds = [&](int ks, bf16x8 &ppk, bf16x8 &pdk) {
                const int rb = ks / 2, hh = ks % 2;
                u32x4 a4, b4;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i0 = 8 * hh + 2 * j, i1 = i0 + 1;
                    const float p0 = exp2_fast(s[rb][i0]), p1 = exp2_fast(s[rb][i1]);
                    a4[j] = pack_bf16(p0, p1);
                    b4[j] = pack_bf16(p0 * dp[rb][i0], p1 * dp[rb][i1]);
                }
                ppk = to_bf16x8(a4);
                pdk = to_bf16x8(b4);
            };
            // dV^T += dO^T P and dK^T += Q^T dS, k-step by k-step; P and dS of
            // step ks+1 are computed between the MFMAs of step ks, whose A
            // operands were read from LDS during step ks-1
            constexpr int NK = 2 * RB;
            bf16x8 fg[2][C::DB], fq[2][C::DB];
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
                fg[0][db] = vfrag<C>(gt, vaddr, 0, db);
                fq[0][db] = vfrag<C>(qt, vaddr, 0, db);
            }
            bf16x8 pp, pd;
            p_ds(0, pp, pd);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < NK; ++ks) {
                if (ks + 1 < NK) {
#pragma unroll
                    for (int db = 0; db < C::DB; ++db) {
                        fg[(ks + 1) & 1][db] = vfrag<C>(gt, vaddr, ks + 1, db);
                        fq[(ks + 1) & 1][db] = vfrag<C>(qt, vaddr, ks + 1, db);
                    }
                }
#pragma unroll
                for (int db = 0; db < C::DB; ++db) {
                    dv[db] = mfma(fg[ks & 1][db], pp, dv[db]);
                    dk[db] = mfma(fq[ks & 1][db], pd, dk[db]);
                }
                if (ks + 1 < NK) {
                    p_ds(ks + 1, pp, pd);
#pragma unroll
                    for (int n = 0; n < 2 * C::DB; ++n) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
                        __builtin_amdgcn_sched_group_barrier(0x002, RA_TUNE_KV_VALU, 0);  // VALU
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // (after the last tile too, where nothing is in flight: every path
        // round the loop then ends with a wait the compiler can see, and it
        // adds no wait for the next tile's loads before this tile's reads)
        wait_for(it + 1, it + NS - 1 < ntiles ? it + NS - 1 : ntiles - 1);
    });

    if (!key_ok) return;
    // element i of block db in lane l is d = 32db + 8(i/4) + 4g + i%4 of the lane's key
    const int64_t off = ((b * len + key) * a.Hkv + hk) * D + 4 * g;
    float *pk = A.dk + off, *pv = A.dv + off;
    // with ACCUMULATE every old value is loaded before any store
    f32x4 ok[C::DB][4], ov[C::DB][4];
    if (A.accumulate) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                ok[db][i4] = *(const f32x4 *)(pk + 32 * db + 8 * i4);
                ov[db][i4] = *(const f32x4 *)(pv + 32 * db + 8 * i4);
            }
    }
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int e = 32 * db + 8 * i4;
            f32x4 x, y;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[j] = A.scale * dk[db][4 * i4 + j];
                y[j] = dv[db][4 * i4 + j];
            }
            if (A.accumulate) {
                x += ok[db][i4];
                y += ov[db][i4];
            }
            *(f32x4 *)(pk + e) = x;
            *(f32x4 *)(pv + e) = y;
        }
}


// ---------------------------------------------------------------------------
// d = 512: the four waves of a workgroup split the head dimension
// ---------------------------------------------------------------------------
// A workgroup owns one 32-row (dQ) or 32-key (dK/dV) block; wave w owns
// dimensions 128w .. 128w+127 of it: its slice of the resident operands and
// of the gradient accumulators.  Per 32-key (or 32-row) tile each wave forms
// the partial S and dP over its dimensions (8 MFMAs each), the four partials
// meet in LDS and every wave adds them in the same order (so all hold the
// same bits), and the wave then takes its slice of the gradient products
// (dQ: 8 MFMAs; dK and dV: 8 each).  Tiles are 32 keys (rows) of 1024-byte
// rows, two stages; the exchange buffer holds 4 x 8 KiB.  One workgroup per
// CU, one wave per SIMD.
namespace bwide {
struct C : Cfg<512, 32, 4, 1> {
    static constexpr int BM = 32;  // rows per workgroup (all four waves share them)
};
constexpr int SL = 128;       // dimensions per wave
constexpr int SDS = SL / 16;  // reduction steps per wave
constexpr int SDB = SL / 32;  // 32-wide gradient blocks per wave
constexpr int XW = 2 * 16 * 64 * 4;  // bytes of one wave's partial S and dP

// Partials: group j (elements 4j .. 4j+3) of block b (0: S, 1: dP) of wave w
// at byte ((2w + b) * 4 + j) * 1024 + 16 * lane.
__device__ inline void exchange_put(char *x, int w, int lane, const f32x16 &s, const f32x16 &dp) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        *reinterpret_cast<f32x4 *>(x + ((2 * w) * 4 + j) * 1024 + 16 * lane) =
            f32x4{s[4 * j], s[4 * j + 1], s[4 * j + 2], s[4 * j + 3]};
        *reinterpret_cast<f32x4 *>(x + ((2 * w + 1) * 4 + j) * 1024 + 16 * lane) =
            f32x4{dp[4 * j], dp[4 * j + 1], dp[4 * j + 2], dp[4 * j + 3]};
    }
}
// The sums over the four waves' partials, in the order 0, 1, 2, 3 (the own
// partial is read back too, so that the code is the same in every wave).
__device__ inline void exchange_sum(const char *x, int lane, f32x16 &s, f32x16 &dp) {
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f32x4 a = *reinterpret_cast<const f32x4 *>(x + ((2 * v) * 4 + j) * 1024 + 16 * lane);
            const f32x4 b = *reinterpret_cast<const f32x4 *>(x + ((2 * v + 1) * 4 + j) * 1024 + 16 * lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s[4 * j + e] = v == 0 ? a[e] : s[4 * j + e] + a[e];
                dp[4 * j + e] = v == 0 ? b[e] : dp[4 * j + e] + b[e];
            }
        }
}

// Partial S (A fragments from tile a) and dP (from tile b) over the wave's
// SDS reduction steps, the B operands of step ds in AGPRs (bs[ds], bd[ds]):
// inline-asm MFMAs whose results stay in VGPRs, where the exchange and the
// vector work read them (the builtin's AGPR form would copy them out).  The
// s_nop in front of each MFMA covers a vector write of a source register just
// before it, the s_nops after the last one the wait states before a vector
// instruction may read the results: the compiler sees neither inside asm.
template <int NS, class KF>
__device__ inline void partial_scores(KF &&frag, const bf16x8 (&bs)[NS], const bf16x8 (&bd)[NS], f32x16 &s,
                                      f32x16 &dp) {
    constexpr int PF = 4;  // fragments read ahead
    bf16x8 fr[PF];
#pragma unroll
    for (int n = 0; n < PF; ++n) fr[n] = frag(n);
#pragma unroll
    for (int n = 0; n < 2 * NS; ++n) {
        const int ds = n / 2;
        if (n == 0)
            asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(fr[0]), "a"(bs[0]));
        else if (n == 1)
            asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(dp) : "v"(fr[1]), "a"(bd[0]));
        else if (n % 2 == 0)
            asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(fr[n % PF]), "a"(bs[ds]));
        else
            asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(dp) : "v"(fr[n % PF]), "a"(bd[ds]));
        if (n + PF < 2 * NS) fr[n % PF] = frag(n + PF);
        if (n % PF == PF - 1) __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" ::: "memory");
}

// Resident B operands moved into AGPRs once (the asm operands then read them there).
template <int N>
__device__ inline void to_agprs(const bf16x8 (&v)[N], bf16x8 (&a)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "=a"(a[i]) : "0"(v[i]));
}
}  // namespace bwide

// dQ for d = 512: 64 query rows per workgroup in two 32-row blocks (S^T =
// K Q^T, rows on the lanes).  Wave w = 2h + r takes row block r and the
// head-dimension half h (256 dimensions): each K/V tile feeds 64 rows, and a
// wave sums its partials with one partner's (wave w ^ 2).
namespace bwq {
struct C : Cfg<512, 32, 4, 1> {
    static constexpr int BM = 64;  // rows per workgroup
};
constexpr int SL = 256;       // dimensions per wave
constexpr int SDS = SL / 16;  // reduction steps per wave
constexpr int SDB = SL / 32;  // 32-wide dQ blocks per wave
}  // namespace bwq

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dq_wide_kernel(const BwdArgs A) {
    using bwq::C;
    using bwq::SDB;
    using bwq::SDS;
    using bwq::SL;
    const FwdArgs &a = A.f;
    constexpr int LPT = 2 * C::LOADS_PER_WAVE;
    RA_STAGE_ARRAYS(2, C::TILE)
    __shared__ __attribute__((aligned(1024))) char xch[4 * bwide::XW];

    const int lane = threadIdx.x & 63, w = wave_index();
    const int r = w & 1, hf = w >> 1;
    const int l32 = lane & 31, g = lane >> 5;
    const WorkTile wt = work_tile<C>(a);
    int64_t wg_tlo, wg_thi;  // the workgroup's rows: tile tests are the same in every wave
    token_range(a, wt.p0, wt.p0 + 64, wg_tlo, wg_thi);
    const LaneRow row = lane_row(a, wt, wt.p0 + 32 * r + l32);

    // the wave's half of the row's queries and output gradients (B operands, moved to AGPRs)
    bf16x8 qa[SDS], ga[SDS];
    {
        bf16x8 qf[SDS], gf[SDS];
        load_q(a, wt, row, g, SL * hf, qf);
        const uint16_t *gp =
            (const uint16_t *)A.dout + wt.b * a.o_sb + row.t * a.o_ss + row.h * a.o_sh + SL * hf + 8 * g;
#pragma unroll
        for (int ds = 0; ds < SDS; ++ds) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row.ok) v = *(const u32x4 *)(gp + 16 * ds);
            gf[ds] = to_bf16x8(v);
        }
        bwide::to_agprs(qf, qa);
        bwide::to_agprs(gf, ga);
    }
    float nl = -kPosInf, nd = 0.f;  // -lse2 and -D of the row (rows past Lq: P = 0)
    if (row.ok) {
        const int64_t idx = (((int64_t)wt.b * a.Hq + row.h) * a.Lq + row.t) * 2;
        nl = A.ld[idx];
        nd = A.ld[idx + 1];
    }
    const float c2 = a.scale_log2;
    f32x16 acc[SDB];
#pragma unroll
    for (int j = 0; j < SDB; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;
    int kaddr[C::NKA];
    k_addrs<C>(0, l32, g, kaddr);
    int vaddr[2][C::NVD];
    v_addrs<C>(0, lane, vaddr);

    for (int c = 0; c < a.n_chunks; ++c) {
        int64_t kbeg, kend;
        int ntiles;
        if (!chunk_range(a, wt, c, 0, kbeg, kend, ntiles, 32) || ntiles == 0) continue;  // uniform
        const ChunkArg ch = a.chunks[c];
        const VisRange vis = visible_range(a, row, ch.start, kbeg, kend);
        const uint16_t *kbase = (const uint16_t *)ch.k + wt.b * a.k_sb + wt.hk * a.k_sh;
        const uint16_t *vbase = (const uint16_t *)ch.v + wt.b * a.v_sb + wt.hk * a.v_sh;
        auto issue = [&](auto u, int t) {
            const int64_t k0 = kbeg + (int64_t)t * 32;
            load_tile<C>(kbase, a.k_ss, k0, kend, kst(u), w, lane);
            load_tile<C>(vbase, a.v_ss, k0, kend, vst(u), w, lane);
        };
        auto wait_for = [&](int need, int last) {
            const int after = last - need;
            wait_tiles_in_flight<LPT>(after < 0 ? 0 : after);
        };
        tile_barrier();  // the previous chunk's tiles and partials are no longer read
        issue(ic<0>{}, 0);
        wait_for(0, 0);
        for_tiles<2>(ntiles, [&](auto u, int it) {
            constexpr int U = decltype(u)::value;
            if (it + 1 < ntiles) issue(ic<(U + 1) % 2>{}, it + 1);
            const int64_t k0 = kbeg + (int64_t)it * 32;
            if (!keys_unseen(a, ch.start, k0, 32, wg_tlo, wg_thi)) {
                const char *kt = kst(u), *vt = vst(u);
                f32x16 s[1], dp;
                bwide::partial_scores([&](int n) { return kfrag<C>(n % 2 ? vt : kt, kaddr, SDS * hf + n / 2, 0); },
                                      qa, ga, s[0], dp);
                bwide::exchange_put(xch, w, lane, s[0], dp);
                tile_barrier();
                // the sums of the row block's two halves, half 0 first (the same bits in both waves)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4 a0 = *reinterpret_cast<const f32x4 *>(xch + ((2 * r) * 4 + j) * 1024 + 16 * lane);
                    const f32x4 b0 = *reinterpret_cast<const f32x4 *>(xch + ((2 * r + 1) * 4 + j) * 1024 + 16 * lane);
                    const f32x4 a1 =
                        *reinterpret_cast<const f32x4 *>(xch + ((2 * (r + 2)) * 4 + j) * 1024 + 16 * lane);
                    const f32x4 b1 =
                        *reinterpret_cast<const f32x4 *>(xch + ((2 * (r + 2) + 1) * 4 + j) * 1024 + 16 * lane);
#pragma unroll
                    for (int e = 0; e < 4; ++e) s[0][4 * j + e] = a0[e] + a1[e], dp[4 * j + e] = b0[e] + b1[e];
                }
                // the K^T fragments of the dQ products, all read before P and dS
                // are computed (read one before each product, every product
                // waited for its own reads)
                bf16x8 kf[2][SDB];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int j = 0; j < SDB; ++j) kf[ks][j] = vfrag<C>(kt, vaddr, ks, SDB * hf + j);
                if (!keys_all_seen(a, ch.start, k0, 32, kend, wg_tlo, wg_thi))
                    mask_scores<C>(s, vis, (int)(k0 - kbeg), g);
                // dS^T = P^T (dP^T - D), packed as the B operands of dQ^T += K^T dS^T
                bf16x8 pf[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    u32x4 pk;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int i0 = 8 * hh + 2 * j, i1 = i0 + 1;
                        const float p0 = exp2_fast(__builtin_fmaf(s[0][i0], c2, nl));
                        const float p1 = exp2_fast(__builtin_fmaf(s[0][i1], c2, nl));
                        pk[j] = pack_bf16(p0 * (dp[i0] + nd), p1 * (dp[i1] + nd));
                    }
                    pf[hh] = to_bf16x8(pk);
                }
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int j = 0; j < SDB; ++j) acc[j] = mfma(kf[ks][j], pf[ks], acc[j]);
            }
            // the next tile is in place; this stage and the partials are free
            // (after the last tile too, where nothing is in flight: every path
            // round the loop then ends with a wait the compiler can see)
            wait_for(it + 1, it + 1);
        });
    }

    if (!row.ok) return;
    // element i of block j in lane l is d = 256h + 32j + 8(i/4) + 4g + i%4; with
    // ACCUMULATE every old value is loaded before any store
    float *dq = A.dq + row.srow * 512 + SL * hf + 4 * g;
#pragma unroll
    for (int j = 0; j < SDB; ++j)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = A.scale * acc[j][4 * i4 + e];
            if (A.accumulate) v += *(const f32x4 *)(dq + 32 * j + 8 * i4);
            *(f32x4 *)(dq + 32 * j + 8 * i4) = v;
        }
}

// dK, dV for d = 512: 32 keys per workgroup (S = Q K^T, keys on the lanes),
// the query rows that can see them walked in tiles of 32.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_wide_kernel(const BwdArgs A) {
    using namespace bwide;
    const FwdArgs &a = A.f;
    constexpr int LPT = 2 * C::LOADS_PER_WAVE;
    RA_STAGE_ARRAYS(2, C::TILE)  // stage u: the Q tile (kst), the dO tile (vst)
    __shared__ __attribute__((aligned(1024))) char xch[4 * XW];

    const int lane = threadIdx.x & 63, w = wave_index();
    const int l32 = lane & 31, g = lane >> 5;
    const ChunkArg ch = a.chunks[A.chunk];
    const int64_t len = ch.len;
    const int nkt = (int)((len + 31) / 32);
    int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int kt = lid % nkt;  // earliest keys (most rows under causal masking) first
    lid /= nkt;
    const int hk = lid % a.Hkv;
    const int b = lid / a.Hkv;
    const int64_t wk0 = (int64_t)kt * 32;  // the workgroup's first key
    const int64_t key = wk0 + l32;         // this lane's key
    const bool key_ok = key < len;

    // the wave's slice of the key's K and V (B operands)
    bf16x8 kf[SDS], vf[SDS];
    {
        const uint16_t *kp = (const uint16_t *)ch.k + b * a.k_sb + key * a.k_ss + hk * a.k_sh + SL * w + 8 * g;
        const uint16_t *vp = (const uint16_t *)ch.v + b * a.v_sb + key * a.v_ss + hk * a.v_sh + SL * w + 8 * g;
#pragma unroll
        for (int ds = 0; ds < SDS; ++ds) {
            u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
            if (key_ok) {
                x = *(const u32x4 *)(kp + 16 * ds);
                y = *(const u32x4 *)(vp + 16 * ds);
            }
            kf[ds] = to_bf16x8(x);
            vf[ds] = to_bf16x8(y);
        }
    }
    bf16x8 ka[SDS], va[SDS];
    to_agprs(kf, ka);
    to_agprs(vf, va);
    f32x16 dk[SDB], dv[SDB];
#pragma unroll
    for (int j = 0; j < SDB; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) dk[j][i] = dv[j][i] = 0.f;

    // query rows that can see any key of the workgroup
    const int64_t kp_lo = ch.start + wk0;
    const int64_t kp_hi = ch.start + (wk0 + 32 < len ? wk0 + 32 : len) - 1;
    int64_t t_lo = 0, t_hi = a.Lq - 1;
    if (a.causal) t_lo = kp_lo - a.q_offset > t_lo ? kp_lo - a.q_offset : t_lo;
    if (a.window > 0) {
        const int64_t hi = kp_hi + a.window - a.q_offset;
        t_hi = hi < t_hi ? hi : t_hi;
        if (!a.causal) {
            const int64_t lo = kp_lo - a.window - a.q_offset;
            t_lo = lo > t_lo ? lo : t_lo;
        }
    }
    const bool no_rows = t_hi < t_lo;  // (rounding t_lo down must not revive an empty range)
    t_lo = t_lo / 32 * 32;
    const int n1 = no_rows ? 0 : (int)((t_hi - t_lo) / 32 + 1);
    const int ntiles = n1 * a.G;

    int kaddr[C::NKA];
    k_addrs<C>(0, l32, g, kaddr);
    int vaddr[2][C::NVD];
    v_addrs<C>(0, lane, vaddr);
    const float c2 = a.scale_log2;
    const int64_t kpos = ch.start + key;

    auto tile_of = [&](int it, int &h, int64_t &t0) {
        h = hk * a.G + it / n1;
        t0 = t_lo + 32 * (int64_t)(it % n1);
    };
    auto issue = [&](auto u, int it) {
        int h;
        int64_t t0;
        tile_of(it, h, t0);
        const uint16_t *qb = (const uint16_t *)a.q + b * a.q_sb + h * a.q_sh;
        const uint16_t *gb = (const uint16_t *)A.dout + b * a.o_sb + h * a.o_sh;
        load_tile<C>(qb, a.q_ss, t0, a.Lq, kst(u), w, lane);
        load_tile<C>(gb, a.o_ss, t0, a.Lq, vst(u), w, lane);
    };
    auto wait_for = [&](int need, int last) {
        const int after = last - need;
        wait_tiles_in_flight<LPT>(after < 0 ? 0 : after);
    };

    if (ntiles > 0) {
        issue(ic<0>{}, 0);
        wait_for(0, 0);
    }
    for_tiles<2>(ntiles, [&](auto u, int it) {
        constexpr int U = decltype(u)::value;
        int h;
        int64_t t0;
        tile_of(it, h, t0);
        // -lse2 and -D of the tile's rows for this lane's elements: element
        // i = 4j + e is row t0 + 8j + 4g + e, pairs (nl, nd) interleaved.
        // Requested before the next tile's loads, so that waiting for them
        // leaves those in flight; rows past Lq read 0 (and are masked).
        f32x4 bx[4], by[4];
        {
            const int64_t nrows = a.Lq - t0 < 32 ? a.Lq - t0 : 32;
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(A.ld + (((int64_t)b * a.Hq + h) * a.Lq + t0) * 2), (short)0, (int)(nrows * 8), kBufferFlags);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bx[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 8 * (8 * j + 4 * g), 0, 0));
                by[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 8 * (8 * j + 4 * g) + 16, 0, 0));
            }
        }
        if (it + 1 < ntiles) issue(ic<(U + 1) % 2>{}, it + 1);
        const int64_t thi = t0 + 31 < a.Lq - 1 ? t0 + 31 : a.Lq - 1;
        // (the same keys in every wave: the tests and the barrier below are uniform)
        if (!(wk0 >= len || keys_unseen(a, ch.start, wk0, 32, t0, thi))) {
            const char *qt = kst(u), *gt = vst(u);
            // partial S = Q K^T and dP = dO V^T over the wave's dimensions: rows on M, keys on N
            f32x16 s, dp;
            partial_scores<SDS>([&](int n) { return kfrag<C>(n % 2 ? gt : qt, kaddr, SDS * w + n / 2, 0); }, ka, va,
                                s, dp);
            exchange_put(xch, w, lane, s, dp);
            tile_barrier();
            exchange_sum(xch, lane, s, dp);
            // the dO^T and Q^T fragments of the dV and dK products, all read
            // before P and dS are computed (as in the dQ kernel)
            bf16x8 gfr[2][SDB], qfr[2][SDB];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int j = 0; j < SDB; ++j) {
                    gfr[ks][j] = vfrag<C>(gt, vaddr, ks, SDB * w + j);
                    qfr[ks][j] = vfrag<C>(qt, vaddr, ks, SDB * w + j);
                }
            if (!(t0 + 31 < a.Lq && keys_all_seen(a, ch.start, wk0, 32, len, t0, thi))) {
                // element i is row t0 + 4g + ro(i), ro(i) = 8(i/4) + i%4, of the lane's key
                const int64_t big = 1 << 30;
                const int64_t base = a.q_offset + t0 + 4 * g - kpos;  // qpos - kpos at ro = 0
                int64_t lo = -big, hi = a.Lq - t0 - 4 * g;
                if (a.causal) lo = -base;
                if (a.window > 0) {
                    hi = a.window - base + 1 < hi ? a.window - base + 1 : hi;
                    if (!a.causal) lo = -a.window - base;
                }
                if (!key_ok) lo = big;
                lo = lo < -big ? -big : (lo > big ? big : lo);
                hi = hi < -big ? -big : (hi > big ? big : hi);
                const int lo32 = (int)lo, hi32 = (int)hi;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int ro = 8 * (i >> 2) + (i & 3);
                    if (ro < lo32 || ro >= hi32) s[i] = kNegInf;
                }
            }
            // P = exp2(S c - lse2) and dS = P (dP - D) of rows 16ks .. 16ks+15, as B operands
            bf16x8 pp[2], pd[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                u32x4 a4, b4;
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const f32x4 x = bx[2 * ks + jj], y = by[2 * ks + jj];  // rows 16ks + 8jj + 4g + 0..3
                    const float l4[4] = {x[0], x[2], y[0], y[2]}, d4[4] = {x[1], x[3], y[1], y[3]};
#pragma unroll
                    for (int r2 = 0; r2 < 2; ++r2) {
                        const int i0 = 8 * ks + 4 * jj + 2 * r2, i1 = i0 + 1;
                        const float p0 = exp2_fast(__builtin_fmaf(s[i0], c2, l4[2 * r2]));
                        const float p1 = exp2_fast(__builtin_fmaf(s[i1], c2, l4[2 * r2 + 1]));
                        a4[2 * jj + r2] = pack_bf16(p0, p1);
                        b4[2 * jj + r2] = pack_bf16(p0 * (dp[i0] + d4[2 * r2]), p1 * (dp[i1] + d4[2 * r2 + 1]));
                    }
                }
                pp[ks] = to_bf16x8(a4);
                pd[ks] = to_bf16x8(b4);
            }
            // dV^T += dO^T P and dK^T += Q^T dS over the wave's dimensions
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int j = 0; j < SDB; ++j) {
                    dv[j] = mfma(gfr[ks][j], pp[ks], dv[j]);
                    dk[j] = mfma(qfr[ks][j], pd[ks], dk[j]);
                }
        }
        // the next tile is in place; this stage and the partials are free
        // (after the last tile too, where nothing is in flight: every path
        // round the loop then ends with a wait the compiler can see)
        wait_for(it + 1, it + 1);
    });

    if (!key_ok) return;
    // element i of block j in lane l is d = 128w + 32j + 8(i/4) + 4g + i%4 of the lane's key
    const int64_t off = ((b * len + key) * a.Hkv + hk) * 512 + SL * w + 4 * g;
    float *pk = A.dk + off, *pv = A.dv + off;
    f32x4 ok[SDB][4], ov[SDB][4];
    if (A.accumulate) {
#pragma unroll
        for (int j = 0; j < SDB; ++j)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                ok[j][i4] = *(const f32x4 *)(pk + 32 * j + 8 * i4);
                ov[j][i4] = *(const f32x4 *)(pv + 32 * j + 8 * i4);
            }
    }
#pragma unroll
    for (int j = 0; j < SDB; ++j)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int e = 32 * j + 8 * i4;
            f32x4 x, y;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                x[q] = A.scale * dk[j][4 * i4 + q];
                y[q] = dv[j][4 * i4 + q];
            }
            if (A.accumulate) {
                x += ok[j][i4];
                y += ov[j][i4];
            }
            *(f32x4 *)(pk + e) = x;
            *(f32x4 *)(pv + e) = y;
        }
}

}  // namespace

int bwd_dq_row_tile(int d) { return d == 512 ? bwq::C::BM : 128; }

hipError_t launch_bwd_pre(const BwdArgs &a, int d, hipStream_t s) {
    const int64_t rows = (int64_t)a.f.B * a.f.Lq * a.f.Hq;
    if (rows == 0) return hipSuccess;
    const unsigned grid = (unsigned)((rows * 16 + 255) / 256);
    if (d == 512)
        hipLaunchKernelGGL(bwd_pre_kernel<512>, dim3(grid), dim3(256), 0, s, a);
    else if (d == 128)
        hipLaunchKernelGGL(bwd_pre_kernel<128>, dim3(grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(bwd_pre_kernel<64>, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int D, int EXT>
static void launch_dq(const BwdArgs &a, unsigned grid, hipStream_t s) {
    hipLaunchKernelGGL((bwd_dq_kernel<D, 64, 4, 2, EXT>), dim3(grid), dim3(256), 0, s, a);
}

template <int D>
static void launch_dq_ext(const BwdArgs &a, unsigned grid, hipStream_t s) {
    const int ext = (a.f.anchor > 0 ? 1 : 0) | (a.f.q_seg != nullptr ? 2 : 0);
    if (ext == 3) launch_dq<D, 3>(a, grid, s);
    else if (ext == 2) launch_dq<D, 2>(a, grid, s);
    else if (ext == 1) launch_dq<D, 1>(a, grid, s);
    else launch_dq<D, 0>(a, grid, s);
}

hipError_t launch_bwd_dq(const BwdArgs &a, int d, hipStream_t s) {
    const unsigned grid = (unsigned)((int64_t)a.f.n_rowtiles * a.f.Hkv * a.f.B);
    if (grid == 0) return hipSuccess;
    if (d == 512) hipLaunchKernelGGL(bwd_dq_wide_kernel, dim3(grid), dim3(256), 0, s, a);
    else if (d == 128) launch_dq_ext<128>(a, grid, s);
    else launch_dq_ext<64>(a, grid, s);
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdArgs &a, int d, hipStream_t s) {
    const int64_t len = a.f.chunks[a.chunk].len;
    if (d == 512) {
        const unsigned grid = (unsigned)((len + 31) / 32 * a.f.Hkv * a.f.B);
        if (grid == 0) return hipSuccess;
        hipLaunchKernelGGL(bwd_dkdv_wide_kernel, dim3(grid), dim3(256), 0, s, a);
        return hipGetLastError();
    }
    const int64_t nkt = (len + kKvKeys - 1) / kKvKeys;
    const unsigned grid = (unsigned)(nkt * a.f.Hkv * a.f.B);
    if (grid == 0) return hipSuccess;
    const bool ext = a.f.anchor > 0 || a.f.q_seg != nullptr;
    const dim3 blk(kKvWaves * 64);
    if (d == 128 && ext)
        hipLaunchKernelGGL((bwd_dkdv_kernel<128, (RA_TUNE_KV_RB < 2 ? RA_TUNE_KV_RB : 2), RA_TUNE_KV_NS, true>), dim3(grid), blk, 0, s, a);
    else if (d == 128)
        hipLaunchKernelGGL((bwd_dkdv_kernel<128, RA_TUNE_KV_RB, RA_TUNE_KV_NS, false>), dim3(grid), blk, 0, s, a);
    else if (ext)
        hipLaunchKernelGGL((bwd_dkdv_kernel<64, (RA_TUNE_KV_RB < 2 ? RA_TUNE_KV_RB : 2), RA_TUNE_KV_NS, true>), dim3(grid), blk, 0, s, a);
    else
        hipLaunchKernelGGL((bwd_dkdv_kernel<64, RA_TUNE_KV_RB, RA_TUNE_KV_NS, false>), dim3(grid), blk, 0, s, a);
    return hipGetLastError();
}

}  // namespace ra
