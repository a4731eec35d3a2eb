// tile_common.h - CDNA4 (gfx950) building blocks shared by the attention
// kernels of libringattn: vector types, MFMA and LDS-transpose wrappers,
// the XOR-swizzled row-major LDS tile layout and its fragment reads, the
// HBM->LDS tile loads, query-row geometry, the causal / local-window masks,
// and the statically named stage buffers with their waits.
//
// Everything here has internal linkage (anonymous namespace); each kernel
// source includes it once.
#pragma once

#include <type_traits>
#include <utility>

#include "ra_internal.h"

// Tuning knobs (compile-time): LDS fragments read ahead of the MFMAs (0 lets
// the compiler schedule them) and whether waves raise their issue priority
// while they feed the matrix cores.
#ifndef RA_TUNE_PF
#define RA_TUNE_PF 4
#endif
#ifndef RA_TUNE_SETPRIO
#define RA_TUNE_SETPRIO 1
#endif

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
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
// v_permlane32_swap exchanges lanes 32..63 of its first operand with lanes
// 0..31 of its second; with both holding x, one holds the low half twice and
// the other the high half twice, so their max is the pair max in every lane.
// It is written as inline asm because the compiler's builtin returns the same
// register for both results.  The s_nops cover the VALU-write -> permlane and
// permlane -> VALU-read wait states, which the compiler does not see inside asm.
__device__ inline float max_pair(float x) {
    float a = x, b = x;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
    return fmaxf(a, b);
}

// Index of the calling wave in its workgroup, as a scalar: the compiler
// cannot see that threadIdx.x >> 6 is uniform across a wave, and would keep
// everything derived from it (row ranges, branch conditions) in vector
// registers and exec-masked branches.
__device__ inline int wave_index() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Workgroup ids are handed to the 8 XCDs round robin; renumber them so that
// each XCD runs a contiguous range of logical tiles (tiles that share K/V then
// share that XCD's L2).
__device__ inline int xcd_remap(int bid, int n) {
    const int q = n >> 3, r = n & 7;
    const int x = bid & 7, s = bid >> 3;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + s;
}

// Swizzle of the 16-byte units of LDS row r (key r of a tile): unit u is
// stored at u ^ swz<D>(r).  gfx950's LDS serves 256 bytes (64 banks) per
// cycle: 16 lanes of a ds_read_b128, 32 lanes of a ds_read_b64_tr_b16.  A K
// fragment read touches 16 consecutive rows at one unit; a transposed V read
// touches 4 consecutive rows x 4 units.  With rows of >= 256 bytes both land on
// 16 distinct units of a 256-byte window when swz(r) = 4(r&3) + ((r>>2)&3).
// 128-byte rows (d=64) pair up in a window, so the row-pair index r>>1 is used.
template <int D>
__device__ inline int swz(int r) {
    if constexpr (D >= 128)
        return ((r & 3) << 2) | ((r >> 2) & 3);
    else
        return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

__device__ inline bf16x8 to_bf16x8(const u32x4 &u) { return __builtin_bit_cast(bf16x8, u); }

__device__ inline unsigned pack_bf16(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

__device__ inline bf16x8 lds_read_b128(const char *lds, int byte) {
    return *reinterpret_cast<const bf16x8 *>(lds + byte);
}

// Two transposed 4-key reads make one V^T A-operand fragment.
__device__ inline bf16x8 lds_read_vt(const char *lds, int byte0, int byte1) {
    const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(lds + byte0));
    const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(lds + byte1));
    const s16x8 xy = __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, xy);
}

__device__ inline f32x16 mfma(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
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
    static constexpr int LOADS = TILE / 1024;    // 1 KiB wave loads per K (or V) tile
    static constexpr int LOADS_PER_WAVE = LOADS / NW;
    static constexpr int PF = RA_TUNE_PF;        // LDS fragments read ahead of the MFMAs
    static constexpr int SWB = D >= 128 ? 16 : 8;  // units covered by the swizzle
    static constexpr int NKA = SWB / 2;            // per-lane K address patterns
    static constexpr int NVD = SWB / 4;            // per-lane V^T address patterns per read
    static_assert(KW % 32 == 0, "each wave needs whole 32-key blocks");
    static_assert(D % 64 == 0, "head size must be a multiple of 64");
    static_assert(LOADS % NW == 0, "tile loads must split evenly over the waves");
};

// ---------------------------------------------------------------------------
// Pieces shared by both kernels
// ---------------------------------------------------------------------------

// Rows and key range of one workgroup.
struct WorkTile {
    int b, hk, split;
    int64_t p0;              // first packed row
    int64_t wg_tlo, wg_thi;  // token range of the workgroup's rows
};

__device__ inline void token_range(const FwdArgs &a, int64_t pa, int64_t pb, int64_t &lo, int64_t &hi) {
    const int64_t pend = (int64_t)a.G * a.Lq_pad;
    pb = (pb < pend ? pb : pend) - 1;
    if (pa / a.Lq_pad == pb / a.Lq_pad) {
        lo = pa % a.Lq_pad;
        hi = pb % a.Lq_pad;
        hi = hi < a.Lq - 1 ? hi : a.Lq - 1;
    } else {
        lo = 0;
        hi = a.Lq - 1;
    }
}

template <class C>
__device__ inline WorkTile work_tile(const FwdArgs &a) {
    WorkTile wt;
    const int nsplit = a.split_mode ? a.n_chunks * a.n_sub : 1;
    int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int rt = lid % a.n_rowtiles;
    lid /= a.n_rowtiles;
    wt.split = lid % nsplit;
    lid /= nsplit;
    wt.hk = lid % a.Hkv;
    wt.b = lid / a.Hkv;
    if (a.Lq_pad % C::BM == 0) {  // one head per tile; heaviest (latest) rows first
        const int64_t ntt = a.Lq_pad / C::BM;
        const int gq = rt % a.G;
        const int64_t tt = ntt - 1 - rt / a.G;
        wt.p0 = gq * a.Lq_pad + tt * C::BM;
    } else {
        wt.p0 = (int64_t)rt * C::BM;
    }
    token_range(a, wt.p0, wt.p0 + C::BM, wt.wg_tlo, wt.wg_thi);
    return wt;
}

// The query row a lane owns.
struct LaneRow {
    int64_t t, qpos, srow;
    int h;
    bool ok;
};

__device__ inline LaneRow lane_row(const FwdArgs &a, const WorkTile &wt, int64_t prow) {
    LaneRow r;
    const int gq = (int)(prow / a.Lq_pad);
    r.t = prow % a.Lq_pad;
    r.ok = prow < (int64_t)a.G * a.Lq_pad && r.t < a.Lq;
    r.h = wt.hk * a.G + gq;
    r.qpos = a.q_offset + r.t;
    r.srow = ((int64_t)wt.b * a.Lq + r.t) * a.Hq + r.h;  // state row index
    return r;
}

// Resident query fragments (B operand of S^T = K Q^T) for dimensions d0 ..
// d0 + 16*NDS - 1: fragment ds of a lane holds d = d0 + 16ds + 8g .. +8.
template <int NDS>
__device__ inline void load_q(const FwdArgs &a, const WorkTile &wt, const LaneRow &r, int g, int d0,
                              bf16x8 (&qf)[NDS]) {
    const uint16_t *qp = (const uint16_t *)a.q + wt.b * a.q_sb + r.t * a.q_ss + r.h * a.q_sh + d0 + 8 * g;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r.ok) v = *(const u32x4 *)(qp + 16 * ds);
        qf[ds] = to_bf16x8(v);
    }
}

// Per-lane LDS byte addresses.  The swizzle only touches the low 4 bits of a
// unit index (3 for d=64), so every read is a per-lane base plus a
// compile-time offset.
// K fragment (kb, ds): row r0 + 32kb + l32, unit u = 2ds+g, stored at u ^ swz(row)
// (r0 and 32kb keep the low 4 bits of the row).
template <class C>
__device__ inline void k_addrs(int r0, int l32, int g, int (&kaddr)[C::NKA]) {
    const int sw = swz<C::DB * 32>(l32);
    const int rowb = (r0 + l32) * C::ROWB;
#pragma unroll
    for (int x = 0; x < C::NKA; ++x) kaddr[x] = rowb + (((2 * x + g) ^ sw) << 4);
}
// V^T fragment (ks, db), read hh of 2: lane = 16G + 4k + q provides V[key][d]
// with key = r0 + 16ks + 4(G>>1) + 8hh + k and d = 32db + 16(G&1) + 4q,
// i.e. unit u = 4db + 2(G&1) + (q>>1), half q&1.
template <class C>
__device__ inline void v_addrs(int r0, int lane, int (&vaddr)[2][C::NVD]) {
    const int G = lane >> 4, k = (lane >> 2) & 3, q = lane & 3;
    const int gi = G & 1, gk = G >> 1;
    const int c = 2 * gi + (q >> 1);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int row = r0 + 4 * gk + 8 * hh + k;
        const int sw = swz<C::DB * 32>(row);
#pragma unroll
        for (int dbl = 0; dbl < C::NVD; ++dbl)
            vaddr[hh][dbl] = row * C::ROWB + (((4 * dbl + c) ^ sw) << 4) + ((q & 1) << 3);
    }
}

template <class C>
__device__ inline bf16x8 kfrag(const char *kt, const int (&kaddr)[C::NKA], int ds, int kb) {
    return lds_read_b128(kt, kaddr[ds % C::NKA] + 16 * C::SWB * (ds / C::NKA) + 32 * kb * C::ROWB);
}

template <class C>
__device__ inline bf16x8 vfrag(const char *vt, const int (&vaddr)[2][C::NVD], int ks, int db) {
    const int off = 16 * C::SWB * (db / C::NVD) + 16 * ks * C::ROWB;
    return lds_read_vt(vt, vaddr[0][db % C::NVD] + off, vaddr[1][db % C::NVD] + off);
}

// One K (or V) tile, keys k0 .. k0+BN-1 of a chunk, HBM -> LDS; keys >= kend
// are zero-filled by the descriptor.  Each wave issues LOADS_PER_WAVE loads.
// The host keeps token strides below 2^24 elements, so the byte offsets
// within a tile (< BN x stride x 2 < 2^31) are computed in 32 bits.
template <class C>
__device__ inline void load_tile(const uint16_t *base, int64_t stride, int64_t k0, int64_t kend, char *dst,
                                 int w, int lane) {
    constexpr int BN = C::TILE / C::ROWB;
    const unsigned stride_b = (unsigned)stride * 2u;
    const unsigned nvalid = (unsigned)(kend - k0 < BN ? kend - k0 : BN);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(base + k0 * stride), (short)0, (int)(nvalid * stride_b), kBufferFlags);
#pragma unroll
    for (int j = 0; j < C::LOADS_PER_WAVE; ++j) {
        const int inst = j * (C::NT / 64) + w;
        const int pos = inst * 64 + lane;
        const int r = pos / C::UPR, u = (pos % C::UPR) ^ swz<C::DB * 32>(r);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(dst + inst * 1024), 16,
                                                 (unsigned)r * stride_b + (unsigned)(u * 16), 0, 0, 0);
    }
}

// Keys of a chunk a lane's row may see, as a range [lo, hi) of key indices
// counted from the chunk's first processed key kbeg: below kend, not after
// the row's position under causal masking, and within the local window.
// Clamped to +-2^30 so that per-tile offsets stay in 32 bits.
struct VisRange {
    int lo, hi;
};

__device__ inline VisRange visible_range(const FwdArgs &a, const LaneRow &r, int64_t cstart, int64_t kbeg,
                                         int64_t kend) {
    const int64_t rel = r.qpos - cstart - kbeg;  // the row's own key index
    int64_t lo = -(1 << 30), hi = kend - kbeg;
    if (a.causal) hi = rel + 1 < hi ? rel + 1 : hi;
    if (a.window > 0) {
        lo = rel - a.window;
        if (!a.causal) hi = rel + a.window + 1 < hi ? rel + a.window + 1 : hi;
    }
    const int64_t big = 1 << 30;
    lo = lo < -big ? -big : (lo > big ? big : lo);
    hi = hi < -big ? -big : (hi > big ? big : hi);
    return VisRange{(int)lo, (int)hi};
}

// Mask the keys a lane's row must not see in a tile whose first key is
// `rel` keys after kbeg: element i of block kb is key 32kb + 8(i/4) + 4g +
// i%4 of the tile, visible iff it lies in [lo - rel, hi - rel).
template <class C>
__device__ inline void mask_scores(f32x16 (&s)[C::KB], VisRange v, int rel, int g) {
    const int hi = v.hi - rel - 4 * g;  // compare against the lane-independent part of the key
    const int lo = v.lo - rel - 4 * g;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = 32 * kb + 8 * (i >> 2) + (i & 3);
            if (key >= hi || key < lo) s[kb][i] = kNegInf;
        }
}

// Keys k0 .. k0+n-1 of a chunk (absolute k0 + cstart) against the rows of
// positions q_offset + tlo .. q_offset + thi: none visible to any row
// (skipped) / all visible to all rows (no mask needed).
__device__ inline bool keys_unseen(const FwdArgs &a, int64_t cstart, int64_t k0, int64_t n, int64_t tlo,
                                   int64_t thi) {
    const int64_t first = cstart + k0, last = first + n - 1;
    if (a.causal && first > a.q_offset + thi) return true;
    if (a.window > 0) {
        if (last < a.q_offset + tlo - a.window) return true;
        if (!a.causal && first > a.q_offset + thi + a.window) return true;
    }
    return false;
}

__device__ inline bool keys_all_seen(const FwdArgs &a, int64_t cstart, int64_t k0, int64_t n, int64_t kend,
                                     int64_t tlo, int64_t thi) {
    const int64_t first = cstart + k0, last = first + n - 1;
    if (k0 + n > kend) return false;
    if (a.causal && last > a.q_offset + tlo) return false;
    if (a.window > 0) {
        if (first < a.q_offset + thi - a.window) return false;
        if (!a.causal && last > a.q_offset + tlo + a.window) return false;
    }
    return true;
}

// keys_unseen / keys_all_seen for every tile of a chunk at once.  A wave
// walks keys kbeg + t*step + woff .. + n-1 for tiles t = 0, 1, ...; both
// tests are monotone in t (each condition holds below or above one bound),
// so once per chunk they reduce to tile-index bounds:
//   unseen(t)   <=>  t < un_lo || t >= un_hi
//   all_seen(t) <=>  fu_lo <= t < fu_hi
// and the tile loop compares 32-bit integers instead of positions.
struct TileSpan {
    int un_lo, un_hi, fu_lo, fu_hi;
    __device__ bool unseen(int t) const { return t < un_lo || t >= un_hi; }
    __device__ bool all_seen(int t) const { return t >= fu_lo && t < fu_hi; }
};

__device__ inline TileSpan tile_span(const FwdArgs &a, int64_t cstart, int64_t kbeg, int64_t kend, int64_t step,
                                     int64_t woff, int64_t n, int64_t tlo, int64_t thi, int ntiles) {
    // tiles t >= 0 with t*step <= v, and the first t with t*step >= v
    auto upto = [&](int64_t v) -> int64_t { return v < 0 ? 0 : v / step + 1; };
    auto from = [&](int64_t v) -> int64_t { return v <= 0 ? 0 : (v + step - 1) / step; };
    auto clamp = [&](int64_t t) -> int { return (int)(t < 0 ? 0 : (t > ntiles ? ntiles : t)); };
    const int64_t base = cstart + kbeg + woff;  // absolute position of the wave's first key of tile 0
    const int64_t W = a.window;
    int64_t un_lo = 0, un_hi = from(kend - kbeg - woff);  // tiles at or past kend hold no key of the wave
    int64_t fu_lo = 0, fu_hi = upto(kend - kbeg - woff - n);
    if (a.causal) {
        un_hi = un_hi < upto(a.q_offset + thi - base) ? un_hi : upto(a.q_offset + thi - base);
        const int64_t f = upto(a.q_offset + tlo - base - n + 1);
        fu_hi = fu_hi < f ? fu_hi : f;
    }
    if (W > 0) {
        un_lo = from(a.q_offset + tlo - W - base - n + 1);
        fu_lo = from(a.q_offset + thi - W - base);
        if (!a.causal) {
            const int64_t u = upto(a.q_offset + thi + W - base);
            un_hi = un_hi < u ? un_hi : u;
            const int64_t f = upto(a.q_offset + tlo + W - base - n + 1);
            fu_hi = fu_hi < f ? fu_hi : f;
        }
    }
    return TileSpan{clamp(un_lo), clamp(un_hi), clamp(fu_lo), clamp(fu_hi)};
}

// ---------------------------------------------------------------------------
// Anchor tokens and segment labels (kernels instantiated with EXT)
// ---------------------------------------------------------------------------
// A query at p also sees the keys at A - 1, A and A + S, A = S floor(p / S),
// whatever the window and causal rules say; with segment labels it sees only
// keys of its own label.  Labels travel with the K tiles (one 4-byte label
// per key, each wave its own keys) and are zero when the call has none.
constexpr int kNoKey = -2147483647 - 1;  // matches no key index

struct Anchors {
    int a0, a1, a2;  // key indices relative to kbeg, or kNoKey
};

// The anchors of a row at position qpos among the keys [kbase, kend) of a
// chunk starting at cstart, relative to kbeg.
__device__ inline Anchors row_anchors(const FwdArgs &a, int64_t qpos, int64_t cstart, int64_t kbase, int64_t kbeg,
                                      int64_t kend) {
    Anchors r{kNoKey, kNoKey, kNoKey};
    if (a.anchor <= 0) return r;
    const int64_t A = qpos / a.anchor * a.anchor - cstart;
    auto pick = [&](int64_t x) { return x >= kbase && x < kend ? (int)(x - kbeg) : kNoKey; };
    r.a0 = pick(A - 1);
    r.a1 = pick(A);
    r.a2 = pick(A + a.anchor);
    return r;
}

// Does the tile of keys k0 .. k0+n-1 (absolute k0 + cstart) hold an anchor of
// a row at positions q_offset + tlo .. q_offset + thi?  Rows spanning more
// than two anchor blocks are answered yes.
__device__ inline bool tile_has_anchor(const FwdArgs &a, int64_t cstart, int64_t k0, int64_t n, int64_t tlo,
                                       int64_t thi) {
    if (a.anchor <= 0) return false;
    const int64_t S = a.anchor;
    const int64_t A0 = (a.q_offset + tlo) / S * S, A1 = (a.q_offset + thi) / S * S;
    if (A1 - A0 > S) return true;
    const int64_t first = cstart + k0, last = first + n - 1;
    auto in = [&](int64_t x) { return x >= first && x <= last; };
    return in(A0 - 1) || in(A0) || in(A0 + S) || in(A1 - 1) || in(A1) || in(A1 + S);
}

// mask_scores with anchors and labels: a key is visible iff (it lies in
// [lo, hi) or is one of the row's anchors) and (LAB) its label (the wave's
// labels of the tile, at lab) equals the row's label ql.
template <class C, bool LAB = true>
__device__ inline void mask_scores_ext(f32x16 (&s)[C::KB], VisRange v, Anchors an, int rel, int g, const char *lab,
                                       int ql) {
    const int off = rel + 4 * g;  // key index of element (0, 0) minus the lane-independent part
    const int hi = v.hi - off, lo = v.lo - off;
    auto shift = [&](int x) { return x == kNoKey ? kNoKey : x - off; };
    const int a0 = shift(an.a0), a1 = shift(an.a1), a2 = shift(an.a2);
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // four keys at a time (few registers live)
            i32x4 lk = {0, 0, 0, 0};
            if constexpr (LAB) lk = *(const i32x4 *)(lab + 4 * (32 * kb + 8 * j + 4 * g));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int key = 32 * kb + 8 * j + e;
                const bool in = (key >= lo && key < hi) || key == a0 || key == a1 || key == a2;
                if (!in || (LAB && lk[e] != ql)) s[kb][4 * j + e] = kNegInf;
            }
        }
}

// The rows' common label L of a wave (uniform = every valid row has it).
__device__ inline void wave_label(int ql, bool ok, int &L, bool &uniform) {
    const uint64_t okm = __builtin_amdgcn_ballot_w64(ok);
    const int first = okm ? __builtin_ctzll(okm) : 0;
    L = __builtin_amdgcn_readlane(ql, first);
    uniform = __builtin_amdgcn_ballot_w64(ok && ql != L) == 0;
}

// Minimum and maximum of x over the workgroup's NW waves (red: 2 NW ints of
// LDS; every wave must call it).
template <int NW>
__device__ inline void wg_min_max(int lo, int hi, int *red, int w, int lane, int &gmin, int &gmax) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const int l2 = __shfl_xor(lo, o), h2 = __shfl_xor(hi, o);
        lo = l2 < lo ? l2 : lo;
        hi = h2 > hi ? h2 : hi;
    }
    if (lane == 0) red[w] = lo, red[NW + w] = hi;
    __syncthreads();
    gmin = red[0], gmax = red[NW];
#pragma unroll
    for (int i = 1; i < NW; ++i) {
        gmin = red[i] < gmin ? red[i] : gmin;
        gmax = red[NW + i] > gmax ? red[NW + i] : gmax;
    }
    __syncthreads();  // red may be written again
}

// First and last key in [k0, k1) of a chunk (labels kseg) whose label lies
// in [lo, hi], over the workgroup's NW waves: kl < kf when there is none.
// With packed documents (labels that never decrease) this is the span of
// the rows' documents.  Each thread keeps kScanLoads label loads in flight
// per pass (indexes past the end re-read the last key, which changes
// neither end), so a pass costs one memory round trip.
constexpr int kScanLoads = 8;
template <int NW>
__device__ inline void label_key_span(const int32_t *kseg, int64_t k0, int64_t k1, int lo, int hi, int *red, int w,
                                      int lane, int64_t &kf, int64_t &kl) {
    constexpr int T = NW * 64;
    const int n = k1 > k0 ? (int)(k1 - k0) : 0;  // chunk lengths stay below 2^31
    const int32_t *p = kseg + k0;
    int first = 2147483647, last = -1;
    for (int base = 0; base < n; base += T * kScanLoads) {
        int r[kScanLoads], L[kScanLoads];
#pragma unroll
        for (int u = 0; u < kScanLoads; ++u) {
            const int i = base + u * T + (int)threadIdx.x;
            r[u] = i < n ? i : n - 1;
            L[u] = p[r[u]];
        }
#pragma unroll
        for (int u = 0; u < kScanLoads; ++u) {
            if (L[u] >= lo && L[u] <= hi) {
                first = r[u] < first ? r[u] : first;
                last = r[u] > last ? r[u] : last;
            }
        }
    }
    int f, l;
    wg_min_max<NW>(first, last, red, w, lane, f, l);
    kf = l < 0 ? 1 : k0 + f;
    kl = l < 0 ? 0 : k0 + l;
}

// Label test of a wave's n (<= 64) tile entries (keys, or rows in the
// dK/dV kernel; the label of entry `lane` at lab; entries at or past nvalid
// do not exist) against each lane's own label x (valid where ok; L and
// uniform as wave_label gives them):
//   all       every entry is visible to every valid lane: no label mask;
//   none      no valid lane shares a label with an entry: the tile is skipped;
//   per_lane  the entries carry one label, so the test reduces to `hit`
//             (x equals it) per lane: a lane without a hit sees nothing.
// A wave whose lanes straddle a document boundary thus masks whole lanes on
// the tiles inside one document instead of testing every element.
struct LabelTest {
    bool all, none, per_lane, hit;
};
// (label_test takes the entry label lk = lab[lane] already read, so that the
// read can be issued ahead of other work.)
__device__ inline LabelTest label_test(int lk, int n, int64_t nvalid, int lane, int x, bool ok, int L, bool uniform) {
    LabelTest t;
    const bool mine = lane < n;
    const bool valid = mine && lane < nvalid;
    const uint64_t vm = __builtin_amdgcn_ballot_w64(valid);
    const int KL = __builtin_amdgcn_readlane(lk, vm ? __builtin_ctzll(vm) : 0);
    const bool kuni = __builtin_amdgcn_ballot_w64(valid && lk != KL) == 0;
    t.hit = ok && x == KL;
    t.per_lane = kuni;
    t.all = kuni && __builtin_amdgcn_ballot_w64(mine && !valid) == 0 && __builtin_amdgcn_ballot_w64(ok && !t.hit) == 0;
    t.none = vm == 0 || (kuni ? __builtin_amdgcn_ballot_w64(t.hit) == 0
                              : uniform && __builtin_amdgcn_ballot_w64(valid && lk == L) == 0);
    return t;
}
__device__ inline LabelTest label_tile(const char *lab, int n, int64_t nvalid, int lane, int x, bool ok, int L,
                                       bool uniform) {
    return label_test(reinterpret_cast<const int *>(lab)[lane], n, nvalid, lane, x, ok, L, uniform);
}

// Every score of a lane without a label hit masked.
template <int N>
__device__ inline void mask_lane(f32x16 (&s)[N], bool hit) {
#pragma unroll
    for (int b = 0; b < N; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[b][i] = hit ? s[b][i] : kNegInf;
}

// Key labels of one wave's 64 keys k0 .. k0+63 of a chunk, HBM -> LDS (one
// dword per lane); zero past kend or when the chunk has none.
__device__ inline void load_labels(const int32_t *kseg, int64_t k0, int64_t kend, char *dst, int lane) {
    const unsigned nvalid = kseg ? (unsigned)(kend - k0 < 64 ? (kend - k0 > 0 ? kend - k0 : 0) : 64) : 0u;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(kseg ? kseg + k0 : nullptr), (short)0, (int)(nvalid * 4), kBufferFlags);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)dst, 4, (unsigned)lane * 4u, 0, 0, 0);
}

// S^T (KB 32-key blocks) = K Q^T from an LDS tile over the NDS reduction
// steps whose K units start at kt, PF fragments in flight.
template <class C, int NDS>
__device__ inline void scores(const char *kt, const int (&kaddr)[C::NKA], const bf16x8 (&qf)[NDS],
                              f32x16 (&s)[C::KB]) {
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
    constexpr int N = NDS * C::KB;
    constexpr int PF = C::PF > 0 ? C::PF : N;
    bf16x8 fr[PF];
#pragma unroll
    for (int n = 0; n < PF && n < N; ++n) fr[n] = kfrag<C>(kt, kaddr, n / C::KB, n % C::KB);
#pragma unroll
    for (int n = 0; n < N; ++n) {
        s[n % C::KB] = mfma(fr[n % PF], qf[n / C::KB], s[n % C::KB]);
        if (n + PF < N) fr[n % PF] = kfrag<C>(kt, kaddr, (n + PF) / C::KB, (n + PF) % C::KB);
        if (C::PF > 0 && n % PF == PF - 1) __builtin_amdgcn_sched_barrier(0);
    }
}

// S^T = K Q^T + bias for the KB key blocks of a tile (the chains start from
// the bias block instead of zero).
template <class C, int NDS>
__device__ inline void scores_biased(const char *kt, const int (&kaddr)[C::NKA], const bf16x8 (&qf)[NDS],
                                     const f32x16 &bias, f32x16 (&s)[C::KB]) {
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) s[kb] = bias;
    constexpr int N = NDS * C::KB;
    constexpr int PF = C::PF > 0 ? C::PF : N;
    bf16x8 fr[PF];
#pragma unroll
    for (int n = 0; n < PF && n < N; ++n) fr[n] = kfrag<C>(kt, kaddr, n / C::KB, n % C::KB);
#pragma unroll
    for (int n = 0; n < N; ++n) {
        s[n % C::KB] = mfma(fr[n % PF], qf[n / C::KB], s[n % C::KB]);
        if (n + PF < N) fr[n % PF] = kfrag<C>(kt, kaddr, (n + PF) / C::KB, (n + PF) % C::KB);
        if (C::PF > 0 && n % PF == PF - 1) __builtin_amdgcn_sched_barrier(0);
    }
}

// Operand fragments (queries, keys) times c, rounded to bf16.
template <int NDS>
__device__ inline void scale_q(bf16x8 (&qf)[NDS], float c) {
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
        const u32x4 u = __builtin_bit_cast(u32x4, qf[ds]);
        u32x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float lo = __builtin_bit_cast(float, u[j] << 16), hi = __builtin_bit_cast(float, u[j] & 0xffff0000u);
            v[j] = pack_bf16(lo * c, hi * c);
        }
        qf[ds] = to_bf16x8(v);
    }
}
// O^T += V^T P^T over the wave's keys of an LDS tile, for the NDB output
// blocks whose V units start at vt, PF fragments in flight.  (Any product
// X^T += T^T Y^T of an LDS tile T with B operands Y^T in the P^T layout.)
template <class C, int NDB>
__device__ inline void accumulate_pv(const char *vt, const int (&vaddr)[2][C::NVD], const bf16x8 (&pf)[2 * C::KB],
                                     f32x16 (&o)[NDB]) {
    constexpr int N = 2 * C::KB * NDB;
    constexpr int PF = C::PF > 0 ? C::PF : N;
    bf16x8 fr[PF];
#pragma unroll
    for (int n = 0; n < PF && n < N; ++n) fr[n] = vfrag<C>(vt, vaddr, n / NDB, n % NDB);
#pragma unroll
    for (int n = 0; n < N; ++n) {
        o[n % NDB] = mfma(fr[n % PF], pf[n / NDB], o[n % NDB]);
        if (n + PF < N) fr[n % PF] = vfrag<C>(vt, vaddr, (n + PF) / NDB, (n + PF) % NDB);
        if (C::PF > 0 && n % PF == PF - 1) __builtin_amdgcn_sched_barrier(0);
    }
}

// Key range of chunk c for this workgroup; returns false when nothing is
// visible.  With a local window the first tile is the one holding the
// earliest key any of the workgroup's rows may see (kbeg moves by whole
// tiles, so tiles stay aligned to the chunk or sub-range start).
__device__ inline bool chunk_range(const FwdArgs &a, const WorkTile &wt, int c, int sub, int64_t &kbeg,
                                   int64_t &kend, int &ntiles, int bn) {
    const ChunkArg &ch = a.chunks[c];
    kbeg = 0;
    kend = ch.len;
    if (a.split_mode) {
        kbeg = sub * a.sub_len;
        kend = kbeg + a.sub_len < ch.len ? kbeg + a.sub_len : ch.len;
    }
    int64_t kstop = kend;
    if (a.causal || a.window > 0) {
        // keys < vis can be visible to the last row
        const int64_t vis = a.q_offset + wt.wg_thi - ch.start + 1 + (a.causal ? 0 : a.window);
        kstop = vis < kstop ? vis : kstop;
    }
    if (a.window > 0) {
        const int64_t lo = a.q_offset + wt.wg_tlo - a.window - ch.start;  // first key the first row may see
        if (lo > kbeg) kbeg += (lo - kbeg) / bn * bn;
    }
    if (kstop <= kbeg) return false;
    ntiles = (int)((kstop - kbeg + bn - 1) / bn);
    return true;
}

// Tiles of chunk c a workgroup walks: the main range of chunk_range, plus
// (kernels with anchors) up to five tiles holding anchors of its rows that
// lie outside it.  Rows spanning more than two anchor blocks take every
// tile of the chunk.  All fields are uniform across the workgroup.
struct TileRange {
    int64_t kbase, kbeg, kend;  // first key of the chunk or sub-range, first main tile, end of keys
    int nmain, ntot;
    // first keys of the anchor tiles outside the main range: six fixed
    // candidate slots and a mask of the used ones, read with constant
    // indices only (a compacted list indexed by the tile counter would live
    // in scratch memory, and every scratch load waits for the tile loads in
    // flight)
    int64_t cand[6];
    unsigned used;
    __device__ int64_t start(int it, int bn) const {
        if (it < nmain) return kbeg + (int64_t)it * bn;
        int j = it - nmain;
        int64_t r = 0;
#pragma unroll
        for (int i = 0; i < 6; ++i) {
            const int u = (used >> i) & 1;
            if (u && j == 0) r = cand[i];
            j -= u;
        }
        return r;
    }
};

// Keys outside [kf, kl] carry no label of the workgroup's rows: (CLAMP) the
// main tiles and (EXT) the anchor tiles are cut to that range.  EXT adds the
// anchor tiles; labels without anchors take CLAMP alone.
template <bool EXT, bool CLAMP = EXT>
__device__ inline bool chunk_tiles(const FwdArgs &a, const WorkTile &wt, int c, int sub, int bn, TileRange &tr,
                                   int64_t kf = 0, int64_t kl = INT64_MAX) {
    const ChunkArg &ch = a.chunks[c];
    tr.kbase = a.split_mode ? sub * a.sub_len : 0;
    int64_t kbeg, kend;
    int nmain = 0;
    if (!chunk_range(a, wt, c, sub, kbeg, kend, nmain, bn)) {
        nmain = 0;
        kbeg = tr.kbase;
        kend = a.split_mode ? (tr.kbase + a.sub_len < ch.len ? tr.kbase + a.sub_len : ch.len) : ch.len;
    }
    if (CLAMP && nmain > 0) {  // main tiles cut to [kf, kl], on the same tile grid
        const int64_t mend = kbeg + (int64_t)nmain * bn;
        const int64_t end = kl < mend ? kl + 1 : mend;
        if (kf > kbeg) kbeg += (kf - kbeg) / bn * bn;
        nmain = end > kbeg ? (int)((end - kbeg + bn - 1) / bn) : 0;
    }
    tr.kbeg = kbeg, tr.kend = kend, tr.nmain = nmain, tr.ntot = nmain;
    tr.used = 0;
#pragma unroll
    for (int i = 0; i < 6; ++i) tr.cand[i] = 0;
    if constexpr (EXT) {
        if (a.anchor > 0 && kend > tr.kbase) {
            const int64_t S = a.anchor;
            const int64_t A0 = (a.q_offset + wt.wg_tlo) / S * S, A1 = (a.q_offset + wt.wg_thi) / S * S;
            if (A1 - A0 > S) {  // every tile of the chunk (within [kf, kl])
                int64_t b0 = tr.kbase;
                const int64_t e = kl < kend ? kl + 1 : kend;
                if (kf > b0) b0 += (kf - b0) / bn * bn;
                tr.kbeg = b0;
                tr.nmain = tr.ntot = e > b0 ? (int)((e - b0 + bn - 1) / bn) : 0;
            } else {
                const int64_t pos[6] = {A0 - 1, A0, A0 + S, A1 - 1, A1, A1 + S};
#pragma unroll
                for (int i = 0; i < 6; ++i) {
                    const int64_t x = pos[i] - ch.start;
                    if (x < tr.kbase || x >= kend || x < kf || x > kl) continue;
                    const int64_t ts = tr.kbase + (x - tr.kbase) / bn * bn;
                    if (ts >= tr.kbeg && ts < tr.kbeg + (int64_t)tr.nmain * bn) continue;
                    bool dup = false;  // the tile of an earlier candidate
#pragma unroll
                    for (int j = 0; j < i; ++j) dup = dup || (((tr.used >> j) & 1) && tr.cand[j] == ts);
                    if (dup) continue;
                    tr.cand[i] = ts;
                    tr.used |= 1u << i;
                    ++tr.ntot;
                }
            }
        }
    }
    return tr.ntot > 0;
}

// ---------------------------------------------------------------------------
// Tile stages: NS statically named K and V buffers per workgroup.  Tile t
// lives in stage t % NS; loads run NS-1 tiles ahead of the compute, and each
// wait lets the loads of later tiles stay in flight.
// ---------------------------------------------------------------------------
// K and V of a tile share one array (K first, V at +TILE); the compiler
// tracks in-flight HBM->LDS loads per array, and a handful of arrays stays
// within what it can tell apart.
#define RA_STAGE_ARRAYS(NS, TILE)                                                      \
    __shared__ __attribute__((aligned(1024))) char kv0[2 * (TILE)];                   \
    __shared__ __attribute__((aligned(1024))) char kv1[2 * (TILE)];                   \
    __shared__ __attribute__((aligned(1024))) char kv2[(NS) > 2 ? 2 * (TILE) : 16];   \
    __shared__ __attribute__((aligned(1024))) char kv3[(NS) > 3 ? 2 * (TILE) : 16];   \
    __shared__ __attribute__((aligned(1024))) char kv4[(NS) > 4 ? 2 * (TILE) : 16];   \
    auto kst = [&](auto u) -> char * {                                                \
        constexpr int U = decltype(u)::value % (NS);                                  \
        if constexpr (U == 0) return kv0;                                             \
        else if constexpr (U == 1) return kv1;                                        \
        else if constexpr (U == 2) return kv2;                                        \
        else if constexpr (U == 3) return kv3;                                        \
        else return kv4;                                                              \
    };                                                                                \
    auto vst = [&](auto u) -> char * { return kst(u) + (TILE); };

template <int N>
using ic = std::integral_constant<int, N>;

// Workgroup barrier for the tile buffers: each wave's own LDS reads and
// writes have completed (lgkmcnt 0) and the compiler may not move memory
// operations across it.  Unlike __syncthreads() it does not wait for the
// wave's in-flight HBM->LDS tile loads (that fence would drain vmcnt and
// serialise the prefetch); their completion is waited for explicitly.
__device__ inline void tile_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// s_waitcnt vmcnt(N) as the builtin rather than asm: the compiler's own wait
// insertion then knows which loads have landed, and does not add a wait for
// every load in flight (the next tile's prefetch included) before the first
// LDS read after a loop back edge.
template <int N>
__device__ inline void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt has six bits");
    // gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt (6:4) and lgkmcnt (11:8) at their maxima
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
}

// Wait until at most `tiles` tiles' loads (LPT load instructions each) of
// this wave are still in flight, then synchronise the workgroup.
template <int LPT>
__device__ inline void wait_tiles_in_flight(int tiles) {
    switch (tiles) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<LPT>(); break;
    case 2: wait_vmcnt<2 * LPT>(); break;
    default: wait_vmcnt<3 * LPT>(); break;
    }
    tile_barrier();
}

// Run f(ic<t % NS>{}, t) for tiles t = 0 .. n-1: the stage of every call is a
// compile-time constant, so each call names its LDS buffers statically.
template <int NS, class F>
__device__ inline void for_tiles(int n, F &&f) {
    static_assert(NS >= 2 && NS <= 5, "2..5 stages");
    for (int t = 0; t < n; t += NS) {
        f(ic<0>{}, t);
        if (t + 1 < n) f(ic<1>{}, t + 1);
        if constexpr (NS > 2) if (t + 2 < n) f(ic<2 % NS>{}, t + 2);
        if constexpr (NS > 3) if (t + 3 < n) f(ic<3 % NS>{}, t + 3);
        if constexpr (NS > 4) if (t + 4 < n) f(ic<4 % NS>{}, t + 4);
    }
}

}  // namespace
}  // namespace ra
