// merge.hip - combine partial softmax states computed over disjoint key sets
// into the global softmax, and optionally normalise it into the output: the
// "attention fusion layer" of page "从百毫秒到百万Token：长上下文推理优化的
// 工程实践" (section 系统架构设计, item 注意力融合层), which collects the
// per-node local outputs and normalises them with one global softmax.  Also
// the last step of split-KV decoding, whose key ranges play the nodes.
//
// For each row: m = max_i m_i, w_i = e^(m_i - m) (0 for m_i = -inf),
// l = sum_i w_i l_i, O = sum_i w_i O_i, out = O / l (0 when l = 0).
//
// HBM-bound: one wave per row group of 64/(d_v/4) rows would waste lanes for
// small d_v, so each thread owns 4 consecutive elements of one row and the
// workgroup covers 256 threads' worth of (row, element) pairs.  The row's
// n weights are computed by every thread of the row from the m values (n is
// small), so no cross-thread exchange is needed.
#include "ra_internal.h"

namespace ra {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();

__device__ inline unsigned pack_bf16(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

__global__ __launch_bounds__(256) void merge_kernel(const MergeArgs a) {
    const int per_row = a.d_v / 4;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gid / per_row;
    const int e = (int)(gid % per_row) * 4;
    if (row >= a.rows) return;

    float mx = kNegInf;
    for (int i = 0; i < a.n_parts; ++i) mx = fmaxf(mx, a.pm[i * a.rows + row]);
    // weights are branch free (a part with m = -inf gets 0 and holds O = 0), so
    // the loads of consecutive parts are independent and stay in flight together
    const float mref = mx == kNegInf ? 0.f : mx;
    float l = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    int i = 0;
    for (; i + 4 <= a.n_parts; i += 4) {
        float w[4], li[4];
        f32x4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float mi = a.pm[(i + j) * a.rows + row];
            li[j] = a.pl[(i + j) * a.rows + row];
            v[j] = *(const f32x4 *)(a.pO + ((i + j) * a.rows + row) * a.d_v + e);
            w[j] = mi == kNegInf ? 0.f : expf(mi - mref);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            l += w[j] * li[j];
            o += w[j] * v[j];
        }
    }
    for (; i < a.n_parts; ++i) {
        const float mi = a.pm[i * a.rows + row];
        const float w = mi == kNegInf ? 0.f : expf(mi - mref);
        l += w * a.pl[i * a.rows + row];
        o += w * *(const f32x4 *)(a.pO + (i * a.rows + row) * a.d_v + e);
    }
    if (a.m) {
        if (e == 0) {
            a.m[row] = mx;
            a.l[row] = l;
        }
        *(f32x4 *)(a.O + row * a.d_v + e) = o;
    }
    if (a.out) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        if (a.out_bf16) {
            u32x2 v = {pack_bf16(o[0] * inv, o[1] * inv), pack_bf16(o[2] * inv, o[3] * inv)};
            *(u32x2 *)((uint16_t *)a.out + row * a.d_v + e) = v;
        } else {
            *(f32x4 *)((float *)a.out + row * a.d_v + e) = o * inv;
        }
    }
}

}  // namespace

hipError_t launch_merge(const MergeArgs &a, hipStream_t s) {
    const int64_t threads = a.rows * (a.d_v / 4);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace ra
