// stage_check.hip - perturbations of the staged ring for validating its
// ordering (page "Ring Attention：百万 Token 上下文的秘密", §3.2 通信-计算重叠:
// a step may read a received block only once it has arrived, and a buffer
// may be refilled only once the step reading it is done).  A context can
// delay the side stream before each staging copy and the compute stream
// before each launch with a bounded spin, and overwrite each staging buffer
// with NaN right after the step that read it.  With correct event ordering
// none of this changes a single output bit; a missing wait turns into stale
// or NaN values.
#include "ra_internal.h"

namespace ra {
namespace {

// Spin one wave for `ticks` of the constant 100 MHz real-time counter; always
// exits (the bound is the caller's and is capped on the host).
__global__ __launch_bounds__(64) void spin_kernel(uint64_t ticks) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__builtin_amdgcn_s_memrealtime() - t0 < ticks) __builtin_amdgcn_s_sleep(1);
}

// Fill n 16-byte units at p with all-ones bytes (NaN in bf16 and fp32).
__global__ __launch_bounds__(256) void fill_kernel(uint4 *p, size_t n) {
    const uint4 ones = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = ones;
}

}  // namespace

hipError_t launch_spin(uint32_t microseconds, hipStream_t s) {
    hipLaunchKernelGGL(spin_kernel, dim3(1), dim3(64), 0, s, (uint64_t)microseconds * 100u);
    return hipGetLastError();
}

hipError_t launch_fill_nan(void *p, size_t bytes, hipStream_t s) {
    const size_t n = bytes / 16;  // staging buffers are whole 16-byte units
    if (n == 0) return hipSuccess;
    const size_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint4 *)p, n);
    return hipGetLastError();
}

}  // namespace ra
