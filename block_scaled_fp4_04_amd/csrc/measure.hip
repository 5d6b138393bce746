// measure.hip -- a load-only pass over a device buffer: what the memory system
// delivers to one kernel that streams bytes once, with nothing else to do.  It
// is the reference point for the decode GEMV, which reads its weight exactly
// once per call (a memory-bound operation: the edge-FP4 article, eefocus.com,
// section on the trade-offs of compute, memory and precision).  Not part of
// the quantization or GEMM path.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"

namespace fp4k {
namespace {

// Each of the grid's threads reads 16-byte words i, i + T, i + 2T, ... (T the
// number of threads), U of them in flight per iteration, with nontemporal loads
// (the data is not reused); the words are folded into an XOR so the loads stay
// live, and the fold is written only when it equals a value that random data
// all but never produces.
template <int U>
__global__ __launch_bounds__(512) void k_read_ceiling(const u32x4 *__restrict__ p, size_t n16,
                                                      uint32_t *__restrict__ sink)
{
    const size_t T = (size_t)gridDim.x * 512;
    size_t i = (size_t)blockIdx.x * 512 + threadIdx.x;
    u32x4 acc = {0, 0, 0, 0};
    for (; i + (U - 1) * T < n16; i += U * T) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * T);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    for (; i < n16; i += T) acc ^= p[i];
    if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x9E3779B9u) sink[0] = 1;
}

}  // namespace

fp4_status launch_read_ceiling(const void *buf, size_t bytes, int grid, uint32_t *sink, hipStream_t st)
{
    hipLaunchKernelGGL(k_read_ceiling<4>, dim3(grid), dim3(512), 0, st, (const u32x4 *)buf, bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

}  // namespace fp4k
