// copy.hip -- plain 16-byte-vector device copy: the streaming ceiling the
// chain's kernels are measured against, and the known-size workload that
// calibrates hardware byte counters.  Same access pattern as the chain's
// streaming kernels: non-temporal 16-byte loads and stores, U vectors in
// flight per thread, one workgroup-width apart.
#include "device_common.hpp"
#include "launch.hpp"

namespace dit {
namespace {

constexpr int kCopyU = 4;
constexpr int kCopyThreads = 256;

__global__ __launch_bounds__(256) void copy16_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                     int64_t nvec)
{
    const int64_t chunk = (int64_t)kCopyThreads * kCopyU;
    for (int64_t c0 = (int64_t)blockIdx.x * chunk + threadIdx.x; c0 < nvec; c0 += (int64_t)gridDim.x * chunk) {
        u32x4 v[kCopyU];
#pragma unroll
        for (int k = 0; k < kCopyU; ++k) {
            const int64_t c = c0 + (int64_t)k * kCopyThreads;
            if (c < nvec)
                v[k] = load_stream(src + c);
        }
#pragma unroll
        for (int k = 0; k < kCopyU; ++k) {
            const int64_t c = c0 + (int64_t)k * kCopyThreads;
            if (c < nvec)
                store_stream(dst + c, v[k]);
        }
    }
}

} // namespace

hipError_t launch_copy16(const void *src, void *dst, int64_t bytes, hipStream_t stream)
{
    const int64_t nvec = bytes / 16;
    const int64_t chunk = (int64_t)kCopyThreads * kCopyU;
    int64_t blocks = (nvec + chunk - 1) / chunk;
    if (blocks > (1 << 20))
        blocks = 1 << 20;
    hipLaunchKernelGGL(copy16_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, stream,
                       static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), nvec);
    return hipGetLastError();
}

} // namespace dit
