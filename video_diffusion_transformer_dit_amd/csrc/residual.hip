// residual.hip -- fused gated residual, out = x + gate[b] * y.
//
// Operation: named among the fused kernels in the xhh.club summary of the
// SGLang MiniMax-H3 benchmark, Q&A (fused-kernel answer); the gate is a
// per-sample vector applied raw.  One pass: x and y are read once, out is
// written once (6 bytes per element).
//
// Mapping (gfx950): the grid is (row, segment); a workgroup of up to 256
// threads covers one segment of one row, each thread U 16-byte vectors spaced
// one workgroup-width apart, so each wave instruction touches 1 KiB of
// contiguous memory and every thread has 2U loads in flight.  The sample index
// of a row is one scalar division per workgroup; the gate vector (8 KiB per
// sample) is re-read from cache, never from HBM more than once per XCD.
#include "device_common.hpp"
#include "launch.hpp"

namespace dit {
namespace {

constexpr int kResidualU = 2;

template <int U>
__global__ __launch_bounds__(256) void gated_residual_kernel(const u32x4 *x, const u32x4 *y,
                                                             const u32x4 *__restrict__ gate, u32x4 *out, int N,
                                                             int C)
{
    const int row = blockIdx.x;
    const int b = row / N;
    const size_t base = (size_t)row * C;
    const u32x4 *g = gate + (size_t)b * C;
    const int c0 = blockIdx.y * blockDim.x * U + threadIdx.x;

    u32x4 xv[U], yv[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int c = c0 + k * blockDim.x;
        if (c < C) {
            xv[k] = load_stream(x + base + c);
            yv[k] = load_stream(y + base + c);
        }
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int c = c0 + k * blockDim.x;
        if (c < C) {
            const u32x4 gv = load_cached(g + c);
            u32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float lo = fmaf(bf16_lo(gv[i]), bf16_lo(yv[k][i]), bf16_lo(xv[k][i]));
                const float hi = fmaf(bf16_hi(gv[i]), bf16_hi(yv[k][i]), bf16_hi(xv[k][i]));
                o[i] = pack_bf16x2(lo, hi);
            }
            store_stream(out + base + c, o);
        }
    }
}

} // namespace

hipError_t launch_gated_residual(const void *x, const void *y, const void *gate, void *out, int64_t rows, int64_t N,
                                 int64_t D, hipStream_t stream)
{
    const int C = (int)(D / 8);
    int threads = 256;
    while (threads > kWave && threads / 2 * kResidualU >= C)
        threads /= 2;
    const int per_block = threads * kResidualU;
    const int segs = (C + per_block - 1) / per_block;
    if (segs > 65535)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gated_residual_kernel<kResidualU>), dim3((unsigned)rows, (unsigned)segs), dim3(threads), 0,
                       stream, static_cast<const u32x4 *>(x), static_cast<const u32x4 *>(y),
                       static_cast<const u32x4 *>(gate), static_cast<u32x4 *>(out), (int)N, C);
    return hipGetLastError();
}

} // namespace dit
