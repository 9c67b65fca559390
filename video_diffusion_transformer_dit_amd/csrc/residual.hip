// residual.hip -- fused gated residual, out = x + gate[b] * y.
//
// Operation: named among the fused kernels in the xhh.club summary of the
// SGLang MiniMax-H3 benchmark, Q&A (fused-kernel answer); the gate is a
// per-sample vector applied raw.  One pass: x and y are read once, out is
// written once (6 bytes per element).
//
// Mapping (gfx950): each thread handles one 16-byte vector; a 64-thread
// workgroup (one wave) covers one segment of 64 vectors (1 KiB of each
// stream).  The grid is 1-D over (row, segment) tiles in row-major order, one
// tile per workgroup, so consecutive workgroups stream consecutive memory.
// One-wave workgroups measured 465 us at 1344x768 5 s against 471-476 us for
// 128, 256 or 512 threads (same bits).  The gate
// vector (8 KiB per sample) is re-read from cache.  With a single sample the
// sample index is 0 and no division is needed.
#include "device_common.hpp"
#include "launch.hpp"

namespace dit {
namespace {

constexpr int kResidualThreads = 64;

template <bool POW2>
__global__ __launch_bounds__(kResidualThreads) void gated_residual_kernel(const u32x4 *x, const u32x4 *y,
                                                                          const u32x4 *__restrict__ gate, u32x4 *out,
                                                                          int N, int B, int C, unsigned segs,
                                                                          unsigned seg_shift, unsigned tiles)
{
    for (unsigned tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        const unsigned row = POW2 ? tile >> seg_shift : tile / segs;
        const int c = (int)(tile - row * segs) * kResidualThreads + threadIdx.x;
        if (c < C) {
            const int b = B == 1 ? 0 : (int)row / N;
            const size_t at = (size_t)row * C + c;
            const u32x4 xv = load_stream(x + at);
            const u32x4 yv = load_stream(y + at);
            const u32x4 gv = load_cached(gate + (size_t)b * C + c);
            u32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                o[i] = pack_bf16x2(fmaf(bf16_lo(gv[i]), bf16_lo(yv[i]), bf16_lo(xv[i])),
                                   fmaf(bf16_hi(gv[i]), bf16_hi(yv[i]), bf16_hi(xv[i])));
            store_stream(out + at, o);
        }
    }
}

// A dispatch holds fewer than 2^32 work-items: beyond 2^23 - 1 workgroups the
// grid stays at that size and workgroups loop over tiles, and the kernel's
// 32-bit tile counter must not wrap on its last step (tile + grid).
constexpr uint64_t kGridCap = (1u << 23) - 1;

uint64_t residual_tiles(int64_t rows, int64_t D)
{
    const uint64_t segs = (uint64_t)((D / 8 + kResidualThreads - 1) / kResidualThreads);
    return (uint64_t)rows * segs;
}

} // namespace

bool gated_residual_fits(int64_t rows, int64_t D)
{
    const uint64_t tiles = residual_tiles(rows, D);
    return tiles <= 0xffffffffull - (tiles < kGridCap ? tiles : kGridCap);
}

hipError_t launch_gated_residual(const void *x, const void *y, const void *gate, void *out, int64_t rows, int64_t N,
                                 int64_t D, hipStream_t stream)
{
    const int C = (int)(D / 8);
    const unsigned segs = (unsigned)((C + kResidualThreads - 1) / kResidualThreads);
    const uint64_t tiles = residual_tiles(rows, D);
    const unsigned grid = (unsigned)(tiles < kGridCap ? tiles : kGridCap); // < 2^32 work-items
    if (!gated_residual_fits(rows, D)) // the entry point refuses these sizes first
        return hipErrorInvalidConfiguration;
    const int B = (int)(rows / N);
    const auto *xv = static_cast<const u32x4 *>(x);
    const auto *yv = static_cast<const u32x4 *>(y);
    const auto *gv = static_cast<const u32x4 *>(gate);
    auto *ov = static_cast<u32x4 *>(out);
    if ((segs & (segs - 1)) == 0) {
        const unsigned shift = (unsigned)__builtin_ctz(segs);
        hipLaunchKernelGGL((gated_residual_kernel<true>), dim3(grid), dim3(kResidualThreads), 0, stream, xv, yv, gv,
                           ov, (int)N, B, C, segs, shift, (unsigned)tiles);
    } else {
        hipLaunchKernelGGL((gated_residual_kernel<false>), dim3(grid), dim3(kResidualThreads), 0, stream, xv, yv, gv,
                           ov, (int)N, B, C, segs, 0u, (unsigned)tiles);
    }
    return hipGetLastError();
}

} // namespace dit
