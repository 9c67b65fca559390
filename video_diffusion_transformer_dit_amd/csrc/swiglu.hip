// swiglu.hip -- fused SwiGLU activation, out[r][j] = silu(a) * b with
// a = in[r][j], b = in[r][F + j], silu(a) = a / (1 + e^-a).
//
// Operation: named among the fused kernels in the xhh.club summary of the
// SGLang MiniMax-H3 benchmark, Q&A (fused-kernel answer), and in the
// stamatios.com summary, "De onde vêm os ganhos".  Each row of the up
// projection holds the gated half a and the linear half b side by side; the
// fused kernel reads both once and writes the product once (6 bytes per
// output element), with no intermediate silu tensor.
//
// Arithmetic: e^-a = 2^(-a log2 e) on the hardware exp2 (v_exp_f32) and the
// quotient as a times the hardware reciprocal (v_rcp_f32).  For very negative
// a the exponential overflows to +inf and the reciprocal gives 0, so the
// result saturates to (-)0 rather than NaN; for large a it is a * b.
//
// Mapping (gfx950): each thread handles one 16-byte vector (8 outputs); a
// 64-thread workgroup (one wave) covers one 1 KiB segment of an output row.
// The grid is 1-D over (row, segment) tiles in row-major order, so
// consecutive workgroups -- which the dispatcher spreads round-robin over the
// 8 XCDs -- walk consecutive memory in all three streams (a, b, out).  One
// tile per workgroup and a full grid: measured on MI355X, many short-lived
// workgroups keep more requests in flight than fewer workgroups looping over
// tiles or threads holding several vectors, and one-wave workgroups beat
// larger ones: at 1344x768 5 s 1810 us against 1862 us for 256 threads, 2080
// us for 128 and 1915 us for 512, same bits.
#include "device_common.hpp"
#include "launch.hpp"

namespace dit {
namespace {

constexpr int kSwigluThreads = 64;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float silu_mul(float a, float b)
{
    const float e = __builtin_amdgcn_exp2f(-a * kLog2e);
    return a * __builtin_amdgcn_rcpf(1.f + e) * b;
}

// segs is the number of segments per row; when it is a power of two the row
// index is a shift (seg_shift), otherwise a scalar division.
template <bool POW2>
__global__ __launch_bounds__(kSwigluThreads) void swiglu_kernel(const u32x4 *__restrict__ in, u32x4 *__restrict__ out,
                                                                int C, unsigned segs, unsigned seg_shift,
                                                                unsigned tiles)
{
    for (unsigned tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        const unsigned row = POW2 ? tile >> seg_shift : tile / segs;
        const int c = (int)(tile - row * segs) * kSwigluThreads + threadIdx.x;
        if (c < C) {
            const u32x4 *a = in + (size_t)row * 2 * C;
            const u32x4 av = load_stream(a + c);
            const u32x4 bv = load_stream(a + C + c);
            u32x4 r;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                r[i] = pack_bf16x2(silu_mul(bf16_lo(av[i]), bf16_lo(bv[i])), silu_mul(bf16_hi(av[i]), bf16_hi(bv[i])));
            store_stream(out + (size_t)row * C + c, r);
        }
    }
}

// A dispatch holds fewer than 2^32 work-items: beyond 2^24 - 1 workgroups the
// grid stays at that size and workgroups loop over tiles, and the kernel's
// 32-bit tile counter must not wrap on its last step (tile + grid).
constexpr uint64_t kGridCap = (1u << 24) - 1;

uint64_t swiglu_tiles(int64_t M, int64_t F)
{
    const uint64_t segs = (uint64_t)((F / 8 + kSwigluThreads - 1) / kSwigluThreads);
    return (uint64_t)M * segs;
}

} // namespace

bool swiglu_fits(int64_t M, int64_t F)
{
    const uint64_t tiles = swiglu_tiles(M, F);
    return tiles <= 0xffffffffull - (tiles < kGridCap ? tiles : kGridCap);
}

hipError_t launch_swiglu(const void *in, void *out, int64_t M, int64_t F, hipStream_t stream)
{
    const int C = (int)(F / 8);
    const unsigned segs = (unsigned)((C + kSwigluThreads - 1) / kSwigluThreads);
    const uint64_t tiles = swiglu_tiles(M, F);
    const unsigned grid = (unsigned)(tiles < kGridCap ? tiles : kGridCap);
    if (!swiglu_fits(M, F)) // the entry point refuses these sizes first
        return hipErrorInvalidConfiguration;
    const auto *src = static_cast<const u32x4 *>(in);
    auto *dst = static_cast<u32x4 *>(out);
    if ((segs & (segs - 1)) == 0) {
        const unsigned shift = (unsigned)__builtin_ctz(segs);
        hipLaunchKernelGGL((swiglu_kernel<true>), dim3(grid), dim3(kSwigluThreads), 0, stream, src, dst, C, segs,
                           shift, (unsigned)tiles);
    } else {
        hipLaunchKernelGGL((swiglu_kernel<false>), dim3(grid), dim3(kSwigluThreads), 0, stream, src, dst, C, segs,
                           0u, (unsigned)tiles);
    }
    return hipGetLastError();
}

} // namespace dit
