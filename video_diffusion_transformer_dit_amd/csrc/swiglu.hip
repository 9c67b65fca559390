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
// Mapping (gfx950): grid (row, segment), each thread U 16-byte vectors of a
// and of b in flight, spaced one workgroup-width apart (1 KiB contiguous per
// wave instruction).
#include "device_common.hpp"
#include "launch.hpp"

namespace dit {
namespace {

constexpr int kSwigluU = 4;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float silu_mul(float a, float b)
{
    const float e = __builtin_amdgcn_exp2f(-a * kLog2e);
    return a * __builtin_amdgcn_rcpf(1.f + e) * b;
}

template <int U>
__global__ __launch_bounds__(256) void swiglu_kernel(const u32x4 *__restrict__ in, u32x4 *__restrict__ out, int C)
{
    const size_t row = blockIdx.x;
    const u32x4 *a = in + row * 2 * C;
    const u32x4 *bh = a + C;
    u32x4 *o = out + row * C;
    const int c0 = blockIdx.y * blockDim.x * U + threadIdx.x;

    u32x4 av[U], bv[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int c = c0 + k * blockDim.x;
        if (c < C) {
            av[k] = load_stream(a + c);
            bv[k] = load_stream(bh + c);
        }
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int c = c0 + k * blockDim.x;
        if (c < C) {
            u32x4 r;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                r[i] = pack_bf16x2(silu_mul(bf16_lo(av[k][i]), bf16_lo(bv[k][i])),
                                   silu_mul(bf16_hi(av[k][i]), bf16_hi(bv[k][i])));
            store_stream(o + c, r);
        }
    }
}

} // namespace

hipError_t launch_swiglu(const void *in, void *out, int64_t M, int64_t F, hipStream_t stream)
{
    const int C = (int)(F / 8);
    int threads = 256;
    while (threads > kWave && threads / 2 * kSwigluU >= C)
        threads /= 2;
    const int per_block = threads * kSwigluU;
    const int segs = (C + per_block - 1) / per_block;
    if (segs > 65535)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((swiglu_kernel<kSwigluU>), dim3((unsigned)M, (unsigned)segs), dim3(threads), 0, stream,
                       static_cast<const u32x4 *>(in), static_cast<u32x4 *>(out), C);
    return hipGetLastError();
}

} // namespace dit
