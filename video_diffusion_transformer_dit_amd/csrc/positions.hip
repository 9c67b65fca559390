// positions.hip -- packed (t, h, w) token coordinates for the 3D rotary
// embedding.
//
// The stamatios.com summary of the SGLang MiniMax-H3 benchmark, section
// "Resultado principal", describes video and audio tokens sharing one packed
// DiT sequence; "3D RoPE" in the xhh.club Q&A rotates by each token's latent
// coordinate.  Video tokens come first in row-major (t, h, w) order of the
// T x Hg x Wg latent grid; the n_extra tokens after them carry the
// temporal-only coordinate (a, 0, 0), a = their index among the extras.
//
// One thread per token; 12 bytes per token, written once.
#include "device_common.hpp"
#include "launch.hpp"

namespace dit {
namespace {

__global__ __launch_bounds__(256) void packed_positions_kernel(int32_t *__restrict__ pos, int n_total, int n_video,
                                                               int hw, int wg)
{
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= n_total)
        return;
    int t, h, w;
    if (n < n_video) {
        t = n / hw;
        const int rem = n - t * hw;
        h = rem / wg;
        w = rem - h * wg;
    } else {
        t = n - n_video;
        h = 0;
        w = 0;
    }
    int32_t *p = pos + 3 * (size_t)n;
    p[0] = t;
    p[1] = h;
    p[2] = w;
}

} // namespace

hipError_t launch_packed_positions(int32_t *pos, int64_t T, int64_t Hg, int64_t Wg, int64_t n_extra,
                                   hipStream_t stream)
{
    const int64_t n_video = T * Hg * Wg;
    const int64_t n_total = n_video + n_extra;
    const int threads = 256;
    const int blocks = (int)((n_total + threads - 1) / threads);
    hipLaunchKernelGGL(packed_positions_kernel, dim3(blocks), dim3(threads), 0, stream, pos, (int)n_total,
                       (int)n_video, (int)(Hg * Wg), (int)Wg);
    return hipGetLastError();
}

} // namespace dit
