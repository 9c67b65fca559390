// adaln.hip -- fused AdaLN modulation, y = LN(x) * (1 + scale[b]) + shift[b].
//
// Operation: named among the fused kernels in the xhh.club summary of the
// SGLang MiniMax-H3 benchmark, Q&A (fused-kernel answer); LayerNorm without
// affine parameters (biased variance, eps under the root), then the per-sample
// modulation.  Fusing keeps the normalised row in registers, so the row is
// read from HBM once and written once (4 bytes per element, the minimum).
//
// Mapping (gfx950): row_group.hpp's -- two rows per workgroup, each thread
// two 16-byte vectors of each row, all loads issued first through a buffer
// descriptor over the workgroup's rows, one-pass (count, sum, M2) statistics
// combined across the wave by DPP and across the waves through LDS after one
// barrier for both rows.  Each thread keeps (1 + scale) and shift of its 16
// columns in registers as fp32, so the expression below is the same for every
// row of every sample.
#include "launch.hpp"
#include "row_group.hpp"

namespace dit {
namespace {

template <bool FULL>
__global__ __launch_bounds__(kGroupMaxThreads) void adaln_modulate_kernel(const u32x4 *x,
                                                                          const u32x4 *__restrict__ shift,
                                                                          const u32x4 *__restrict__ scale, u32x4 *y,
                                                                          int rows, int N, int C, float inv_d,
                                                                          float eps)
{
    __shared__ float4 part[kGroupRows * kGroupMaxWaves];
    const int T = blockDim.x, tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave, nw = T / kWave;
    const int r0 = blockIdx.x * kGroupRows;
    const int nr = min(rows - r0, kGroupRows);
    int c[kGroupVecs];
    bool ok[kGroupVecs];
    int nvec = 0;
#pragma unroll
    for (int k = 0; k < kGroupVecs; ++k) {
        c[k] = tid + T * k;
        ok[k] = FULL || c[k] < C;
        nvec += ok[k] ? 1 : 0;
    }
    const float n_t = 8.f * (float)nvec;

    // Both rows' loads first (rows past the end, and vectors past C, read 0).
    const __amdgpu_buffer_rsrc_t rx = group_rows_rsrc(x + (size_t)r0 * C, nr, C);
    u32x4 raw[kGroupRows][kGroupVecs];
#pragma unroll
    for (int j = 0; j < kGroupRows; ++j)
#pragma unroll
        for (int k = 0; k < kGroupVecs; ++k)
            raw[j][k] = group_load(rx, ok[k] ? (j * C + c[k]) * 16 : kOutOfRange);

    int b = -1;
    float ps[kGroupVecs][8], sh[kGroupVecs][8];
    auto load_modulation = [&](int sample) {
#pragma unroll
        for (int k = 0; k < kGroupVecs; ++k) {
            const int cc = ok[k] ? c[k] : 0;
            float s[8];
            unpack8(load_cached(scale + (size_t)sample * C + cc), s);
            unpack8(load_cached(shift + (size_t)sample * C + cc), sh[k]);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                ps[k][i] = 1.f + s[i];
        }
        b = sample;
    };

    float v[kGroupRows][kGroupVecs][8];
#pragma unroll
    for (int j = 0; j < kGroupRows; ++j)
#pragma unroll
        for (int k = 0; k < kGroupVecs; ++k)
            unpack8(raw[j][k], v[j][k]);
    float mean[kGroupRows], rstd[kGroupRows];
    group_row_stats<FULL>(v, ok, n_t, lane, wave, nw, part, inv_d, eps, mean, rstd);

    // Normalise, modulate, round once, store.  The modulation vectors are read
    // here, after the barrier, not right after the rows' loads: that order
    // measured 338 us against 330 us at 1344x768 5 s.
#pragma unroll
    for (int j = 0; j < kGroupRows; ++j) {
        if (j >= nr) // workgroup-uniform
            break;
        const int r = r0 + j;
        if (r / N != b) // the first row, or a second row that starts a new sample (workgroup-uniform)
            load_modulation(r / N);
#pragma unroll
        for (int k = 0; k < kGroupVecs; ++k) {
            if (FULL || ok[k]) {
                float o[8];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    o[i] = fmaf((v[j][k][i] - mean[j]) * rstd[j], ps[k][i], sh[k][i]);
                store_stream(y + (size_t)r * C + c[k], pack8(o));
            }
        }
    }
}

} // namespace

hipError_t launch_adaln_modulate(const void *x, const void *shift, const void *scale, void *y, int64_t rows, int64_t N,
                                 int64_t D, float eps, hipStream_t stream)
{
    const auto *xv = static_cast<const u32x4 *>(x);
    const auto *shv = static_cast<const u32x4 *>(shift);
    const auto *scv = static_cast<const u32x4 *>(scale);
    auto *yv = static_cast<u32x4 *>(y);
    const int C = (int)(D / 8);
    const RowGroupShape shape = row_group_shape(C);
    const dim3 grid((unsigned)((rows + kGroupRows - 1) / kGroupRows)), block((unsigned)shape.threads);
    const float inv_d = 1.f / (float)D;
    if (shape.full)
        hipLaunchKernelGGL(adaln_modulate_kernel<true>, grid, block, 0, stream, xv, shv, scv, yv, (int)rows, (int)N,
                           C, inv_d, eps);
    else
        hipLaunchKernelGGL(adaln_modulate_kernel<false>, grid, block, 0, stream, xv, shv, scv, yv, (int)rows, (int)N,
                           C, inv_d, eps);
    return hipGetLastError();
}

} // namespace dit
