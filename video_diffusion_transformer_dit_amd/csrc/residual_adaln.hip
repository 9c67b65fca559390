// residual_adaln.hip -- gated residual fused with the AdaLN modulation that
// follows it:  x_out = x + gate[b] * y  (stored as bf16), then
// z = LN(x_out) * (1 + scale[b]) + shift[b]  over the stored x_out.
//
// Operations: both named among the fused kernels in the xhh.club summary of
// the SGLang MiniMax-H3 benchmark, Q&A (fused-kernel answer); fusing adjacent
// kernels is the search the Sol-H3 abstract describes, and the stamatios.com
// summary ("Resultado principal") says fusion leaves the arithmetic unchanged.
// In a DiT block each residual update is immediately normalised for the next
// sub-layer, so the unfused pair writes x_out and reads it straight back:
// 6 + 4 = 10 bytes per element.  Fused, x and y are read once and x_out and z
// written once: 8 bytes per element.  The normalisation runs on the bf16
// values actually stored in x_out, so the result equals the unfused pipeline.
//
// Mapping (gfx950): row_group.hpp's, as adaln.hip -- two rows per workgroup,
// each thread two 16-byte vectors of each row of x and of y, all eight loads
// issued first; the residual of both rows is rounded and stored before the
// statistics' barrier, so those stores drain while the waves combine their
// partials.  gate, (1 + scale) and shift of the thread's 16 columns are read
// with the rows and held in registers as fp32 (109 registers, four waves per
// SIMD).  Reading (1 + scale) and shift only after the barrier, as adaln.hip
// does, cut that to 77 registers and six waves per SIMD but measured 705 us
// against 675 us at 1344x768 5 s; so did holding the rows and the vectors
// as bf16, widened at each use (68 registers, 698 us).  The statistics and the modulation are adaln.hip's
// operations in the same order, so z equals dit_adaln_modulate(x_out) bit for
// bit, and a row's result does not depend on where it sits in the batch.
#include "launch.hpp"
#include "row_group.hpp"

namespace dit {
namespace {

template <bool FULL>
__global__ __launch_bounds__(kGroupMaxThreads) void gated_residual_adaln_kernel(
    const u32x4 *x, const u32x4 *y, const u32x4 *__restrict__ gate, const u32x4 *__restrict__ shift,
    const u32x4 *__restrict__ scale, u32x4 *x_out, u32x4 *z, int rows, int N, int C, float inv_d, float eps)
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

    // Both rows of x and y first (rows past the end, and vectors past C, read 0).
    const __amdgpu_buffer_rsrc_t rx = group_rows_rsrc(x + (size_t)r0 * C, nr, C);
    const __amdgpu_buffer_rsrc_t ry = group_rows_rsrc(y + (size_t)r0 * C, nr, C);
    u32x4 xr[kGroupRows][kGroupVecs], yr[kGroupRows][kGroupVecs];
#pragma unroll
    for (int j = 0; j < kGroupRows; ++j)
#pragma unroll
        for (int k = 0; k < kGroupVecs; ++k) {
            const int off = ok[k] ? (j * C + c[k]) * 16 : kOutOfRange;
            xr[j][k] = group_load(rx, off);
            yr[j][k] = group_load(ry, off);
        }

    int b = -1;
    float g[kGroupVecs][8], ps[kGroupVecs][8], sh[kGroupVecs][8];
    auto load_modulation = [&](int sample) {
#pragma unroll
        for (int k = 0; k < kGroupVecs; ++k) {
            const int cc = ok[k] ? c[k] : 0;
            float s[8];
            unpack8(load_cached(gate + (size_t)sample * C + cc), g[k]);
            unpack8(load_cached(scale + (size_t)sample * C + cc), s);
            unpack8(load_cached(shift + (size_t)sample * C + cc), sh[k]);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                ps[k][i] = 1.f + s[i];
        }
        b = sample;
    };

    // Residual update: round once to bf16, store, and keep the stored values.
    float v[kGroupRows][kGroupVecs][8];
#pragma unroll
    for (int j = 0; j < kGroupRows; ++j) {
        const int r = r0 + (j < nr ? j : 0); // a row past the end computes on zeros and stores nothing
        if (r / N != b) // workgroup-uniform
            load_modulation(r / N);
#pragma unroll
        for (int k = 0; k < kGroupVecs; ++k) {
            float xf[8], yf[8], o[8];
            unpack8(xr[j][k], xf);
            unpack8(yr[j][k], yf);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                o[i] = fmaf(g[k][i], yf[i], xf[i]);
            const u32x4 stored = pack8(o);
            if ((FULL || ok[k]) && j < nr)
                store_stream(x_out + (size_t)r * C + c[k], stored);
            unpack8(stored, v[j][k]);
        }
    }

    float mean[kGroupRows], rstd[kGroupRows];
    group_row_stats<FULL>(v, ok, n_t, lane, wave, nw, part, inv_d, eps, mean, rstd);

    // Modulate, round once, store (adaln.hip's expression).
#pragma unroll
    for (int j = 0; j < kGroupRows; ++j) {
        if (j >= nr) // workgroup-uniform
            break;
        const int r = r0 + j;
        if (r / N != b)
            load_modulation(r / N);
#pragma unroll
        for (int k = 0; k < kGroupVecs; ++k) {
            if (FULL || ok[k]) {
                float o[8];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    o[i] = fmaf((v[j][k][i] - mean[j]) * rstd[j], ps[k][i], sh[k][i]);
                store_stream(z + (size_t)r * C + c[k], pack8(o));
            }
        }
    }
}

} // namespace

hipError_t launch_gated_residual_adaln(const void *x, const void *y, const void *gate, const void *shift,
                                       const void *scale, void *x_out, void *z, int64_t rows, int64_t N, int64_t D,
                                       float eps, hipStream_t stream)
{
    const auto *xv = static_cast<const u32x4 *>(x);
    const auto *yv = static_cast<const u32x4 *>(y);
    const auto *gv = static_cast<const u32x4 *>(gate);
    const auto *shv = static_cast<const u32x4 *>(shift);
    const auto *scv = static_cast<const u32x4 *>(scale);
    auto *xo = static_cast<u32x4 *>(x_out);
    auto *zv = static_cast<u32x4 *>(z);
    const int C = (int)(D / 8);
    const RowGroupShape shape = row_group_shape(C);
    const dim3 grid((unsigned)((rows + kGroupRows - 1) / kGroupRows)), block((unsigned)shape.threads);
    const float inv_d = 1.f / (float)D;
    if (shape.full)
        hipLaunchKernelGGL(gated_residual_adaln_kernel<true>, grid, block, 0, stream, xv, yv, gv, shv, scv, xo, zv,
                           (int)rows, (int)N, C, inv_d, eps);
    else
        hipLaunchKernelGGL(gated_residual_adaln_kernel<false>, grid, block, 0, stream, xv, yv, gv, shv, scv, xo, zv,
                           (int)rows, (int)N, C, inv_d, eps);
    return hipGetLastError();
}

} // namespace dit
