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
// Mapping (gfx950) as in adaln.hip: one wave per row, four rows per
// workgroup, the row's loads issued first, the row held in registers (here
// the stored residual), row statistics from per-lane (count, mean, M2)
// partials combined across the wave with the parallel-variance identity, and
// the per-sample vectors (gate, 1 + scale, shift) staged once per workgroup
// in LDS as fp32 for rows up to 4096 wide (48 KiB).
#include "device_common.hpp"
#include "launch.hpp"

namespace dit {
namespace {

constexpr int kRowsPerBlock = 256 / kWave;

__device__ __forceinline__ void lds_read8(const float4 *base, int at, float out[8])
{
    const float4 a = base[at], b = base[at + kWave];
    out[0] = a.x, out[1] = a.y, out[2] = a.z, out[3] = a.w;
    out[4] = b.x, out[5] = b.y, out[6] = b.z, out[7] = b.w;
}

template <int VPL, bool FULL, bool STAGE>
__global__ __launch_bounds__(256) void gated_residual_adaln_kernel(
    const u32x4 *x, const u32x4 *y, const u32x4 *__restrict__ gate, const u32x4 *__restrict__ shift,
    const u32x4 *__restrict__ scale, u32x4 *x_out, u32x4 *z, int rows, int N, int C, float inv_d, float eps)
{
    // [k][half][lane]: elements 4*half .. 4*half+3 of vector lane + 64k.
    __shared__ float4 lds_g[STAGE ? VPL * 2 * kWave : 1];
    __shared__ float4 lds_ps[STAGE ? VPL * 2 * kWave : 1];
    __shared__ float4 lds_sh[STAGE ? VPL * 2 * kWave : 1];

    const int lane = threadIdx.x & (kWave - 1);
    const int row0 = blockIdx.x * kRowsPerBlock;
    const int row = row0 + (threadIdx.x / kWave);
    const int b0 = row0 / N;
    // The row's loads go out before the staging below: they do not depend on
    // it, so the HBM latency of x and y overlaps the cached reads of the
    // modulation vectors and the barrier (measured 3% faster at 4096 wide).
    // A wave past the last row loads nothing and leaves after the barrier.
    const size_t base = (size_t)row * C;
    u32x4 xr[VPL], yr[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int c = lane + kWave * k;
        xr[k] = yr[k] = u32x4{0u, 0u, 0u, 0u};
        if (row < rows && (FULL || c < C)) {
            xr[k] = load_stream(x + base + c);
            yr[k] = load_stream(y + base + c);
        }
    }

    if constexpr (STAGE) {
        for (int c = threadIdx.x; c < C; c += blockDim.x) {
            float g[8], s[8], t[8];
            unpack8(load_cached(gate + (size_t)b0 * C + c), g);
            unpack8(load_cached(scale + (size_t)b0 * C + c), s);
            unpack8(load_cached(shift + (size_t)b0 * C + c), t);
            const int at = (c / kWave) * 2 * kWave + (c % kWave);
            lds_g[at] = make_float4(g[0], g[1], g[2], g[3]);
            lds_g[at + kWave] = make_float4(g[4], g[5], g[6], g[7]);
            lds_ps[at] = make_float4(1.f + s[0], 1.f + s[1], 1.f + s[2], 1.f + s[3]);
            lds_ps[at + kWave] = make_float4(1.f + s[4], 1.f + s[5], 1.f + s[6], 1.f + s[7]);
            lds_sh[at] = make_float4(t[0], t[1], t[2], t[3]);
            lds_sh[at + kWave] = make_float4(t[4], t[5], t[6], t[7]);
        }
        __syncthreads();
    }
    if (row >= rows) // wave-uniform
        return;

    const int b = row / N;
    const bool staged = STAGE && b == b0; // wave-uniform
    const u32x4 *gv = gate + (size_t)b * C;

    // Residual update: round once to bf16, store, and keep the stored values.
    float v[VPL][8];
    int nvec = 0;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int c = lane + kWave * k;
        if (FULL || c < C) {
            float g[8], xf[8], yf[8], o[8];
            if (staged)
                lds_read8(lds_g, k * 2 * kWave + lane, g);
            else
                unpack8(load_cached(gv + c), g);
            unpack8(xr[k], xf);
            unpack8(yr[k], yf);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                o[i] = fmaf(g[i], yf[i], xf[i]);
            const u32x4 stored = pack8(o);
            store_stream(x_out + base + c, stored);
            unpack8(stored, v[k]);
            ++nvec;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[k][i] = 0.f;
        }
    }

    // Row statistics of the stored residual (see adaln.hip).
    float lsum = 0.f;
#pragma unroll
    for (int k = 0; k < VPL; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            lsum += v[k][i];
    const float n_l = 8.f * (float)nvec;
    const float m_l = nvec > 0 ? lsum / n_l : 0.f;
    float lm2 = 0.f;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const bool valid = FULL || lane + kWave * k < C;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float d = v[k][i] - m_l;
            lm2 = valid ? fmaf(d, d, lm2) : lm2;
        }
    }
    const float mean = wave_sum(lsum) * inv_d;
    const float dm = m_l - mean;
    const float m2 = wave_sum(fmaf(n_l * dm, dm, lm2));
    const float rstd = 1.f / sqrtf(fmaf(m2, inv_d, eps));

    // Modulate, round once, store.
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int c = lane + kWave * k;
        if (FULL || c < C) {
            // One expression on both paths, the same as adaln.hip's: the fused
            // op matches the two separate calls bit for bit, and a row's result
            // does not depend on where it sits in the batch.
            float t[8], o[8];
            if (staged) {
                float ps[8];
                lds_read8(lds_ps, k * 2 * kWave + lane, ps);
                lds_read8(lds_sh, k * 2 * kWave + lane, t);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    o[i] = fmaf((v[k][i] - mean) * rstd, ps[i], t[i]);
            } else {
                float s[8];
                unpack8(load_cached(scale + (size_t)b * C + c), s);
                unpack8(load_cached(shift + (size_t)b * C + c), t);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    o[i] = fmaf((v[k][i] - mean) * rstd, 1.f + s[i], t[i]);
            }
            store_stream(z + base + c, pack8(o));
        }
    }
}

template <int VPL>
hipError_t launch_vpl(const u32x4 *x, const u32x4 *y, const u32x4 *g, const u32x4 *sh, const u32x4 *sc, u32x4 *xo,
                      u32x4 *z, int rows, int N, int C, float eps, hipStream_t stream)
{
    constexpr bool kStage = VPL <= 8; // 96*C bytes of LDS
    const dim3 grid((rows + kRowsPerBlock - 1) / kRowsPerBlock), block(256);
    const float inv_d = 1.f / (8.f * (float)C);
    if (C == kWave * VPL)
        hipLaunchKernelGGL((gated_residual_adaln_kernel<VPL, true, kStage>), grid, block, 0, stream, x, y, g, sh, sc,
                           xo, z, rows, N, C, inv_d, eps);
    else
        hipLaunchKernelGGL((gated_residual_adaln_kernel<VPL, false, kStage>), grid, block, 0, stream, x, y, g, sh, sc,
                           xo, z, rows, N, C, inv_d, eps);
    return hipGetLastError();
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
    const int r = (int)rows, n = (int)N;
    if (C <= kWave) return launch_vpl<1>(xv, yv, gv, shv, scv, xo, zv, r, n, C, eps, stream);
    if (C <= 2 * kWave) return launch_vpl<2>(xv, yv, gv, shv, scv, xo, zv, r, n, C, eps, stream);
    if (C <= 4 * kWave) return launch_vpl<4>(xv, yv, gv, shv, scv, xo, zv, r, n, C, eps, stream);
    if (C <= 8 * kWave) return launch_vpl<8>(xv, yv, gv, shv, scv, xo, zv, r, n, C, eps, stream);
    return launch_vpl<16>(xv, yv, gv, shv, scv, xo, zv, r, n, C, eps, stream);
}

} // namespace dit
