// adaln.hip -- fused AdaLN modulation, y = LN(x) * (1 + scale[b]) + shift[b].
//
// Operation: named among the fused kernels in the xhh.club summary of the
// SGLang MiniMax-H3 benchmark, Q&A (fused-kernel answer); LayerNorm without
// affine parameters (biased variance, eps under the root), then the per-sample
// modulation.  Fusing keeps the normalised row in registers, so the row is
// read from HBM once and written once (4 bytes per element, the minimum).
//
// Mapping (gfx950): one 64-lane wavefront per row, four rows per 256-thread
// workgroup.  Lane l holds the 16-byte vectors l, l+64, l+128, ... of its row
// (VPL vectors, 8*VPL values) in registers, so every load instruction of the
// wave reads 1 KiB of contiguous memory.  Row statistics take one pass over
// memory: each lane forms its partial (count, mean, M2) from its registers, and
// the wave combines the partials with the parallel-variance identity
//   M2 = sum_l [ M2_l + n_l (mean_l - mean)^2 ],  mean = sum_l n_l mean_l / D,
// using DPP row sums and cross-half lane swaps, never LDS.  Centring each lane
// on its own mean keeps the squared deviations free of cancellation even for
// rows whose mean is large against their spread.
//
// The modulation vectors are the same for every row of a sample, so for rows
// up to 4096 wide the workgroup first stages (1 + scale) and shift as fp32 in
// LDS (32 KiB), laid out [vector k][half][lane] so each lane's float4 reads
// are contiguous across the wave (no bank conflicts).  That replaces two
// cached loads and sixteen bf16 unpacks per vector per row with four LDS
// reads, which measurably shortens the ALU phase each wave runs between its
// loads and its stores.  A wave whose row belongs to a different sample than
// the workgroup's first row (rows straddling a sample boundary) reads the
// vectors from cache instead, and evaluates the same expression, so a row's
// result does not depend on where it sits in the batch.
#include "device_common.hpp"
#include "launch.hpp"

namespace dit {
namespace {

constexpr int kRowsPerBlock = 256 / kWave;

template <int VPL, bool FULL, bool STAGE>
__global__ __launch_bounds__(256) void adaln_modulate_kernel(const u32x4 *x, const u32x4 *__restrict__ shift,
                                                             const u32x4 *__restrict__ scale, u32x4 *y, int rows,
                                                             int N, int C, float inv_d, float eps)
{
    // [k][half][lane]: elements 4*half .. 4*half+3 of vector lane + 64k.
    __shared__ float4 lds_ps[STAGE ? VPL * 2 * kWave : 1];
    __shared__ float4 lds_sh[STAGE ? VPL * 2 * kWave : 1];

    const int lane = threadIdx.x & (kWave - 1);
    const int row0 = blockIdx.x * kRowsPerBlock;
    const int row = row0 + (threadIdx.x / kWave);
    const int b0 = row0 / N;
    if constexpr (STAGE) {
        for (int c = threadIdx.x; c < C; c += blockDim.x) {
            float s[8], t[8];
            unpack8(load_cached(scale + (size_t)b0 * C + c), s);
            unpack8(load_cached(shift + (size_t)b0 * C + c), t);
            const int at = (c / kWave) * 2 * kWave + (c % kWave);
            lds_ps[at] = make_float4(1.f + s[0], 1.f + s[1], 1.f + s[2], 1.f + s[3]);
            lds_ps[at + kWave] = make_float4(1.f + s[4], 1.f + s[5], 1.f + s[6], 1.f + s[7]);
            lds_sh[at] = make_float4(t[0], t[1], t[2], t[3]);
            lds_sh[at + kWave] = make_float4(t[4], t[5], t[6], t[7]);
        }
        __syncthreads();
    }
    if (row >= rows) // wave-uniform: whole waves retire together
        return;

    const size_t base = (size_t)row * C;

    // Load the lane's share of the row (all loads issued before any use).
    u32x4 raw[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int c = lane + kWave * k;
        raw[k] = u32x4{0u, 0u, 0u, 0u};
        if (FULL || c < C)
            raw[k] = load_stream(x + base + c);
    }
    float v[VPL][8];
    int nvec = 0;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        unpack8(raw[k], v[k]);
        nvec += (FULL || lane + kWave * k < C) ? 1 : 0;
    }

    // Lane partials: sum, then M2 about the lane mean.
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

    // Wave combine (all 64 lanes active here).
    const float mean = wave_sum(lsum) * inv_d;
    const float dm = m_l - mean;
    const float m2 = wave_sum(fmaf(n_l * dm, dm, lm2));
    const float rstd = 1.f / sqrtf(fmaf(m2, inv_d, eps));

    // Normalise, modulate, round once, store.
    const int b = row / N;
    if (STAGE && b == b0) {
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int c = lane + kWave * k;
            if (FULL || c < C) {
                const int at = k * 2 * kWave + lane;
                const float4 p0 = lds_ps[at], p1 = lds_ps[at + kWave];
                const float4 t0 = lds_sh[at], t1 = lds_sh[at + kWave];
                const float ps[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
                const float t[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
                float o[8];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    o[i] = fmaf((v[k][i] - mean) * rstd, ps[i], t[i]);
                store_stream(y + base + c, pack8(o));
            }
        }
    } else {
        const u32x4 *sh = shift + (size_t)b * C;
        const u32x4 *sc = scale + (size_t)b * C;
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int c = lane + kWave * k;
            if (FULL || c < C) {
                float s[8], t[8], o[8];
                unpack8(load_cached(sc + c), s);
                unpack8(load_cached(sh + c), t);
#pragma unroll
                for (int i = 0; i < 8; ++i) // the staged path's expression: same bits in any sample
                    o[i] = fmaf((v[k][i] - mean) * rstd, 1.f + s[i], t[i]);
                store_stream(y + base + c, pack8(o));
            }
        }
    }
}

template <int VPL>
hipError_t launch_vpl(const u32x4 *x, const u32x4 *sh, const u32x4 *sc, u32x4 *y, int rows, int N, int C, float eps,
                      hipStream_t stream)
{
    // Staging needs 64*C bytes of LDS: used for rows up to 512 vectors (4096 wide).
    constexpr bool kStage = VPL <= 8;
    const dim3 grid((rows + kRowsPerBlock - 1) / kRowsPerBlock), block(256);
    const float inv_d = 1.f / (8.f * (float)C);
    if (C == kWave * VPL)
        hipLaunchKernelGGL((adaln_modulate_kernel<VPL, true, kStage>), grid, block, 0, stream, x, sh, sc, y, rows, N,
                           C, inv_d, eps);
    else
        hipLaunchKernelGGL((adaln_modulate_kernel<VPL, false, kStage>), grid, block, 0, stream, x, sh, sc, y, rows, N,
                           C, inv_d, eps);
    return hipGetLastError();
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
    const int r = (int)rows, n = (int)N;
    if (C <= kWave) return launch_vpl<1>(xv, shv, scv, yv, r, n, C, eps, stream);
    if (C <= 2 * kWave) return launch_vpl<2>(xv, shv, scv, yv, r, n, C, eps, stream);
    if (C <= 4 * kWave) return launch_vpl<4>(xv, shv, scv, yv, r, n, C, eps, stream);
    if (C <= 8 * kWave) return launch_vpl<8>(xv, shv, scv, yv, r, n, C, eps, stream);
    return launch_vpl<16>(xv, shv, scv, yv, r, n, C, eps, stream);
}

} // namespace dit
