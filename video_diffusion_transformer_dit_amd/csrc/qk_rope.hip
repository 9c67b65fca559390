// qk_rope.hip -- fused per-head RMSNorm of q and k followed by the 3D rotary
// embedding driven by each token's (t, h, w) latent coordinate.
//
// Operation: the xhh.club summary of the SGLang MiniMax-H3 benchmark, Q&A
// (fused-kernel answer), names "QK RMSNorm fused with 3D RoPE".  Per head:
// u = v / sqrt(mean(v^2) + eps) * w, then the head's channels form three
// contiguous bands (t, h, w); in a band of width d at coordinate p the
// adjacent pair (2j, 2j+1) turns counter-clockwise by p * theta^(-2j/d).
// Fused, q and k are read once and written once (8 bytes per channel pair of
// q and k together), and no cos/sin table is read: the angles come from the
// token's integer coordinate in registers.
//
// Mapping (gfx950): one 64-lane wavefront per token at a time, four waves per
// 256-thread workgroup, waves striding over the tokens.  A head of Dh channels is Dh/8 lanes holding 8 channels (16 bytes)
// each, so a wave instruction covers 64*8 channels = 512/Dh heads and lane l
// always holds channels 8*(l mod Dh/8) .. +7 of some head.  Hence:
//   - the head's sum of squares is a DPP sum over Dh/8 adjacent lanes;
//   - a lane's 4 channel pairs, their bands and frequencies are fixed for the
//     whole kernel (computed once, in fp64, as turns per unit coordinate);
//   - per token a lane evaluates 4 (cos, sin) pairs, reused for every head of
//     q and of k.
// The angle is reduced to [-1/2, 1/2] turn in fp64 before the hardware sine
// and cosine (v_sin_f32 / v_cos_f32 take turns), so coordinates in the
// hundreds lose no accuracy.
#include "device_common.hpp"
#include "launch.hpp"

namespace dit {
namespace {

constexpr int kTokensPerBlock = 256 / kWave;
constexpr int kGroup = 8; // vectors per lane per tensor loaded together
// Waves loop over tokens; the grid is capped so each wave amortises its
// per-lane constants over several tokens while still oversubscribing the
// 256 CUs many times.
constexpr int kMaxBlocks = 2048;

template <int LPH>
__device__ __forceinline__ u32x4 norm_rotate(u32x4 raw, const float w[8], const float cs[4], const float sn[4],
                                             float inv_dh, float eps)
{
    float v[8];
    unpack8(raw, v);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        ss = fmaf(v[i], v[i], ss);
    ss = group_sum<LPH>(ss);
    const float rstd = __builtin_amdgcn_rsqf(fmaf(ss, inv_dh, eps));
    float o[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float u0 = v[2 * j] * rstd * w[2 * j];
        const float u1 = v[2 * j + 1] * rstd * w[2 * j + 1];
        o[2 * j] = fmaf(u0, cs[j], -u1 * sn[j]);
        o[2 * j + 1] = fmaf(u0, sn[j], u1 * cs[j]);
    }
    return pack8(o);
}

template <int LPH>
__global__ __launch_bounds__(256) void qk_rmsnorm_rope3d_kernel(const u32x4 *q, const u32x4 *k, u32x4 *q_out,
                                                                u32x4 *k_out, const u32x4 *__restrict__ wq,
                                                                const u32x4 *__restrict__ wk,
                                                                const int32_t *__restrict__ pos, int rows, int N,
                                                                int VPR, int d_t, int d_h, int d_w, double log2_theta,
                                                                float inv_dh, float eps)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = blockIdx.x * kTokensPerBlock + (threadIdx.x / kWave);
    const int nwaves = gridDim.x * kTokensPerBlock;

    // Lane constants, fixed for every token this wave visits: the lane's slot
    // inside a head, its 8 weights of q and of k, and for each of its 4
    // channel pairs the band axis and theta^(-2i/d) / (2 pi) turns per unit
    // coordinate (2i = the pair's first channel relative to its band start).
    const int slot = lane % LPH;
    float wqf[8], wkf[8];
    unpack8(load_cached(wq + slot), wqf);
    unpack8(load_cached(wk + slot), wkf);
    int axis[4];
    double turns_per_unit[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int ch = slot * 8 + 2 * j;
        int lo, width;
        if (ch < d_t) {
            axis[j] = 0, lo = 0, width = d_t;
        } else if (ch < d_t + d_h) {
            axis[j] = 1, lo = d_t, width = d_h;
        } else {
            axis[j] = 2, lo = d_t + d_h, width = d_w;
        }
        turns_per_unit[j] = exp2(-(double)(ch - lo) / (double)width * log2_theta) * 0.15915494309189535;
    }

    for (int row = wave; row < rows; row += nwaves) { // wave-uniform loop
        const int n = row % N;
        const int32_t *p = pos + 3 * (size_t)n;
        const int coord[3] = {p[0], p[1], p[2]};
        float cs[4], sn[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const double turns = (double)coord[axis[j]] * turns_per_unit[j];
            const float r = (float)(turns - rint(turns)); // [-1/2, 1/2] turn
            cs[j] = __builtin_amdgcn_cosf(r);
            sn[j] = __builtin_amdgcn_sinf(r);
        }

        const size_t base = (size_t)row * VPR;
        for (int g0 = 0; g0 < VPR; g0 += kGroup * kWave) {
            u32x4 qv[kGroup], kv[kGroup];
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                const int c = g0 + lane + kWave * i;
                qv[i] = kv[i] = u32x4{0u, 0u, 0u, 0u};
                if (c < VPR) {
                    qv[i] = load_stream(q + base + c);
                    kv[i] = load_stream(k + base + c);
                }
            }
            // Lanes past the last head hold zeros; whole heads are either in or
            // out (VPR is a multiple of LPH), so the group sums stay per head.
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                const int c = g0 + lane + kWave * i;
                const u32x4 r = norm_rotate<LPH>(qv[i], wqf, cs, sn, inv_dh, eps);
                if (c < VPR)
                    store_stream(q_out + base + c, r);
            }
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                const int c = g0 + lane + kWave * i;
                const u32x4 r = norm_rotate<LPH>(kv[i], wkf, cs, sn, inv_dh, eps);
                if (c < VPR)
                    store_stream(k_out + base + c, r);
            }
        }
    }
}

template <int LPH>
hipError_t launch_lph(const u32x4 *q, const u32x4 *k, u32x4 *qo, u32x4 *ko, const u32x4 *wq, const u32x4 *wk,
                      const int32_t *pos, int rows, int N, int VPR, int d_t, int d_h, int d_w, double log2_theta,
                      float inv_dh, float eps, hipStream_t stream)
{
    const int blocks = (rows + kTokensPerBlock - 1) / kTokensPerBlock;
    const dim3 grid(blocks < kMaxBlocks ? blocks : kMaxBlocks), block(256);
    hipLaunchKernelGGL((qk_rmsnorm_rope3d_kernel<LPH>), grid, block, 0, stream, q, k, qo, ko, wq, wk, pos, rows, N,
                       VPR, d_t, d_h, d_w, log2_theta, inv_dh, eps);
    return hipGetLastError();
}

} // namespace

hipError_t launch_qk_rmsnorm_rope3d(const void *q, const void *k, void *q_out, void *k_out, const void *wq,
                                    const void *wk, const int32_t *pos, int64_t rows, int64_t N, int64_t H,
                                    int64_t Dh, int d_t, int d_h, int d_w, float theta, float eps, hipStream_t stream)
{
    const auto *qv = static_cast<const u32x4 *>(q);
    const auto *kv = static_cast<const u32x4 *>(k);
    auto *qo = static_cast<u32x4 *>(q_out);
    auto *ko = static_cast<u32x4 *>(k_out);
    const auto *wqv = static_cast<const u32x4 *>(wq);
    const auto *wkv = static_cast<const u32x4 *>(wk);
    const int VPR = (int)(H * Dh / 8);
    const double log2_theta = log2((double)theta);
    const float inv_dh = 1.f / (float)Dh;
    const int r = (int)rows, n = (int)N;
    switch (Dh) {
    case 8: return launch_lph<1>(qv, kv, qo, ko, wqv, wkv, pos, r, n, VPR, d_t, d_h, d_w, log2_theta, inv_dh, eps, stream);
    case 16: return launch_lph<2>(qv, kv, qo, ko, wqv, wkv, pos, r, n, VPR, d_t, d_h, d_w, log2_theta, inv_dh, eps, stream);
    case 32: return launch_lph<4>(qv, kv, qo, ko, wqv, wkv, pos, r, n, VPR, d_t, d_h, d_w, log2_theta, inv_dh, eps, stream);
    case 64: return launch_lph<8>(qv, kv, qo, ko, wqv, wkv, pos, r, n, VPR, d_t, d_h, d_w, log2_theta, inv_dh, eps, stream);
    case 128: return launch_lph<16>(qv, kv, qo, ko, wqv, wkv, pos, r, n, VPR, d_t, d_h, d_w, log2_theta, inv_dh, eps, stream);
    case 256: return launch_lph<32>(qv, kv, qo, ko, wqv, wkv, pos, r, n, VPR, d_t, d_h, d_w, log2_theta, inv_dh, eps, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace dit
