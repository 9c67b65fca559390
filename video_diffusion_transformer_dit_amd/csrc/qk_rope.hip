// qk_rope.hip -- fused per-head RMSNorm of q and k followed by the 3D rotary
// embedding driven by each token's (t, h, w) latent coordinate.
//
// Operation: the xhh.club summary of the SGLang MiniMax-H3 benchmark, Q&A
// (fused-kernel answer), names "QK RMSNorm fused with 3D RoPE".  Per head:
// u = v / sqrt(mean(v^2) + eps) * w, then the head's channels form three
// contiguous bands (t, h, w); in a band of width d at coordinate p the
// adjacent pair (2j, 2j+1) turns counter-clockwise by p * theta^(-2j/d).
// Fused, q and k are read once and written once (8 bytes per channel of q
// and k together), and no cos/sin table is read from memory: the angles come
// from the token's integer coordinate.
//
// Mapping (gfx950): each thread handles one 16-byte vector (8 channels of one
// head); a 256-thread workgroup covers 256 vectors of one token's q or k row,
// i.e. 256*8/Dh heads.  The grid is 2-D: x = token, y = part, where parts
// 0 .. P-1 cover q and P .. 2P-1 cover k.  The dispatcher runs x fastest, so
// each part streams token after token: at any time the workgroups in flight
// read one input stream and write one output stream, which the MI355X
// memory system serves faster than interleaving q, k and both outputs.
//   - A head is Dh/8 adjacent lanes, so its sum of squares is a DPP sum over
//     those lanes (no LDS).
//   - The token's Dh/2 (cos, sin) pairs are computed once per workgroup by
//     its first Dh/2 threads into LDS and read by all: the angle in turns is
//     coordinate * theta^(-2i/d) / (2 pi), formed and reduced to [-1/2, 1/2]
//     in fp64, then fed to the hardware v_cos_f32 / v_sin_f32 (which take
//     turns), so coordinates in the hundreds lose no accuracy.  The per-pair
//     factor theta^(-2i/d) / (2 pi) and band axis depend only on (Dh, bands,
//     theta): the launcher computes them once in double and passes them in
//     the kernel arguments, so no cos/sin table and no exponential is
//     evaluated per token.
#include <math.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace dit {
namespace {

constexpr int kQKThreads = 256;
constexpr int kMaxPairs = 128; // Dh / 2 for Dh <= 256

// Per channel pair i of a head: theta^(-2i'/d) / (2 pi) turns per unit
// coordinate (2i' = the pair's first channel relative to its band start, d =
// the band width) and the coordinate axis (0 = t, 1 = h, 2 = w) of its band.
struct RotaryPlan {
    double turns_per_unit[kMaxPairs];
    int32_t axis[kMaxPairs];
};

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

// LPH = Dh/8 lanes per head.  half_parts = workgroups per q (or k) row.
// in_stride = vectors from one token's q (or k) to the next token's.
// HEAD_MAJOR: outputs [B][H][N][Dh] instead of [B][N][H][Dh].
template <int LPH, bool HEAD_MAJOR>
__global__ __launch_bounds__(kQKThreads) void qk_rmsnorm_rope3d_kernel(
    const u32x4 *q, const u32x4 *k, u32x4 *q_out, u32x4 *k_out, const u32x4 *__restrict__ wq,
    const u32x4 *__restrict__ wk, const int32_t *__restrict__ pos, int N, int B, int H, int VPR, int64_t in_stride,
    int half_parts, float inv_dh, float eps, const RotaryPlan plan)
{
    __shared__ float2 rot[4 * LPH]; // (cos, sin) of each channel pair of a head
    const int tid = threadIdx.x;
    const unsigned row = blockIdx.x;
    const int which = (int)blockIdx.y >= half_parts; // 0: q, 1: k
    const int c = ((int)blockIdx.y - which * half_parts) * kQKThreads + tid;
    const bool valid = c < VPR;
    const int n = B == 1 ? (int)row : (int)(row % (unsigned)N);
    const size_t src = (size_t)row * in_stride + c;
    size_t dst;
    if constexpr (HEAD_MAJOR) {
        const int b = B == 1 ? 0 : (int)(row / (unsigned)N);
        const int h = c / LPH; // LPH is a power of two
        dst = ((size_t)(b * H + h) * N + n) * LPH + (c % LPH);
    } else {
        dst = (size_t)row * VPR + c;
    }

    // The lane's weights and the pair's rotary plan entry are read before the
    // row, so that waiting for them leaves the row load in flight (vector
    // loads complete in order).
    const int slot = tid % LPH; // the lane's 8 channels are 8*slot .. 8*slot+7 of its head
    const u32x4 wraw = load_cached((which ? wk : wq) + slot);
    double turns_per_unit = 0.0;
    int axis = 0;
    if (tid < 4 * LPH) {
        turns_per_unit = plan.turns_per_unit[tid];
        axis = plan.axis[tid];
    }
    // Unconditional load (lanes past the row read the row's first vector and
    // then zero it), so no branch forces a full wait on the plan load above.
    u32x4 raw = load_stream((which ? k : q) + (valid ? src : (size_t)row * in_stride));
    if (!valid)
        raw = u32x4{0u, 0u, 0u, 0u};

    // The token's coordinates are the same for the whole workgroup: three
    // scalar loads, then a per-lane select of the pair's axis.
    const int32_t *p = pos + 3 * (size_t)n;
    const int p_t = p[0], p_h = p[1], p_w = p[2];
    if (tid < 4 * LPH) {
        const int coord = axis == 0 ? p_t : (axis == 1 ? p_h : p_w);
        const double turns = (double)coord * turns_per_unit;
        const float r = (float)(turns - rint(turns));
        rot[tid] = make_float2(__builtin_amdgcn_cosf(r), __builtin_amdgcn_sinf(r));
    }
    float w[8];
    unpack8(wraw, w);
    __syncthreads();
    float cs[4], sn[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float2 t = rot[4 * slot + j];
        cs[j] = t.x;
        sn[j] = t.y;
    }
    // Threads past the last head hold zeros; heads are LPH-aligned and VPR is
    // a multiple of LPH, so every DPP group is wholly in or wholly out.
    const u32x4 o = norm_rotate<LPH>(raw, w, cs, sn, inv_dh, eps);
    if (valid)
        store_stream((which ? k_out : q_out) + dst, o);
}

template <int LPH>
hipError_t launch_lph(const u32x4 *q, const u32x4 *k, u32x4 *qo, u32x4 *ko, const u32x4 *wq, const u32x4 *wk,
                      const int32_t *pos, int rows, int N, int H, int VPR, int64_t in_stride, bool head_major,
                      float inv_dh, float eps, const RotaryPlan &plan, hipStream_t stream)
{
    const int half_parts = (VPR + kQKThreads - 1) / kQKThreads;
    const dim3 grid((unsigned)rows, (unsigned)(2 * half_parts)), block(kQKThreads);
    if (head_major)
        hipLaunchKernelGGL((qk_rmsnorm_rope3d_kernel<LPH, true>), grid, block, 0, stream, q, k, qo, ko, wq, wk, pos,
                           N, rows / N, H, VPR, in_stride, half_parts, inv_dh, eps, plan);
    else
        hipLaunchKernelGGL((qk_rmsnorm_rope3d_kernel<LPH, false>), grid, block, 0, stream, q, k, qo, ko, wq, wk, pos,
                           N, rows / N, H, VPR, in_stride, half_parts, inv_dh, eps, plan);
    return hipGetLastError();
}

} // namespace

hipError_t launch_qk_rmsnorm_rope3d(const void *q, const void *k, void *q_out, void *k_out, const void *wq,
                                    const void *wk, const int32_t *pos, int64_t rows, int64_t N, int64_t H,
                                    int64_t Dh, int64_t in_token_stride, bool head_major, int d_t, int d_h, int d_w,
                                    float theta, float eps, hipStream_t stream)
{
    const auto *qv = static_cast<const u32x4 *>(q);
    const auto *kv = static_cast<const u32x4 *>(k);
    auto *qo = static_cast<u32x4 *>(q_out);
    auto *ko = static_cast<u32x4 *>(k_out);
    const auto *wqv = static_cast<const u32x4 *>(wq);
    const auto *wkv = static_cast<const u32x4 *>(wk);
    const int VPR = (int)(H * Dh / 8);
    const int64_t in_stride = in_token_stride / 8;
    const float inv_dh = 1.f / (float)Dh;
    const int r = (int)rows, n = (int)N, h = (int)H;

    RotaryPlan plan = {};
    const double log2_theta = log2((double)theta);
    for (int i = 0; i < (int)Dh / 2; ++i) {
        const int ch = 2 * i;
        int axis, lo, width;
        if (ch < d_t) {
            axis = 0, lo = 0, width = d_t;
        } else if (ch < d_t + d_h) {
            axis = 1, lo = d_t, width = d_h;
        } else {
            axis = 2, lo = d_t + d_h, width = d_w;
        }
        plan.axis[i] = axis;
        plan.turns_per_unit[i] = exp2(-(double)(ch - lo) / (double)width * log2_theta) / (2.0 * M_PI);
    }
#define DIT_QK_LAUNCH(L) launch_lph<L>(qv, kv, qo, ko, wqv, wkv, pos, r, n, h, VPR, in_stride, head_major, inv_dh, eps, plan, stream)
    switch (Dh) {
    case 8: return DIT_QK_LAUNCH(1);
    case 16: return DIT_QK_LAUNCH(2);
    case 32: return DIT_QK_LAUNCH(4);
    case 64: return DIT_QK_LAUNCH(8);
    case 128: return DIT_QK_LAUNCH(16);
    case 256: return DIT_QK_LAUNCH(32);
    default: return hipErrorInvalidValue;
    }
#undef DIT_QK_LAUNCH
}

} // namespace dit
