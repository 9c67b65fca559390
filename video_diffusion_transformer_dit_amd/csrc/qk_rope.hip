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
// Mapping (gfx950), token-major outputs: each thread handles one 16-byte
// vector (8 channels of one head); a 256-thread workgroup covers 256 vectors
// of one token's q or k row, i.e. 256*8/Dh heads.  (Head-major outputs use
// the same arithmetic on four tokens per workgroup staged through LDS; see
// qk_rmsnorm_rope3d_head_major_kernel.)  The grid is 2-D: x = token, y = part, where parts
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

// The token-major kernel's output store.  A workgroup writes one contiguous
// run of kQKThreads vectors, so the run's start is uniform and fits a buffer
// resource descriptor, with the lane's byte offset in the instruction.  That
// lets the store carry the system-scope bit (sc1) on top of the non-temporal
// hint, which a plain global store cannot express from C++.  At 1344x768 5 s
// it measured 609-612 us against 617-620 us for the global non-temporal store,
// bit-identical; AdaLN, SwiGLU and the block-means variant of this kernel
// gained nothing from it and keep their global stores.
__device__ __forceinline__ void store_run_sc1(u32x4 *run, int vec, int run_vectors, u32x4 v)
{
    constexpr int kRawFormat = 0x00020000; // descriptor dword 3: 32-bit data format, no swizzle or stride
    constexpr int kNtSc1 = 2 | 16;         // cache policy bits: nt, sc1
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc((void *)run, 0, run_vectors * 16, kRawFormat);
    __builtin_amdgcn_raw_buffer_store_b128(v, rd, vec * 16, 0, kNtSc1);
}

// LPH = Dh/8 lanes per head.  half_parts = workgroups per q (or k) row.
// in_stride = vectors from one token's q (or k) to the next token's.
// Outputs token-major [B][N][H][Dh].
template <int LPH>
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
    if (valid) // the workgroup's run: from vector row * VPR + part * kQKThreads on
        store_run_sc1((which ? k_out : q_out) + (size_t)row * VPR + ((int)blockIdx.y - which * half_parts) * kQKThreads,
                      tid, kQKThreads, o);
}

// Head-major outputs [B][H][N][Dh], head plane (b, h) starting `plane`
// vectors after plane (b, h - 1) (plane = N * Dh / 8 when packed).  Packed,
// at 1344x768 5 s a plane is 1953 * 16 KiB, so the planes all start at the
// same offset modulo 4 KiB; a caller-chosen plane stride can pad that away.  Writing one token's
// heads with one store instruction (as the token-major mapping does) then
// sends its 256-byte pieces to the same offset in several planes at once,
// which measured 13-18% slower than token-major output.  Here a workgroup
// loads kHmTokens consecutive tokens of one part (each thread one column,
// four 16-byte loads, every load instruction still 1 KiB of one token row),
// normalises and rotates them as the token-major kernel does, stages the
// results in LDS, and each store instruction then writes one head's
// kHmTokens tokens: kHmTokens * Dh contiguous values of its plane (measured
// 4% faster than storing one token at a time; 2 and 8 tokens were slower).
// The (cos, sin) pairs of the kHmTokens tokens are computed once per
// workgroup, one pair per thread at Dh = 128.
constexpr int kHmTokens = 4;

template <int LPH>
__global__ __launch_bounds__(kQKThreads) void qk_rmsnorm_rope3d_head_major_kernel(
    const u32x4 *q, const u32x4 *k, u32x4 *q_out, u32x4 *k_out, const u32x4 *__restrict__ wq,
    const u32x4 *__restrict__ wk, const int32_t *__restrict__ pos, int N, int B, int H, int VPR, int64_t in_stride,
    int64_t plane, int half_parts, int rows, float inv_dh, float eps, const RotaryPlan plan)
{
    constexpr int kPairs = 4 * LPH;
    __shared__ float2 rot[kHmTokens * kPairs];
    __shared__ u32x4 stage[kHmTokens][kQKThreads];
    const int tid = threadIdx.x;
    const unsigned r0 = blockIdx.x * kHmTokens;
    const int which = (int)blockIdx.y >= half_parts; // 0: q, 1: k
    const int part = (int)blockIdx.y - which * half_parts;
    const int c = part * kQKThreads + tid;
    const bool col_ok = c < VPR;
    const int slot = tid % LPH;

    const u32x4 wraw = load_cached((which ? wk : wq) + slot);
    // Unconditional loads (absent tokens and columns read the group's first
    // row or column and are then zeroed), so no branch waits on the loads.
    u32x4 raw[kHmTokens];
#pragma unroll
    for (int t = 0; t < kHmTokens; ++t) {
        const bool ok = col_ok && r0 + t < (unsigned)rows;
        raw[t] = load_stream((which ? k : q) + (size_t)(ok ? r0 + t : r0) * in_stride + (col_ok ? c : 0));
        if (!ok)
            raw[t] = u32x4{0u, 0u, 0u, 0u};
    }
    for (int e = tid; e < kHmTokens * kPairs; e += kQKThreads) {
        const unsigned r = r0 + e / kPairs;
        const int pr = e % kPairs;
        float2 cs = make_float2(1.f, 0.f);
        if (r < (unsigned)rows) {
            const int32_t *p = pos + 3 * (size_t)(B == 1 ? r : r % (unsigned)N);
            const int axis = plan.axis[pr];
            const int coord = axis == 0 ? p[0] : (axis == 1 ? p[1] : p[2]);
            const double turns = (double)coord * plan.turns_per_unit[pr];
            const float rr = (float)(turns - rint(turns));
            cs = make_float2(__builtin_amdgcn_cosf(rr), __builtin_amdgcn_sinf(rr));
        }
        rot[e] = cs;
    }
    float w[8];
    unpack8(wraw, w);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kHmTokens; ++t) {
        float cs[4], sn[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float2 v = rot[t * kPairs + 4 * slot + j];
            cs[j] = v.x;
            sn[j] = v.y;
        }
        // all lanes active: the DPP group sums inside need every lane
        stage[t][tid] = norm_rotate<LPH>(raw[t], w, cs, sn, inv_dh, eps);
    }
    __syncthreads();

    // Vector m of a head's kHmTokens * LPH run is token m / LPH, slot m % LPH;
    // consecutive threads take consecutive vectors of a run.
    constexpr int kRun = kHmTokens * LPH;
#pragma unroll
    for (int i = 0; i < kHmTokens; ++i) {
        const int idx = tid + kQKThreads * i; // < kHmTokens * kQKThreads
        const int hl = idx / kRun, m = idx % kRun;
        const int t = m / LPH, s = m % LPH;
        const int col = part * kQKThreads + hl * LPH + s;
        const unsigned r = r0 + t;
        if (col < VPR && r < (unsigned)rows) {
            const int h = col / LPH;
            const unsigned b = B == 1 ? 0u : r / (unsigned)N, n = B == 1 ? r : r % (unsigned)N;
            store_stream((which ? k_out : q_out) + ((size_t)b * (unsigned)H + h) * plane + (size_t)n * LPH + s,
                         stage[t][hl * LPH + s]);
        }
    }
}

// Per channel pair: turns per unit coordinate and band axis, from (Dh, bands,
// theta), evaluated once on the host in double.
RotaryPlan make_rotary_plan(int64_t Dh, int d_t, int d_h, int d_w, float theta)
{
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
    (void)d_w;
    return plan;
}

// QK RMSNorm + RoPE fused with the SubBlock block means of its outputs.
// grid (chunks * nb, 2 (q then k), B), 512
// threads.  A workgroup covers one 64-token block and one chunk of 64 vector
// columns (64 * 8 / Dh heads): wave w handles tokens w, w+8, ..., w+56 of the
// block, each across its 64 columns just as the QK kernel handles a token (a
// head is LPH adjacent lanes), stores every normalised, rotated vector, and
// adds the stored bf16 values into eight fp32 sums per lane.  Wave 0 then adds
// the other waves' sums in order and writes the means -- the order of the
// standalone pooling kernel, so the means equal pooling the stored q', k'
// bit for bit, and q', k' equal the QK kernel's bit for bit (same rotary
// arithmetic, same norm_rotate).  The token's (cos, sin) pairs are computed
// once per wave and token, pair p by lane p % 64, and fetched with lane
// shuffles.  Pooling this way costs no HBM traffic beyond QK's own.
constexpr int kQKPoolWaves = 8;
constexpr int kQKPoolTokens = 64; // SubBlock block size

// in_stride = vectors from one token's q (or k) to the next token's (C for
// contiguous inputs, more for q and k inside a fused QKV projection).
// HEAD_MAJOR: q', k' written [B][H][N][Dh] with `plane` vectors between head
// planes; the workgroup's 64 tokens of a head are then 64 * Dh contiguous
// values of its plane.
template <int LPH, bool HEAD_MAJOR>
__global__ __launch_bounds__(kQKPoolWaves * kWave) void qk_rmsnorm_rope3d_pool_kernel(
    const u32x4 *q, const u32x4 *k, u32x4 *q_out, u32x4 *k_out, const u32x4 *__restrict__ wq,
    const u32x4 *__restrict__ wk, const int32_t *__restrict__ pos, float *__restrict__ qp, float *__restrict__ kp,
    int N, int nb, int C, int64_t in_stride, int64_t plane, int chunks, float inv_dh, float eps,
    const RotaryPlan plan)
{
    constexpr int kPerWave = kQKPoolTokens / kQKPoolWaves;
    constexpr int kPairs = 4 * LPH;                       // channel pairs per head
    constexpr int kPairSlots = kPairs > kWave ? kPairs / kWave : 1; // pairs computed per lane
    __shared__ float4 part[kQKPoolWaves - 1][2][kWave];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int chunk = blockIdx.x % chunks, blk = blockIdx.x / chunks;
    const int which = blockIdx.y; // 0: q, 1: k
    const size_t b = blockIdx.z;
    const u32x4 *src = which ? k : q;
    u32x4 *dst = which ? k_out : q_out;
    const int c = chunk * kWave + lane;
    const bool valid = c < C;
    const int n0 = blk * kQKPoolTokens;
    const int count = min(kQKPoolTokens, N - n0);
    const int slot = lane % LPH; // chunks start on head boundaries: c % LPH == lane % LPH

    float w[8];
    unpack8(load_cached((which ? wk : wq) + slot), w);
    double tpu[kPairSlots];
    int axis[kPairSlots];
#pragma unroll
    for (int m = 0; m < kPairSlots; ++m) {
        const int pr = (lane + kWave * m) % kPairs;
        tpu[m] = plan.turns_per_unit[pr];
        axis[m] = plan.axis[pr];
    }

    const size_t row0 = (size_t)b * N + n0;
    const int H = C / LPH, h = c / LPH;
    // output vector of token n0 + n: token-major row, or the head's plane
    const size_t out0 = HEAD_MAJOR ? ((size_t)b * H + h) * plane + (size_t)n0 * LPH + slot : row0 * C + c;
    const size_t out_step = HEAD_MAJOR ? LPH : C;
    u32x4 raw[kPerWave];
#pragma unroll
    for (int t = 0; t < kPerWave; ++t) {
        const int n = wave + kQKPoolWaves * t; // wave-uniform
        raw[t] = (valid && n < count) ? load_stream(src + (row0 + n) * in_stride + c) : u32x4{0u, 0u, 0u, 0u};
    }

    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < kPerWave; ++t) {
        const int n = wave + kQKPoolWaves * t;
        if (n < count) { // wave-uniform
            const int32_t *p = pos + 3 * (size_t)(n0 + n);
            const int p_t = p[0], p_h = p[1], p_w = p[2];
            float2 mine[kPairSlots];
#pragma unroll
            for (int m = 0; m < kPairSlots; ++m) {
                const int coord = axis[m] == 0 ? p_t : (axis[m] == 1 ? p_h : p_w);
                const double turns = (double)coord * tpu[m];
                const float r = (float)(turns - rint(turns));
                mine[m] = make_float2(__builtin_amdgcn_cosf(r), __builtin_amdgcn_sinf(r));
            }
            float cs[4], sn[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int pr = 4 * slot + j;
                const int from = pr % kWave;
                float cj = __shfl(mine[0].x, from, kWave), sj = __shfl(mine[0].y, from, kWave);
#pragma unroll
                for (int m = 1; m < kPairSlots; ++m) {
                    const float cm = __shfl(mine[m].x, from, kWave), sm = __shfl(mine[m].y, from, kWave);
                    cj = pr / kWave == m ? cm : cj;
                    sj = pr / kWave == m ? sm : sj;
                }
                cs[j] = cj;
                sn[j] = sj;
            }
            const u32x4 o = norm_rotate<LPH>(raw[t], w, cs, sn, inv_dh, eps);
            if (valid)
                store_stream(dst + out0 + (size_t)n * out_step, o);
            float f[8];
            unpack8(o, f);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[i] += valid ? f[i] : 0.f;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[i] += 0.f; // the standalone pooling adds the zero vectors of absent tokens
        }
    }
    if (wave > 0) {
        part[wave - 1][0][lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        part[wave - 1][1][lane] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
    __syncthreads();
    if (wave == 0 && valid) {
#pragma unroll
        for (int v = 0; v < kQKPoolWaves - 1; ++v) {
            const float4 lo = part[v][0][lane], hi = part[v][1][lane];
            acc[0] += lo.x, acc[1] += lo.y, acc[2] += lo.z, acc[3] += lo.w;
            acc[4] += hi.x, acc[5] += hi.y, acc[6] += hi.z, acc[7] += hi.w;
        }
        const int Dh = 8 * LPH;
        float *o = (which ? kp : qp) + (((size_t)b * H + h) * nb + blk) * Dh + slot * 8;
        float4 *o4 = reinterpret_cast<float4 *>(o);
        const float cnt = (float)count;
        o4[0] = make_float4(acc[0] / cnt, acc[1] / cnt, acc[2] / cnt, acc[3] / cnt);
        o4[1] = make_float4(acc[4] / cnt, acc[5] / cnt, acc[6] / cnt, acc[7] / cnt);
    }
}

template <int LPH>
hipError_t launch_pool_lph(const u32x4 *q, const u32x4 *k, u32x4 *qo, u32x4 *ko, const u32x4 *wq, const u32x4 *wk,
                           const int32_t *pos, float *qp, float *kp, int B, int N, int C, int64_t in_stride,
                           bool head_major, int64_t plane, float inv_dh, float eps, const RotaryPlan &plan,
                           hipStream_t stream)
{
    const int nb = (N + kQKPoolTokens - 1) / kQKPoolTokens;
    const int chunks = (C + kWave - 1) / kWave;
    const dim3 grid((unsigned)(chunks * nb), 2u, (unsigned)B), block(kQKPoolWaves * kWave);
    if (head_major)
        hipLaunchKernelGGL((qk_rmsnorm_rope3d_pool_kernel<LPH, true>), grid, block, 0, stream, q, k, qo, ko, wq, wk,
                           pos, qp, kp, N, nb, C, in_stride, plane, chunks, inv_dh, eps, plan);
    else
        hipLaunchKernelGGL((qk_rmsnorm_rope3d_pool_kernel<LPH, false>), grid, block, 0, stream, q, k, qo, ko, wq, wk,
                           pos, qp, kp, N, nb, C, in_stride, plane, chunks, inv_dh, eps, plan);
    return hipGetLastError();
}

template <int LPH>
hipError_t launch_lph(const u32x4 *q, const u32x4 *k, u32x4 *qo, u32x4 *ko, const u32x4 *wq, const u32x4 *wk,
                      const int32_t *pos, int rows, int N, int H, int VPR, int64_t in_stride, bool head_major,
                      int64_t plane, float inv_dh, float eps, const RotaryPlan &plan, hipStream_t stream)
{
    const int half_parts = (VPR + kQKThreads - 1) / kQKThreads;
    const dim3 block(kQKThreads);
    if (head_major)
        hipLaunchKernelGGL((qk_rmsnorm_rope3d_head_major_kernel<LPH>),
                           dim3((unsigned)((rows + kHmTokens - 1) / kHmTokens), (unsigned)(2 * half_parts)), block, 0,
                           stream, q, k, qo, ko, wq, wk, pos, N, rows / N, H, VPR, in_stride, plane, half_parts, rows,
                           inv_dh, eps, plan);
    else
        hipLaunchKernelGGL((qk_rmsnorm_rope3d_kernel<LPH>), dim3((unsigned)rows, (unsigned)(2 * half_parts)), block, 0,
                           stream, q, k, qo, ko, wq, wk, pos, N, rows / N, H, VPR, in_stride, half_parts, inv_dh, eps,
                           plan);
    return hipGetLastError();
}

} // namespace

hipError_t launch_qk_rmsnorm_rope3d(const void *q, const void *k, void *q_out, void *k_out, const void *wq,
                                    const void *wk, const int32_t *pos, int64_t rows, int64_t N, int64_t H,
                                    int64_t Dh, int64_t in_token_stride, bool head_major, int64_t out_plane_stride,
                                    int d_t, int d_h, int d_w, float theta, float eps, hipStream_t stream)
{
    const auto *qv = static_cast<const u32x4 *>(q);
    const auto *kv = static_cast<const u32x4 *>(k);
    auto *qo = static_cast<u32x4 *>(q_out);
    auto *ko = static_cast<u32x4 *>(k_out);
    const auto *wqv = static_cast<const u32x4 *>(wq);
    const auto *wkv = static_cast<const u32x4 *>(wk);
    const int VPR = (int)(H * Dh / 8);
    const int64_t in_stride = in_token_stride / 8;
    const int64_t plane = out_plane_stride / 8;
    const float inv_dh = 1.f / (float)Dh;
    const int r = (int)rows, n = (int)N, h = (int)H;

    const RotaryPlan plan = make_rotary_plan(Dh, d_t, d_h, d_w, theta);
#define DIT_QK_LAUNCH(L)                                                                                             \
    launch_lph<L>(qv, kv, qo, ko, wqv, wkv, pos, r, n, h, VPR, in_stride, head_major, plane, inv_dh, eps, plan, stream)
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

hipError_t launch_qk_rmsnorm_rope3d_pool(const void *q, const void *k, void *q_out, void *k_out, const void *wq,
                                         const void *wk, const int32_t *pos, float *q_pooled, float *k_pooled,
                                         int64_t B, int64_t N, int64_t H, int64_t Dh, int64_t in_token_stride,
                                         bool head_major, int64_t out_plane_stride, int d_t, int d_h, int d_w,
                                         float theta, float eps, hipStream_t stream)
{
    const auto *qv = static_cast<const u32x4 *>(q);
    const auto *kv = static_cast<const u32x4 *>(k);
    auto *qo = static_cast<u32x4 *>(q_out);
    auto *ko = static_cast<u32x4 *>(k_out);
    const auto *wqv = static_cast<const u32x4 *>(wq);
    const auto *wkv = static_cast<const u32x4 *>(wk);
    const int C = (int)(H * Dh / 8);
    const float inv_dh = 1.f / (float)Dh;
    const RotaryPlan plan = make_rotary_plan(Dh, d_t, d_h, d_w, theta);
    const int b = (int)B, n = (int)N;
    const int64_t in_stride = in_token_stride / 8;
    const int64_t plane = out_plane_stride / 8;
#define DIT_QK_POOL_LAUNCH(L)                                                                                        \
    launch_pool_lph<L>(qv, kv, qo, ko, wqv, wkv, pos, q_pooled, k_pooled, b, n, C, in_stride, head_major, plane,      \
                       inv_dh, eps, plan, stream)
    switch (Dh) {
    case 16: return DIT_QK_POOL_LAUNCH(2);
    case 32: return DIT_QK_POOL_LAUNCH(4);
    case 64: return DIT_QK_POOL_LAUNCH(8);
    case 128: return DIT_QK_POOL_LAUNCH(16);
    case 256: return DIT_QK_POOL_LAUNCH(32);
    default: return hipErrorInvalidValue;
    }
#undef DIT_QK_POOL_LAUNCH
}

} // namespace dit
