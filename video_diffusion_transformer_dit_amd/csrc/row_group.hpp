// row_group.hpp -- the row mapping shared by AdaLN (adaln.hip) and the fused
// residual -> AdaLN (residual_adaln.hip), so that the two compute a row's
// statistics with the same operations in the same order and the fused op
// equals the two separate calls bit for bit.
//
// A workgroup of T threads (T = 256 at 4096 wide) owns kGroupRows = 2
// consecutive rows.  Thread t holds the 16-byte vectors t and t + T of each
// of them (kGroupVecs = 2), so every load instruction of a wave reads 1 KiB of
// contiguous memory, and all four of a thread's loads per input are issued
// before any arithmetic.  The loads go through a buffer descriptor that spans
// only the workgroup's rows: a vector past the last row, or past C at the end
// of a row, is out of its range and reads 0 without a memory access, so no
// load needs a branch.  The per-sample modulation vectors are held in the
// thread's registers as fp32 for both rows (read again only when the second
// row starts a new sample).
//
// Row statistics in one pass over the registers: each thread forms its
// (count, sum, M2 about its own mean) over its 16 values of the row, the wave
// combines the threads with the parallel-variance identity
//   M2_w = sum_t [ M2_t + n_t (mean_t - mean_w)^2 ]
// using DPP and lane reads, and after one barrier for both rows every thread
// combines the waves' (n_w, sum_w, mean_w, M2_w) the same way, in wave order.
// Centring on the thread's and then the wave's mean keeps rows whose mean is
// large against their spread free of cancellation.
//
// Measured at 1344x768 5 s (124,992 rows of 4096) against the earlier mapping
// (one wave per row, four rows per workgroup, modulation staged in LDS), each
// kernel timed after the rest of the chain, after a 2 GiB copy and back to
// back: AdaLN 329-332 us against 328-337 us; the fused residual -> AdaLN
// 675-676 us against 695-702 us.  Four rows per workgroup, one row per
// thread vector (512 threads), or rows walked by longer-lived workgroups
// with the next row's loads in flight all measured slower.
#pragma once

#include "device_common.hpp"

namespace dit {

constexpr int kGroupRows = 2;
constexpr int kGroupVecs = 2;
constexpr int kGroupMaxThreads = 512; // rows up to 1024 vectors (8192 wide)
constexpr int kGroupMaxWaves = kGroupMaxThreads / kWave;

// Threads per workgroup for rows of C 16-byte vectors: ceil(C / 2) rounded up
// to whole waves.  `full` when the vectors fill every thread's two slots.
struct RowGroupShape {
    int threads;
    bool full;
};

inline RowGroupShape row_group_shape(int C)
{
    const int per = (C + kGroupVecs - 1) / kGroupVecs;
    const int t = (per + kWave - 1) / kWave * kWave;
    return RowGroupShape{t, t * kGroupVecs == C};
}

constexpr int kRawBufferFormat = 0x00020000; // descriptor dword 3: 32-bit data, no swizzle, no stride
constexpr int kLoadNt = 2;                   // cache policy: non-temporal

// Descriptor over `rows` rows of C vectors starting at `first`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t group_rows_rsrc(const u32x4 *first, int rows, int C)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)first, 0, rows * C * 16, kRawBufferFormat);
}

constexpr int kOutOfRange = 0x7ffffff0; // a byte offset past any group's range

__device__ __forceinline__ u32x4 group_load(__amdgpu_buffer_rsrc_t rd, int byte_offset)
{
    return __builtin_amdgcn_raw_buffer_load_b128(rd, byte_offset, 0, kLoadNt);
}

// Mean and 1/sqrt(var + eps) of the workgroup's rows from the registers v
// (invalid vectors hold 0 and are flagged in ok).  n_t = 8 * (valid vectors
// of the thread); part holds kGroupRows * kGroupMaxWaves float4.  Contains
// the workgroup's one barrier.
template <bool FULL>
__device__ __forceinline__ void group_row_stats(const float (&v)[kGroupRows][kGroupVecs][8],
                                                const bool (&ok)[kGroupVecs], float n_t, int lane, int wave, int nw,
                                                float4 *part, float inv_d, float eps, float (&mean)[kGroupRows],
                                                float (&rstd)[kGroupRows])
{
#pragma unroll
    for (int j = 0; j < kGroupRows; ++j) {
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < kGroupVecs; ++k)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                s += v[j][k][i];
        const float m_t = n_t > 0.f ? s / n_t : 0.f;
        float q = 0.f;
#pragma unroll
        for (int k = 0; k < kGroupVecs; ++k)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float d = v[j][k][i] - m_t;
                q = (FULL || ok[k]) ? fmaf(d, d, q) : q;
            }
        const float s_w = wave_sum(s);
        // every wave holds at least one valid vector (the launch shape)
        const float n_w = FULL ? (float)(kWave * kGroupVecs * 8) : wave_sum(n_t);
        const float m_w = s_w / n_w;
        const float dm = m_t - m_w;
        const float q_w = wave_sum(fmaf(n_t * dm, dm, q));
        if (lane == 0)
            part[j * kGroupMaxWaves + wave] = make_float4(s_w, q_w, n_w, m_w);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kGroupRows; ++j) {
        float S = 0.f;
        for (int w = 0; w < nw; ++w)
            S += part[j * kGroupMaxWaves + w].x;
        mean[j] = S * inv_d;
        float M2 = 0.f;
        for (int w = 0; w < nw; ++w) {
            const float4 p = part[j * kGroupMaxWaves + w];
            const float d = p.w - mean[j];
            M2 += fmaf(p.z * d, d, p.y);
        }
        rstd[j] = 1.f / sqrtf(fmaf(M2, inv_d, eps));
    }
}

} // namespace dit
