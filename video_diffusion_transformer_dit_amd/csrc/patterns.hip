// patterns.hip -- access-pattern streams: the chain's memory traffic with no
// arithmetic, one kernel per shape, as ceilings for the kernels that carry
// that traffic.  Measurement only (not operators of the chain): each stream
// keeps the launch shape of the kernel it stands for, so "X% of its pattern"
// compares a kernel with the same loads and stores minus its arithmetic.
//   READ           one 16-byte non-temporal load per thread, 256-thread
//                  workgroups over consecutive 4 KiB tiles (copy16's shape
//                  without the stores); the loaded words are folded into one
//                  value that is stored only if it equals `sink_key`, so the
//                  loads cannot be dropped and nearly nothing is written
//   WRITE          one 16-byte non-temporal store per thread, same tiling
//   SPLIT_ROWS     [rows][2W] -> [rows][W] bytes, out = a ^ b of the two
//                  halves: SwiGLU's tiling (256 threads per 4 KiB output
//                  segment, 1-D grid over (row, segment))
//   TWO_IN         two [rows][W] inputs -> one output (a ^ b): the gated
//                  residual's tiling (512 threads per 8 KiB segment)
//   ROW_WAVE       [rows][W] -> [rows][W]: AdaLN's mapping (one wave per row,
//                  four rows per 256-thread workgroup, each lane's vectors
//                  lane, lane + 64, ..., every load issued before any store)
//   ROW_WAVE_2X2   two [rows][W] inputs -> two outputs with ROW_WAVE's
//                  mapping: the fused residual -> AdaLN's traffic
//   HEAD_MAJOR     [rows][heads][W/heads] -> [heads][rows][W/heads]: a
//                  token-major to head-major copy, one vector per thread,
//                  grid (row, 4 KiB part) as the token-major QK kernel
#include "device_common.hpp"
#include "launch.hpp"

namespace dit {
namespace {

constexpr unsigned kGridCap = (1u << 24) - 1; // < 2^32 work-items per dispatch at 256 threads

__device__ __forceinline__ u32x4 xor4(u32x4 a, u32x4 b) { return a ^ b; }

__global__ __launch_bounds__(256) void pattern_read_kernel(const u32x4 *__restrict__ src, int64_t nvec,
                                                           u32x4 *__restrict__ sink, uint32_t sink_key)
{
    uint32_t acc = 0u;
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < nvec; c += (int64_t)gridDim.x * 256) {
        const u32x4 v = load_stream(src + c);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if (acc == sink_key)
        sink[0] = u32x4{acc, acc, acc, acc};
}

__global__ __launch_bounds__(256) void pattern_write_kernel(u32x4 *__restrict__ dst, int64_t nvec)
{
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < nvec; c += (int64_t)gridDim.x * 256) {
        const uint32_t w = (uint32_t)c;
        store_stream(dst + c, u32x4{w, w, w, w});
    }
}

// C = 16-byte vectors per output row.
__global__ __launch_bounds__(256) void pattern_split_rows_kernel(const u32x4 *__restrict__ in,
                                                                 u32x4 *__restrict__ out, int C, unsigned segs,
                                                                 unsigned tiles)
{
    for (unsigned tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        const unsigned row = tile / segs;
        const int c = (int)(tile - row * segs) * 256 + threadIdx.x;
        if (c < C) {
            const u32x4 *a = in + (size_t)row * 2 * C;
            store_stream(out + (size_t)row * C + c, xor4(load_stream(a + c), load_stream(a + C + c)));
        }
    }
}

__global__ __launch_bounds__(512) void pattern_two_in_kernel(const u32x4 *__restrict__ x, const u32x4 *__restrict__ y,
                                                             u32x4 *__restrict__ out, int C, unsigned segs,
                                                             unsigned tiles)
{
    for (unsigned tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        const unsigned row = tile / segs;
        const int c = (int)(tile - row * segs) * 512 + threadIdx.x;
        if (c < C) {
            const size_t at = (size_t)row * C + c;
            store_stream(out + at, xor4(load_stream(x + at), load_stream(y + at)));
        }
    }
}

// FULL: the row is exactly 64 * VPL vectors, so no load is conditional (as in
// AdaLN's kernels: conditional loads into an array make the compiler wait for
// each load before the next).
template <int VPL, bool TWO, bool FULL>
__global__ __launch_bounds__(256) void pattern_row_wave_kernel(const u32x4 *__restrict__ x,
                                                               const u32x4 *__restrict__ y, u32x4 *__restrict__ ox,
                                                               u32x4 *__restrict__ oy, int rows, int C)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int row = blockIdx.x * 4 + threadIdx.x / kWave;
    if (row >= rows) // wave-uniform
        return;
    const size_t base = (size_t)row * C;
    u32x4 a[VPL], b[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int c = lane + kWave * k;
        a[k] = b[k] = u32x4{0u, 0u, 0u, 0u};
        if (FULL || c < C) {
            a[k] = load_stream(x + base + c);
            if (TWO)
                b[k] = load_stream(y + base + c);
        }
    }
    // the kernels this stands for store only after the whole row is in (their
    // row statistics need it): keep the scheduler from moving stores earlier
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int c = lane + kWave * k;
        if (FULL || c < C) {
            store_stream(ox + base + c, a[k]);
            if (TWO)
                store_stream(oy + base + c, b[k]);
        }
    }
}

// VPH = vectors per head, H heads, C = H * VPH vectors per row; grid (rows, parts).
__global__ __launch_bounds__(256) void pattern_head_major_kernel(const u32x4 *__restrict__ in, u32x4 *__restrict__ out,
                                                                 int rows, int H, int VPH)
{
    const int C = H * VPH;
    const int c = blockIdx.y * 256 + threadIdx.x;
    const unsigned row = blockIdx.x;
    if (c < C) {
        const int h = c / VPH, s = c - h * VPH;
        store_stream(out + ((size_t)h * rows + row) * VPH + s, load_stream(in + (size_t)row * C + c));
    }
}

unsigned capped(uint64_t tiles) { return tiles < kGridCap ? (unsigned)tiles : kGridCap; }

template <bool TWO>
hipError_t launch_row_wave(const u32x4 *x, const u32x4 *y, u32x4 *ox, u32x4 *oy, int rows, int C, hipStream_t stream)
{
    const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
#define DIT_ROW_WAVE(V)                                                                                              \
    do {                                                                                                             \
        if (C == kWave * (V))                                                                                        \
            hipLaunchKernelGGL((pattern_row_wave_kernel<V, TWO, true>), grid, block, 0, stream, x, y, ox, oy, rows,   \
                               C);                                                                                   \
        else                                                                                                         \
            hipLaunchKernelGGL((pattern_row_wave_kernel<V, TWO, false>), grid, block, 0, stream, x, y, ox, oy, rows,  \
                               C);                                                                                   \
    } while (0)
    if (C <= kWave) DIT_ROW_WAVE(1);
    else if (C <= 2 * kWave) DIT_ROW_WAVE(2);
    else if (C <= 4 * kWave) DIT_ROW_WAVE(4);
    else if (C <= 8 * kWave) DIT_ROW_WAVE(8);
    else DIT_ROW_WAVE(16);
#undef DIT_ROW_WAVE
    return hipGetLastError();
}

} // namespace

hipError_t launch_stream_pattern(int kind, const void *in0, const void *in1, void *out0, void *out1, int64_t rows,
                                 int64_t row_bytes, int64_t heads, hipStream_t stream)
{
    const auto *a = static_cast<const u32x4 *>(in0);
    const auto *b = static_cast<const u32x4 *>(in1);
    auto *o = static_cast<u32x4 *>(out0);
    auto *o2 = static_cast<u32x4 *>(out1);
    const int64_t C = row_bytes / 16;
    switch (kind) {
    case kPatternRead: {
        const int64_t nvec = rows * C;
        hipLaunchKernelGGL(pattern_read_kernel, dim3(capped((uint64_t)(nvec + 255) / 256)), dim3(256), 0, stream, a,
                           nvec, o, 0x9e3779b9u);
        break;
    }
    case kPatternWrite: {
        const int64_t nvec = rows * C;
        hipLaunchKernelGGL(pattern_write_kernel, dim3(capped((uint64_t)(nvec + 255) / 256)), dim3(256), 0, stream, o,
                           nvec);
        break;
    }
    case kPatternSplitRows: {
        const unsigned segs = (unsigned)((C + 255) / 256);
        const uint64_t tiles = (uint64_t)rows * segs;
        hipLaunchKernelGGL(pattern_split_rows_kernel, dim3(capped(tiles)), dim3(256), 0, stream, a, o, (int)C, segs,
                           (unsigned)tiles);
        break;
    }
    case kPatternTwoIn: {
        const unsigned segs = (unsigned)((C + 511) / 512);
        const uint64_t tiles = (uint64_t)rows * segs;
        const unsigned grid = tiles < (1u << 23) - 1 ? (unsigned)tiles : (1u << 23) - 1;
        hipLaunchKernelGGL(pattern_two_in_kernel, dim3(grid), dim3(512), 0, stream, a, b, o, (int)C, segs,
                           (unsigned)tiles);
        break;
    }
    case kPatternRowWave: return launch_row_wave<false>(a, a, o, o, (int)rows, (int)C, stream);
    case kPatternRowWave2x2: return launch_row_wave<true>(a, b, o, o2, (int)rows, (int)C, stream);
    case kPatternHeadMajor: {
        const int H = (int)heads, VPH = (int)(C / heads);
        hipLaunchKernelGGL(pattern_head_major_kernel, dim3((unsigned)rows, (unsigned)((C + 255) / 256)), dim3(256), 0,
                           stream, a, o, (int)rows, H, VPH);
        break;
    }
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

} // namespace dit
