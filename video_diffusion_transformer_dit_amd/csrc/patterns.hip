// patterns.hip -- access-pattern streams: the chain's memory traffic with no
// arithmetic, one kernel per shape, as ceilings for the kernels that carry
// that traffic.  Measurement only (not operators of the chain): each stream
// keeps the launch shape of the kernel it stands for, so "X% of its pattern"
// compares a kernel with the same loads and stores minus its arithmetic.
//   READ           one 16-byte non-temporal load per thread, 256-thread
//                  workgroups over consecutive 4 KiB tiles (a one-way
//                  stream: the fastest workgroup size for it, see below); the
//                  loaded words are folded into one value that is stored
//                  only if it equals `sink_key`, so the loads cannot be
//                  dropped and nearly nothing is written
//   WRITE          one 16-byte non-temporal store per thread, same tiling
//   SPLIT_ROWS     [rows][2W] -> [rows][W] bytes, out = a ^ b of the two
//                  halves: SwiGLU's tiling (64 threads per 1 KiB output
//                  segment, 1-D grid over (row, segment))
//   TWO_IN         two [rows][W] inputs -> one output (a ^ b): the gated
//                  residual's tiling (64 threads per 1 KiB segment)
//   ROW_GROUP      [rows][W] -> [rows][W]: AdaLN's mapping (row_group.hpp:
//                  two rows per workgroup, thread t holding vectors t and
//                  t + T of each, loaded through the workgroup's buffer
//                  descriptor, every load issued before any store)
//   ROW_GROUP_2X2  two [rows][W] inputs -> two outputs with ROW_GROUP's
//                  mapping, the first output stored before the second: the
//                  fused residual -> AdaLN's traffic
//   HEAD_MAJOR     [rows][heads][W/heads] -> [heads][rows][W/heads]: a
//                  token-major to head-major copy in the head-major QK
//                  kernel's shape: grid (group of 4 tokens, 4 KiB part),
//                  each thread one column of the 4 tokens, staged in LDS so
//                  that each store instruction writes runs of one head's 4
//                  tokens
//   SCORE_TILES    the SubBlock block-score kernel's traffic at head dim 128:
//                  its persistent 512-thread workgroups (one per CU), its
//                  order of (plane, query tile, key tile) items, the query
//                  tile loaded when it changes and the next key tile
//                  prefetched, and each 128 x 128 tile of fp32 words stored
//                  as 512-byte row segments; no products, no LDS staging
//   TOPK_ROWS      the SubBlock top-k kernel's traffic: one wave per row of
//                  n scores read with its buffer loads (n / 64 rounded up to
//                  4, 8, 16, 32 or 64 per lane), then ceil(n / 4) words of the
//                  row's kept list written (the kept count at sparsity 0.75);
//                  no selection
#include "device_common.hpp"
#include "launch.hpp"
#include "row_group.hpp"

namespace dit {
namespace {

constexpr unsigned kGridCap = (1u << 24) - 1; // < 2^32 work-items per dispatch
// Workgroup size of the streaming kernels these shapes stand for (dit_copy16,
// SwiGLU, the gated residual): one wave per workgroup.
constexpr int kStreamThreads = 64;
// The one-way streams keep 256-thread workgroups: with one wave a workgroup
// moves only 1 KiB, and an 8 GB read then ran at the rate workgroups are
// dispatched (1.69 ms against 1.16 ms with 256 threads at 1344x768 5 s).
constexpr int kOneWayThreads = 256;

__device__ __forceinline__ u32x4 xor4(u32x4 a, u32x4 b) { return a ^ b; }

__global__ __launch_bounds__(kOneWayThreads) void pattern_read_kernel(const u32x4 *__restrict__ src, int64_t nvec,
                                                           u32x4 *__restrict__ sink, uint32_t sink_key)
{
    uint32_t acc = 0u;
    for (int64_t c = (int64_t)blockIdx.x * kOneWayThreads + threadIdx.x; c < nvec;
         c += (int64_t)gridDim.x * kOneWayThreads) {
        const u32x4 v = load_stream(src + c);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if (acc == sink_key)
        sink[0] = u32x4{acc, acc, acc, acc};
}

__global__ __launch_bounds__(kOneWayThreads) void pattern_write_kernel(u32x4 *__restrict__ dst, int64_t nvec)
{
    for (int64_t c = (int64_t)blockIdx.x * kOneWayThreads + threadIdx.x; c < nvec;
         c += (int64_t)gridDim.x * kOneWayThreads) {
        const uint32_t w = (uint32_t)c;
        store_stream(dst + c, u32x4{w, w, w, w});
    }
}

// C = 16-byte vectors per output row.
__global__ __launch_bounds__(kStreamThreads) void pattern_split_rows_kernel(const u32x4 *__restrict__ in,
                                                                 u32x4 *__restrict__ out, int C, unsigned segs,
                                                                 unsigned tiles)
{
    for (unsigned tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        const unsigned row = tile / segs;
        const int c = (int)(tile - row * segs) * kStreamThreads + threadIdx.x;
        if (c < C) {
            const u32x4 *a = in + (size_t)row * 2 * C;
            store_stream(out + (size_t)row * C + c, xor4(load_stream(a + c), load_stream(a + C + c)));
        }
    }
}

__global__ __launch_bounds__(kStreamThreads) void pattern_two_in_kernel(const u32x4 *__restrict__ x, const u32x4 *__restrict__ y,
                                                             u32x4 *__restrict__ out, int C, unsigned segs,
                                                             unsigned tiles)
{
    for (unsigned tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        const unsigned row = tile / segs;
        const int c = (int)(tile - row * segs) * kStreamThreads + threadIdx.x;
        if (c < C) {
            const size_t at = (size_t)row * C + c;
            store_stream(out + at, xor4(load_stream(x + at), load_stream(y + at)));
        }
    }
}

// The loads and stores of adaln.hip (TWO = false) and residual_adaln.hip
// (TWO = true) with nothing computed in between.
template <bool TWO, bool FULL>
__global__ __launch_bounds__(kGroupMaxThreads) void pattern_row_group_kernel(const u32x4 *__restrict__ x,
                                                                             const u32x4 *__restrict__ y,
                                                                             u32x4 *__restrict__ ox,
                                                                             u32x4 *__restrict__ oy, int rows, int C)
{
    const int T = blockDim.x, tid = threadIdx.x;
    const int r0 = blockIdx.x * kGroupRows;
    const int nr = min(rows - r0, kGroupRows);
    int c[kGroupVecs];
    bool ok[kGroupVecs];
#pragma unroll
    for (int k = 0; k < kGroupVecs; ++k) {
        c[k] = tid + T * k;
        ok[k] = FULL || c[k] < C;
    }
    const __amdgpu_buffer_rsrc_t rx = group_rows_rsrc(x + (size_t)r0 * C, nr, C);
    const __amdgpu_buffer_rsrc_t ry = group_rows_rsrc((TWO ? y : x) + (size_t)r0 * C, nr, C);
    u32x4 a[kGroupRows][kGroupVecs], b[kGroupRows][kGroupVecs];
#pragma unroll
    for (int j = 0; j < kGroupRows; ++j)
#pragma unroll
        for (int k = 0; k < kGroupVecs; ++k) {
            const int off = ok[k] ? (j * C + c[k]) * 16 : kOutOfRange;
            a[j][k] = group_load(rx, off);
            if (TWO)
                b[j][k] = group_load(ry, off);
        }
    // the kernels this stands for store only after their rows are in: keep
    // the scheduler from moving stores earlier
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kGroupRows; ++j)
#pragma unroll
        for (int k = 0; k < kGroupVecs; ++k)
            if ((FULL || ok[k]) && j < nr)
                store_stream(ox + (size_t)(r0 + j) * C + c[k], a[j][k]);
    if (TWO) {
#pragma unroll
        for (int j = 0; j < kGroupRows; ++j)
#pragma unroll
            for (int k = 0; k < kGroupVecs; ++k)
                if ((FULL || ok[k]) && j < nr)
                    store_stream(oy + (size_t)(r0 + j) * C + c[k], b[j][k]);
    }
}

// VPH = vectors per head (a divisor of 256, so no head straddles two parts),
// C vectors per row; grid (ceil(rows / kHmTokens), parts).  Loads and stores
// of qk_rmsnorm_rope3d_head_major_kernel without its arithmetic.
constexpr int kHmTokens = 4;
__global__ __launch_bounds__(256) void pattern_head_major_kernel(const u32x4 *__restrict__ in, u32x4 *__restrict__ out,
                                                                 int rows, int C, int VPH)
{
    __shared__ u32x4 stage[kHmTokens][256];
    const int tid = threadIdx.x;
    const unsigned r0 = blockIdx.x * kHmTokens;
    const int c = blockIdx.y * 256 + tid;
    const bool col_ok = c < C;
    // absent tokens and columns read the group's first row or column and are never stored
    u32x4 raw[kHmTokens];
#pragma unroll
    for (int t = 0; t < kHmTokens; ++t) {
        const bool ok = col_ok && r0 + t < (unsigned)rows;
        raw[t] = load_stream(in + (size_t)(ok ? r0 + t : r0) * C + (col_ok ? c : 0));
    }
#pragma unroll
    for (int t = 0; t < kHmTokens; ++t)
        stage[t][tid] = raw[t];
    __syncthreads();
    // vector m of a head's run of kHmTokens * VPH is token m / VPH, slot m % VPH
    const int run = kHmTokens * VPH;
#pragma unroll
    for (int i = 0; i < kHmTokens; ++i) {
        const int idx = tid + 256 * i;
        const int hl = idx / run, m = idx % run;
        const int t = m / VPH, s = m % VPH;
        const int col = blockIdx.y * 256 + hl * VPH + s;
        const unsigned r = r0 + t;
        if (col < C && r < (unsigned)rows)
            store_stream(out + ((size_t)(col / VPH) * (unsigned)rows + r) * VPH + s, stage[t][hl * VPH + s]);
    }
}

// SCORE_TILES: P planes of n x n fp32 words (row stride ld4 vectors), the
// block-score kernel's item order and loads.  A stored word is its tag
// (plane row * 65536 + column, mod 2^32) XOR the fold of the words this thread
// loaded for the tile, so all-zero means give the bare tags.  The LDS array
// is never touched; it holds occupancy at the kernel's one workgroup per CU.
constexpr int kScoreTile = 128, kScoreDh = 128, kScoreLds = 135168;

__global__ __launch_bounds__(512) void pattern_score_tiles_kernel(const u32x4 *__restrict__ qm,
                                                                  const u32x4 *__restrict__ km,
                                                                  u32x4 *__restrict__ out, int n, int ld4, int tiles,
                                                                  unsigned total)
{
    constexpr int kThreads = 512, kF4PerRow = kScoreDh / 4;
    constexpr int kLoads = kScoreTile * kF4PerRow / kThreads;
    constexpr int kStores = kScoreTile * kScoreTile / 4 / kThreads;
    __shared__ uint32_t lds_hold[kScoreLds / 4];
    asm volatile("" : : "v"(lds_hold) : "memory"); // the array's address escapes: the allocation stays

    const unsigned per = gridDim.x / 8, xcd = blockIdx.x % 8, j = blockIdx.x / 8;
    const unsigned span = (total + 7) / 8;
    const unsigned first = xcd * span, last = min(total, first + span);
    const unsigned run = (span + per - 1) / per;
    const unsigned begin = min(last, first + j * run), end = min(last, begin + run);
    const unsigned per_plane = (unsigned)(tiles * tiles);

    u32x4 kr[kLoads];
    auto load_k = [&](unsigned it) {
        const size_t p = it / per_plane;
        const int tj = (int)(it % per_plane) % tiles;
        const u32x4 *kb = km + (p * n + (size_t)tj * kScoreTile) * kF4PerRow;
        const int k_rows = min(kScoreTile, n - tj * kScoreTile);
#pragma unroll
        for (int m = 0; m < kLoads; ++m) {
            const int e = threadIdx.x + kThreads * m;
            kr[m] = e / kF4PerRow < k_rows ? kb[e] : u32x4{0u, 0u, 0u, 0u};
        }
    };
    if (begin < end)
        load_k(begin);
    size_t held_p = ~(size_t)0;
    int held_ti = -1;
    uint32_t qfold = 0u;
    for (unsigned item = begin; item < end; ++item) {
        const size_t p = item / per_plane;
        const int tile = (int)(item % per_plane), ti = tile / tiles, tj = tile % tiles;
        const int q_rows = min(kScoreTile, n - ti * kScoreTile), k_rows = min(kScoreTile, n - tj * kScoreTile);
        if (p != held_p || ti != held_ti) { // workgroup-uniform
            const u32x4 *qa = qm + (p * n + (size_t)ti * kScoreTile) * kF4PerRow;
            qfold = 0u;
#pragma unroll
            for (int m = 0; m < kLoads; ++m) {
                const int e = threadIdx.x + kThreads * m;
                const u32x4 a = e / kF4PerRow < q_rows ? qa[e] : u32x4{0u, 0u, 0u, 0u};
                qfold ^= a[0] ^ a[1] ^ a[2] ^ a[3];
            }
            held_p = p, held_ti = ti;
        }
        uint32_t x = qfold;
#pragma unroll
        for (int m = 0; m < kLoads; ++m)
            x ^= kr[m][0] ^ kr[m][1] ^ kr[m][2] ^ kr[m][3];
        __syncthreads(); // the kernel's barrier before the key tile is replaced
        if (item + 1 < end)
            load_k(item + 1);
        const uint32_t row_tag = (uint32_t)(p * n + (size_t)ti * kScoreTile) * 65536u;
        u32x4 *o = out + (p * n + (size_t)ti * kScoreTile) * ld4 + (size_t)tj * (kScoreTile / 4);
#pragma unroll
        for (int m = 0; m < kStores; ++m) {
            const int idx = threadIdx.x + kThreads * m;
            const int row = idx / (kScoreTile / 4), c4 = idx % (kScoreTile / 4);
            if (row < q_rows && 4 * c4 < k_rows) {
                const uint32_t t = row_tag + (uint32_t)row * 65536u + (uint32_t)(tj * kScoreTile + 4 * c4);
                store_stream(o + (size_t)row * ld4 + c4, u32x4{t ^ x, (t + 1u) ^ x, (t + 2u) ^ x, (t + 3u) ^ x});
            }
        }
    }
}

// TOPK_ROWS: row r of in [rows][ld] (n words read), ceil(n / 4) words written
// to out [rows][keep]: word j = (r * 65536 + j) XOR the fold of the words the
// lane loaded, so an all-zero input gives the bare tags.  The loads are the
// top-k kernel's (out-of-range words read as 0 by the buffer's range check,
// the same 4 KiB split of the offset); the LDS array holds its occupancy.
template <int S>
__global__ __launch_bounds__(kWave) void pattern_topk_rows_kernel(const float *__restrict__ in, uint32_t *__restrict__ out,
                                                                  int n, int ld, int keep)
{
    constexpr int kRawFormat = 0x00020000;
    constexpr int kSlotsPerOffset = 4096 / (4 * kWave);
    __shared__ uint32_t lds_hold[1024];
    asm volatile("" : : "v"(lds_hold) : "memory"); // the array's address escapes: the allocation stays
    const int lane = threadIdx.x;
    const size_t row = (size_t)blockIdx.y * n + blockIdx.x;
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc((void *)(in + row * ld), 0, n * 4, kRawFormat);
    uint32_t fold = 0u;
#pragma unroll
    for (int q = 0; q < S; ++q) {
        const int base = 4 * lane + 4096 * (q / kSlotsPerOffset);
        fold ^= __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(
                                                 rd, base + 4 * kWave * (q % kSlotsPerOffset), 0, 2 /* nt */));
    }
    uint32_t *o = out + row * keep;
    const uint32_t tag = (uint32_t)row * 65536u;
    for (int j = lane; j < keep; j += kWave)
        o[j] = (tag + (uint32_t)j) ^ fold;
}

unsigned capped(uint64_t tiles) { return tiles < kGridCap ? (unsigned)tiles : kGridCap; }

template <bool TWO>
hipError_t launch_row_group(const u32x4 *x, const u32x4 *y, u32x4 *ox, u32x4 *oy, int rows, int C, hipStream_t stream)
{
    const RowGroupShape shape = row_group_shape(C);
    const dim3 grid((unsigned)((rows + kGroupRows - 1) / kGroupRows)), block((unsigned)shape.threads);
    if (shape.full)
        hipLaunchKernelGGL((pattern_row_group_kernel<TWO, true>), grid, block, 0, stream, x, y, ox, oy, rows, C);
    else
        hipLaunchKernelGGL((pattern_row_group_kernel<TWO, false>), grid, block, 0, stream, x, y, ox, oy, rows, C);
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
        hipLaunchKernelGGL(pattern_read_kernel, dim3(capped((uint64_t)(nvec + kOneWayThreads - 1) / kOneWayThreads)),
                           dim3(kOneWayThreads), 0, stream, a, nvec, o, 0x9e3779b9u);
        break;
    }
    case kPatternWrite: {
        const int64_t nvec = rows * C;
        hipLaunchKernelGGL(pattern_write_kernel, dim3(capped((uint64_t)(nvec + kOneWayThreads - 1) / kOneWayThreads)),
                           dim3(kOneWayThreads), 0, stream, o, nvec);
        break;
    }
    case kPatternSplitRows: {
        const unsigned segs = (unsigned)((C + kStreamThreads - 1) / kStreamThreads);
        const uint64_t tiles = (uint64_t)rows * segs;
        hipLaunchKernelGGL(pattern_split_rows_kernel, dim3(capped(tiles)), dim3(kStreamThreads), 0, stream, a, o,
                           (int)C, segs, (unsigned)tiles);
        break;
    }
    case kPatternTwoIn: {
        const unsigned segs = (unsigned)((C + kStreamThreads - 1) / kStreamThreads);
        const uint64_t tiles = (uint64_t)rows * segs;
        const unsigned grid = tiles < (1u << 23) - 1 ? (unsigned)tiles : (1u << 23) - 1; // the residual's cap
        hipLaunchKernelGGL(pattern_two_in_kernel, dim3(grid), dim3(kStreamThreads), 0, stream, a, b, o, (int)C, segs,
                           (unsigned)tiles);
        break;
    }
    case kPatternRowGroup: return launch_row_group<false>(a, a, o, o, (int)rows, (int)C, stream);
    case kPatternRowGroup2x2: return launch_row_group<true>(a, b, o, o2, (int)rows, (int)C, stream);
    case kPatternHeadMajor: {
        const int VPH = (int)(C / heads);
        hipLaunchKernelGGL(pattern_head_major_kernel,
                           dim3((unsigned)((rows + kHmTokens - 1) / kHmTokens), (unsigned)((C + 255) / 256)), dim3(256),
                           0, stream, a, o, (int)rows, (int)C, VPH);
        break;
    }
    case kPatternScoreTiles: {
        // rows = P * n, heads = n: the grid the block-score kernel takes at
        // head dim 128, one workgroup per CU (a multiple of 8), no more than
        // there are tiles
        const int n = (int)heads, tiles = (n + kScoreTile - 1) / kScoreTile;
        const unsigned total = (unsigned)((uint64_t)(rows / heads) * (uint64_t)tiles * (uint64_t)tiles);
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8) {
            (void)hipGetLastError();
            cus = 256;
        }
        const unsigned resident = (unsigned)cus / 8 * 8, need = (total + 7) / 8 * 8;
        hipLaunchKernelGGL(pattern_score_tiles_kernel, dim3(resident < need ? resident : need), dim3(512), 0, stream,
                           a, b, o, n, (int)C, tiles, total);
        break;
    }
    case kPatternTopkRows: {
        // rows = P * n, heads = n; the top-k kernel's grid (n, P) of single waves
        const int n = (int)heads, ld = (int)(row_bytes / 4), keep = (n + 3) / 4;
        const dim3 grid((unsigned)n, (unsigned)(rows / heads));
        const float *in = static_cast<const float *>(in0);
        auto *out = static_cast<uint32_t *>(out0);
        if (n <= 256) hipLaunchKernelGGL(pattern_topk_rows_kernel<4>, grid, dim3(kWave), 0, stream, in, out, n, ld, keep);
        else if (n <= 512) hipLaunchKernelGGL(pattern_topk_rows_kernel<8>, grid, dim3(kWave), 0, stream, in, out, n, ld, keep);
        else if (n <= 1024) hipLaunchKernelGGL(pattern_topk_rows_kernel<16>, grid, dim3(kWave), 0, stream, in, out, n, ld, keep);
        else if (n <= 2048) hipLaunchKernelGGL(pattern_topk_rows_kernel<32>, grid, dim3(kWave), 0, stream, in, out, n, ld, keep);
        else hipLaunchKernelGGL(pattern_topk_rows_kernel<64>, grid, dim3(kWave), 0, stream, in, out, n, ld, keep);
        break;
    }
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

} // namespace dit
