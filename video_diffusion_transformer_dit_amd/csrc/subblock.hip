// subblock.hip -- front-end of the SubBlock sparse-attention router:
//   1. block pooling:  per sample and head, the mean of each 64-token block of
//      q' and of k' (after RMSNorm + RoPE), as fp32;
//   2. block scores:   s[i][j] = bf16(qp[i]) . bf16(kp[j]) per sample and head,
//      on the matrix cores (bf16 operands, fp32 accumulation);
//   3. kept blocks:    per query block, the `keep` key blocks of largest score
//      (ties to the lower index), listed in ascending order.
//
// SubBlock attention cuts the sequence into 64-token blocks and keeps only part
// of the key blocks, dropping those of smaller estimated contribution
// ("SGLang acelera vídeo do MiniMax-H3…", stamatios.com, "De onde vêm os
// ganhos" and "Resultado principal"); sparsity is the dropped share, so 0.75
// keeps about a quarter ("8×H200 上的 MiniMax-H3…", xhh.club, Q&A on the
// sparsity parameter).
//
// Roofline per step (1344x768 5 s: 124,992 tokens, 1953 blocks, 32 x 128 heads):
//   pooling reads q' and k' once (2 x 1.02 GB) and writes 2 x 32 MB: HBM-bound;
//   scores are a batched 1953 x 1953 x 128 product per head (31 GFLOP, bf16
//   matrix cores) whose cost is writing 488 MB of fp32 scores;
//   selection reads the scores once and writes the kept indices.
// The pooling can instead be done by the QK kernel while it writes q', k'
// (qk_rmsnorm_rope3d_pool_kernel, qk_rope.hip), which spares the read.
#include "device_common.hpp"
#include "launch.hpp"

namespace dit {
namespace {

constexpr int kBlockTokens = 64;

// ---------------------------------------------------------------- pooling

__device__ __forceinline__ void add8(float acc[8], u32x4 v)
{
    float f[8];
    unpack8(v, f);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        acc[i] += f[i];
}

__device__ __forceinline__ void store_mean8(float *o, const float acc[8], float count)
{
    float4 *o4 = reinterpret_cast<float4 *>(o);
    o4[0] = make_float4(acc[0] / count, acc[1] / count, acc[2] / count, acc[3] / count);
    o4[1] = make_float4(acc[4] / count, acc[5] / count, acc[6] / count, acc[7] / count);
}

// Token-major input [B][N][H][Dh], C = H*Dh/8 16-byte vectors per token.
// grid (chunks * nb, 2 (q then k), B), 512 threads.  A workgroup pools one
// 64-vector column chunk of one block: lane = vector column, wave w adds tokens
// w, w+8, ..., w+56 (eight loads in flight), then wave 0 adds the other
// waves' partials in order and writes the means.  (Eight waves of eight tokens
// measured 4% faster than four of sixteen or sixteen of four.)
constexpr int kPoolWaves = 8;
__global__ __launch_bounds__(kPoolWaves * kWave) void subblock_pool_token_major_kernel(const u32x4 *__restrict__ q,
                                                                        const u32x4 *__restrict__ k,
                                                                        float *__restrict__ qp,
                                                                        float *__restrict__ kp, int N, int nb,
                                                                        int C, int chunks, int vph_shift)
{
    constexpr int kWaves = kPoolWaves, kPerWave = kBlockTokens / kWaves;
    __shared__ float4 part[kWaves - 1][2][kWave];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int chunk = blockIdx.x % chunks, blk = blockIdx.x / chunks;
    const size_t b = blockIdx.z;
    const u32x4 *src = blockIdx.y ? k : q;
    float *dst = blockIdx.y ? kp : qp;
    const int c = chunk * kWave + lane;
    const int n0 = blk * kBlockTokens;
    const int count = min(kBlockTokens, N - n0);

    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (c < C) {
        const u32x4 *base = src + ((size_t)b * N + n0) * C + c;
        u32x4 v[kPerWave];
#pragma unroll
        for (int t = 0; t < kPerWave; ++t) {
            const int n = wave + kWaves * t; // wave-uniform
            v[t] = n < count ? load_stream(base + (size_t)n * C) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int t = 0; t < kPerWave; ++t)
            add8(acc, v[t]);
    }
    if (wave > 0) {
        part[wave - 1][0][lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        part[wave - 1][1][lane] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
    __syncthreads();
    if (wave == 0 && c < C) {
#pragma unroll
        for (int w = 0; w < kWaves - 1; ++w) {
            const float4 lo = part[w][0][lane], hi = part[w][1][lane];
            acc[0] += lo.x, acc[1] += lo.y, acc[2] += lo.z, acc[3] += lo.w;
            acc[4] += hi.x, acc[5] += hi.y, acc[6] += hi.z, acc[7] += hi.w;
        }
        const int H = C >> vph_shift;
        const int h = c >> vph_shift, dv = c & ((1 << vph_shift) - 1);
        const int Dh = 8 << vph_shift;
        store_mean8(dst + (((size_t)b * H + h) * nb + blk) * Dh + dv * 8, acc, (float)count);
    }
}

// Head-major input [B][H][N][Dh]: a block of one head is 64*Dh contiguous
// values.  grid (nb, 2*H (q heads then k heads), B), 256 threads.  Thread t
// reads vectors t, t+256, ... of the block; with VPT = Dh/8 vectors per token
// every one of them is column t % VPT.  Lanes of one column are summed with
// lane swaps, then the four waves through LDS in order.
template <int VPT>
__global__ __launch_bounds__(256) void subblock_pool_head_major_kernel(const u32x4 *__restrict__ q,
                                                                       const u32x4 *__restrict__ k,
                                                                       float *__restrict__ qp,
                                                                       float *__restrict__ kp, int N, int nb, int H)
{
    constexpr int kVectors = kBlockTokens * VPT;              // per block of one head
    constexpr int kLoads = kVectors >= 256 ? kVectors / 256 : 1;
    constexpr int kDh = VPT * 8;
    __shared__ float4 part[4][2][VPT];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int blk = blockIdx.x;
    const bool is_k = blockIdx.y >= (unsigned)H;
    const int h = is_k ? blockIdx.y - H : blockIdx.y;
    const size_t b = blockIdx.z;
    const u32x4 *src = (is_k ? k : q) + (((size_t)b * H + h) * N + (size_t)blk * kBlockTokens) * VPT;
    const int count = min(kBlockTokens, N - blk * kBlockTokens);

    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    u32x4 v[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
        const int e = threadIdx.x + 256 * u;
        v[u] = (e < kVectors && e / VPT < count) ? load_stream(src + e) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kLoads; ++u)
        add8(acc, v[u]);
    // lanes l, l + VPT, l + 2 VPT, ... hold the same column
#pragma unroll
    for (int off = VPT; off < kWave; off <<= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[i] += __shfl_xor(acc[i], off, kWave);
    if (lane < VPT) {
        part[wave][0][lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        part[wave][1][lane] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
    __syncthreads();
    if (threadIdx.x < VPT) {
        float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float4 lo = part[w][0][threadIdx.x], hi = part[w][1][threadIdx.x];
            s[0] += lo.x, s[1] += lo.y, s[2] += lo.z, s[3] += lo.w;
            s[4] += hi.x, s[5] += hi.y, s[6] += hi.z, s[7] += hi.w;
        }
        float *dst = is_k ? kp : qp;
        store_mean8(dst + (((size_t)b * H + h) * nb + blk) * kDh + threadIdx.x * 8, s, (float)count);
    }
}

// ---------------------------------------------------------------- scores

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// grid (tiles * tiles, H, B), 4 * TILE threads; tiles = ceil(nb / TILE), the
// (head, tile) pairs renumbered per XCD (below).  A workgroup computes a
// TILE x TILE tile of one head's score matrix.  The route runs it for
// Dh = 256 with TILE = 64 (two 128-row operand tiles would fill most of the
// LDS); smaller heads take the persistent form below, whose tiles are 128:
// both TILE-row operand tiles are rounded to bf16 into LDS (rows padded by 4
// values so the 16 rows one MFMA reads fall in different banks).  The waves
// form a 4 x (TILE/64) grid; each multiplies TILE/64 strips of 16 query rows
// with 64 key rows, Dh/16 MFMA 16x16x16 steps per 16 x 16 output tile, so a
// wave reuses each operand fragment it reads from LDS in several products.
// Operand layout of v_mfma_f32_16x16x16_bf16: lane l supplies row l % 16,
// reduction elements 4(l/16) .. 4(l/16)+3 of A and of B; it receives output
// rows 4(l/16) .. +3 of column l % 16.  The 128-row tile halves the operand
// bytes each score costs in L2 reads, bf16 conversion and LDS reads against
// a 64-row tile, and measured 8-15% faster at 1953 blocks; every score is the
// same sum of the same products in the same order either way.
template <int DH, int TILE>
__global__ __launch_bounds__(4 * TILE) void subblock_scores_kernel(const float *__restrict__ qp,
                                                                   const float *__restrict__ kp,
                                                                   float *__restrict__ scores, int nb, int ld,
                                                                   int tiles, int H)
{
    constexpr int kThreads = 4 * TILE;
    constexpr int kStrips = TILE / 64; // 16-row query strips per wave, and wave columns
    constexpr int kRow = DH + 4;       // bf16 per padded LDS row
    constexpr int kF4PerRow = DH / 4;
    constexpr int kOutRow = TILE + 4; // floats per padded LDS row of the output tile
    constexpr int kOperandBytes = 2 * TILE * kRow * 2, kOutBytes = TILE * kOutRow * 4;
    __shared__ __align__(16) unsigned char lds_raw[kOperandBytes > kOutBytes ? kOperandBytes : kOutBytes];
    uint16_t *lds_q = reinterpret_cast<uint16_t *>(lds_raw);
    uint16_t *lds_k = lds_q + TILE * kRow;

    // Workgroups go to the 8 XCDs round-robin in dispatch order; renumber
    // them so that XCD x takes the x-th contiguous eighth of the (head, tile)
    // list and its L2 holds one head's means at a time (a bijection on the
    // grid, also when the count is not a multiple of 8).
    const size_t per_head = (size_t)tiles * tiles;
    const size_t total = per_head * H * gridDim.z;
    const size_t lin = blockIdx.x + per_head * (blockIdx.y + (size_t)H * blockIdx.z);
    const size_t q8 = total / 8, r8 = total % 8, xcd = lin % 8, k8 = lin / 8;
    const size_t item = xcd < r8 ? xcd * (q8 + 1) + k8 : r8 * (q8 + 1) + (xcd - r8) * q8 + k8;
    const size_t bh = item / per_head;
    const int tile = (int)(item % per_head);
    const int ti = tile / tiles, tj = tile % tiles;
    const float4 *qa = reinterpret_cast<const float4 *>(qp + (bh * nb + (size_t)ti * TILE) * DH);
    const float4 *kb = reinterpret_cast<const float4 *>(kp + (bh * nb + (size_t)tj * TILE) * DH);
    const int q_rows = min(TILE, nb - ti * TILE);
    const int k_rows = min(TILE, nb - tj * TILE);

    for (int e = threadIdx.x; e < TILE * kF4PerRow; e += kThreads) {
        const int r = e / kF4PerRow, c4 = e % kF4PerRow;
        const float4 a = r < q_rows ? qa[e] : make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 c = r < k_rows ? kb[e] : make_float4(0.f, 0.f, 0.f, 0.f);
        uint2 pa, pc;
        pa.x = pack_bf16x2(a.x, a.y), pa.y = pack_bf16x2(a.z, a.w);
        pc.x = pack_bf16x2(c.x, c.y), pc.y = pack_bf16x2(c.z, c.w);
        *reinterpret_cast<uint2 *>(&lds_q[r * kRow + 4 * c4]) = pa;
        *reinterpret_cast<uint2 *>(&lds_k[r * kRow + 4 * c4]) = pc;
    }
    __syncthreads();

    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int r16 = lane & 15, quad = lane >> 4;
    const int row0 = 16 * kStrips * (wave / kStrips), col0 = 64 * (wave % kStrips);
    f32x4 acc[kStrips][4];
#pragma unroll
    for (int i = 0; i < kStrips; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t)
            acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < DH / 16; ++s) {
        const int kof = 16 * s + 4 * quad;
        s16x4 a[kStrips];
#pragma unroll
        for (int i = 0; i < kStrips; ++i)
            a[i] = *reinterpret_cast<const s16x4 *>(&lds_q[(row0 + 16 * i + r16) * kRow + kof]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const s16x4 bv = *reinterpret_cast<const s16x4 *>(&lds_k[(col0 + 16 * t + r16) * kRow + kof]);
#pragma unroll
            for (int i = 0; i < kStrips; ++i)
                acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a[i], bv, acc[i][t], 0, 0, 0);
        }
    }

    // The tile goes out through LDS as whole-row segments: TILE/4 lanes store
    // 4 * TILE contiguous bytes of one row with non-temporal 16-byte stores, so
    // each 128-byte line of a (128-byte-aligned) row is written whole by one
    // instruction and nothing is read back or kept in the caches.
    float *lds_s = reinterpret_cast<float *>(lds_raw);
    __syncthreads(); // every wave has finished reading the operand tiles
#pragma unroll
    for (int i = 0; i < kStrips; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                lds_s[(row0 + 16 * i + 4 * quad + e) * kOutRow + col0 + 16 * t + r16] = acc[i][t][e];
    __syncthreads();
    float *out = scores + (bh * nb + (size_t)ti * TILE) * ld + (size_t)tj * TILE;
#pragma unroll
    for (int m = 0; m < TILE * TILE / 4 / kThreads; ++m) {
        const int idx = threadIdx.x + kThreads * m;
        const int row = idx / (TILE / 4), c4 = idx % (TILE / 4);
        if (row < q_rows && 4 * c4 < k_rows) // columns up to nb rounded up to 4, all inside ld
            __builtin_nontemporal_store(*reinterpret_cast<const f32x4 *>(&lds_s[row * kOutRow + 4 * c4]),
                                        reinterpret_cast<f32x4 *>(out + (size_t)row * ld + 4 * c4));
    }
}

// Persistent form of the 128 x 128 tile for Dh <= 128 (what the route runs):
// one 512-thread workgroup per resident slot, each walking a contiguous run of
// tiles.  The XCD of workgroup w (w % 8, dispatch is round-robin) takes the
// (w % 8)-th contiguous eighth of the (head, tile) list and splits it into
// one run per workgroup, so each XCD's L2 holds one head's means at a time.
// Tiles are numbered query-tile-major, so consecutive tiles of a run share
// their query tile: it stays in LDS (bf16) and is loaded again only when the
// run moves to the next query tile, about once per nb/128 tiles.  The key
// tile is prefetched: once the current one is in LDS, the next one's fp32
// values are loaded into registers, in flight while the current tile is
// multiplied, staged out through its own LDS buffer and stored.  The score
// stores thus overlap the next tile's loads, which the short-lived
// workgroups of subblock_scores_kernel (storing only at their end) could not
// do.  The arithmetic per tile is that kernel's, so the scores are the same
// bit for bit.  At 1953 blocks: 102 us, against 121 us with both operands
// prefetched per tile and 135 us with one workgroup per tile.  Registers and
// the three LDS tiles (135 KB at Dh = 128) leave one workgroup per CU.
template <int DH>
__global__ __launch_bounds__(512) void subblock_scores_persistent_kernel(const float *__restrict__ qp,
                                                                         const float *__restrict__ kp,
                                                                         float *__restrict__ scores, int nb, int ld,
                                                                         int tiles, unsigned total)
{
    constexpr int TILE = 128, kThreads = 512, kStrips = 2;
    constexpr int kRow = DH + 4; // bf16 per padded LDS row
    constexpr int kF4PerRow = DH / 4;
    constexpr int kLoads = TILE * kF4PerRow / kThreads; // float4 per thread and operand
    constexpr int kOutRow = TILE + 4;
    __shared__ __align__(16) uint16_t lds_q[TILE * kRow];
    __shared__ __align__(16) uint16_t lds_k[TILE * kRow];
    __shared__ __align__(16) float lds_s[TILE * kOutRow];

    // gridDim.x is a multiple of 8; items [first, last) belong to this XCD and
    // [begin, end) to this workgroup
    const unsigned per = gridDim.x / 8, xcd = blockIdx.x % 8, j = blockIdx.x / 8;
    const unsigned span = (total + 7) / 8;
    const unsigned first = xcd * span, last = min(total, first + span);
    const unsigned run = (span + per - 1) / per;
    const unsigned begin = min(last, first + j * run), end = min(last, begin + run);
    const unsigned per_head = (unsigned)(tiles * tiles);

    float4 kr[kLoads];
    auto load_k = [&](unsigned it) {
        const size_t bh = it / per_head;
        const int tj = (int)(it % per_head) % tiles;
        const float4 *kb = reinterpret_cast<const float4 *>(kp + (bh * nb + (size_t)tj * TILE) * DH);
        const int k_rows = min(TILE, nb - tj * TILE);
#pragma unroll
        for (int m = 0; m < kLoads; ++m) {
            const int e = threadIdx.x + kThreads * m;
            kr[m] = e / kF4PerRow < k_rows ? kb[e] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int r16 = lane & 15, quad = lane >> 4;
    const int row0 = 16 * kStrips * (wave / kStrips), col0 = 64 * (wave % kStrips);

    if (begin < end)
        load_k(begin);
    size_t held_bh = ~(size_t)0; // the (head, query tile) whose operand is in lds_q
    int held_ti = -1;
    for (unsigned item = begin; item < end; ++item) { // the same trip count for the whole workgroup
        const size_t bh = item / per_head;
        const int tile = (int)(item % per_head), ti = tile / tiles, tj = tile % tiles;
        const int q_rows = min(TILE, nb - ti * TILE), k_rows = min(TILE, nb - tj * TILE);
        __syncthreads(); // the previous tile's operand and score reads are over
        if (bh != held_bh || ti != held_ti) { // workgroup-uniform
            const float4 *qa = reinterpret_cast<const float4 *>(qp + (bh * nb + (size_t)ti * TILE) * DH);
#pragma unroll
            for (int m = 0; m < kLoads; ++m) {
                const int e = threadIdx.x + kThreads * m;
                const int r = e / kF4PerRow, c4 = e % kF4PerRow;
                const float4 a = r < q_rows ? qa[e] : make_float4(0.f, 0.f, 0.f, 0.f);
                uint2 pa;
                pa.x = pack_bf16x2(a.x, a.y), pa.y = pack_bf16x2(a.z, a.w);
                *reinterpret_cast<uint2 *>(&lds_q[r * kRow + 4 * c4]) = pa;
            }
            held_bh = bh, held_ti = ti;
        }
#pragma unroll
        for (int m = 0; m < kLoads; ++m) {
            const int e = threadIdx.x + kThreads * m;
            const int r = e / kF4PerRow, c4 = e % kF4PerRow;
            uint2 pc;
            pc.x = pack_bf16x2(kr[m].x, kr[m].y), pc.y = pack_bf16x2(kr[m].z, kr[m].w);
            *reinterpret_cast<uint2 *>(&lds_k[r * kRow + 4 * c4]) = pc;
        }
        __syncthreads();
        if (item + 1 < end)
            load_k(item + 1); // in flight during the products and the stores below

        f32x4 acc[kStrips][4];
#pragma unroll
        for (int i = 0; i < kStrips; ++i)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DH / 16; ++s) {
            const int kof = 16 * s + 4 * quad;
            s16x4 a[kStrips];
#pragma unroll
            for (int i = 0; i < kStrips; ++i)
                a[i] = *reinterpret_cast<const s16x4 *>(&lds_q[(row0 + 16 * i + r16) * kRow + kof]);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const s16x4 bv = *reinterpret_cast<const s16x4 *>(&lds_k[(col0 + 16 * t + r16) * kRow + kof]);
#pragma unroll
                for (int i = 0; i < kStrips; ++i)
                    acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a[i], bv, acc[i][t], 0, 0, 0);
            }
        }

        // lds_s has its own space; the barrier at the loop top ordered the
        // previous tile's reads of it before these writes
#pragma unroll
        for (int i = 0; i < kStrips; ++i)
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    lds_s[(row0 + 16 * i + 4 * quad + e) * kOutRow + col0 + 16 * t + r16] = acc[i][t][e];
        __syncthreads();
        float *out = scores + (bh * nb + (size_t)ti * TILE) * ld + (size_t)tj * TILE;
#pragma unroll
        for (int m = 0; m < TILE * TILE / 4 / kThreads; ++m) {
            const int idx = threadIdx.x + kThreads * m;
            const int row = idx / (TILE / 4), c4 = idx % (TILE / 4);
            if (row < q_rows && 4 * c4 < k_rows) // columns up to nb rounded up to 4, all inside ld
                __builtin_nontemporal_store(*reinterpret_cast<const f32x4 *>(&lds_s[row * kOutRow + 4 * c4]),
                                            reinterpret_cast<f32x4 *>(out + (size_t)row * ld + 4 * c4));
        }
    }
}

// ---------------------------------------------------------------- selection

// Order-preserving map of an fp32 score to an unsigned key; -0 and +0 map to
// the same key so that they tie, as equal scores do.  Positive scores (and
// +0) take u + 2^31, negative ones 2^32 - u, which sends -0 to +0's key and
// every other negative below it in reverse order of magnitude.  No score maps
// to 0, which marks the slots past the last key block.
__device__ __forceinline__ uint32_t score_key(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (int32_t)u < 0 ? 0u - u : u ^ 0x80000000u;
}

__device__ __forceinline__ int lanes_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// x from the lane `ctrl` names (DPP), 0 where the source lane is out of
// range or the row / bank masks leave the lane out.
template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_or_zero(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, BANK_MASK, true);
}

// Sum of x over lanes 0 .. lane: within each row of 16 lanes by row shifts
// (1, 2, 3, then 4 and 8 on the upper banks), then across rows by broadcasting
// lane 15 into row 1 and 3 and lane 31 into rows 2 and 3 (the GCN DPP scan).
__device__ __forceinline__ uint32_t prefix_sum(uint32_t x)
{
    uint32_t t = x + dpp_or_zero<0x111>(x); // row_shr:1
    t += dpp_or_zero<0x112>(x);             // row_shr:2
    t += dpp_or_zero<0x113>(x);             // row_shr:3
    t += dpp_or_zero<0x114, 0xf, 0xe>(t);   // row_shr:4, banks 1-3
    t += dpp_or_zero<0x118, 0xf, 0xc>(t);   // row_shr:8, banks 2-3
    t += dpp_or_zero<0x142, 0xa, 0xf>(t);   // row_bcast:15 into rows 1, 3
    t += dpp_or_zero<0x143, 0xc, 0xf>(t);   // row_bcast:31 into rows 2, 3
    return t;
}

// Sum of x over lanes lane .. 63: the wave total less the sum below the lane.
__device__ __forceinline__ uint32_t suffix_sum(uint32_t x)
{
    const uint32_t incl = prefix_sum(x);
    const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
    return total - incl + x;
}

// Radix-select state: keys matching `prefix` under `mask` are still
// candidates, `need` of them are kept, and `in_bin` of them share the prefix.
struct RadixState {
    uint32_t prefix, mask, need, in_bin;
};

constexpr int kTopBits = 10;                   // the first digit: ten bits, just below those all of a row's keys share
constexpr int kTopBins = 1 << kTopBits;
constexpr int kMaxSurvivors = 512;
constexpr int kSelectWords = kTopBins; // LDS words one selecting wave uses (survivors overlay the histogram)
static_assert(256 + kMaxSurvivors <= kTopBins, "survivors sit past the 256 bins the later digits use");

// Least and greatest x over the wave: four row shifts leave each row's
// extreme in its lane 15 (a lane whose source lies outside its row keeps its
// own value), and the four rows' extremes are combined from those lanes.
__device__ __forceinline__ uint32_t wave_min(uint32_t x)
{
    x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x111, 0xf, 0xf, false)); // row_shr:1
    x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x112, 0xf, 0xf, false)); // row_shr:2
    x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x114, 0xf, 0xf, false)); // row_shr:4
    x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x118, 0xf, 0xf, false)); // row_shr:8
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)x, 15), b = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)x, 47), d = (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
    return min(min(a, b), min(c, d));
}

__device__ __forceinline__ uint32_t wave_max(uint32_t x)
{
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x111, 0xf, 0xf, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x112, 0xf, 0xf, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x114, 0xf, 0xf, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x118, 0xf, 0xf, false));
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)x, 15), b = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)x, 47), d = (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
    return max(max(a, b), max(c, d));
}

// Picks the first digit, bits shift .. shift + 9 of the keys (all keys share
// `high`, their bits above those), from its 1024-bin histogram: the largest
// digit whose keys, with those of all larger digits, reach `need`.  Lane l
// sums bins 16 l .. 16 l + 15; a suffix sum over the lanes finds the lane
// holding the digit, then sixteen lanes take one bin each of that lane's range.
__device__ __forceinline__ void choose_top_digit(const uint32_t *hist, int lane, int shift, uint32_t high,
                                                 RadixState &st)
{
    const uint4 *h4 = reinterpret_cast<const uint4 *>(hist) + 4 * lane;
    const uint4 a = h4[0], b = h4[1], c = h4[2], d = h4[3];
    const uint32_t cnt = (a.x + a.y + a.z + a.w) + (b.x + b.y + b.z + b.w) + (c.x + c.y + c.z + c.w) +
                         (d.x + d.y + d.z + d.w);
    const uint32_t suffix = suffix_sum(cnt);
    const uint32_t above = suffix - cnt;
    const int L = __builtin_ctzll(__ballot(above < st.need && st.need <= suffix)); // exactly one lane
    const uint32_t above_l = (uint32_t)__builtin_amdgcn_readlane(above, L);
    uint32_t h = hist[(16 * L + lane) & (kTopBins - 1)];
    h = lane < 16 ? h : 0u;
    const uint32_t greater = above_l + suffix_sum(h) - h; // keys of the larger digits
    const int D = __builtin_ctzll(__ballot(greater < st.need && st.need <= greater + h));
    st.prefix = high | ((uint32_t)(16 * L + D) << shift);
    st.mask = ~0u << shift;
    st.need -= (uint32_t)__builtin_amdgcn_readlane(greater, D);
    st.in_bin = (uint32_t)__builtin_amdgcn_readlane(h, D);
}

// The same for an 8-bit digit at `shift` from a 256-bin histogram (lane l
// reads digits 4l .. 4l+3).
__device__ __forceinline__ void choose_digit(const uint32_t *hist, int lane, int shift, RadixState &st)
{
    const uint4 h4 = reinterpret_cast<const uint4 *>(hist)[lane];
    const uint32_t c = h4.x + h4.y + h4.z + h4.w;
    const uint32_t suffix = suffix_sum(c); // keys of digits >= 4l
    const uint32_t above = suffix - c;
    const bool mine = above < st.need && st.need <= suffix; // exactly one lane
    uint32_t digit = 4u * lane, greater = above, count = h4.x;
    if (mine) {
        if (above + h4.w >= st.need) {
            digit += 3u, count = h4.w;
        } else if (above + h4.w + h4.z >= st.need) {
            digit += 2u, greater += h4.w, count = h4.z;
        } else if (above + h4.w + h4.z + h4.y >= st.need) {
            digit += 1u, greater += h4.w + h4.z, count = h4.y;
        } else {
            greater += h4.w + h4.z + h4.y;
        }
    }
    const int src = __builtin_ctzll(__ballot(mine));
    st.prefix |= (uint32_t)__builtin_amdgcn_readlane(digit, src) << shift;
    st.mask |= 0xffu << shift;
    st.need -= (uint32_t)__builtin_amdgcn_readlane(greater, src);
    st.in_bin = (uint32_t)__builtin_amdgcn_readlane(count, src);
}

// Orders the LDS accesses of one wave across its lanes: a wavefront's LDS
// operations execute in order, so fences at wavefront scope that keep the
// compiler from moving memory operations across the point are enough (no
// workgroup barrier, so waves of a larger workgroup select independently).
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A wave-uniform value the compiler cannot see through: each loop over the
// slots tests `64 s < nb` against its own copy, so the tests are not merged
// across loops into per-slot flags held for the whole selection.
__device__ __forceinline__ int fresh_uniform(int x)
{
    asm volatile("" : "+s"(x));
    return x;
}

// The keep largest of one query block's keys, written as ascending key-block
// indices to out[0 .. keep-1]; executed by one whole wave, 1 <= keep <= nb.
// Lane l holds the key of block 64 s + l in key[s] (s < S, 64 S >= nb, and
// 64 S / 2 < nb when S > 4, so the first half of the slots is whole), and 0
// in the slots of blocks at or past nb: below every score's key and past
// every real block's index, so those slots are never among the kept ones and
// need no test.  `lds` is the wave's own kSelectWords words, 16-byte aligned:
// the 1024-bin histogram of the first digit; once that digit is chosen,
// words 256 .. 256 + kMaxSurvivors - 1 take the survivors and words 0 .. 255
// the 256-bin histograms of the later digits.
// A radix select finds the keep-th largest key T, most significant digit
// first.  The bits above the highest one in which the least and the greatest
// key differ are the same in every key, so the first digit is the ten bits
// just below them: keys crowded into a narrow range (scores of one sign and
// magnitude) still spread over the 1024 bins.  A histogram of that digit
// (LDS atomics, one per key) fixes it, the keys sharing it are compacted into LDS (each slot's
// matching lanes found by one ballot), and 8-bit digits over those few fix
// the rest, each again taken just below the bits the remaining candidates
// share -- stopping as soon as every key left in the bin is kept (keys >=
// the prefix are then exactly the kept ones) or the candidates are all equal.
// A row whose keys are all equal skips the digits.  Only when T splits a run of
// equal keys do ties need ranks (lowest index first).  Kept blocks are
// written slot by slot: a ballot of the slot's kept lanes gives each lane its
// place, so the list comes out ascending with no sort.
template <int S>
__device__ __forceinline__ void select_keep(const uint32_t (&key)[S], int nb, int keep, int lane, uint32_t *lds,
                                            int32_t *__restrict__ out)
{
    uint32_t *hist = lds;
    uint32_t *survivors = lds + 256;
    RadixState st = {0u, 0u, (uint32_t)keep, 0u};
    constexpr int kWhole = S > 4 ? S / 2 : 0; // slots known to be whole: no test

#pragma unroll
    for (int i = 0; i < kTopBins / (4 * kWave); ++i)
        reinterpret_cast<uint4 *>(hist)[lane + kWave * i] = make_uint4(0u, 0u, 0u, 0u);
    wave_sync();
    // The keys' range; key 0 (slots past the last block) wraps to the top
    // under key - 1 and so is left out of the least.
    uint32_t lo = ~0u, hi = 0u;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        lo = min(lo, key[s] - 1u);
        hi = max(hi, key[s]);
    }
    lo = wave_min(lo) + 1u;
    hi = wave_max(hi);
    const uint32_t diff = lo ^ hi;
    const int varying = diff ? 32 - __builtin_clz(diff) : 0; // low bits in which the keys differ
    const int shift0 = varying > kTopBits ? varying - kTopBits : 0;
    const uint32_t high = shift0 + kTopBits >= 32 ? 0u : lo & (~0u << (shift0 + kTopBits));

    int n;
    if (lo == hi) { // wave-uniform: every key of the row is the same, all are ties
        st.prefix = lo, st.mask = ~0u, st.in_bin = (uint32_t)nb;
    } else {
        n = fresh_uniform(nb);
        uint32_t one; // held in a register (the compiler would set it again before every atomic)
        asm volatile("v_mov_b32 %0, 1" : "=v"(one));
#pragma unroll
        for (int s = 0; s < S; ++s) {
            if (s < kWhole) // every lane holds a block's key
                atomicAdd(&hist[(key[s] >> shift0) & (kTopBins - 1)], one);
            else if (kWave * s < n && key[s] != 0u) // wave-uniform slot test; lanes past the last block left out
                atomicAdd(&hist[(key[s] >> shift0) & (kTopBins - 1)], one);
        }
        wave_sync();
        choose_top_digit(hist, lane, shift0, high, st);
        wave_sync();

        if (st.need < st.in_bin && shift0 > 0) {
            // the bin holds keys that are not kept: resolve the remaining bits
            const bool compact = st.in_bin <= (uint32_t)kMaxSurvivors; // wave-uniform
            uint32_t n_surv = 0u;
            if (compact) {
                n = fresh_uniform(nb);
                char *surv_bytes = reinterpret_cast<char *>(survivors);
#pragma unroll
                for (int s = 0; s < S; ++s)
                    if (s < kWhole || kWave * s < n) {
                        const bool m = (key[s] & st.mask) == st.prefix;
                        const uint64_t mm = __ballot(m);
                        if (mm) { // wave-uniform
                            // exactly in_bin keys match, so every place is below the bound (the
                            // mask only keeps the address inside the list whatever happens)
                            if (m)
                                *reinterpret_cast<uint32_t *>(
                                    surv_bytes + ((((uint32_t)lanes_below(mm) << 2) + (n_surv << 2)) &
                                                  (uint32_t)(4 * kMaxSurvivors - 1))) = key[s];
                            n_surv += (uint32_t)__builtin_popcountll(mm);
                        }
                    }
                wave_sync();
            }
#pragma unroll 1
            for (;;) {
                // The candidates' range (keys under the prefix): bits they all
                // share are fixed at once, and the next 8-bit digit is the one
                // just below them; equal candidates end the search (ties).
                uint32_t clo = ~0u, chi = 0u;
                if (compact) {
                    for (uint32_t c = lane; c < n_surv; c += kWave) {
                        const uint32_t k = survivors[c];
                        if ((k & st.mask) == st.prefix)
                            clo = min(clo, k), chi = max(chi, k);
                    }
                } else {
                    n = fresh_uniform(nb);
#pragma unroll
                    for (int s = 0; s < S; ++s)
                        if ((s < kWhole || kWave * s < n) && (key[s] & st.mask) == st.prefix)
                            clo = min(clo, key[s]), chi = max(chi, key[s]);
                }
                clo = wave_min(clo);
                chi = wave_max(chi);
                if (clo == chi) {
                    st.prefix = clo, st.mask = ~0u;
                    break; // every candidate is the keep-th largest key
                }
                const int vary = 32 - __builtin_clz(clo ^ chi); // below the bits already fixed
                const int shift = vary > 8 ? vary - 8 : 0;
                st.prefix = clo & (~0u << vary);
                st.mask = ~0u << vary;
                reinterpret_cast<uint4 *>(hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
                wave_sync();
                if (compact) {
                    for (uint32_t c = lane; c < n_surv; c += kWave) {
                        const uint32_t k = survivors[c];
                        if ((k & st.mask) == st.prefix)
                            atomicAdd(&hist[(k >> shift) & 0xffu], 1u);
                    }
                } else {
                    n = fresh_uniform(nb);
#pragma unroll
                    for (int s = 0; s < S; ++s)
                        if ((s < kWhole || kWave * s < n) && (key[s] & st.mask) == st.prefix)
                            atomicAdd(&hist[(key[s] >> shift) & 0xffu], 1u);
                }
                wave_sync();
                choose_digit(hist, lane, shift, st);
                wave_sync();
                if (shift == 0 || st.need == st.in_bin)
                    break; // every bit fixed, or every key left in the bin is kept
            }
        }
    }

    // Kept: every key above T = st.prefix and, of the in_bin keys equal to
    // it, the st.need of lowest index -- when st.need == st.in_bin simply
    // every key >= st.prefix (the bits below the mask are zero in it).  A
    // slot whose kept keys would run past keep (never, as exactly keep are
    // kept) writes nothing: the test is on wave-uniform counts.
    const uint32_t T = st.prefix;
    int32_t block; // lane's block index in the current slot, advanced per slot
    asm volatile("v_mov_b32 %0, %1" : "=v"(block) : "v"(lane));
    char *out_bytes = reinterpret_cast<char *>(out);
    uint32_t written = 0u;
    auto emit = [&](bool sel) {
        const uint64_t ms = __ballot(sel);
        const uint32_t cnt = (uint32_t)__builtin_popcountll(ms);
        if (written + cnt <= (uint32_t)keep && sel)
            *reinterpret_cast<int32_t *>(out_bytes + (((uint32_t)lanes_below(ms) << 2) + (written << 2))) = block;
        written += cnt;
        block += kWave;
    };
    n = fresh_uniform(nb);
    if (st.need == st.in_bin) { // wave-uniform
#pragma unroll
        for (int s = 0; s < S; ++s)
            if (s < kWhole || kWave * s < n)
                emit(key[s] >= T);
    } else {
        uint32_t ties = 0u;
#pragma unroll
        for (int s = 0; s < S; ++s)
            if (s < kWhole || kWave * s < n) {
                const bool eq = key[s] == T;
                const uint64_t me = __ballot(eq);
                emit(key[s] > T || (eq && ties + (uint32_t)lanes_below(me) < st.need));
                ties += (uint32_t)__builtin_popcountll(me);
            }
    }
}

// One wave (one workgroup) per query block; grid (nb, H, B).  Lane l loads
// the scores of key blocks l, l + 64, ... (S of them) and keeps their keys in
// registers, then selects (select_keep).  The loads go through a buffer
// descriptor over the row's nb scores: lane offset and slot offset are fixed
// (no address arithmetic per slot), every load is issued before any is used,
// and blocks past nb read 0 from the range check and are then given key 0.
// The launcher picks the smallest S with 64 S >= nb, so for S > 4 the first
// S / 2 slots are whole and need no test.
template <int S>
__global__ __launch_bounds__(kWave) void subblock_topk_kernel(const float *__restrict__ scores,
                                                              int32_t *__restrict__ kept, int nb, int ld, int keep,
                                                              int H)
{
    __shared__ __align__(16) uint32_t lds[kSelectWords];
    constexpr int kRawFormat = 0x00020000; // descriptor dword 3: 32-bit data format, no swizzle or stride
    constexpr int kWhole = S > 4 ? S / 2 : 0;
    constexpr int kSlotsPerOffset = 4096 / (4 * kWave); // slots the 12-bit instruction offset reaches
    const int lane = threadIdx.x;
    const size_t row = ((size_t)blockIdx.z * H + blockIdx.y) * nb + blockIdx.x;
    const __amdgpu_buffer_rsrc_t rd =
        __builtin_amdgcn_make_buffer_rsrc((void *)(scores + row * ld), 0, nb * 4, kRawFormat);

    float v[S];
#pragma unroll
    for (int q = 0; q < S; ++q) {
        // lane offset + a multiple of 4 KiB in the register, the rest in the instruction
        const int base = 4 * lane + 4096 * (q / kSlotsPerOffset);
        v[q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                             rd, base + 4 * kWave * (q % kSlotsPerOffset), 0, 2 /* nt */));
    }
    uint32_t key[S];
#pragma unroll
    for (int q = 0; q < S; ++q)
        key[q] = (q < kWhole || kWave * q + lane < nb) ? score_key(v[q]) : 0u;
    select_keep<S>(key, nb, keep, lane, lds, kept + row * keep);
}

// ---------------------------------------------------------------- fused route

// Scores and kept blocks in one kernel, for callers that do not need the
// score matrix: the scores of a strip of query blocks go from the matrix
// cores through LDS into the registers of the waves that select on them, and
// never to memory.  Only the means are read and the kept indices written.
//
// Workgroup = 16 waves and a strip of ROWS = 16 * RPW query blocks of one
// (sample, head); wave w selects for query blocks RPW w .. RPW w + RPW - 1 of
// the strip.  Phase 1 walks the key blocks in chunks of 256: the chunk's fp32
// means are loaded by the whole workgroup (consecutive bytes per load
// instruction), rounded to bf16 into LDS (KD <= 128 dimensions at a time),
// and wave w multiplies key tile w (16 key blocks) with each 16-row block of
// the strip's bf16 query means on the matrix cores -- the same operands and
// the same MFMA 16x16x16 sequence over the dimensions as the score kernels,
// so every score is the same bits.  The order-preserving keys of the chunk's
// scores are staged in LDS, and each wave reads its own query blocks' 256
// keys into the register slots of the chunk: lane l ends up with key block
// 64 s + l in slot s, the layout select_keep takes (0 past the last block).
// Phase 2 reuses the LDS as one selection area per wave and the waves select
// independently.
//
// RV = ceil(nb / 256) chunks, so 4 RV key slots per query block; RPW = 2
// query blocks per wave while RV <= 8 (up to 64 key registers of the 128 a
// wave has when 16 share a CU), else 1.  Workgroups walk (sample, head, strip) items; the
// XCD of workgroup g (g % 8, dispatch is round-robin) takes the (g % 8)-th
// contiguous eighth of the items, so the 32 workgroups an XCD runs at once
// share one head's key means in its L2.
//
// What bounds it (1344x768 5 s, 1953 blocks, 32 heads): each strip re-reads
// its head's key means, 16 bytes of L2 traffic per score against the score
// kernel's 4 (128 x 128 tiles): 2 GB in all, which L2 serves at about 9 TB/s
// (a copy of the kernel that only streams the chunks takes ~230 us).  The
// keys of a strip fill the register file, so the strip cannot grow, one
// workgroup runs per CU, and its load, multiply and select phases do not
// overlap with another's.
constexpr int kRouteWaves = 16;
constexpr int kChunkKeys = 256;

template <int DH, int RV, int RPW>
__global__ __launch_bounds__(kRouteWaves * kWave) void subblock_route_fused_kernel(
    const float *__restrict__ qp, const float *__restrict__ kp, int32_t *__restrict__ kept, int nb, int keep,
    int strips, uint64_t total)
{
    constexpr int kThreads = kRouteWaves * kWave;
    constexpr int ROWS = kRouteWaves * RPW;   // query blocks per strip
    constexpr int NRB = ROWS / 16;            // 16-row MFMA blocks of the strip
    constexpr int KD = DH < 128 ? DH : 128;   // key dimensions staged per pass
    constexpr int PASSES = DH / KD;
    constexpr int kQRow = DH + 4;             // bf16 per padded LDS row (rows 8 bytes apart in bank)
    constexpr int kKRow = KD + 4;
    constexpr int kSRow = kChunkKeys + 4;     // keys per padded staging row
    constexpr int kQBytes = ROWS * kQRow * 2, kKBytes = kChunkKeys * kKRow * 2, kSBytes = ROWS * kSRow * 4;
    constexpr int kPhase1 = kQBytes + kKBytes + kSBytes;
    constexpr int kPhase2 = kRouteWaves * kSelectWords * 4;
    constexpr int kF4 = kChunkKeys * KD / 4 / kThreads; // float4 of the key chunk per thread and pass
    static_assert(kF4 >= 1, "tile shapes");
    __shared__ __align__(16) unsigned char lds_raw[kPhase1 > kPhase2 ? kPhase1 : kPhase2];
    uint16_t *lds_q = reinterpret_cast<uint16_t *>(lds_raw);
    uint16_t *lds_k = reinterpret_cast<uint16_t *>(lds_raw + kQBytes);
    uint32_t *lds_s = reinterpret_cast<uint32_t *>(lds_raw + kQBytes + kKBytes);

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int r16 = lane & 15, quad = lane >> 4;

    const uint64_t per = gridDim.x / 8, xcd = blockIdx.x % 8, g = blockIdx.x / 8;
    const uint64_t span = (total + 7) / 8, first = xcd * span;
    const uint64_t last = first + span < total ? first + span : total;
    for (uint64_t item = first + g; item < last; item += per) { // the same trip count for the whole workgroup
        const uint64_t bh = item / (uint64_t)strips;
        const int i0 = (int)(item % (uint64_t)strips) * ROWS; // first query block of the strip
        const float *qrow = qp + (bh * nb) * DH;
        const float *krow = kp + (bh * nb) * DH;

        __syncthreads(); // the previous item's selection areas are free
        // the strip's query means, bf16, rows past nb zero
        for (int e = tid; e < ROWS * DH / 4; e += kThreads) {
            const int r = e / (DH / 4), c4 = e % (DH / 4);
            const float4 a = i0 + r < nb ? reinterpret_cast<const float4 *>(qrow + (size_t)(i0 + r) * DH)[c4]
                                         : make_float4(0.f, 0.f, 0.f, 0.f);
            uint2 pa;
            pa.x = pack_bf16x2(a.x, a.y), pa.y = pack_bf16x2(a.z, a.w);
            *reinterpret_cast<uint2 *>(&lds_q[r * kQRow + 4 * c4]) = pa;
        }

        // A runtime loop over the chunks (unrolled, the compiler would hold the
        // addresses of every chunk's loads at once, and spill); each chunk's
        // keys enter the last four register slots and the earlier ones move
        // down four, so after RV chunks slots 4 r .. 4 r + 3 hold chunk r.
        uint32_t key[RPW][4 * RV];
#pragma unroll 1
        for (int c = 0; c < RV; ++c) {
            f32x4 acc[NRB];
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
                acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < PASSES; ++p) {
                float4 v[kF4];
#pragma unroll
                for (int m = 0; m < kF4; ++m) {
                    const int e = tid + kThreads * m;
                    const int kr = e / (KD / 4), c4 = e % (KD / 4);
                    const int j = kChunkKeys * c + kr;
                    v[m] = j < nb ? reinterpret_cast<const float4 *>(krow + (size_t)j * DH + p * KD)[c4]
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
                }
                __syncthreads(); // every wave is done with the previous pass's key tile
#pragma unroll
                for (int m = 0; m < kF4; ++m) {
                    const int e = tid + kThreads * m;
                    const int kr = e / (KD / 4), c4 = e % (KD / 4);
                    uint2 pc;
                    pc.x = pack_bf16x2(v[m].x, v[m].y), pc.y = pack_bf16x2(v[m].z, v[m].w);
                    *reinterpret_cast<uint2 *>(&lds_k[kr * kKRow + 4 * c4]) = pc;
                }
                __syncthreads();
#pragma unroll
                for (int s = 0; s < KD / 16; ++s) {
                    const int kof = 16 * s + 4 * quad;
                    const s16x4 bv = *reinterpret_cast<const s16x4 *>(&lds_k[(16 * wave + r16) * kKRow + kof]);
#pragma unroll
                    for (int rb = 0; rb < NRB; ++rb) {
                        const s16x4 a = *reinterpret_cast<const s16x4 *>(
                            &lds_q[(16 * rb + r16) * kQRow + p * KD + kof]);
                        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bv, acc[rb], 0, 0, 0);
                    }
                }
            }
            // query block 16 rb + 4 quad + e, key block 256 c + 16 wave + r16
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    lds_s[(16 * rb + 4 * quad + e) * kSRow + 16 * wave + r16] =
                        kChunkKeys * c + 16 * wave + r16 < nb ? score_key(acc[rb][e]) : 0u;
            __syncthreads();
#pragma unroll
            for (int j = 0; j < RPW; ++j) {
#pragma unroll
                for (int q = 0; q + 4 < 4 * RV; ++q)
                    key[j][q] = key[j][q + 4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    key[j][4 * RV - 4 + e] = lds_s[(RPW * wave + j) * kSRow + kWave * e + lane];
            }
            // the staging rows are written again only after the next chunk's barriers
        }
        __syncthreads(); // phase 1's LDS is dead: the selection areas overlay it
        uint32_t *sel = reinterpret_cast<uint32_t *>(lds_raw) + wave * kSelectWords;
#pragma unroll
        for (int j = 0; j < RPW; ++j) {
            const int i = i0 + RPW * wave + j;
            if (i < nb) // wave-uniform
                select_keep<4 * RV>(key[j], nb, keep, lane, sel, kept + (bh * nb + (uint64_t)i) * keep);
        }
    }
}

template <int DH, int RV>
void launch_route_fused_dh_rv(const float *qp, const float *kp, int32_t *kept, int nb, int keep, int H, int B,
                              hipStream_t stream)
{
    constexpr int RPW = RV <= 8 ? 2 : 1;
    constexpr int ROWS = kRouteWaves * RPW;
    const int strips = (nb + ROWS - 1) / ROWS;
    const uint64_t total = (uint64_t)B * (uint64_t)H * (uint64_t)strips;
    // at most 8 * 4096 workgroups (each then walks its items); a multiple of 8
    const uint64_t grid = ((total + 7) / 8 * 8) < 32768u ? (total + 7) / 8 * 8 : 32768u;
    hipLaunchKernelGGL((subblock_route_fused_kernel<DH, RV, RPW>), dim3((unsigned)grid), dim3(kRouteWaves * kWave), 0,
                       stream, qp, kp, kept, nb, keep, strips, total);
}

template <int DH>
void launch_route_fused_dh(const float *qp, const float *kp, int32_t *kept, int nb, int keep, int H, int B,
                           hipStream_t stream)
{
    if (nb <= 256) launch_route_fused_dh_rv<DH, 1>(qp, kp, kept, nb, keep, H, B, stream);
    else if (nb <= 512) launch_route_fused_dh_rv<DH, 2>(qp, kp, kept, nb, keep, H, B, stream);
    else if (nb <= 1024) launch_route_fused_dh_rv<DH, 4>(qp, kp, kept, nb, keep, H, B, stream);
    else if (nb <= 2048) launch_route_fused_dh_rv<DH, 8>(qp, kp, kept, nb, keep, H, B, stream);
    else launch_route_fused_dh_rv<DH, 16>(qp, kp, kept, nb, keep, H, B, stream);
}

template <int S>
void launch_topk_s(const float *scores, int32_t *kept, int nb, int ld, int keep, int H, int B, hipStream_t stream)
{
    hipLaunchKernelGGL(subblock_topk_kernel<S>, dim3((unsigned)nb, (unsigned)H, (unsigned)B), dim3(kWave), 0, stream,
                       scores, kept, nb, ld, keep, H);
}

template <int DH>
void launch_scores_dh(const float *qp, const float *kp, float *scores, int nb, int ld, int H, int B,
                      hipStream_t stream)
{
    const uint64_t tiles128 = (uint64_t)((nb + 127) / 128);
    if (DH <= 128 && tiles128 * tiles128 * (uint64_t)H * (uint64_t)B > 0x7fffffffull) {
        // beyond the persistent kernel's 32-bit tile count: one workgroup per tile
        constexpr int kTile = 128;
        const int tiles = (nb + kTile - 1) / kTile;
        hipLaunchKernelGGL((subblock_scores_kernel<DH, kTile>),
                           dim3((unsigned)(tiles * tiles), (unsigned)H, (unsigned)B), dim3(4 * kTile), 0, stream, qp,
                           kp, scores, nb, ld, tiles, H);
        return;
    }
    if constexpr (DH <= 128) {
        // as many workgroups as the device holds at once (a multiple of 8 for
        // the per-XCD ranges), no more than there are tiles (rounded up to 8)
        const int tiles = (nb + 127) / 128;
        const unsigned total = (unsigned)(tiles * tiles) * (unsigned)(H * B);
        int dev = 0, cus = 0, per_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8) {
            (void)hipGetLastError(); // a failed query: fall back to the MI355X's 256 CUs
            cus = 256;
        }
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, subblock_scores_persistent_kernel<DH>, 512, 0) !=
                hipSuccess || per_cu < 1) {
            (void)hipGetLastError();
            per_cu = 1;
        }
        const unsigned resident = (unsigned)(cus * per_cu) / 8 * 8, need = (total + 7) / 8 * 8;
        hipLaunchKernelGGL(subblock_scores_persistent_kernel<DH>, dim3(resident < need ? resident : need), dim3(512),
                           0, stream, qp, kp, scores, nb, ld, tiles, total);
    } else {
        constexpr int kTile = 64;
        const int tiles = (nb + kTile - 1) / kTile;
        hipLaunchKernelGGL((subblock_scores_kernel<DH, kTile>),
                           dim3((unsigned)(tiles * tiles), (unsigned)H, (unsigned)B), dim3(4 * kTile), 0, stream, qp,
                           kp, scores, nb, ld, tiles, H);
    }
}

template <int VPT>
void launch_pool_head_major(const u32x4 *q, const u32x4 *k, float *qp, float *kp, int N, int nb, int H, int B,
                            hipStream_t stream)
{
    hipLaunchKernelGGL(subblock_pool_head_major_kernel<VPT>, dim3((unsigned)nb, (unsigned)(2 * H), (unsigned)B),
                       dim3(256), 0, stream, q, k, qp, kp, N, nb, H);
}

} // namespace

hipError_t launch_subblock_pool(const void *q, const void *k, float *q_pooled, float *k_pooled, int64_t B, int64_t N,
                                int64_t H, int64_t Dh, bool head_major, hipStream_t stream)
{
    const int nb = (int)((N + kBlockTokens - 1) / kBlockTokens);
    const auto *qv = static_cast<const u32x4 *>(q);
    const auto *kv = static_cast<const u32x4 *>(k);
    const int vph = (int)(Dh / 8);
    if (!head_major) {
        const int C = (int)(H * Dh / 8);
        const int chunks = (C + kWave - 1) / kWave;
        const int vph_shift = __builtin_ctz((unsigned)vph);
        hipLaunchKernelGGL(subblock_pool_token_major_kernel, dim3((unsigned)(chunks * nb), 2u, (unsigned)B),
                           dim3(kPoolWaves * kWave), 0, stream, qv, kv, q_pooled, k_pooled, (int)N, nb, C, chunks, vph_shift);
        return hipGetLastError();
    }
    const int h = (int)H, n = (int)N, b = (int)B;
    switch (vph) {
    case 2: launch_pool_head_major<2>(qv, kv, q_pooled, k_pooled, n, nb, h, b, stream); break;
    case 4: launch_pool_head_major<4>(qv, kv, q_pooled, k_pooled, n, nb, h, b, stream); break;
    case 8: launch_pool_head_major<8>(qv, kv, q_pooled, k_pooled, n, nb, h, b, stream); break;
    case 16: launch_pool_head_major<16>(qv, kv, q_pooled, k_pooled, n, nb, h, b, stream); break;
    case 32: launch_pool_head_major<32>(qv, kv, q_pooled, k_pooled, n, nb, h, b, stream); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_subblock_route(const float *q_pooled, const float *k_pooled, float *scores, int32_t *kept,
                                 int64_t B, int64_t H, int64_t nb, int64_t Dh, int64_t ld, int64_t keep,
                                 hipStream_t stream)
{
    const int n = (int)nb, l = (int)ld, h = (int)H, b = (int)B;
    if (!scores) { // kept blocks only: one fused kernel, no score matrix
        if (keep == 0)
            return hipSuccess;
        const int kp = (int)keep;
        switch (Dh) {
        case 16: launch_route_fused_dh<16>(q_pooled, k_pooled, kept, n, kp, h, b, stream); break;
        case 32: launch_route_fused_dh<32>(q_pooled, k_pooled, kept, n, kp, h, b, stream); break;
        case 64: launch_route_fused_dh<64>(q_pooled, k_pooled, kept, n, kp, h, b, stream); break;
        case 128: launch_route_fused_dh<128>(q_pooled, k_pooled, kept, n, kp, h, b, stream); break;
        case 256: launch_route_fused_dh<256>(q_pooled, k_pooled, kept, n, kp, h, b, stream); break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    switch (Dh) {
    case 16: launch_scores_dh<16>(q_pooled, k_pooled, scores, n, l, h, b, stream); break;
    case 32: launch_scores_dh<32>(q_pooled, k_pooled, scores, n, l, h, b, stream); break;
    case 64: launch_scores_dh<64>(q_pooled, k_pooled, scores, n, l, h, b, stream); break;
    case 128: launch_scores_dh<128>(q_pooled, k_pooled, scores, n, l, h, b, stream); break;
    case 256: launch_scores_dh<256>(q_pooled, k_pooled, scores, n, l, h, b, stream); break;
    default: return hipErrorInvalidValue;
    }
    if (keep == 0)
        return hipGetLastError();
    const int kp = (int)keep;
    if (n <= 256) launch_topk_s<4>(scores, kept, n, l, kp, h, b, stream);
    else if (n <= 512) launch_topk_s<8>(scores, kept, n, l, kp, h, b, stream);
    else if (n <= 1024) launch_topk_s<16>(scores, kept, n, l, kp, h, b, stream);
    else if (n <= 2048) launch_topk_s<32>(scores, kept, n, l, kp, h, b, stream);
    else launch_topk_s<64>(scores, kept, n, l, kp, h, b, stream);
    return hipGetLastError();
}

} // namespace dit
