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
// the same key so that they tie, as equal scores do.
__device__ __forceinline__ uint32_t score_key(float f)
{
    uint32_t u = __float_as_uint(f);
    u = (u == 0x80000000u) ? 0u : u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lanes_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Radix-select state: keys matching `prefix` under `mask` are still
// candidates, `need` of them are kept, and `in_bin` of them share the prefix.
struct RadixState {
    uint32_t prefix, mask, need, in_bin;
};

// Picks the next 8-bit digit from a 256-bin histogram (lane l reads digits
// 4l .. 4l+3): the largest digit whose keys, with those of all larger digits,
// reach `need`.
__device__ __forceinline__ void choose_digit(const uint32_t *hist, int lane, int shift, RadixState &st)
{
    const uint4 h4 = reinterpret_cast<const uint4 *>(hist)[lane];
    const uint32_t c = h4.x + h4.y + h4.z + h4.w;
    uint32_t suffix = c; // keys of digits >= 4l
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t o = __shfl_down(suffix, off, kWave);
        suffix += (lane + off < kWave) ? o : 0u;
    }
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

// Exclusive prefix sum over the wave of per-lane counts in 0 .. 7, and the
// total, from one ballot per bit.
__device__ __forceinline__ uint32_t lane_offset(uint32_t c, uint32_t &total)
{
    uint32_t excl = 0u;
    total = 0u;
#pragma unroll
    for (int bit = 0; bit < 3; ++bit) {
        const uint64_t m = __ballot((c >> bit) & 1u);
        excl += (uint32_t)lanes_below(m) << bit;
        total += (uint32_t)__builtin_popcountll(m) << bit;
    }
    return excl;
}

constexpr int kMaxSurvivors = 256;

// One wave (one workgroup) per query block; grid (nb, H, B).  Lane l loads
// key blocks 256 r + 4 l .. 256 r + 4 l + 3 with one 16-byte load per r and
// keeps their keys in registers.  A radix select over four 8-bit digits, most
// significant first, finds the keep-th largest key T and how many keys equal
// to T are kept (LDS histogram of the keys still matching the chosen prefix,
// then a suffix scan across lanes).  After two digits the few keys that still
// match are compacted into LDS and the last two digits count only those.  The
// kept blocks -- every key above T and the lowest-indexed keys equal to T --
// are written in ascending order, each lane's offset taken from ballots.
// Counting never branches: a key that does not count adds to its lane's own
// trash slot after the 256 bins (and a survivor past the bound to a trash
// slot after the list), so the waves issue no exec-mask bookkeeping per key;
// when the first digit's likeliest crowded bin pair holds most keys, that pair
// is counted by ballots instead.
template <int RV>
__global__ __launch_bounds__(kWave) void subblock_topk_kernel(const float *__restrict__ scores,
                                                              int32_t *__restrict__ kept, int nb, int ld, int keep,
                                                              int H)
{
    __shared__ __align__(16) uint32_t hist[256 + kWave]; // 256 digits, then one trash slot per lane
    __shared__ uint32_t survivors[kMaxSurvivors + kWave]; // then one trash slot per lane
    const int lane = threadIdx.x;
    const size_t row = ((size_t)blockIdx.z * H + blockIdx.y) * nb + blockIdx.x;
    const float *s = scores + row * ld;
    int32_t *out = kept + row * keep;

    uint32_t key[RV][4];
#pragma unroll
    for (int r = 0; r < RV; ++r) {
        const int j0 = 256 * r + 4 * lane;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (j0 < nb) // the row is 16-byte aligned and ld >= nb rounded up to 4
            v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(s + j0));
#pragma unroll
        for (int e = 0; e < 4; ++e)
            key[r][e] = score_key(v[e]);
    }
    const int limit = nb - 4 * lane; // key (r, e) is a real block when 256 r + e < limit
    auto valid = [&](int r, int e) { return 256 * r + e < limit; };

    RadixState st = {0u, 0u, (uint32_t)keep, 0u};
    // Every key adds to a bin without branching: keys that do not count go to
    // the lane's own trash slot.
    auto count_registers = [&](int shift) {
#pragma unroll
        for (int r = 0; r < RV; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool counts = valid(r, e) && (key[r][e] & st.mask) == st.prefix;
                atomicAdd(&hist[counts ? (key[r][e] >> shift) & 0xffu : 256u + lane], 1u);
            }
    };
    // First digit: every valid key counts.  The first digit is the sign and
    // the top of the exponent, so a row's keys can crowd into a few bins, and
    // LDS atomics on one address serialise.  The candidate crowded bin is the
    // first key's, paired with its mirror 255 - it (the key of -x is the
    // bitwise inverse of the key of x, so that bin holds the same magnitudes
    // with the other sign).  When the pair holds more than half of the first
    // 256 keys (a wave-uniform test), the keys in it are counted with one
    // ballot per bin and key slot and added once, and only the others go to
    // the atomics.  Otherwise the ballots would cost more than the conflicts
    // they remove, and every key adds to its bin.  The counts, and so the
    // selection, are the same either way.
    reinterpret_cast<uint4 *>(hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    {
        const uint32_t hot = (uint32_t)__builtin_amdgcn_readfirstlane((int)(key[0][0] >> 24)); // lane 0's key 0 is real
        const uint32_t mirror = 255u - hot;
        uint32_t in_pair = 0u, sampled = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t d = key[0][e] >> 24;
            in_pair += (uint32_t)__builtin_popcountll(__ballot(valid(0, e) && (d == hot || d == mirror)));
            sampled += (uint32_t)__builtin_popcountll(__ballot(valid(0, e)));
        }
        if (2u * in_pair > sampled) {
            uint32_t hot_count = 0u, mirror_count = 0u;
#pragma unroll
            for (int r = 0; r < RV; ++r)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t d = key[r][e] >> 24;
                    const bool v = valid(r, e);
                    const bool h = v && d == hot, m = v && d == mirror;
                    hot_count += (uint32_t)__builtin_popcountll(__ballot(h));
                    mirror_count += (uint32_t)__builtin_popcountll(__ballot(m));
                    atomicAdd(&hist[(v && !h && !m) ? d : 256u + lane], 1u);
                }
            if (lane == 0) {
                atomicAdd(&hist[hot], hot_count);
                atomicAdd(&hist[mirror], mirror_count);
            }
        } else {
#pragma unroll
            for (int r = 0; r < RV; ++r)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    atomicAdd(&hist[valid(r, e) ? key[r][e] >> 24 : 256u + lane], 1u);
        }
    }
    __syncthreads();
    choose_digit(hist, lane, 24, st);
    __syncthreads();
    reinterpret_cast<uint4 *>(hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    count_registers(16);
    __syncthreads();
    choose_digit(hist, lane, 16, st);
    __syncthreads();
    const bool compact = st.in_bin <= (uint32_t)kMaxSurvivors; // wave-uniform
    uint32_t n_surv = 0u;
    if (compact) {
#pragma unroll
        for (int r = 0; r < RV; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool m = valid(r, e) && (key[r][e] & st.mask) == st.prefix;
                const uint64_t mm = __ballot(m);
                const uint32_t at = n_surv + (uint32_t)lanes_below(mm);
                // exactly in_bin keys match; the bound only guards the store
                survivors[(m && at < (uint32_t)kMaxSurvivors) ? at : kMaxSurvivors + lane] = key[r][e];
                n_surv += (uint32_t)__builtin_popcountll(mm);
            }
    }
#pragma unroll 1
    for (int pass = 2; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        reinterpret_cast<uint4 *>(hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
        __syncthreads();
        if (compact) {
            for (uint32_t c = lane; c < n_surv; c += kWave) {
                const uint32_t k = survivors[c];
                if ((k & st.mask) == st.prefix)
                    atomicAdd(&hist[(k >> shift) & 0xffu], 1u);
            }
        } else {
            count_registers(shift);
        }
        __syncthreads();
        choose_digit(hist, lane, shift, st);
        __syncthreads();
    }

    // st.prefix is now the keep-th largest key T; st.in_bin keys equal T and
    // st.need of them are kept.  Exactly keep blocks are selected; the bound
    // on `at` only guards the stores.
    const uint32_t T = st.prefix;
    const bool all_ties = st.need == st.in_bin; // wave-uniform
    uint32_t written = 0u, ties = 0u;
#pragma unroll
    for (int r = 0; r < RV; ++r) {
        bool sel[4];
        uint32_t c = 0u;
        if (all_ties) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sel[e] = valid(r, e) && key[r][e] >= T;
                c += sel[e] ? 1u : 0u;
            }
        } else {
            bool eq[4];
            uint32_t c_eq = 0u, eq_total;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                eq[e] = valid(r, e) && key[r][e] == T;
                c_eq += eq[e] ? 1u : 0u;
            }
            uint32_t rank = ties + lane_offset(c_eq, eq_total); // tie rank of this lane's first tie
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sel[e] = (valid(r, e) && key[r][e] > T) || (eq[e] && rank < st.need);
                rank += eq[e] ? 1u : 0u;
                c += sel[e] ? 1u : 0u;
            }
            ties += eq_total;
        }
        uint32_t total;
        uint32_t at = written + lane_offset(c, total);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (sel[e]) {
                if (at < (uint32_t)keep)
                    out[at] = 256 * r + 4 * lane + e;
                ++at;
            }
        written += total;
    }
}

template <int RV>
void launch_topk_rv(const float *scores, int32_t *kept, int nb, int ld, int keep, int H, int B, hipStream_t stream)
{
    hipLaunchKernelGGL(subblock_topk_kernel<RV>, dim3((unsigned)nb, (unsigned)H, (unsigned)B), dim3(kWave), 0, stream,
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
    if (n <= 256) launch_topk_rv<1>(scores, kept, n, l, kp, h, b, stream);
    else if (n <= 512) launch_topk_rv<2>(scores, kept, n, l, kp, h, b, stream);
    else if (n <= 1024) launch_topk_rv<4>(scores, kept, n, l, kp, h, b, stream);
    else if (n <= 2048) launch_topk_rv<8>(scores, kept, n, l, kp, h, b, stream);
    else launch_topk_rv<16>(scores, kept, n, l, kp, h, b, stream);
    return hipGetLastError();
}

} // namespace dit
