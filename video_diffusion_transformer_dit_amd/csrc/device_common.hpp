// device_common.hpp -- gfx950 device helpers shared by the chain's kernels:
// 16-byte vector memory access, bf16 <-> fp32 conversion, and cross-lane sums
// built on DPP (data-parallel primitives inside a 16-lane row) and wave-wide
// lane swaps.  Written for CDNA4's 64-wide wavefronts; no other target.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

constexpr int kWave = 64;

// Eight bf16 values (16 bytes) as four dwords; the unit of every HBM access.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- memory access
// Streaming data is touched exactly once, so it is loaded and stored with the
// non-temporal hint; small per-sample vectors and weights that every row
// re-reads use ordinary cached loads.

__device__ __forceinline__ u32x4 load_stream(const u32x4 *p) { return __builtin_nontemporal_load(p); }

__device__ __forceinline__ u32x4 load_cached(const u32x4 *p) { return *p; }

__device__ __forceinline__ void store_stream(u32x4 *p, u32x4 v) { __builtin_nontemporal_store(v, p); }

// ---------------------------------------------------------------- bf16 <-> fp32
// A bf16 value is the high half of an fp32, so widening is a shift or a mask.

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }

__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> two bf16 in one dword, round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ void unpack8(u32x4 v, float f[8])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_lo(v[i]);
        f[2 * i + 1] = bf16_hi(v[i]);
    }
}

__device__ __forceinline__ u32x4 pack8(const float f[8])
{
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return v;
}

// ---------------------------------------------------------------- cross-lane sums
// DPP control words (GFX9 encoding).
constexpr int kDppQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppRowHalfMirror = 0x141; // lane i <- lane 7-i inside each 8-lane half row
constexpr int kDppRowMirror = 0x140;     // lane i <- lane 15-i inside each 16-lane row

template <int Ctrl>
__device__ __forceinline__ float dpp_read(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), Ctrl, 0xf, 0xf, false));
}

// Sum over aligned groups of L consecutive lanes (L a power of two, <= 64);
// every lane of a group receives the group total.  Must be called with all 64
// lanes active.  Groups of up to 16 lanes stay inside one DPP row: after the
// two quad swaps each quad holds its sum, the half-row mirror pairs quad 0
// with quad 1, and the row mirror pairs the two halves.  Wider groups then add
// the row totals read out of lanes 0, 16, 32 and 48 with v_readlane (scalar
// registers, a few cycles) instead of a round trip through the LDS crossbar.
__device__ __forceinline__ float lane_value(float v, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

template <int L>
__device__ __forceinline__ float group_sum(float v)
{
    static_assert(L >= 1 && L <= 64 && (L & (L - 1)) == 0, "group width must be a power of two");
    if constexpr (L >= 2) v += dpp_read<kDppQuadSwap1>(v);
    if constexpr (L >= 4) v += dpp_read<kDppQuadSwap2>(v);
    if constexpr (L >= 8) v += dpp_read<kDppRowHalfMirror>(v);
    if constexpr (L >= 16) v += dpp_read<kDppRowMirror>(v);
    if constexpr (L == 32) {
        const float lo = lane_value(v, 0) + lane_value(v, 16);
        const float hi = lane_value(v, 32) + lane_value(v, 48);
        v = (__lane_id() < 32) ? lo : hi;
    }
    if constexpr (L == 64)
        v = (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<kWave>(v); }

} // namespace dit
