// launch.hpp -- host-side launchers of the chain's kernels.  Each assumes its
// arguments were validated by the C entry points in abi.hip (sizes in range,
// pointers 16-byte aligned) and enqueues on `stream` without synchronising.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

// y = LN(x) * (1 + scale[b]) + shift[b]; rows = B*N, D % 8 == 0, D <= 8192.
hipError_t launch_adaln_modulate(const void *x, const void *shift, const void *scale, void *y,
                                 int64_t rows, int64_t N, int64_t D, float eps, hipStream_t stream);

// out = x + gate[b] * y; rows = B*N, D % 8 == 0.
hipError_t launch_gated_residual(const void *x, const void *y, const void *gate, void *out,
                                 int64_t rows, int64_t N, int64_t D, hipStream_t stream);

// Whether rows x ceil(D / 4096) residual tiles fit the kernel's 32-bit tile counter.
bool gated_residual_fits(int64_t rows, int64_t D);

// Whether M x ceil(F / 2048) SwiGLU tiles fit the kernel's 32-bit tile counter.
bool swiglu_fits(int64_t M, int64_t F);

// out[r][j] = silu(in[r][j]) * in[r][F+j]; F % 8 == 0.
hipError_t launch_swiglu(const void *in, void *out, int64_t M, int64_t F, hipStream_t stream);

// Per-head RMSNorm + 3D RoPE of q and k; Dh in {8,...,256} (power of two).  Inputs have
// in_token_stride elements (a multiple of 8, >= H*Dh) between consecutive tokens; outputs are
// [B][N][H][Dh], or [B][H][N][Dh] when head_major, with out_plane_stride elements (a multiple
// of 8, >= N*Dh) between consecutive head planes.
hipError_t launch_qk_rmsnorm_rope3d(const void *q, const void *k, void *q_out, void *k_out,
                                    const void *wq, const void *wk, const int32_t *pos,
                                    int64_t rows, int64_t N, int64_t H, int64_t Dh,
                                    int64_t in_token_stride, bool head_major, int64_t out_plane_stride,
                                    int d_t, int d_h, int d_w, float theta, float eps,
                                    hipStream_t stream);

// x_out = x + gate[b] * y (bf16), z = LN(x_out) * (1 + scale[b]) + shift[b]; D % 8 == 0, D <= 8192.
hipError_t launch_gated_residual_adaln(const void *x, const void *y, const void *gate, const void *shift,
                                       const void *scale, void *x_out, void *z, int64_t rows, int64_t N, int64_t D,
                                       float eps, hipStream_t stream);

// Workgroup tiles per sample of the residual-change statistic (workspace holds B * tiles * 16 bytes).
int64_t residual_change_tiles(int64_t N, int64_t D);

// out[b] = (sum |r - r_cached|, sum |r_cached|, ratio) per sample, via per-tile partials in workspace.
hipError_t launch_residual_change(const void *r, const void *r_cached, double *out, void *workspace, int64_t B,
                                  int64_t N, int64_t D, hipStream_t stream);

// Capacity, in (num, den) partials, of the library's static scratch array used by the
// allocation-free residual-change entry point: 2 MiB per device.
constexpr int64_t kResidualChangeScratchPartials = 131072;

// Device address of that scratch array on the current device (looked up once per device).
hipError_t residual_change_scratch(void **ptr);

// QK RMSNorm + 3D RoPE and the means of each 64-token block of the stored q', k':
// [B][H][ceil(N/64)][Dh] fp32.  Inputs with in_token_stride elements between tokens; outputs
// [B][N][H][Dh] or [B][H][N][Dh] (head_major, out_plane_stride elements between head planes).
// Dh in {16,...,256}, power of two.
hipError_t launch_qk_rmsnorm_rope3d_pool(const void *q, const void *k, void *q_out, void *k_out, const void *wq,
                                         const void *wk, const int32_t *pos, float *q_pooled, float *k_pooled,
                                         int64_t B, int64_t N, int64_t H, int64_t Dh, int64_t in_token_stride,
                                         bool head_major, int64_t out_plane_stride, int d_t, int d_h, int d_w,
                                         float theta, float eps, hipStream_t stream);

// Means of each 64-token block of q and of k, per sample and head: [B][H][ceil(N/64)][Dh] fp32.
// Inputs [B][N][H][Dh] (token-major) or [B][H][N][Dh] (head_major); Dh in {16,...,256}, power of two.
hipError_t launch_subblock_pool(const void *q, const void *k, float *q_pooled, float *k_pooled, int64_t B, int64_t N,
                                int64_t H, int64_t Dh, bool head_major, hipStream_t stream);

// Block scores [B][H][nb][ld] (bf16 operands, fp32 accumulation) and, for keep > 0, the keep
// highest-scoring key blocks of every query block, ascending: kept [B][H][nb][keep].
hipError_t launch_subblock_route(const float *q_pooled, const float *k_pooled, float *scores, int32_t *kept,
                                 int64_t B, int64_t H, int64_t nb, int64_t Dh, int64_t ld, int64_t keep,
                                 hipStream_t stream);

// Packed (t, h, w) coordinates of T*Hg*Wg video tokens then n_extra tokens.
hipError_t launch_packed_positions(int32_t *pos, int64_t T, int64_t Hg, int64_t Wg, int64_t n_extra,
                                   hipStream_t stream);

// dst = src, bytes % 16 == 0.
hipError_t launch_copy16(const void *src, void *dst, int64_t bytes, hipStream_t stream);

// Access-pattern streams (measurement only); kinds as the DIT_STREAM_* values of dit_ops.h.
enum : int {
    kPatternRead = 0,
    kPatternWrite = 1,
    kPatternSplitRows = 2,
    kPatternTwoIn = 3,
    kPatternRowGroup = 4,
    kPatternRowGroup2x2 = 5,
    kPatternHeadMajor = 6,
    kPatternScoreTiles = 7,
    kPatternTopkRows = 8,
};
hipError_t launch_stream_pattern(int kind, const void *in0, const void *in1, void *out0, void *out1, int64_t rows,
                                 int64_t row_bytes, int64_t heads, hipStream_t stream);

} // namespace dit
