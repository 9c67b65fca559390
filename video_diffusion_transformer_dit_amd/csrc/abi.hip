// abi.hip -- the library's C entry points (declared in include/dit_ops.h).
//
// Each entry point validates its arguments on the host, in a fixed order,
// before any HIP call:
//   1. sizes negative or beyond the limits     -> DIT_ERR_ARG
//   2. widths, head size or RoPE bands invalid  -> DIT_ERR_SHAPE
//   3. eps / theta out of range                 -> DIT_ERR_ARG
//   4. zero rows                                -> DIT_OK (nothing enqueued;
//                                                  pointers not examined)
//   5. NULL pointers                            -> DIT_ERR_NULL
//   6. misaligned pointers                      -> DIT_ERR_ALIGN
//   7. forbidden overlaps                       -> DIT_ERR_ARG
// and only then launches on the caller's stream; a failed launch returns
// DIT_ERR_HIP.  Nothing is allocated or synchronised; the only state is the
// per-device address of the allocation-free residual-change entry point's
// static scratch array, looked up on its first call on a device.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "dit_ops.h"
#include "launch.hpp"

namespace {

// Largest row (token) count accepted by one call: below 2^24 rows every grid
// dimension stays within the 32-bit work-item count of a dispatch (a
// workgroup per row spans up to 256 work-items) and every row index fits in
// 32 bits.
constexpr int64_t kMaxRows = (int64_t(1) << 24) - 1;
constexpr int64_t kMaxAdaLNWidth = 8192; // rows of up to 1024 vectors: 512 threads per workgroup
constexpr int64_t kMaxWidth = int64_t(1) << 24;
constexpr int64_t kMaxHeadRow = 65536; // H * Dh

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Byte ranges [a, a+na) and [b, b+nb) intersect.
bool overlap(const void *a, int64_t na, const void *b, int64_t nb)
{
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
}

// Overlap that is not the exact in-place case (same start, same extent).
bool bad_alias(const void *out, const void *in, int64_t n) { return out != in && overlap(out, n, in, n); }

// rows = a * b without overflow, or -1 when either is negative or the product
// exceeds kMaxRows.
int64_t row_count(int64_t a, int64_t b)
{
    if (a < 0 || b < 0)
        return -1;
    if (a != 0 && b > kMaxRows / a)
        return -1;
    const int64_t r = a * b;
    return r > kMaxRows ? -1 : r;
}

dit_status launched(hipError_t e) { return e == hipSuccess ? DIT_OK : DIT_ERR_HIP; }

// Largest head-plane stride of a head-major QK output (elements).
constexpr int64_t kMaxPlaneStride = int64_t(1) << 40;

// Resolved head-plane stride of a QK output (0 selects N*Dh, the packed
// layout; token-major outputs take only 0), or a status: DIT_ERR_ARG for a
// negative or oversized stride, a stride with a token-major output, or an
// output extent past 2^62 bytes; DIT_ERR_SHAPE for a stride that is not a
// multiple of 8 or is shorter than a plane.
dit_status plane_stride(int64_t requested, int32_t out_layout, int64_t B, int64_t N, int64_t H, int64_t Dh,
                        int64_t *plane)
{
    if (requested < 0 || requested > kMaxPlaneStride || (out_layout == DIT_QK_TOKEN_MAJOR && requested != 0))
        return DIT_ERR_ARG;
    *plane = requested == 0 ? N * Dh : requested;
    if (out_layout == DIT_QK_HEAD_MAJOR && (*plane % 8 != 0 || *plane < N * Dh))
        return DIT_ERR_SHAPE;
    const int64_t planes = B * H; // B < 2^24, H <= 2^16: no overflow
    if (planes > 1 && *plane > ((int64_t(1) << 61) - N * Dh) / (planes - 1))
        return DIT_ERR_ARG;
    return DIT_OK;
}

// Bytes from the first to one past the last element of a QK output.
int64_t qk_out_extent(int32_t out_layout, int64_t B, int64_t N, int64_t H, int64_t Dh, int64_t plane)
{
    if (out_layout == DIT_QK_TOKEN_MAJOR || B * N == 0)
        return B * N * H * Dh * 2;
    return ((B * H - 1) * plane + N * Dh) * 2;
}

} // namespace

extern "C" {

const char *dit_status_str(int status)
{
    switch (status) {
    case DIT_OK: return "DIT_OK";
    case DIT_ERR_NULL: return "DIT_ERR_NULL: a required pointer is NULL";
    case DIT_ERR_SHAPE: return "DIT_ERR_SHAPE: unsupported width, head size or RoPE bands";
    case DIT_ERR_ALIGN: return "DIT_ERR_ALIGN: pointer not aligned (bf16 tensors need 16 bytes)";
    case DIT_ERR_ARG: return "DIT_ERR_ARG: size, eps, theta or buffer overlap out of range";
    case DIT_ERR_HIP: return "DIT_ERR_HIP: kernel launch failed";
    case DIT_ERR_SCRATCH: return "DIT_ERR_SCRATCH: sizes exceed the library's static scratch buffer";
    default: return "unknown dit_status";
    }
}

int dit_abi_version(void) { return DIT_ABI_VERSION; }

dit_status dit_adaln_modulate(const dit_bf16 *x, const dit_bf16 *shift, const dit_bf16 *scale, dit_bf16 *y,
                              int64_t B, int64_t N, int64_t D, float eps, void *stream)
{
    const int64_t rows = row_count(B, N);
    if (rows < 0 || D < 0)
        return DIT_ERR_ARG;
    if (D < 8 || D % 8 != 0 || D > kMaxAdaLNWidth)
        return DIT_ERR_SHAPE;
    if (!(eps > 0.f) || !isfinite(eps))
        return DIT_ERR_ARG;
    if (rows == 0)
        return DIT_OK;
    if (!x || !shift || !scale || !y)
        return DIT_ERR_NULL;
    if (!aligned(x, 16) || !aligned(shift, 16) || !aligned(scale, 16) || !aligned(y, 16))
        return DIT_ERR_ALIGN;
    const int64_t nx = rows * D * 2, nv = B * D * 2;
    if (bad_alias(y, x, nx) || overlap(y, nx, shift, nv) || overlap(y, nx, scale, nv))
        return DIT_ERR_ARG;
    return launched(dit::launch_adaln_modulate(x, shift, scale, y, rows, N, D, eps, (hipStream_t)stream));
}

dit_status dit_gated_residual(const dit_bf16 *x, const dit_bf16 *y, const dit_bf16 *gate, dit_bf16 *out, int64_t B,
                              int64_t N, int64_t D, void *stream)
{
    const int64_t rows = row_count(B, N);
    if (rows < 0 || D < 0)
        return DIT_ERR_ARG;
    if (D < 8 || D % 8 != 0 || D > kMaxWidth)
        return DIT_ERR_SHAPE;
    if (!dit::gated_residual_fits(rows, D))
        return DIT_ERR_ARG;
    if (rows == 0)
        return DIT_OK;
    if (!x || !y || !gate || !out)
        return DIT_ERR_NULL;
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(gate, 16) || !aligned(out, 16))
        return DIT_ERR_ALIGN;
    const int64_t nx = rows * D * 2, ng = B * D * 2;
    if (bad_alias(out, x, nx) || bad_alias(out, y, nx) || overlap(out, nx, gate, ng))
        return DIT_ERR_ARG;
    return launched(dit::launch_gated_residual(x, y, gate, out, rows, N, D, (hipStream_t)stream));
}

dit_status dit_swiglu(const dit_bf16 *in, dit_bf16 *out, int64_t M, int64_t F, void *stream)
{
    if (M < 0 || M > kMaxRows || F < 0)
        return DIT_ERR_ARG;
    if (F < 8 || F % 8 != 0 || F > kMaxWidth)
        return DIT_ERR_SHAPE;
    if (!dit::swiglu_fits(M, F))
        return DIT_ERR_ARG;
    if (M == 0)
        return DIT_OK;
    if (!in || !out)
        return DIT_ERR_NULL;
    if (!aligned(in, 16) || !aligned(out, 16))
        return DIT_ERR_ALIGN;
    if (overlap(out, M * F * 2, in, M * F * 4))
        return DIT_ERR_ARG;
    return launched(dit::launch_swiglu(in, out, M, F, (hipStream_t)stream));
}

dit_status dit_qk_rmsnorm_rope3d_layout(const dit_bf16 *q, const dit_bf16 *k, dit_bf16 *q_out, dit_bf16 *k_out,
                                        const dit_bf16 *wq, const dit_bf16 *wk, const int32_t *pos, int64_t B,
                                        int64_t N, int64_t H, int64_t Dh, int64_t in_token_stride,
                                        int32_t out_layout, int64_t out_plane_stride, int32_t d_t, int32_t d_h,
                                        int32_t d_w, float theta, float eps, void *stream)
{
    const int64_t rows = row_count(B, N);
    if (rows < 0 || H < 0 || Dh < 0 || in_token_stride < 0 || in_token_stride > kMaxWidth)
        return DIT_ERR_ARG;
    if (out_layout != DIT_QK_TOKEN_MAJOR && out_layout != DIT_QK_HEAD_MAJOR)
        return DIT_ERR_ARG;
    const bool dh_ok = Dh == 8 || Dh == 16 || Dh == 32 || Dh == 64 || Dh == 128 || Dh == 256;
    if (!dh_ok || H < 1 || H * Dh > kMaxHeadRow || d_t < 0 || d_h < 0 || d_w < 0 || (d_t | d_h | d_w) & 1 ||
        (int64_t)d_t + d_h + d_w != Dh || in_token_stride % 8 != 0 || in_token_stride < H * Dh)
        return DIT_ERR_SHAPE;
    int64_t plane = 0;
    const dit_status ps = plane_stride(out_plane_stride, out_layout, B, N, H, Dh, &plane);
    if (ps != DIT_OK)
        return ps;
    if (!(eps > 0.f) || !isfinite(eps) || !(theta > 1.f) || !isfinite(theta))
        return DIT_ERR_ARG;
    if (rows == 0)
        return DIT_OK;
    if (!q || !k || !q_out || !k_out || !wq || !wk || !pos)
        return DIT_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(q_out, 16) || !aligned(k_out, 16) || !aligned(wq, 16) ||
        !aligned(wk, 16) || !aligned(pos, 4))
        return DIT_ERR_ALIGN;
    const int64_t nt = qk_out_extent(out_layout, B, N, H, Dh, plane); // byte extent of each output
    const int64_t ni = ((rows - 1) * in_token_stride + H * Dh) * 2;   // byte extent of each input
    const int64_t nw = Dh * 2, np = N * 12;
    // In place (q_out == q, k_out == k) only where the layouts coincide.
    const bool same_layout = in_token_stride == H * Dh && out_layout == DIT_QK_TOKEN_MAJOR;
    const bool q_bad = same_layout ? bad_alias(q_out, q, nt) : overlap(q_out, nt, q, ni);
    const bool k_bad = same_layout ? bad_alias(k_out, k, nt) : overlap(k_out, nt, k, ni);
    if (q_bad || k_bad || overlap(q_out, nt, k, ni) || overlap(k_out, nt, q, ni) || overlap(k_out, nt, q_out, nt))
        return DIT_ERR_ARG;
    const void *small[3] = {wq, wk, pos};
    const int64_t small_n[3] = {nw, nw, np};
    for (int i = 0; i < 3; ++i)
        if (overlap(q_out, nt, small[i], small_n[i]) || overlap(k_out, nt, small[i], small_n[i]))
            return DIT_ERR_ARG;
    return launched(dit::launch_qk_rmsnorm_rope3d(q, k, q_out, k_out, wq, wk, pos, rows, N, H, Dh, in_token_stride,
                                                  out_layout == DIT_QK_HEAD_MAJOR, plane, d_t, d_h, d_w, theta, eps,
                                                  (hipStream_t)stream));
}

dit_status dit_qk_rmsnorm_rope3d(const dit_bf16 *q, const dit_bf16 *k, dit_bf16 *q_out, dit_bf16 *k_out,
                                 const dit_bf16 *wq, const dit_bf16 *wk, const int32_t *pos, int64_t B, int64_t N,
                                 int64_t H, int64_t Dh, int32_t d_t, int32_t d_h, int32_t d_w, float theta, float eps,
                                 void *stream)
{
    // Token-major q and k in, token-major out: the layout entry point with the plain layout.
    if (H < 0 || Dh < 0 || H > kMaxHeadRow || Dh > kMaxHeadRow)
        return H < 0 || Dh < 0 ? DIT_ERR_ARG : DIT_ERR_SHAPE;
    return dit_qk_rmsnorm_rope3d_layout(q, k, q_out, k_out, wq, wk, pos, B, N, H, Dh, H * Dh, DIT_QK_TOKEN_MAJOR, 0,
                                        d_t, d_h, d_w, theta, eps, stream);
}

dit_status dit_gated_residual_adaln(const dit_bf16 *x, const dit_bf16 *y, const dit_bf16 *gate, const dit_bf16 *shift,
                                    const dit_bf16 *scale, dit_bf16 *x_out, dit_bf16 *z, int64_t B, int64_t N,
                                    int64_t D, float eps, void *stream)
{
    const int64_t rows = row_count(B, N);
    if (rows < 0 || D < 0)
        return DIT_ERR_ARG;
    if (D < 8 || D % 8 != 0 || D > kMaxAdaLNWidth)
        return DIT_ERR_SHAPE;
    if (!(eps > 0.f) || !isfinite(eps))
        return DIT_ERR_ARG;
    if (rows == 0)
        return DIT_OK;
    if (!x || !y || !gate || !shift || !scale || !x_out || !z)
        return DIT_ERR_NULL;
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(gate, 16) || !aligned(shift, 16) || !aligned(scale, 16) ||
        !aligned(x_out, 16) || !aligned(z, 16))
        return DIT_ERR_ALIGN;
    const int64_t nx = rows * D * 2, nv = B * D * 2;
    // x_out may be x exactly and z may be y exactly; nothing else may overlap.
    if (bad_alias(x_out, x, nx) || overlap(x_out, nx, y, nx) || bad_alias(z, y, nx) || overlap(z, nx, x, nx) ||
        overlap(z, nx, x_out, nx))
        return DIT_ERR_ARG;
    const void *vecs[3] = {gate, shift, scale};
    for (const void *v : vecs)
        if (overlap(x_out, nx, v, nv) || overlap(z, nx, v, nv))
            return DIT_ERR_ARG;
    return launched(
        dit::launch_gated_residual_adaln(x, y, gate, shift, scale, x_out, z, rows, N, D, eps, (hipStream_t)stream));
}

// Samples per call of the residual-change statistic (one grid row each) and
// tiles per sample: the grid's x extent in 1024-thread workgroups, so that its
// work-item count stays below 2^32.
constexpr int64_t kMaxSamples = 65535;
constexpr int64_t kMaxChangeTiles = (int64_t(1) << 22) - 1;

int64_t dit_residual_change_workspace_bytes(int64_t B, int64_t N, int64_t D)
{
    if (B < 0 || N < 0 || D < 8 || D % 8 != 0 || D > kMaxWidth || B > kMaxSamples || N > kMaxRows)
        return -1;
    const int64_t tiles = dit::residual_change_tiles(N, D);
    if (tiles > kMaxChangeTiles)
        return -1;
    return B * tiles * 16;
}

dit_status dit_residual_change(const dit_bf16 *r, const dit_bf16 *r_cached, double *out, void *workspace,
                               int64_t workspace_bytes, int64_t B, int64_t N, int64_t D, void *stream)
{
    if (B < 0 || N < 0 || D < 0 || workspace_bytes < 0 || B > kMaxSamples || N > kMaxRows)
        return DIT_ERR_ARG;
    if (D < 8 || D % 8 != 0 || D > kMaxWidth)
        return DIT_ERR_SHAPE;
    const int64_t need = dit_residual_change_workspace_bytes(B, N, D);
    if (need < 0)
        return DIT_ERR_ARG;
    if (B == 0)
        return DIT_OK;
    if (!out || (N > 0 && (!r || !r_cached)) || (need > 0 && !workspace))
        return DIT_ERR_NULL;
    if (!aligned(out, 8) || (N > 0 && (!aligned(r, 16) || !aligned(r_cached, 16))) ||
        (need > 0 && !aligned(workspace, 16)))
        return DIT_ERR_ALIGN;
    if (workspace_bytes < need)
        return DIT_ERR_ARG;
    const int64_t nin = B * N * D * 2, nout = B * 3 * 8;
    if (overlap(out, nout, workspace, need) || (N > 0 && (overlap(out, nout, r, nin) || overlap(out, nout, r_cached, nin) ||
                                                          overlap(workspace, need, r, nin) ||
                                                          overlap(workspace, need, r_cached, nin))))
        return DIT_ERR_ARG;
    return launched(dit::launch_residual_change(r, r_cached, out, workspace, B, N, D, (hipStream_t)stream));
}

dit_status dit_residual_change_noalloc(const dit_bf16 *r, const dit_bf16 *r_cached, double *out, int64_t B,
                                      int64_t N, int64_t D, void *stream)
{
    if (B < 0 || N < 0 || D < 0 || B > kMaxSamples || N > kMaxRows)
        return DIT_ERR_ARG;
    if (D < 8 || D % 8 != 0 || D > kMaxWidth)
        return DIT_ERR_SHAPE;
    const int64_t need = dit_residual_change_workspace_bytes(B, N, D);
    if (need < 0)
        return DIT_ERR_ARG;
    if (need > dit::kResidualChangeScratchPartials * 16)
        return DIT_ERR_SCRATCH;
    if (B == 0)
        return DIT_OK;
    if (!out || (N > 0 && (!r || !r_cached)))
        return DIT_ERR_NULL;
    if (!aligned(out, 8) || (N > 0 && (!aligned(r, 16) || !aligned(r_cached, 16))))
        return DIT_ERR_ALIGN;
    const int64_t nin = B * N * D * 2, nout = B * 3 * 8;
    if (N > 0 && (overlap(out, nout, r, nin) || overlap(out, nout, r_cached, nin)))
        return DIT_ERR_ARG;
    void *ws = nullptr;
    if (dit::residual_change_scratch(&ws) != hipSuccess)
        return DIT_ERR_HIP;
    return launched(dit::launch_residual_change(r, r_cached, out, ws, B, N, D, (hipStream_t)stream));
}

// SubBlock routing: at most 4096 blocks of 64 tokens per sample (262,144 tokens).
constexpr int64_t kMaxSubBlocks = 4096;

static bool subblock_head_ok(int64_t H, int64_t Dh)
{
    const bool dh_ok = Dh == 16 || Dh == 32 || Dh == 64 || Dh == 128 || Dh == 256;
    return dh_ok && H >= 1 && H * Dh <= kMaxHeadRow;
}

int64_t dit_subblock_keep(int64_t nb, double sparsity)
{
    if (nb < 0 || !(sparsity >= 0.0) || !(sparsity < 1.0))
        return -1;
    if (nb == 0)
        return 0;
    const int64_t keep = nb - (int64_t)floor(sparsity * (double)nb);
    return keep < 1 ? 1 : keep;
}

int64_t dit_subblock_scores_ld(int64_t nb)
{
    if (nb < 0 || nb > kMaxSubBlocks)
        return -1;
    return (nb + 31) / 32 * 32;
}

dit_status dit_subblock_pool(const dit_bf16 *q, const dit_bf16 *k, float *q_pooled, float *k_pooled, int64_t B,
                             int64_t N, int64_t H, int64_t Dh, int32_t layout, void *stream)
{
    if (B < 0 || N < 0 || H < 0 || Dh < 0 || B > kMaxSamples || N > kMaxSubBlocks * DIT_SUBBLOCK_TOKENS)
        return DIT_ERR_ARG;
    if (layout != DIT_QK_TOKEN_MAJOR && layout != DIT_QK_HEAD_MAJOR)
        return DIT_ERR_ARG;
    if (!subblock_head_ok(H, Dh))
        return DIT_ERR_SHAPE;
    if (B == 0 || N == 0)
        return DIT_OK;
    if (!q || !k || !q_pooled || !k_pooled)
        return DIT_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(q_pooled, 16) || !aligned(k_pooled, 16))
        return DIT_ERR_ALIGN;
    const int64_t nb = (N + DIT_SUBBLOCK_TOKENS - 1) / DIT_SUBBLOCK_TOKENS;
    const int64_t ni = B * N * H * Dh * 2, no = B * H * nb * Dh * 4;
    // q and k may be one buffer (they are only read); the outputs overlap nothing.
    if (overlap(q_pooled, no, k_pooled, no) || overlap(q_pooled, no, q, ni) || overlap(q_pooled, no, k, ni) ||
        overlap(k_pooled, no, q, ni) || overlap(k_pooled, no, k, ni))
        return DIT_ERR_ARG;
    return launched(dit::launch_subblock_pool(q, k, q_pooled, k_pooled, B, N, H, Dh, layout == DIT_QK_HEAD_MAJOR,
                                              (hipStream_t)stream));
}

dit_status dit_qk_rmsnorm_rope3d_pool(const dit_bf16 *q, const dit_bf16 *k, dit_bf16 *q_out, dit_bf16 *k_out,
                                      const dit_bf16 *wq, const dit_bf16 *wk, const int32_t *pos, float *q_pooled,
                                      float *k_pooled, int64_t B, int64_t N, int64_t H, int64_t Dh,
                                      int64_t in_token_stride, int32_t out_layout, int64_t out_plane_stride,
                                      int32_t d_t, int32_t d_h, int32_t d_w, float theta, float eps, void *stream)
{
    if (B < 0 || N < 0 || H < 0 || Dh < 0 || B > kMaxSamples || N > kMaxSubBlocks * DIT_SUBBLOCK_TOKENS ||
        in_token_stride < 0 || in_token_stride > kMaxWidth)
        return DIT_ERR_ARG;
    if (out_layout != DIT_QK_TOKEN_MAJOR && out_layout != DIT_QK_HEAD_MAJOR)
        return DIT_ERR_ARG;
    if (!subblock_head_ok(H, Dh) || d_t < 0 || d_h < 0 || d_w < 0 || (d_t | d_h | d_w) & 1 ||
        (int64_t)d_t + d_h + d_w != Dh || in_token_stride % 8 != 0 || in_token_stride < H * Dh)
        return DIT_ERR_SHAPE;
    int64_t plane = 0;
    const dit_status ps = plane_stride(out_plane_stride, out_layout, B, N, H, Dh, &plane);
    if (ps != DIT_OK)
        return ps;
    if (!(eps > 0.f) || !isfinite(eps) || !(theta > 1.f) || !isfinite(theta))
        return DIT_ERR_ARG;
    if (B == 0 || N == 0)
        return DIT_OK;
    if (!q || !k || !q_out || !k_out || !wq || !wk || !pos || !q_pooled || !k_pooled)
        return DIT_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(q_out, 16) || !aligned(k_out, 16) || !aligned(wq, 16) ||
        !aligned(wk, 16) || !aligned(pos, 4) || !aligned(q_pooled, 16) || !aligned(k_pooled, 16))
        return DIT_ERR_ALIGN;
    const int64_t rows = B * N;
    const int64_t nb = (N + DIT_SUBBLOCK_TOKENS - 1) / DIT_SUBBLOCK_TOKENS;
    const int64_t nt = qk_out_extent(out_layout, B, N, H, Dh, plane); // byte extent of each output
    const int64_t ni = ((rows - 1) * in_token_stride + H * Dh) * 2;   // byte extent of each input
    const int64_t npool = B * H * nb * Dh * 4, nw = Dh * 2, np = N * 12;
    // q' may overwrite q and k' k exactly, where the two layouts coincide; the
    // inputs may share a buffer (fused QKV); nothing else overlaps.
    const bool same_layout = in_token_stride == H * Dh && out_layout == DIT_QK_TOKEN_MAJOR;
    const bool q_bad = same_layout ? bad_alias(q_out, q, nt) : overlap(q_out, nt, q, ni);
    const bool k_bad = same_layout ? bad_alias(k_out, k, nt) : overlap(k_out, nt, k, ni);
    if (q_bad || k_bad || overlap(q_out, nt, k, ni) || overlap(k_out, nt, q, ni) || overlap(k_out, nt, q_out, nt))
        return DIT_ERR_ARG;
    const void *rd[5] = {q, k, wq, wk, pos};
    const int64_t rd_n[5] = {ni, ni, nw, nw, np};
    const void *wr[4] = {q_out, k_out, q_pooled, k_pooled};
    const int64_t wr_n[4] = {nt, nt, npool, npool};
    for (int i = 0; i < 4; ++i) {
        for (int j = i < 2 ? 2 : 0; j < 5; ++j) // q_out, k_out against q, k are checked above
            if (overlap(wr[i], wr_n[i], rd[j], rd_n[j]))
                return DIT_ERR_ARG;
        for (int j = 2; j < 4; ++j)
            if (j != i && overlap(wr[i], wr_n[i], wr[j], wr_n[j]))
                return DIT_ERR_ARG;
    }
    return launched(dit::launch_qk_rmsnorm_rope3d_pool(q, k, q_out, k_out, wq, wk, pos, q_pooled, k_pooled, B, N, H,
                                                       Dh, in_token_stride, out_layout == DIT_QK_HEAD_MAJOR, plane,
                                                       d_t, d_h, d_w, theta, eps, (hipStream_t)stream));
}

dit_status dit_subblock_route(const float *q_pooled, const float *k_pooled, float *scores, int32_t *kept, int64_t B,
                              int64_t H, int64_t nb, int64_t Dh, int64_t keep, void *stream)
{
    if (B < 0 || H < 0 || nb < 0 || Dh < 0 || keep < 0 || B > kMaxSamples || nb > kMaxSubBlocks)
        return DIT_ERR_ARG;
    if (!subblock_head_ok(H, Dh))
        return DIT_ERR_SHAPE;
    if (keep > nb)
        return DIT_ERR_ARG;
    if (B == 0 || nb == 0 || (!scores && keep == 0)) // nothing to compute
        return DIT_OK;
    if (!q_pooled || !k_pooled || (keep > 0 && !kept))
        return DIT_ERR_NULL;
    if (!aligned(q_pooled, 16) || !aligned(k_pooled, 16) || !aligned(scores, 16) || (keep > 0 && !aligned(kept, 4)))
        return DIT_ERR_ALIGN;
    const int64_t ld = dit_subblock_scores_ld(nb);
    const int64_t np = B * H * nb * Dh * 4, ns = scores ? B * H * nb * ld * 4 : 0, nk = B * H * nb * keep * 4;
    if (scores && (overlap(scores, ns, q_pooled, np) || overlap(scores, ns, k_pooled, np)))
        return DIT_ERR_ARG;
    if (keep > 0 && ((scores && overlap(kept, nk, scores, ns)) || overlap(kept, nk, q_pooled, np) ||
                     overlap(kept, nk, k_pooled, np)))
        return DIT_ERR_ARG;
    return launched(
        dit::launch_subblock_route(q_pooled, k_pooled, scores, kept, B, H, nb, Dh, ld, keep, (hipStream_t)stream));
}

dit_status dit_packed_positions(int32_t *pos, int64_t T, int64_t Hg, int64_t Wg, int64_t n_extra, void *stream)
{
    if (T < 0 || Hg < 0 || Wg < 0 || n_extra < 0 || n_extra > kMaxRows)
        return DIT_ERR_ARG;
    const int64_t hw = row_count(Hg, Wg);
    const int64_t video = hw < 0 ? -1 : row_count(T, hw);
    if (video < 0 || video + n_extra > kMaxRows)
        return DIT_ERR_ARG;
    if (video + n_extra == 0)
        return DIT_OK;
    if (!pos)
        return DIT_ERR_NULL;
    if (!aligned(pos, 4))
        return DIT_ERR_ALIGN;
    return launched(dit::launch_packed_positions(pos, T, Hg, Wg, n_extra, (hipStream_t)stream));
}

static_assert(DIT_STREAM_READ == dit::kPatternRead && DIT_STREAM_WRITE == dit::kPatternWrite &&
                  DIT_STREAM_SPLIT_ROWS == dit::kPatternSplitRows && DIT_STREAM_TWO_IN == dit::kPatternTwoIn &&
                  DIT_STREAM_ROW_GROUP == dit::kPatternRowGroup && DIT_STREAM_ROW_GROUP_2X2 == dit::kPatternRowGroup2x2 &&
                  DIT_STREAM_HEAD_MAJOR == dit::kPatternHeadMajor && DIT_STREAM_SCORE_TILES == dit::kPatternScoreTiles &&
                  DIT_STREAM_TOPK_ROWS == dit::kPatternTopkRows,
              "pattern kinds");

dit_status dit_stream_pattern(int32_t kind, const void *in0, const void *in1, void *out0, void *out1, int64_t rows,
                              int64_t row_bytes, int64_t heads, void *stream)
{
    if (kind < DIT_STREAM_READ || kind > DIT_STREAM_TOPK_ROWS || rows < 0 || rows > kMaxRows || row_bytes < 0 ||
        heads < 0)
        return DIT_ERR_ARG;
    if (row_bytes < 16 || row_bytes % 16 != 0 || row_bytes > 2 * kMaxWidth)
        return DIT_ERR_SHAPE;
    if (kind == DIT_STREAM_ROW_GROUP || kind == DIT_STREAM_ROW_GROUP_2X2) {
        if (row_bytes > 2 * kMaxAdaLNWidth)
            return DIT_ERR_SHAPE;
    }
    if (kind == DIT_STREAM_HEAD_MAJOR) {
        if (heads < 1 || (row_bytes / 16) % heads != 0 || 256 % ((row_bytes / 16) / heads) != 0)
            return DIT_ERR_SHAPE;
        if (rows * ((row_bytes / 16 + 255) / 256) > kMaxRows)
            return DIT_ERR_ARG;
    }
    const bool score_tiles = kind == DIT_STREAM_SCORE_TILES;
    if (score_tiles) {
        if (heads < 1 || rows % heads != 0 || row_bytes < 16 * ((heads + 3) / 4))
            return DIT_ERR_SHAPE;
        const int64_t tiles = (heads + 127) / 128;
        if ((rows / heads) * tiles * tiles >= (int64_t)1 << 31)
            return DIT_ERR_ARG;
    }
    const bool topk_rows = kind == DIT_STREAM_TOPK_ROWS;
    if (topk_rows) {
        if (heads < 1 || heads > 4096 || rows % heads != 0 || row_bytes < 4 * heads)
            return DIT_ERR_SHAPE;
        if (rows / heads > 65535)
            return DIT_ERR_ARG;
    }
    if ((kind == DIT_STREAM_SPLIT_ROWS && !dit::swiglu_fits(rows, row_bytes / 2)) ||
        (kind == DIT_STREAM_TWO_IN && !dit::gated_residual_fits(rows, row_bytes / 2)))
        return DIT_ERR_ARG;
    if (rows == 0)
        return DIT_OK;
    const bool two_in = kind == DIT_STREAM_TWO_IN || kind == DIT_STREAM_ROW_GROUP_2X2 || score_tiles;
    if ((kind != DIT_STREAM_WRITE && !in0) || (two_in && !in1) || !out0 || (kind == DIT_STREAM_ROW_GROUP_2X2 && !out1))
        return DIT_ERR_NULL;
    if (!aligned(in0, 16) || !aligned(in1, 16) || !aligned(out0, 16) || !aligned(out1, 16))
        return DIT_ERR_ALIGN;
    const int64_t n = rows * row_bytes;
    const int64_t nin = kind == DIT_STREAM_SPLIT_ROWS ? 2 * n : score_tiles ? rows * 512 : n;
    const int64_t nout = kind == DIT_STREAM_READ ? 16 : topk_rows ? rows * ((heads + 3) / 4) * 4 : n;
    const void *ins[2] = {kind == DIT_STREAM_WRITE ? nullptr : in0, two_in ? in1 : nullptr};
    void *outs[2] = {out0, kind == DIT_STREAM_ROW_GROUP_2X2 ? out1 : nullptr};
    for (void *o : outs) {
        if (!o)
            continue;
        for (const void *i : ins)
            if (i && overlap(o, nout, i, nin))
                return DIT_ERR_ARG;
    }
    if (outs[1] && overlap(outs[0], nout, outs[1], nout))
        return DIT_ERR_ARG;
    return launched(dit::launch_stream_pattern(kind, in0, in1, out0, out1, rows, row_bytes, heads,
                                               (hipStream_t)stream));
}

dit_status dit_copy16(const void *src, void *dst, int64_t bytes, void *stream)
{
    if (bytes < 0)
        return DIT_ERR_ARG;
    if (bytes % 16 != 0)
        return DIT_ERR_SHAPE;
    if (bytes == 0)
        return DIT_OK;
    if (!src || !dst)
        return DIT_ERR_NULL;
    if (!aligned(src, 16) || !aligned(dst, 16))
        return DIT_ERR_ALIGN;
    if (overlap(src, bytes, dst, bytes))
        return DIT_ERR_ARG;
    return launched(dit::launch_copy16(src, dst, bytes, (hipStream_t)stream));
}

} // extern "C"
