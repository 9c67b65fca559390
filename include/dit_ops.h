/*
 * dit_ops.h -- C ABI of the fused non-GEMM operator chain of a video+audio
 * diffusion-transformer (DiT) denoising block, for AMD Instinct MI355X (gfx950).
 *
 * Where the operations come from:
 *   "8×H200 上的 MiniMax-H3:无损加速 1.95 倍,SSIM 0.76–0.91 下最高 6.24 倍"
 *   (xhh.club), section Q&A, the answer on which operations the fused kernels
 *   optimise: AdaLN modulation, gated residual, SwiGLU activation, and QK
 *   RMSNorm fused with 3D RoPE.
 *   "SGLang acelera vídeo do MiniMax-H3 em até 6,2x em GPUs H200"
 *   (stamatios.com), section "Resultado principal": the fused kernels remove
 *   memory traffic, intermediate tensors and launches without changing the
 *   arithmetic; video and audio tokens form one packed DiT sequence.
 *   "Sol-H3: Recursive Self-Improvement for MiniMax-H3 Inference Acceleration
 *   on Sol-Engine across Cloud and Edge", abstract: operator work is a search
 *   over kernel fusions and memory layouts judged by latency together with
 *   numerical agreement.
 * The pages name these operations but print no formulas; each entry point
 * states the standard definition it computes and the readings it takes.
 *
 * Conventions shared by every entry point:
 *   - Tensors are bf16 (raw bit patterns, dit_bf16), row-major and contiguous,
 *     last dimension unit-stride, batch-major [B][N][...].  Arithmetic is fp32
 *     with a single round-to-nearest-even to bf16 at each output element.
 *   - Every pointer is a DEVICE pointer on the current HIP device.  The caller
 *     owns all buffers; the library allocates nothing, keeps no state between
 *     calls (one exception: the static scratch array of
 *     dit_residual_change_noalloc), and never synchronises.  Work is enqueued on `stream` (a
 *     hipStream_t cast to void*; NULL = the default stream) and completes
 *     asynchronously, in stream order.
 *   - Arguments are validated on the host BEFORE any HIP call or write; a
 *     rejected call touches no memory and enqueues nothing:
 *       DIT_ERR_NULL   a required pointer is NULL
 *       DIT_ERR_SHAPE  a width is not a multiple of 8, exceeds a stated limit,
 *                      or RoPE bands are odd or do not sum to the head width
 *       DIT_ERR_ALIGN  a bf16 pointer is not 16-byte aligned (int32 pointers:
 *                      4-byte)
 *       DIT_ERR_ARG    a negative size, eps <= 0 or not finite, theta <= 1 or
 *                      not finite, more than 2^24 - 1 rows (tokens) in one
 *                      call, or outputs that overlap inputs in a way the entry
 *                      point forbids
 *       DIT_ERR_HIP    the kernel launch itself failed (hipGetLastError)
 *       DIT_ERR_SCRATCH  the sizes need more than the fixed capacity of the
 *                      library's static scratch array (allocation-free entry
 *                      points only)
 *     A call with zero rows is a no-op returning DIT_OK (its pointers are not
 *     examined).  Faults inside a
 *     kernel (for example a pointer that is not device memory) surface at the
 *     caller's next synchronisation, as for any HIP work.  The library never
 *     aborts and never prints.
 */
#ifndef DIT_OPS_H
#define DIT_OPS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t dit_bf16; /* raw bfloat16 bits */

typedef enum {
    DIT_OK = 0,
    DIT_ERR_NULL = 1,
    DIT_ERR_SHAPE = 2,
    DIT_ERR_ALIGN = 3,
    DIT_ERR_ARG = 4,
    DIT_ERR_HIP = 5,
    DIT_ERR_SCRATCH = 6 /* sizes beyond a static scratch buffer's capacity */
} dit_status;

#define DIT_ABI_VERSION 5

/* Human-readable name of a status code; never NULL. */
const char *dit_status_str(int status);

/* DIT_ABI_VERSION of the built library. */
int dit_abi_version(void);

/*
 * AdaLN modulation: y = LayerNorm(x) * (1 + scale[b]) + shift[b].
 * Cited: xhh.club summary, Q&A (fused-kernel answer), "AdaLN modulation".
 * LayerNorm runs over the D channels of each token with no affine parameters:
 * mean, biased variance (divide by D), y_i = (x_i - mean) / sqrt(var + eps).
 * shift and scale are per sample and apply to all N tokens of that sample.
 *   x      [B][N][D]  input
 *   shift  [B][D]
 *   scale  [B][D]
 *   y      [B][N][D]  output; y == x (in place) is allowed, any other overlap
 *                     with x, shift or scale is rejected (DIT_ERR_ARG)
 *   D      multiple of 8, 8 <= D <= 8192
 *   eps    > 0 (1e-6 in the shipped workloads)
 */
dit_status dit_adaln_modulate(const dit_bf16 *x, const dit_bf16 *shift,
                              const dit_bf16 *scale, dit_bf16 *y, int64_t B,
                              int64_t N, int64_t D, float eps, void *stream);

/*
 * Gated residual: out = x + gate[b] * y.
 * Cited: xhh.club summary, Q&A (fused-kernel answer), "gated residual".
 * The gate is used as given (no sigmoid or tanh); it is per sample and
 * applies to all N tokens of that sample.
 *   x, y   [B][N][D]
 *   gate   [B][D]
 *   out    [B][N][D]; out == x or out == y (in place) is allowed, any other
 *          overlap with an input is rejected (DIT_ERR_ARG)
 *   D      multiple of 8, 8 <= D <= 2^24
 *   B * N * ceil(D / 4096) <= 4,286,578,688 (2^32 - 2^23) row segments, else
 *          DIT_ERR_ARG
 */
dit_status dit_gated_residual(const dit_bf16 *x, const dit_bf16 *y,
                              const dit_bf16 *gate, dit_bf16 *out, int64_t B,
                              int64_t N, int64_t D, void *stream);

/*
 * SwiGLU activation: out[r][j] = silu(in[r][j]) * in[r][F + j],
 * silu(a) = a / (1 + exp(-a)).
 * Cited: xhh.club summary, Q&A (fused-kernel answer), and the stamatios.com
 * summary, "De onde vêm os ganhos", both listing SwiGLU.
 * Each input row is the two halves [a | b] of width F each, as an up
 * projection of width 2F emits them; the first half is gated.
 *   in     [M][2F]
 *   out    [M][F]; must not overlap `in` (DIT_ERR_ARG)
 *   F      multiple of 8, 8 <= F <= 2^24
 *   M * ceil(F / 2048) <= 4,278,190,080 (2^32 - 2^24) row segments, else
 *          DIT_ERR_ARG
 * Finite inputs give finite outputs: silu saturates to a for large a and to
 * (-)0 for very negative a.
 */
dit_status dit_swiglu(const dit_bf16 *in, dit_bf16 *out, int64_t M, int64_t F,
                      void *stream);

/*
 * Per-head QK RMSNorm fused with 3D rotary embedding, for q and k.
 * Cited: xhh.club summary, Q&A (fused-kernel answer), "QK RMSNorm fused with
 * 3D RoPE".
 * For every sample b, token n and head h, separately for q (weight wq) and
 * k (weight wk), over the Dh channels v of that head:
 *   u_i = v_i / sqrt(mean(v^2) + eps) * w_i
 * then the head's channels are split into three contiguous bands t, h, w of
 * widths d_t, d_h, d_w; in a band of width d driven by the token's integer
 * coordinate p (pos[n][0], pos[n][1] or pos[n][2]), the adjacent pair
 * (2j, 2j+1), j < d/2, is rotated counter-clockwise by p * theta^(-2j/d):
 *   (u0, u1) -> (u0 cos f - u1 sin f, u0 sin f + u1 cos f).
 *   q, k          [B][N][H][Dh] inputs
 *   q_out, k_out  [B][N][H][Dh] outputs; q_out == q and k_out == k are
 *                 allowed, any other overlap is rejected (DIT_ERR_ARG)
 *   wq, wk        [Dh] RMSNorm weights shared by all heads
 *   pos           [N][3] int32 (t, h, w) coordinates, shared by all B samples;
 *                 entries must lie in [0, 2^24) so they convert to fp32 exactly
 *   Dh            one of 8, 16, 32, 64, 128, 256
 *   d_t, d_h, d_w even, >= 0, d_t + d_h + d_w == Dh
 *   theta > 1 (1e4 in the shipped workloads), eps > 0
 */
dit_status dit_qk_rmsnorm_rope3d(const dit_bf16 *q, const dit_bf16 *k,
                                 dit_bf16 *q_out, dit_bf16 *k_out,
                                 const dit_bf16 *wq, const dit_bf16 *wk,
                                 const int32_t *pos, int64_t B, int64_t N,
                                 int64_t H, int64_t Dh, int32_t d_t,
                                 int32_t d_h, int32_t d_w, float theta,
                                 float eps, void *stream);

/* Output layouts of dit_qk_rmsnorm_rope3d_layout. */
#define DIT_QK_TOKEN_MAJOR 0 /* [B][N][H][Dh] */
#define DIT_QK_HEAD_MAJOR 1  /* [B][H][N][Dh], head planes out_plane_stride apart */

/*
 * dit_qk_rmsnorm_rope3d with the memory layouts around it made explicit:
 * q and k are read with a token stride, so they can be the q and k parts of a
 * fused QKV projection [B][N][3][H][Dh] (q = qkv, k = qkv + H*Dh, stride
 * 3*H*Dh) with no split pass, and q_out, k_out can be written head-major
 * [B][H][N][Dh], the layout an attention kernel reads, with no transpose pass.
 * Head-major planes may be padded apart (out_plane_stride), so that they do
 * not all start at the same offset modulo the memory system's interleave.
 * The arithmetic is exactly that of dit_qk_rmsnorm_rope3d.
 * Cited: the Sol-H3 abstract (its search covers memory layouts as well as
 * kernel fusions); xhh.club Q&A for the operation itself.
 *   q, k             token (b, n), head h, channel i at
 *                    (b*N + n) * in_token_stride + h*Dh + i
 *   in_token_stride  elements between consecutive tokens: a multiple of 8 and
 *                    >= H*Dh (DIT_ERR_SHAPE otherwise)
 *   out_layout       DIT_QK_TOKEN_MAJOR or DIT_QK_HEAD_MAJOR (else DIT_ERR_ARG)
 *   out_plane_stride head-major: elements from head plane (b, h) to the next,
 *                    element (b, h, n, i) at (b*H + h) * out_plane_stride +
 *                    n*Dh + i; 0 selects N*Dh (packed [B][H][N][Dh]); else a
 *                    multiple of 8 and >= N*Dh (DIT_ERR_SHAPE otherwise), at
 *                    most 2^40, with the whole output under 2^62 bytes
 *                    (DIT_ERR_ARG otherwise).  The padding between planes is
 *                    never read or written.  Token-major: must be 0
 *                    (DIT_ERR_ARG otherwise)
 *   q_out, k_out     [B][N][H][Dh] or [B][H][N][Dh]; in place (q_out == q,
 *                    k_out == k) only when in_token_stride == H*Dh and the
 *                    layout is token-major; any other overlap (over the
 *                    output's whole extent, padding included) is rejected
 * All other arguments and limits as for dit_qk_rmsnorm_rope3d.
 */
dit_status dit_qk_rmsnorm_rope3d_layout(const dit_bf16 *q, const dit_bf16 *k,
                                        dit_bf16 *q_out, dit_bf16 *k_out,
                                        const dit_bf16 *wq, const dit_bf16 *wk,
                                        const int32_t *pos, int64_t B, int64_t N,
                                        int64_t H, int64_t Dh,
                                        int64_t in_token_stride,
                                        int32_t out_layout,
                                        int64_t out_plane_stride, int32_t d_t,
                                        int32_t d_h, int32_t d_w, float theta,
                                        float eps, void *stream);

/*
 * Gated residual fused with the AdaLN modulation that follows it:
 *   x_out = x + gate[b] * y                       (rounded once to bf16)
 *   z     = LayerNorm(x_out) * (1 + scale[b]) + shift[b]
 * where LayerNorm (as in dit_adaln_modulate) runs over the bf16 values stored
 * in x_out, so the result equals calling dit_gated_residual and then
 * dit_adaln_modulate on its output.
 * Cited: xhh.club summary, Q&A (fused-kernel answer) names both operations;
 * the Sol-H3 abstract describes searching over such fusions; the
 * stamatios.com summary, "Resultado principal", says fusion leaves the
 * arithmetic unchanged.  Reads x and y once and writes x_out and z once:
 * 8 bytes per element instead of 10 for the two separate calls.
 *   x, y          [B][N][D] inputs
 *   gate, shift, scale  [B][D]
 *   x_out         [B][N][D]; x_out == x (in-place residual update) is allowed
 *   z             [B][N][D]; z == y (reuse of the branch buffer) is allowed
 *   any other overlap among the buffers is rejected (DIT_ERR_ARG)
 *   D             multiple of 8, 8 <= D <= 8192
 *   eps           > 0
 */
dit_status dit_gated_residual_adaln(const dit_bf16 *x, const dit_bf16 *y,
                                    const dit_bf16 *gate, const dit_bf16 *shift,
                                    const dit_bf16 *scale, dit_bf16 *x_out,
                                    dit_bf16 *z, int64_t B, int64_t N,
                                    int64_t D, float eps, void *stream);

/*
 * Cache-DiT residual-change statistic, per sample b over every token (video
 * and audio alike) and channel of the packed sequence:
 *   out[3b + 0] = sum |r - r_cached|
 *   out[3b + 1] = sum |r_cached|
 *   out[3b + 2] = out[3b] / out[3b + 1]   (0 if both sums are 0, +inf if only
 *                                          the second is)
 * Cited: xhh.club summary, Q&A on Cache-DiT (after warm-up, boundary blocks'
 * normalised residual change against the cached state decides whether the
 * middle blocks are reused); stamatios.com summary, "Resultado principal"
 * (one joint decision for the packed video+audio stack).  Reading: the
 * normalised change is this relative L1 distance; the threshold and the
 * reuse policy are the caller's.
 *   r, r_cached   [B][N][D] bf16
 *   out           [B][3] double, device memory, 8-byte aligned
 *   workspace     device scratch owned by the caller, 16-byte aligned, at
 *                 least dit_residual_change_workspace_bytes(B, N, D) bytes
 *                 (DIT_ERR_ARG if smaller); its contents on entry do not
 *                 matter and on return are unspecified
 *   D             multiple of 8; B <= 65535; per sample at most
 *                 4,194,303 tiles of 2048 16-byte vectors, i.e. N * D <=
 *                 68,719,460,352 (else DIT_ERR_ARG)
 * Sums are fp32 over each 8-value vector and fp64 above, in a fixed order:
 * repeated calls give bit-identical results.  B == 0 is a no-op; N == 0
 * writes zeros.  No buffer may overlap another (DIT_ERR_ARG).
 */
dit_status dit_residual_change(const dit_bf16 *r, const dit_bf16 *r_cached,
                               double *out, void *workspace,
                               int64_t workspace_bytes, int64_t B, int64_t N,
                               int64_t D, void *stream);

/*
 * Bytes of workspace dit_residual_change needs for these sizes (16 bytes per
 * 2048 16-byte vectors of each sample, rounded up), or -1 if the sizes are
 * invalid.  Host-only; makes no HIP call.
 */
int64_t dit_residual_change_workspace_bytes(int64_t B, int64_t N, int64_t D);

/*
 * dit_residual_change without the workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The per-tile partials live in a static
 * 2 MiB array inside the library's device code (one copy per GPU, held until
 * the process ends), so the call allocates nothing: it makes no hipMalloc or
 * hipFree and calls no allocating library routine.  Results are bit-identical
 * to dit_residual_change on the same inputs (same kernels, same order).
 *   r, r_cached, out, B, N, D  as for dit_residual_change
 *   capacity   B * ceil(N * D / 16384) <= 131,072 partials (2 MiB), else
 *              DIT_ERR_SCRATCH before any HIP call: about 2^31 elements in
 *              all, e.g. one sample of up to 524,288 tokens of width 4096, or
 *              two samples of 124,992 tokens.
 * The first call on a device looks up the array's device address
 * (hipGetSymbolAddress) and caches it; DIT_ERR_HIP if that fails.  Every call
 * on one GPU shares the one array, which keeps the last call's partials: calls
 * that overlap in time on one GPU (on different streams, or from several host
 * threads without stream ordering) race on it and may return wrong sums.
 * Calls ordered on one stream are safe.  Nothing in the array needs clearing
 * between calls: each call writes every partial it reads.
 */
dit_status dit_residual_change_noalloc(const dit_bf16 *r, const dit_bf16 *r_cached,
                                       double *out, int64_t B, int64_t N,
                                       int64_t D, void *stream);

/*
 * SubBlock sparse-attention routing, front-end.
 * Cited: stamatios.com summary, "De onde vêm os ganhos" (SubBlock attention
 * splits the sequence into 64-token blocks and routing keeps only part of the
 * key blocks) and "Resultado principal" (the blocks dropped are those of
 * smaller estimated contribution); xhh.club Q&A on the sparsity parameter
 * (sparsity is the share of key blocks that may be dropped: 0.75 keeps about
 * 25%).  Readings: a block is summarised by the mean of its tokens' q' (or k')
 * head vectors; the estimated contribution of key block j to query block i is
 * the dot product of the two means, rounded to bf16 first (the attention
 * operands' precision), per sample and head, without a 1/sqrt(Dh) factor; ties
 * are kept lowest index first.  Blocks never span two samples; the last block
 * of a sample may be shorter and averages only its own tokens.
 * The dense fallback for short calls and the first steps, and the sparse
 * attention itself, are the caller's.
 */
#define DIT_SUBBLOCK_TOKENS 64

/*
 * Key blocks kept per query block for `nb` blocks at `sparsity`:
 * nb - floor(sparsity * nb), at least 1 (0 when nb == 0); -1 if nb < 0 or
 * sparsity is not in [0, 1).  Host-only; makes no HIP call.
 */
int64_t dit_subblock_keep(int64_t nb, double sparsity);

/*
 * Row stride (in floats) of the score matrix dit_subblock_route writes: nb
 * rounded up to a multiple of 32, so that every row starts on a 128-byte line;
 * -1 if nb < 0 or nb > 4096.  Host-only.
 */
int64_t dit_subblock_scores_ld(int64_t nb);

/*
 * Block means of q' and k':
 *   q_pooled[b][h][i][d] = mean of q[b][n][h][d] over the tokens n of block i
 *   (n = 64 i .. min(64 i + 64, N) - 1), the same for k; fp32 sums of the
 *   bf16 inputs, one fp32 division.
 *   q, k      bf16, [B][N][H][Dh] for layout DIT_QK_TOKEN_MAJOR or
 *             [B][H][N][Dh] for DIT_QK_HEAD_MAJOR (else DIT_ERR_ARG); may be
 *             the same buffer
 *   q_pooled, k_pooled
 *             fp32 [B][H][nb][Dh], nb = ceil(N / 64), 16-byte aligned; they
 *             overlap neither each other nor the inputs (DIT_ERR_ARG)
 *   Dh in {16, 32, 64, 128, 256}, H*Dh <= 65536 (else DIT_ERR_SHAPE);
 *   N <= 262,144 (4096 blocks) and B <= 65535 (else DIT_ERR_ARG).
 * Deterministic: a fixed summation order per layout.  B == 0 or N == 0 is a
 * no-op.
 */
dit_status dit_subblock_pool(const dit_bf16 *q, const dit_bf16 *k,
                             float *q_pooled, float *k_pooled, int64_t B,
                             int64_t N, int64_t H, int64_t Dh, int32_t layout,
                             void *stream);

/*
 * QK RMSNorm + 3D RoPE fused with the block means of its outputs: q_out, k_out
 * are exactly those of dit_qk_rmsnorm_rope3d_layout with the same strides and
 * layout, and q_pooled, k_pooled exactly those dit_subblock_pool computes from
 * the stored q_out, k_out, without reading them back from memory.  With a
 * fused QKV projection as input and head-major outputs this prepares q', k'
 * for attention and the means for SubBlock routing in one pass.
 * Cited: xhh.club Q&A ("QK RMSNorm fused with 3D RoPE"); stamatios.com
 * summary, "De onde vêm os ganhos" (SubBlock 64-token blocks); Sol-H3
 * abstract (search over kernel fusions and memory layouts).  Reading: the
 * routing pools q', k' as stored in bf16.
 *   q, k             bf16; token (b, n), head h at (b*N + n)*in_token_stride +
 *                    h*Dh; in_token_stride a multiple of 8, >= H*Dh, at most
 *                    2^24 (else DIT_ERR_SHAPE / DIT_ERR_ARG); may share a buffer
 *   q_out, k_out     bf16 [B][N][H][Dh] (DIT_QK_TOKEN_MAJOR) or [B][H][N][Dh]
 *                    (DIT_QK_HEAD_MAJOR; else DIT_ERR_ARG); q_out == q and
 *                    k_out == k only when in_token_stride == H*Dh and the output
 *                    is token-major; any other overlap DIT_ERR_ARG
 *   out_plane_stride as for dit_qk_rmsnorm_rope3d_layout
 *   wq, wk, pos      as for dit_qk_rmsnorm_rope3d
 *   q_pooled, k_pooled  fp32 [B][H][ceil(N/64)][Dh], 16-byte aligned,
 *                    overlapping nothing else (DIT_ERR_ARG)
 *   Dh in {16, 32, 64, 128, 256}, bands as for dit_qk_rmsnorm_rope3d, H*Dh <=
 *   65536 (else DIT_ERR_SHAPE); N <= 262,144 and B <= 65535 (else DIT_ERR_ARG).
 * B == 0 or N == 0 is a no-op.
 */
dit_status dit_qk_rmsnorm_rope3d_pool(const dit_bf16 *q, const dit_bf16 *k,
                                      dit_bf16 *q_out, dit_bf16 *k_out,
                                      const dit_bf16 *wq, const dit_bf16 *wk,
                                      const int32_t *pos, float *q_pooled,
                                      float *k_pooled, int64_t B, int64_t N,
                                      int64_t H, int64_t Dh,
                                      int64_t in_token_stride,
                                      int32_t out_layout,
                                      int64_t out_plane_stride, int32_t d_t,
                                      int32_t d_h, int32_t d_w, float theta,
                                      float eps, void *stream);

/*
 * Block scores and the kept key blocks of every query block:
 *   scores[b][h][i][j] = sum_d bf16(q_pooled[b][h][i][d]) *
 *                               bf16(k_pooled[b][h][j][d])
 *   (round-to-nearest-even operands, fp32 accumulation on the matrix cores);
 *   kept[b][h][i][0 .. keep-1] = the keep key blocks j of largest score (equal
 *   scores: lower j first), in ascending order of j.
 *   q_pooled, k_pooled  fp32 [B][H][nb][Dh], 16-byte aligned (as written by
 *                       dit_subblock_pool); may be the same buffer
 *   scores    fp32 [B][H][nb][ld], ld = dit_subblock_scores_ld(nb), 16-byte
 *             aligned, an output; entries j >= nb of a row are unspecified
 *             (the kernel may write them).  NULL: the score matrix is not
 *             written at all -- scores and selection run in one kernel that
 *             keeps each strip's scores on chip, reading only the means and
 *             writing only the kept lists (the same lists, bit for bit, as
 *             with a score matrix); with keep == 0 the call is then a no-op
 *   kept      int32 [B][H][nb][keep], 4-byte aligned; unused if keep == 0
 *   keep      0 <= keep <= nb (else DIT_ERR_ARG); dit_subblock_keep gives the
 *             count for a sparsity
 *   Dh in {16, 32, 64, 128, 256}, H*Dh <= 65536 (else DIT_ERR_SHAPE);
 *   nb <= 4096 and B <= 65535 (else DIT_ERR_ARG).
 * Scores are expected finite; with NaN pooled values the kept lists are still
 * keep distinct, ascending, in-range indices.  scores and kept overlap no
 * other buffer (DIT_ERR_ARG).  Deterministic.  B == 0 or nb == 0 is a no-op.
 */
dit_status dit_subblock_route(const float *q_pooled, const float *k_pooled,
                              float *scores, int32_t *kept, int64_t B,
                              int64_t H, int64_t nb, int64_t Dh, int64_t keep,
                              void *stream);

/*
 * Packed token coordinates for the 3D rotary embedding.
 * Cited: stamatios.com summary, "Resultado principal" (video and audio tokens
 * in one packed DiT sequence); xhh.club Q&A ("3D RoPE").
 * Writes pos[N][3] int32 for N = T*Hg*Wg + n_extra tokens: video token
 * n < T*Hg*Wg gets its row-major latent-grid coordinate
 * (n / (Hg*Wg), (n / Wg) % Hg, n % Wg); the n_extra tokens that follow get the
 * temporal-only coordinate (a, 0, 0), a = 0 .. n_extra-1.
 *   pos    [N][3] device buffer, 4-byte aligned
 *   T, Hg, Wg, n_extra >= 0; N = T*Hg*Wg + n_extra at most 2^24 - 1
 */
dit_status dit_packed_positions(int32_t *pos, int64_t T, int64_t Hg, int64_t Wg,
                                int64_t n_extra, void *stream);

/*
 * Plain 16-byte-vector device copy, dst = src, `bytes` a multiple of 16.
 * Not an operator of the chain: it is the streaming-bandwidth ceiling the
 * chain's kernels are measured against, and the known-size workload used to
 * calibrate hardware byte counters.  src and dst must not overlap.
 */
dit_status dit_copy16(const void *src, void *dst, int64_t bytes, void *stream);

/*
 * Access-pattern streams: the memory traffic of the chain's kernels with no
 * arithmetic, each with the launch shape of the kernel it stands for.  Not
 * operators of the chain: they are the ceilings the kernels are measured
 * against ("X% of its own pattern").  Outputs are plain copies or XORs of the
 * inputs.  `rows` rows of `row_bytes` bytes each (a multiple of 16):
 *   DIT_STREAM_READ          reads in0 [rows][row_bytes]; out0 is a 16-byte
 *                            sink written only when the XOR of everything
 *                            read equals a fixed key (keeps the loads live)
 *   DIT_STREAM_WRITE         writes out0 [rows][row_bytes] (in0 unused)
 *   DIT_STREAM_SPLIT_ROWS    in0 [rows][2*row_bytes] -> out0 [rows][row_bytes],
 *                            out = first half XOR second half (SwiGLU's shape)
 *   DIT_STREAM_TWO_IN        out0 = in0 XOR in1 (the gated residual's shape)
 *   DIT_STREAM_ROW_GROUP     out0 = in0 with AdaLN's mapping: two rows per
 *                            workgroup, each thread two 16-byte vectors of
 *                            each row, every load before any store;
 *                            row_bytes <= 16384
 *   DIT_STREAM_ROW_GROUP_2X2 out0 = in0 and out1 = in1 with ROW_GROUP's
 *                            mapping, out0 stored before out1 (the fused
 *                            residual -> AdaLN's shape)
 *   DIT_STREAM_HEAD_MAJOR    in0 [rows][heads][row_bytes/heads] ->
 *                            out0 [heads][rows][row_bytes/heads] (token-major
 *                            to head-major copy) in the head-major QK
 *                            kernel's shape: four tokens per workgroup,
 *                            staged so each store writes one head's four
 *                            tokens; row_bytes/16 a multiple of heads and
 *                            row_bytes/heads/16 a divisor of 256;
 *                            rows * ceil(row_bytes / 4096) < 2^24
 *   DIT_STREAM_SCORE_TILES   the block-score traffic of dit_subblock_route at
 *                            head dim 128, in that kernel's launch shape and
 *                            tile order: here `heads` is the number of blocks
 *                            n and rows = P * n (P planes).  Reads in0 and in1
 *                            [rows][128] fp32 (query and key means; each query
 *                            tile when it changes, every key tile), writes the
 *                            n x n leading block of each plane of out0
 *                            [rows][row_bytes] (columns up to n rounded up to
 *                            4; row_bytes >= 16 * ceil(n / 4)).  With all-zero
 *                            means the 32-bit word at (row r, column c) is
 *                            (r * 65536 + c) mod 2^32; otherwise it is that
 *                            XOR a fold of the words loaded.  P * ceil(n /
 *                            128)^2 < 2^31
 *   DIT_STREAM_TOPK_ROWS     the top-k traffic of dit_subblock_route, in that
 *                            kernel's launch shape (one wave per row): `heads`
 *                            is n and rows = P * n (P <= 65535, n <= 4096).
 *                            Reads the first n fp32 words of each row of in0
 *                            [rows][row_bytes] (row_bytes >= 4 * n) and writes
 *                            out0 [rows][keep] int32 with keep = ceil(n / 4),
 *                            the kept count at sparsity 0.75.  With an all-zero
 *                            in0, word j of row r is (r * 65536 + j) mod 2^32;
 *                            otherwise that XOR a fold of the words loaded
 * Limits: rows < 2^24; row_bytes <= 2^25; SPLIT_ROWS and TWO_IN as for
 * dit_swiglu and dit_gated_residual on the same rows and widths.  Pointers
 * 16-byte aligned; no output may overlap an input (DIT_ERR_ARG); unused
 * pointers may be NULL.
 */
#define DIT_STREAM_READ 0
#define DIT_STREAM_WRITE 1
#define DIT_STREAM_SPLIT_ROWS 2
#define DIT_STREAM_TWO_IN 3
#define DIT_STREAM_ROW_GROUP 4 /* stream kinds 4 and 5 take this mapping from ABI version 4 */
#define DIT_STREAM_ROW_GROUP_2X2 5
#define DIT_STREAM_HEAD_MAJOR 6
#define DIT_STREAM_SCORE_TILES 7
#define DIT_STREAM_TOPK_ROWS 8
dit_status dit_stream_pattern(int32_t kind, const void *in0, const void *in1,
                              void *out0, void *out1, int64_t rows,
                              int64_t row_bytes, int64_t heads, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DIT_OPS_H */
