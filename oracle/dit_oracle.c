/*
 * dit_oracle.c -- plain fp64 CPU oracle for the fused non-GEMM operator chain
 * of a video+audio DiT denoising block.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  It shares no
 * code, header, table or helper with the HIP kernels, and the product path
 * never links it.
 *
 * What is computed, and why this is the reference:
 *   - The SGLang benchmark summary "8xH200 上的 MiniMax-H3: 无损加速 1.95 倍 ..."
 *     (xhh.club), section Q&A (the question on which operations the fused
 *     kernels cover), names the four fused operations: AdaLN modulation, gated
 *     residual, SwiGLU activation, and per-head QK RMSNorm fused with 3D RoPE.
 *   - "SGLang acelera video do MiniMax-H3 em ate 6,2x em GPUs H200"
 *     (stamatios.com), section "Resultado principal", states that the fused
 *     kernels cut memory traffic, intermediates and launches while leaving the
 *     arithmetic unchanged, and that video and audio tokens share one packed
 *     DiT stack.
 *   - The same stamatios.com summary, "De onde vêm os ganhos" and "Resultado
 *     principal", and the xhh.club Q&A on the sparsity parameter describe the
 *     SubBlock attention router: 64-token blocks, scored by estimated
 *     contribution, a fraction of the key blocks kept per query block.  The
 *     routing functions at the end compute that selection step by step.
 *   So each function below is the plain, unfused definition of its operation,
 *   evaluated in double precision with no blocking or reordering.  Inputs are
 *   raw bf16 bit patterns (decoded exactly to double); outputs are unrounded
 *   doubles.  Formulas the pages only name are the standard definitions of
 *   those operations; every reading taken where the pages are silent is listed
 *   in the project's design notes and repeated at the function it affects.
 *
 * Reductions are the textbook two-pass mean-then-variance in serial order.
 * Build with a plain C compiler, -O2, no -ffast-math, -ffp-contract=off.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG (-1)

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static double bf16_to_double(uint16_t bits)
{
    uint32_t word = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &word, sizeof f);
    return (double)f;
}

/* Exported so tests can check the decoding against known bit patterns. */
double dit_oracle_bf16_decode(uint16_t bits) { return bf16_to_double(bits); }

/*
 * Round a double to the nearest bf16 (8 significant bits, ties to even, the
 * IEEE default), returning its bit pattern.  Used where an operation's
 * definition stores an intermediate tensor in bf16.  Normal numbers keep 8
 * bits below the leading one; below 2^-126 the spacing is fixed at 2^-133
 * (bf16 subnormals); magnitudes that round past the largest finite bf16
 * become infinity.  NaN maps to the canonical quiet NaN.
 */
uint16_t dit_oracle_bf16_encode(double v)
{
    if (isnan(v))
        return 0x7FC0;
    const double max_finite = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
    double mag = fabs(v), q;
    int e;
    if (mag < ldexp(1.0, -126)) {
        q = nearbyint(ldexp(mag, 133)) * ldexp(1.0, -133); /* ties to even */
    } else {
        double m = frexp(mag, &e); /* mag = m * 2^e, 0.5 <= m < 1 */
        q = ldexp(nearbyint(ldexp(m, 8)), e - 8);
    }
    float f = q > max_finite ? INFINITY : (float)q; /* exact: q has <= 8 significant bits */
    uint32_t word;
    memcpy(&word, &f, sizeof word);
    uint16_t bits = (uint16_t)(word >> 16);
    return signbit(v) ? (uint16_t)(bits | 0x8000) : bits;
}

/*
 * Packed token positions.
 * Cited: "SGLang acelera video do MiniMax-H3 ..." (stamatios.com), section
 * "Resultado principal": video and audio tokens run through one packed DiT
 * stack.  "3D RoPE" in the xhh.club Q&A means each video token carries its
 * (t, h, w) latent-grid coordinate.
 * Readings: the video grid is enumerated in row-major (t, h, w) order with
 * integer coordinates from 0; the n_extra tokens appended after it carry a
 * temporal-only coordinate equal to their own index a = 0 .. n_extra-1, with
 * h = w = 0.
 * pos is [T*Hg*Wg + n_extra][3] int32.  Returns the token count written.
 */
int64_t dit_oracle_packed_positions(int32_t *pos, int64_t T, int64_t Hg,
                                    int64_t Wg, int64_t n_extra)
{
    if (!pos || T < 0 || Hg < 0 || Wg < 0 || n_extra < 0)
        return ORACLE_BAD_ARG;
    int64_t n = 0;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t h = 0; h < Hg; ++h)
            for (int64_t w = 0; w < Wg; ++w) {
                pos[3 * n + 0] = (int32_t)t;
                pos[3 * n + 1] = (int32_t)h;
                pos[3 * n + 2] = (int32_t)w;
                ++n;
            }
    for (int64_t a = 0; a < n_extra; ++a) {
        pos[3 * n + 0] = (int32_t)a;
        pos[3 * n + 1] = 0;
        pos[3 * n + 2] = 0;
        ++n;
    }
    return n;
}

/*
 * AdaLN modulation.
 * Cited: xhh.club Q&A (fused-kernel answer) names "AdaLN modulation".
 * Definition: LayerNorm over the hidden dimension with no affine parameters,
 * then y = LN(x) * (1 + scale) + shift.
 * Readings: biased variance (divide by D); eps added to the variance inside
 * the square root; shift/scale are per sample, [B][D], broadcast over all N
 * tokens of that sample (extra tokens included).
 * x, y: [B][N][D]; shift, scale: [B][D].
 */
int dit_oracle_adaln_modulate(const uint16_t *x, const uint16_t *shift,
                              const uint16_t *scale, double *y, int64_t B,
                              int64_t N, int64_t D, double eps)
{
    if (!x || !shift || !scale || !y || B < 0 || N < 0 || D <= 0 || !(eps > 0))
        return ORACLE_BAD_ARG;
    for (int64_t b = 0; b < B; ++b) {
        const uint16_t *sh = shift + b * D;
        const uint16_t *sc = scale + b * D;
        for (int64_t n = 0; n < N; ++n) {
            const uint16_t *xr = x + (b * N + n) * D;
            double *yr = y + (b * N + n) * D;

            double sum = 0.0;
            for (int64_t i = 0; i < D; ++i)
                sum += bf16_to_double(xr[i]);
            double mean = sum / (double)D;

            double sq = 0.0;
            for (int64_t i = 0; i < D; ++i) {
                double d = bf16_to_double(xr[i]) - mean;
                sq += d * d;
            }
            double var = sq / (double)D;
            double denom = sqrt(var + eps);

            for (int64_t i = 0; i < D; ++i) {
                double ln = (bf16_to_double(xr[i]) - mean) / denom;
                yr[i] = ln * (1.0 + bf16_to_double(sc[i])) + bf16_to_double(sh[i]);
            }
        }
    }
    return ORACLE_OK;
}

/*
 * Gated residual.
 * Cited: xhh.club Q&A (fused-kernel answer) names the gated residual.
 * Definition: out = x + gate * y, elementwise, with gate per sample [B][D]
 * broadcast over the N tokens.  Reading: the gate is used raw (no sigmoid or
 * tanh).
 * x, y, out: [B][N][D]; gate: [B][D].
 */
int dit_oracle_gated_residual(const uint16_t *x, const uint16_t *y,
                              const uint16_t *gate, double *out, int64_t B,
                              int64_t N, int64_t D)
{
    if (!x || !y || !gate || !out || B < 0 || N < 0 || D <= 0)
        return ORACLE_BAD_ARG;
    for (int64_t b = 0; b < B; ++b) {
        const uint16_t *g = gate + b * D;
        for (int64_t n = 0; n < N; ++n) {
            int64_t base = (b * N + n) * D;
            for (int64_t i = 0; i < D; ++i)
                out[base + i] = bf16_to_double(x[base + i]) +
                                bf16_to_double(g[i]) * bf16_to_double(y[base + i]);
        }
    }
    return ORACLE_OK;
}

/* Logistic function 1/(1+e^-a), evaluated without overflow for either sign. */
static double logistic(double a)
{
    if (a >= 0.0)
        return 1.0 / (1.0 + exp(-a));
    double e = exp(a);
    return e / (1.0 + e);
}

/*
 * SwiGLU activation.
 * Cited: xhh.club Q&A (fused-kernel answer) and stamatios.com "De onde vem
 * os ganhos" both list SwiGLU among the fused kernels.
 * Definition: out = silu(a) * b with silu(a) = a * logistic(a) (beta = 1).
 * Reading: each input row of width 2F is two contiguous halves [a | b]; the
 * first half is the one passed through silu.
 * in: [M][2F]; out: [M][F].
 */
int dit_oracle_swiglu(const uint16_t *in, double *out, int64_t M, int64_t F)
{
    if (!in || !out || M < 0 || F <= 0)
        return ORACLE_BAD_ARG;
    for (int64_t r = 0; r < M; ++r) {
        const uint16_t *a = in + r * 2 * F;
        const uint16_t *bh = a + F;
        for (int64_t j = 0; j < F; ++j) {
            double av = bf16_to_double(a[j]);
            out[r * F + j] = av * logistic(av) * bf16_to_double(bh[j]);
        }
    }
    return ORACLE_OK;
}

/*
 * RMSNorm of one head vector: u = v / sqrt(mean(v^2) + eps) * w.
 * Cited: xhh.club Q&A names "QK RMSNorm" (per head, fused with 3D RoPE).
 * Reading: the mean runs over the head's Dh channels; w is a [Dh] weight.
 */
int dit_oracle_rmsnorm(const double *v, const double *w, double *u, int64_t n,
                       double eps)
{
    if (!v || !w || !u || n <= 0 || !(eps > 0))
        return ORACLE_BAD_ARG;
    double sq = 0.0;
    for (int64_t i = 0; i < n; ++i)
        sq += v[i] * v[i];
    double denom = sqrt(sq / (double)n + eps);
    for (int64_t i = 0; i < n; ++i)
        u[i] = v[i] / denom * w[i];
    return ORACLE_OK;
}

/*
 * 3D rotary embedding of one head vector, in place.
 * Cited: xhh.club Q&A ("QK RMSNorm fused with 3D RoPE").
 * Readings: the Dh channels are three contiguous bands in the order t, h, w
 * with widths d_t, d_h, d_w (each even, summing to Dh).  Inside a band of
 * width d driven by integer coordinate p, the channel pair (2j, 2j+1),
 * j = 0 .. d/2-1, is rotated by the angle p * theta^(-2j/d) (exponent
 * normalised by the band's own width), counter-clockwise:
 *   (u0, u1) -> (u0 cos f - u1 sin f, u0 sin f + u1 cos f).
 */
int dit_oracle_rope3d(double *u, int64_t Dh, int32_t d_t, int32_t d_h,
                      int32_t d_w, int32_t p_t, int32_t p_h, int32_t p_w,
                      double theta)
{
    if (!u || d_t < 0 || d_h < 0 || d_w < 0 || (d_t | d_h | d_w) & 1 ||
        (int64_t)d_t + d_h + d_w != Dh || !(theta > 0))
        return ORACLE_BAD_ARG;
    const int32_t width[3] = {d_t, d_h, d_w};
    const int32_t coord[3] = {p_t, p_h, p_w};
    int64_t start = 0;
    for (int band = 0; band < 3; ++band) {
        int32_t d = width[band];
        for (int32_t j = 0; j < d / 2; ++j) {
            double angle = (double)coord[band] * pow(theta, -2.0 * j / (double)d);
            double c = cos(angle), s = sin(angle);
            double u0 = u[start + 2 * j], u1 = u[start + 2 * j + 1];
            u[start + 2 * j] = u0 * c - u1 * s;
            u[start + 2 * j + 1] = u0 * s + u1 * c;
        }
        start += d;
    }
    return ORACLE_OK;
}

/*
 * QK RMSNorm followed by 3D RoPE, for every (sample, token, head) of q and of
 * k separately (q uses wq, k uses wk).  Order: normalise, multiply by the
 * weight, rotate.
 * q, k, q_out, k_out: [B][N][H][Dh]; wq, wk: [Dh]; pos: [N][3] shared by all
 * samples of the batch.
 */
int dit_oracle_qk_rmsnorm_rope3d(const uint16_t *q, const uint16_t *k,
                                 const uint16_t *wq, const uint16_t *wk,
                                 const int32_t *pos, double *q_out,
                                 double *k_out, int64_t B, int64_t N, int64_t H,
                                 int64_t Dh, int32_t d_t, int32_t d_h,
                                 int32_t d_w, double theta, double eps)
{
    if (!q || !k || !wq || !wk || !pos || !q_out || !k_out || B < 0 || N < 0 ||
        H <= 0 || Dh <= 0 || !(eps > 0) || !(theta > 0))
        return ORACLE_BAD_ARG;
    if ((d_t | d_h | d_w) & 1 || d_t < 0 || d_h < 0 || d_w < 0 ||
        (int64_t)d_t + d_h + d_w != Dh)
        return ORACLE_BAD_ARG;

    double *w_q = malloc(sizeof(double) * (size_t)Dh);
    double *w_k = malloc(sizeof(double) * (size_t)Dh);
    double *v = malloc(sizeof(double) * (size_t)Dh);
    double *u = malloc(sizeof(double) * (size_t)Dh);
    if (!w_q || !w_k || !v || !u) {
        free(w_q); free(w_k); free(v); free(u);
        return ORACLE_BAD_ARG;
    }
    for (int64_t i = 0; i < Dh; ++i) {
        w_q[i] = bf16_to_double(wq[i]);
        w_k[i] = bf16_to_double(wk[i]);
    }

    int status = ORACLE_OK;
    for (int64_t b = 0; b < B && status == ORACLE_OK; ++b)
        for (int64_t n = 0; n < N && status == ORACLE_OK; ++n) {
            const int32_t *p = pos + 3 * n;
            for (int64_t h = 0; h < H && status == ORACLE_OK; ++h) {
                int64_t base = ((b * N + n) * H + h) * Dh;
                for (int which = 0; which < 2; ++which) {
                    const uint16_t *src = which == 0 ? q : k;
                    double *dst = which == 0 ? q_out : k_out;
                    const double *w = which == 0 ? w_q : w_k;
                    for (int64_t i = 0; i < Dh; ++i)
                        v[i] = bf16_to_double(src[base + i]);
                    status = dit_oracle_rmsnorm(v, w, u, Dh, eps);
                    if (status == ORACLE_OK)
                        status = dit_oracle_rope3d(u, Dh, d_t, d_h, d_w, p[0],
                                                   p[1], p[2], theta);
                    if (status != ORACLE_OK)
                        break;
                    for (int64_t i = 0; i < Dh; ++i)
                        dst[base + i] = u[i];
                }
            }
        }
    free(w_q); free(w_k); free(v); free(u);
    return status;
}

/*
 * Gated residual fused with the AdaLN modulation that follows it.
 * Cited: xhh.club Q&A (fused-kernel answer) names both operations, and the
 * Sol-H3 abstract describes searching over such kernel fusions; the
 * stamatios.com summary ("Resultado principal") says fusion leaves the
 * arithmetic unchanged.  So this is the composition of the two unfused
 * operations exactly as a pipeline would run them:
 *   x_out = x + gate[b] * y                      (returned unrounded)
 *   x_bf  = x_out stored as bf16 (round to nearest even)
 *   z     = LN(x_bf) * (1 + scale[b]) + shift[b] (LN as in adaln_modulate)
 * Reading: the normalisation sees the bf16-stored residual, as the unfused
 * AdaLN reads it back from memory.
 * x, y, x_out, z: [B][N][D]; gate, shift, scale: [B][D].
 */
int dit_oracle_gated_residual_adaln(const uint16_t *x, const uint16_t *y,
                                    const uint16_t *gate, const uint16_t *shift,
                                    const uint16_t *scale, double *x_out,
                                    double *z, int64_t B, int64_t N, int64_t D,
                                    double eps)
{
    if (!x || !y || !gate || !shift || !scale || !x_out || !z || B < 0 ||
        N < 0 || D <= 0 || !(eps > 0))
        return ORACLE_BAD_ARG;
    int status = dit_oracle_gated_residual(x, y, gate, x_out, B, N, D);
    if (status != ORACLE_OK)
        return status;
    size_t count = (size_t)(B * N * D);
    uint16_t *stored = malloc(sizeof(uint16_t) * (count ? count : 1));
    if (!stored)
        return ORACLE_BAD_ARG;
    for (size_t i = 0; i < count; ++i)
        stored[i] = dit_oracle_bf16_encode(x_out[i]);
    status = dit_oracle_adaln_modulate(stored, shift, scale, z, B, N, D, eps);
    free(stored);
    return status;
}

/*
 * QK RMSNorm + 3D RoPE with the memory layouts of a fused QKV projection and
 * of an attention kernel's input.
 * Cited: the Sol-H3 abstract describes searching over memory layouts as well
 * as fusions; the arithmetic is that of dit_oracle_qk_rmsnorm_rope3d.
 * Layouts (element offsets):
 *   input  q, k: token (b, n), head h, channel i at ((b*N + n) * in_stride + h*Dh + i),
 *          in_stride >= H*Dh (3*H*Dh with q, k, v interleaved per token);
 *   output out_layout 0: ((b*N + n) * H + h) * Dh + i      (token-major)
 *          out_layout 1: ((b*H + h) * N + n) * Dh + i      (head-major).
 */
int dit_oracle_qk_rmsnorm_rope3d_layout(const uint16_t *q, const uint16_t *k,
                                        const uint16_t *wq, const uint16_t *wk,
                                        const int32_t *pos, double *q_out,
                                        double *k_out, int64_t B, int64_t N,
                                        int64_t H, int64_t Dh, int64_t in_stride,
                                        int32_t out_layout, int32_t d_t,
                                        int32_t d_h, int32_t d_w, double theta,
                                        double eps)
{
    if (!q || !k || !wq || !wk || !pos || !q_out || !k_out || B < 0 || N < 0 ||
        H <= 0 || Dh <= 0 || in_stride < H * Dh || (out_layout != 0 && out_layout != 1) ||
        !(eps > 0) || !(theta > 0))
        return ORACLE_BAD_ARG;
    if ((d_t | d_h | d_w) & 1 || d_t < 0 || d_h < 0 || d_w < 0 ||
        (int64_t)d_t + d_h + d_w != Dh)
        return ORACLE_BAD_ARG;

    double *w_q = malloc(sizeof(double) * (size_t)Dh);
    double *w_k = malloc(sizeof(double) * (size_t)Dh);
    double *v = malloc(sizeof(double) * (size_t)Dh);
    double *u = malloc(sizeof(double) * (size_t)Dh);
    if (!w_q || !w_k || !v || !u) {
        free(w_q); free(w_k); free(v); free(u);
        return ORACLE_BAD_ARG;
    }
    for (int64_t i = 0; i < Dh; ++i) {
        w_q[i] = bf16_to_double(wq[i]);
        w_k[i] = bf16_to_double(wk[i]);
    }
    int status = ORACLE_OK;
    for (int64_t b = 0; b < B && status == ORACLE_OK; ++b)
        for (int64_t n = 0; n < N && status == ORACLE_OK; ++n)
            for (int64_t h = 0; h < H && status == ORACLE_OK; ++h) {
                int64_t src = (b * N + n) * in_stride + h * Dh;
                int64_t dst = out_layout == 0 ? ((b * N + n) * H + h) * Dh
                                              : ((b * H + h) * N + n) * Dh;
                for (int which = 0; which < 2 && status == ORACLE_OK; ++which) {
                    const uint16_t *in = which == 0 ? q : k;
                    double *out = which == 0 ? q_out : k_out;
                    for (int64_t i = 0; i < Dh; ++i)
                        v[i] = bf16_to_double(in[src + i]);
                    status = dit_oracle_rmsnorm(v, which == 0 ? w_q : w_k, u, Dh, eps);
                    if (status == ORACLE_OK)
                        status = dit_oracle_rope3d(u, Dh, d_t, d_h, d_w, pos[3 * n],
                                                   pos[3 * n + 1], pos[3 * n + 2], theta);
                    for (int64_t i = 0; i < Dh && status == ORACLE_OK; ++i)
                        out[dst + i] = u[i];
                }
            }
    free(w_q); free(w_k); free(v); free(u);
    return status;
}

/*
 * Cache-DiT residual-change statistic.
 * Cited: "8×H200 上的 MiniMax-H3…" (xhh.club), Q&A on how Cache-DiT reuses
 * computation: after warm-up steps the boundary blocks are evaluated and their
 * normalised residual change against the cached state decides reuse; and
 * "SGLang acelera vídeo do MiniMax-H3…" (stamatios.com), "Resultado
 * principal": the packed video+audio stack gets one joint decision.
 * Reading: the normalised change is the relative L1 distance over every
 * token (video and audio alike) and channel of a sample:
 *   num_b = sum |r - r_cached|,  den_b = sum |r_cached|,  ratio_b = num_b / den_b
 * with ratio 0 when both sums are 0 and +inf when only den is 0.
 * r, r_cached: [B][N][D]; out: [B][3] = (num, den, ratio).
 */
int dit_oracle_residual_change(const uint16_t *r, const uint16_t *r_cached,
                               double *out, int64_t B, int64_t N, int64_t D)
{
    if (!r || !r_cached || !out || B < 0 || N < 0 || D <= 0)
        return ORACLE_BAD_ARG;
    for (int64_t b = 0; b < B; ++b) {
        double num = 0.0, den = 0.0;
        for (int64_t i = 0; i < N * D; ++i) {
            double a = bf16_to_double(r[b * N * D + i]);
            double c = bf16_to_double(r_cached[b * N * D + i]);
            num += fabs(a - c);
            den += fabs(c);
        }
        out[3 * b + 0] = num;
        out[3 * b + 1] = den;
        out[3 * b + 2] = den > 0.0 ? num / den : (num > 0.0 ? INFINITY : 0.0);
    }
    return ORACLE_OK;
}


/*
 * SubBlock routing, step 1: block pooling.
 * Cited: "SGLang acelera vídeo do MiniMax-H3…" (stamatios.com), "De onde vêm
 * os ganhos": SubBlock attention cuts the sequence into 64-token blocks and
 * routes over the key blocks; "Resultado principal": the blocks dropped are
 * those whose estimated contribution is smaller.
 * Reading: a block is summarised by the mean of its tokens' head vectors (q or
 * k after RMSNorm and RoPE).  Blocks never span two samples; the last block of
 * a sample may hold fewer tokens and averages only those.
 * x: [B][N][H][Dh] bf16 bits (token-major); out: [B][H][nb][Dh] with
 * nb = ceil(N / block).
 */
int dit_oracle_subblock_pool(const uint16_t *x, double *out, int64_t B, int64_t N,
                             int64_t H, int64_t Dh, int64_t block)
{
    if (!x || !out || B < 0 || N < 0 || H <= 0 || Dh <= 0 || block <= 0)
        return ORACLE_BAD_ARG;
    const int64_t nb = (N + block - 1) / block;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t i = 0; i < nb; ++i) {
                const int64_t first = i * block;
                const int64_t last = first + block < N ? first + block : N;
                double *o = out + ((b * H + h) * nb + i) * Dh;
                for (int64_t d = 0; d < Dh; ++d) {
                    double sum = 0.0;
                    for (int64_t n = first; n < last; ++n)
                        sum += bf16_to_double(x[((b * N + n) * H + h) * Dh + d]);
                    o[d] = sum / (double)(last - first);
                }
            }
    return ORACLE_OK;
}

/*
 * SubBlock routing, step 2: block scores.
 * Cited: as for the pooling (stamatios.com, "De onde vêm os ganhos" and
 * "Resultado principal").
 * Reading: the estimated contribution of key block j to query block i is the
 * dot product of their pooled means, per sample and head, with no 1/sqrt(Dh)
 * factor (a positive scale leaves the order unchanged).  The means enter the
 * product rounded to bf16, the operand precision of the attention path that
 * consumes the routing; the products are exact and summed in double.
 *   s[b][h][i][j] = sum_d bf16(qp[b][h][i][d]) * bf16(kp[b][h][j][d])
 * qp: [B][H][nq][Dh] (any nq query blocks), kp: [B][H][nk][Dh],
 * s: [B][H][nq][nk].
 */
int dit_oracle_subblock_scores(const double *qp, const double *kp, double *s, int64_t B,
                               int64_t H, int64_t nq, int64_t nk, int64_t Dh)
{
    if (!qp || !kp || !s || B < 0 || H <= 0 || nq < 0 || nk < 0 || Dh <= 0)
        return ORACLE_BAD_ARG;
    const int64_t nqe = B * H * nq * Dh, nke = B * H * nk * Dh;
    double *qr = malloc(sizeof(double) * (size_t)(nqe > 0 ? nqe : 1));
    double *kr = malloc(sizeof(double) * (size_t)(nke > 0 ? nke : 1));
    if (!qr || !kr) {
        free(qr); free(kr);
        return ORACLE_BAD_ARG;
    }
    for (int64_t e = 0; e < nqe; ++e)
        qr[e] = bf16_to_double(dit_oracle_bf16_encode(qp[e]));
    for (int64_t e = 0; e < nke; ++e)
        kr[e] = bf16_to_double(dit_oracle_bf16_encode(kp[e]));
    for (int64_t bh = 0; bh < B * H; ++bh)
        for (int64_t i = 0; i < nq; ++i)
            for (int64_t j = 0; j < nk; ++j) {
                const double *qi = qr + (bh * nq + i) * Dh;
                const double *kj = kr + (bh * nk + j) * Dh;
                double acc = 0.0;
                for (int64_t d = 0; d < Dh; ++d)
                    acc += qi[d] * kj[d];
                s[(bh * nq + i) * nk + j] = acc;
            }
    free(qr); free(kr);
    return ORACLE_OK;
}

/*
 * SubBlock routing: key blocks kept per query block.
 * Cited: "8×H200 上的 MiniMax-H3…" (xhh.club), Q&A on the sparsity parameter:
 * sparsity is the fraction of key blocks that may be dropped, so 0.75 keeps
 * about a quarter of them.
 * Reading: floor(sparsity * nb) blocks are dropped and the rest kept, with at
 * least one kept; sparsity must lie in [0, 1).  Returns -1 on bad arguments.
 */
int64_t dit_oracle_subblock_keep(int64_t nb, double sparsity)
{
    if (nb < 0 || !(sparsity >= 0.0) || !(sparsity < 1.0))
        return -1;
    if (nb == 0)
        return 0;
    int64_t keep = nb - (int64_t)floor(sparsity * (double)nb);
    return keep < 1 ? 1 : keep;
}

struct scored_block {
    double score;
    int64_t index;
};

/* Larger score first; equal scores lower block index first. */
static int by_score_then_index(const void *pa, const void *pb)
{
    const struct scored_block *a = pa, *b = pb;
    if (a->score != b->score)
        return a->score > b->score ? -1 : 1;
    return a->index < b->index ? -1 : (a->index > b->index);
}

/*
 * SubBlock routing, step 3: the kept key blocks.
 * Cited: stamatios.com, "Resultado principal" (blocks of smaller estimated
 * contribution are dropped) and "De onde vêm os ganhos" (routing keeps part of
 * the key blocks).
 * Reading: each query block keeps the `keep` key blocks of largest score;
 * among equal scores the lower block index is kept.  The kept indices are
 * listed in ascending block order.  Scores must be finite.
 * s: [B][H][nq][nb] (nq query blocks' rows over nb key blocks);
 * idx: [B][H][nq][keep] int32.
 */
int dit_oracle_subblock_topk(const double *s, int32_t *idx, int64_t B, int64_t H, int64_t nq,
                             int64_t nb, int64_t keep)
{
    if (!s || !idx || B < 0 || H <= 0 || nq < 0 || nb < 0 || keep < 0 || keep > nb)
        return ORACLE_BAD_ARG;
    if (nb == 0)
        return ORACLE_OK;
    struct scored_block *row = malloc(sizeof(*row) * (size_t)nb);
    unsigned char *kept = malloc((size_t)nb);
    if (!row || !kept) {
        free(row); free(kept);
        return ORACLE_BAD_ARG;
    }
    int status = ORACLE_OK;
    for (int64_t r = 0; r < B * H * nq && status == ORACLE_OK; ++r) {
        for (int64_t j = 0; j < nb; ++j) {
            row[j].score = s[r * nb + j];
            row[j].index = j;
            if (!isfinite(row[j].score))
                status = ORACLE_BAD_ARG;
        }
        if (status != ORACLE_OK)
            break;
        qsort(row, (size_t)nb, sizeof(*row), by_score_then_index);
        memset(kept, 0, (size_t)nb);
        for (int64_t t = 0; t < keep; ++t)
            kept[row[t].index] = 1;
        int64_t at = 0;
        for (int64_t j = 0; j < nb; ++j)
            if (kept[j])
                idx[r * keep + at++] = (int32_t)j;
    }
    free(row); free(kept);
    return status;
}

/*
 * QK RMSNorm + 3D RoPE with the SubBlock block means of its outputs.
 * Cited: the xhh.club Q&A (QK RMSNorm fused with 3D RoPE) and the
 * stamatios.com summary, "De onde vêm os ganhos" (SubBlock routing over
 * 64-token blocks); the Sol-H3 abstract describes searching over such kernel
 * fusions.
 * Reading: the routing pools q' and k' as stored, i.e. rounded to bf16, as it
 * does when it reads them back from memory; so this is the QK op, one bf16
 * rounding of each output, then dit_oracle_subblock_pool.
 * q, k: [B][N][H][Dh] bf16 bits; q_out, k_out: [B][N][H][Dh] unrounded;
 * q_pooled, k_pooled: [B][H][nb][Dh], nb = ceil(N / block).
 */
int dit_oracle_qk_rmsnorm_rope3d_pool(const uint16_t *q, const uint16_t *k,
                                      const uint16_t *wq, const uint16_t *wk,
                                      const int32_t *pos, double *q_out, double *k_out,
                                      double *q_pooled, double *k_pooled, int64_t B,
                                      int64_t N, int64_t H, int64_t Dh, int32_t d_t,
                                      int32_t d_h, int32_t d_w, double theta, double eps,
                                      int64_t block)
{
    if (!q_pooled || !k_pooled || block <= 0)
        return ORACLE_BAD_ARG;
    int status = dit_oracle_qk_rmsnorm_rope3d(q, k, wq, wk, pos, q_out, k_out, B, N, H, Dh,
                                              d_t, d_h, d_w, theta, eps);
    if (status != ORACLE_OK)
        return status;
    const int64_t n_el = B * N * H * Dh;
    uint16_t *stored = malloc(sizeof(uint16_t) * (size_t)(n_el > 0 ? n_el : 1));
    if (!stored)
        return ORACLE_BAD_ARG;
    for (int which = 0; which < 2 && status == ORACLE_OK; ++which) {
        const double *u = which == 0 ? q_out : k_out;
        for (int64_t e = 0; e < n_el; ++e)
            stored[e] = dit_oracle_bf16_encode(u[e]);
        status = dit_oracle_subblock_pool(stored, which == 0 ? q_pooled : k_pooled, B, N, H, Dh,
                                          block);
    }
    free(stored);
    return status;
}
