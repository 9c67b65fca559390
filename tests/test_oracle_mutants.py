"""Planted-mistake check of the oracle's pins (CPU only).

Each case below copies oracle/dit_oracle.c, plants one plausible mistake by a
textual edit (a dropped term, a wrong sign or index, a swapped operand, a wrong
normalisation), builds the copy with the same compiler flags into a temporary
directory, and runs every pin of tests/test_oracle_pins.py against it.  The
case passes when at least one pin fails.  The real oracle is never modified.
"""
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as pins

MUTANTS = {
    # AdaLN
    "adaln_unbiased_variance": ("double var = sq / (double)D;", "double var = sq / (double)(D - 1);"),
    "adaln_eps_outside_root": ("double denom = sqrt(var + eps);", "double denom = sqrt(var) + eps;"),
    "adaln_scale_without_one": ("ln * (1.0 + bf16_to_double(sc[i]))", "ln * bf16_to_double(sc[i])"),
    "adaln_shift_scale_swapped": ("const uint16_t *sh = shift + b * D;\n        const uint16_t *sc = scale + b * D;",
                                  "const uint16_t *sh = scale + b * D;\n        const uint16_t *sc = shift + b * D;"),
    "adaln_variance_not_centred": ("double d = bf16_to_double(xr[i]) - mean;", "double d = bf16_to_double(xr[i]);"),
    "adaln_sample_zero_vectors": ("const uint16_t *sh = shift + b * D;", "const uint16_t *sh = shift;"),
    "adaln_mean_not_subtracted": ("double ln = (bf16_to_double(xr[i]) - mean) / denom;",
                                  "double ln = bf16_to_double(xr[i]) / denom;"),
    # gated residual
    "residual_gate_on_x": ("bf16_to_double(x[base + i]) +\n                                bf16_to_double(g[i]) * bf16_to_double(y[base + i]);",
                           "bf16_to_double(g[i]) * bf16_to_double(x[base + i]) +\n                                bf16_to_double(y[base + i]);"),
    "residual_gate_sample_zero": ("const uint16_t *g = gate + b * D;", "const uint16_t *g = gate;"),
    "residual_minus": ("bf16_to_double(x[base + i]) +\n", "bf16_to_double(x[base + i]) -\n"),
    # SwiGLU
    "swiglu_halves_swapped": ("out[r * F + j] = av * logistic(av) * bf16_to_double(bh[j]);",
                              "out[r * F + j] = bf16_to_double(bh[j]) * logistic(bf16_to_double(bh[j])) * av;"),
    "swiglu_sigmoid_sign": ("return 1.0 / (1.0 + exp(-a));", "return 1.0 / (1.0 + exp(a));"),
    "swiglu_drops_a_factor": ("out[r * F + j] = av * logistic(av) * bf16_to_double(bh[j]);",
                              "out[r * F + j] = logistic(av) * bf16_to_double(bh[j]);"),
    "swiglu_negative_branch": ("return e / (1.0 + e);", "return 1.0 / (1.0 + e);"),
    "swiglu_second_half_offset": ("const uint16_t *bh = a + F;", "const uint16_t *bh = a + F - 1;"),
    # RMSNorm
    "rmsnorm_sum_not_mean": ("double denom = sqrt(sq / (double)n + eps);", "double denom = sqrt(sq + eps);"),
    "rmsnorm_no_weight": ("u[i] = v[i] / denom * w[i];", "u[i] = v[i] / denom;"),
    "rmsnorm_eps_outside_root": ("double denom = sqrt(sq / (double)n + eps);", "double denom = sqrt(sq / (double)n) + eps;"),
    # RoPE
    "rope_sin_sign": ("u[start + 2 * j] = u0 * c - u1 * s;", "u[start + 2 * j] = u0 * c + u1 * s;"),
    "rope_exponent_over_dh": ("pow(theta, -2.0 * j / (double)d)", "pow(theta, -2.0 * j / (double)Dh)"),
    "rope_exponent_j_not_2j": ("pow(theta, -2.0 * j / (double)d)", "pow(theta, -1.0 * j / (double)d)"),
    "rope_t_h_swapped": ("const int32_t coord[3] = {p_t, p_h, p_w};", "const int32_t coord[3] = {p_h, p_t, p_w};"),
    "rope_rotate_half_pairing": ("double u0 = u[start + 2 * j], u1 = u[start + 2 * j + 1];\n"
                                 "            u[start + 2 * j] = u0 * c - u1 * s;\n"
                                 "            u[start + 2 * j + 1] = u0 * s + u1 * c;",
                                 "double u0 = u[start + j], u1 = u[start + j + d / 2];\n"
                                 "            u[start + j] = u0 * c - u1 * s;\n"
                                 "            u[start + j + d / 2] = u0 * s + u1 * c;"),
    "rope_band_start_not_advanced": ("        start += d;\n    }\n    return ORACLE_OK;", "    }\n    return ORACLE_OK;"),
    # QK composition
    "qk_k_uses_wq": ("const double *w = which == 0 ? w_q : w_k;", "const double *w = w_q;"),
    "qk_position_of_first_token": ("const int32_t *p = pos + 3 * n;", "const int32_t *p = pos;"),
    "qk_rotate_before_norm_weight": ("status = dit_oracle_rmsnorm(v, w, u, Dh, eps);",
                                     "status = dit_oracle_rmsnorm(v, w, u, Dh, eps);\n"
                                     "                    for (int64_t i = 0; i < Dh; ++i) u[i] /= w[i];"),
    # positions
    "positions_h_w_swapped": ("pos[3 * n + 1] = (int32_t)h;\n                pos[3 * n + 2] = (int32_t)w;",
                              "pos[3 * n + 1] = (int32_t)w;\n                pos[3 * n + 2] = (int32_t)h;"),
    "positions_extra_at_zero": ("pos[3 * n + 0] = (int32_t)a;", "pos[3 * n + 0] = 0;"),
    # bf16 storage rounding
    "encode_ties_away": ("q = ldexp(nearbyint(ldexp(m, 8)), e - 8);", "q = ldexp(round(ldexp(m, 8)), e - 8);"),
    "encode_truncates": ("q = ldexp(nearbyint(ldexp(m, 8)), e - 8);", "q = ldexp(trunc(ldexp(m, 8)), e - 8);"),
    "encode_seven_bits": ("q = ldexp(nearbyint(ldexp(m, 8)), e - 8);", "q = ldexp(nearbyint(ldexp(m, 7)), e - 7);"),
    "encode_no_subnormal_ties": ("q = nearbyint(ldexp(mag, 133)) * ldexp(1.0, -133);",
                                 "q = ceil(ldexp(mag, 133)) * ldexp(1.0, -133);"),
    # fused gated residual + AdaLN
    "fused_normalises_input_x": ("stored[i] = dit_oracle_bf16_encode(x_out[i]);", "stored[i] = x[i];"),
    "fused_truncates_store": ("stored[i] = dit_oracle_bf16_encode(x_out[i]);",
                              "{ float f = (float)x_out[i]; uint32_t w; memcpy(&w, &f, 4); stored[i] = (uint16_t)(w >> 16); }"),
    # QK memory layouts
    "layout_head_major_wrong_order": ("                                              : ((b * H + h) * N + n) * Dh;",
                                      "                                              : ((n * H + h) * B + b) * Dh;"),
    "layout_ignores_stride": ("int64_t src = (b * N + n) * in_stride + h * Dh;", "int64_t src = (b * N + n) * H * Dh + h * Dh;"),
    "layout_k_uses_q": ("const uint16_t *in = which == 0 ? q : k;", "const uint16_t *in = q;"),
    # Cache-DiT residual change
    "change_den_of_r": ("den += fabs(c);", "den += fabs(a);"),
    "change_signed_difference": ("num += fabs(a - c);", "num += a - c;"),
    "change_sample_zero": ("double a = bf16_to_double(r[b * N * D + i]);", "double a = bf16_to_double(r[i]);"),
    "change_zero_den_ratio": ("(num > 0.0 ? INFINITY : 0.0)", "0.0"),
    # SubBlock routing
    "pool_divides_by_block": ("o[d] = sum / (double)(last - first);", "o[d] = sum / (double)block;"),
    "pool_drops_short_block": ("const int64_t nb = (N + block - 1) / block;", "const int64_t nb = N / block;"),
    "pool_ignores_sample": ("sum += bf16_to_double(x[((b * N + n) * H + h) * Dh + d]);",
                            "sum += bf16_to_double(x[(n * H + h) * Dh + d]);"),
    "pool_ignores_head": ("sum += bf16_to_double(x[((b * N + n) * H + h) * Dh + d]);",
                          "sum += bf16_to_double(x[((b * N + n) * H) * Dh + d]);"),
    "scores_unrounded": ("kr[e] = bf16_to_double(dit_oracle_bf16_encode(kp[e]));", "kr[e] = kp[e];"),
    "scores_transposed": ("s[(bh * nq + i) * nk + j] = acc;", "s[(bh * nk + j) * nq + i] = acc;"),
    "scores_k_with_q": ("const double *kj = kr + (bh * nk + j) * Dh;", "const double *kj = qr + (bh * nk + j) * Dh;"),
    "keep_rounds_drop_up": ("int64_t keep = nb - (int64_t)floor(sparsity * (double)nb);",
                            "int64_t keep = nb - (int64_t)ceil(sparsity * (double)nb);"),
    "keep_is_sparsity_share": ("int64_t keep = nb - (int64_t)floor(sparsity * (double)nb);",
                               "int64_t keep = (int64_t)floor(sparsity * (double)nb);"),
    "topk_smallest": ("return a->score > b->score ? -1 : 1;", "return a->score < b->score ? -1 : 1;"),
    "topk_ties_high_index": ("return a->index < b->index ? -1 : (a->index > b->index);",
                             "return a->index > b->index ? -1 : (a->index < b->index);"),
    "topk_score_order": ("        int64_t at = 0;\n        for (int64_t j = 0; j < nb; ++j)\n"
                         "            if (kept[j])\n                idx[r * keep + at++] = (int32_t)j;",
                         "        for (int64_t t = 0; t < keep; ++t)\n"
                         "            idx[r * keep + t] = (int32_t)row[t].index;"),
    # QK + block means of the stored outputs
    "qk_pool_unrounded_store": ("stored[e] = dit_oracle_bf16_encode(u[e]);",
                                "{ float f = (float)u[e]; uint32_t w; memcpy(&w, &f, 4); stored[e] = (uint16_t)(w >> 16); }"),
    "qk_pool_k_into_q": ("status = dit_oracle_subblock_pool(stored, which == 0 ? q_pooled : k_pooled, B, N, H, Dh,",
                         "status = dit_oracle_subblock_pool(stored, q_pooled, B, N, H, Dh,"),
    # bf16 decode
    "decode_wrong_shift": ("uint32_t word = (uint32_t)bits << 16;", "uint32_t word = (uint32_t)bits << 15;"),
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE, encoding="utf-8") as fh:
        return fh.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(source, tmp_path, name):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for {name} not found exactly once"
    src = tmp_path / f"{name}.c"
    src.write_text(source.replace(old, new), encoding="utf-8")
    lib_path = str(tmp_path / f"lib{name}.so")
    subprocess.run(["gcc", *oracle.CFLAGS, "-o", lib_path, str(src), "-lm"], check=True)
    lib = oracle.load(lib_path)
    failed = []
    for pin_name, pin in pins.PINS.items():
        try:
            pin(lib)
        except Exception:  # any failure of a pin counts as catching the mistake
            failed.append(pin_name)
    assert failed, f"planted mistake {name} passed every pin"
    os.remove(lib_path)
