"""Pins of the fp64 oracle to facts it does not compute itself.

Each pin checks the oracle against one of: a closed-form hand case from
tests/golden/, a special case that reduces to a library routine (torch fp64),
an invariant of the operation, or brute force on a tiny input.  They are chosen
so that a dropped term, a wrong sign or index, or a swapped operand in any
oracle function fails at least one of them; tests/test_oracle_mutants.py plants
such mistakes in copies of the oracle and checks exactly that.

Every pin is a function ``pin_*(lib)`` taking the loaded oracle library, so the
same pins run against the real oracle (the tests at the bottom) and against the
planted-mistake builds.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import oracle
from golden_io import cases, evaluate, values
from synthetic_inputs import bits, from_float

REL = 1e-12
BANDS = (16, 24, 24)


def b16(values_, shape=None):
    t = from_float(values_)
    return bits(t.reshape(shape) if shape is not None else t)


def close(a, b, rel=REL, abs_=1e-300):
    return np.allclose(np.asarray(a, np.float64), np.asarray(b, np.float64), rtol=rel, atol=abs_)


def rand_bf16(shape, seed, scale=1.0, loc=0.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale + loc).to(torch.bfloat16)


def f64(t):
    return t.to(torch.float64)


# --------------------------------------------------------------------------- bf16 decode

def pin_bf16_decode(lib):
    for pattern, value in [(0x3F80, 1.0), (0xC000, -2.0), (0x0000, 0.0), (0x4049, 3.140625),
                           (0x7F7F, 3.3895313892515355e38), (0x0001, 2.0 ** -133), (0x3C00, 2.0 ** -7)]:
        assert oracle.bf16_decode(pattern, lib=lib) == value, hex(pattern)
    assert math.copysign(1.0, oracle.bf16_decode(0x8000, lib=lib)) == -1.0


# --------------------------------------------------------------------------- positions

def pin_positions_hand_cases(lib):
    for case in cases("positions_hand.txt"):
        T, Hg, Wg = (int(v) for v in case["grid"])
        extra = int(case["extra"][0])
        n = int(case["n"][0])
        pos = oracle.packed_positions(T, Hg, Wg, extra, lib=lib)
        assert pos.shape == (T * Hg * Wg + extra, 3)
        assert tuple(pos[n]) == tuple(int(v) for v in case["pos"]), case


def pin_positions_brute_force(lib):
    for (T, Hg, Wg), extra in [((2, 4, 4), 0), ((3, 5, 7), 11), ((1, 1, 1), 0), ((4, 1, 3), 2), ((0, 0, 0), 5)]:
        pos = oracle.packed_positions(T, Hg, Wg, extra, lib=lib)
        nv = T * Hg * Wg
        seen = set()
        for n in range(nv):
            t, h, w = (int(v) for v in pos[n])
            assert 0 <= t < T and 0 <= h < Hg and 0 <= w < Wg
            assert t * Hg * Wg + h * Wg + w == n
            seen.add((t, h, w))
        assert len(seen) == nv
        for a in range(extra):
            assert tuple(pos[nv + a]) == (a, 0, 0)


# --------------------------------------------------------------------------- AdaLN

def pin_adaln_hand_cases(lib):
    for case in cases("adaln_hand.txt"):
        eps = float(case["eps"][0])
        D = len(case["x"])
        x = b16([float(v) for v in case["x"]], (1, 1, D))
        sc = b16([float(v) for v in case["scale"]], (1, D))
        sh = b16([float(v) for v in case["shift"]], (1, D))
        y = oracle.adaln_modulate(x, sh, sc, eps=eps, lib=lib)[0, 0]
        assert close(y, values(case["y"])), (case, y)


def pin_adaln_zero_modulation_is_layer_norm(lib):
    for B, N, D in [(2, 7, 96), (1, 3, 4096), (1, 5, 8)]:
        x = rand_bf16((B, N, D), seed=D + N, scale=1.5, loc=0.3)
        zeros = torch.zeros((B, D), dtype=torch.bfloat16)
        y = oracle.adaln_modulate(bits(x), bits(zeros), bits(zeros), eps=1e-6, lib=lib)
        ref = Fn.layer_norm(f64(x), (D,), eps=1e-6).numpy()
        assert close(y, ref, rel=1e-12, abs_=1e-12), (B, N, D)


def pin_adaln_matches_library_composition(lib):
    B, N, D = 2, 6, 64
    x = rand_bf16((B, N, D), seed=1)
    sc = rand_bf16((B, D), seed=2, scale=0.1)
    sh = rand_bf16((B, D), seed=3, scale=0.1)
    y = oracle.adaln_modulate(bits(x), bits(sh), bits(sc), eps=1e-6, lib=lib)
    ln = Fn.layer_norm(f64(x), (D,), eps=1e-6)
    ref = torch.addcmul(f64(sh)[:, None, :], ln, 1.0 + f64(sc)[:, None, :]).numpy()
    assert close(y, ref, rel=1e-12, abs_=1e-12)


def pin_adaln_constant_row_gives_shift(lib):
    D = 32
    x = torch.full((2, 3, D), 2.5, dtype=torch.bfloat16)
    sc = rand_bf16((2, D), seed=5, scale=0.1)
    sh = rand_bf16((2, D), seed=6, scale=0.1)
    y = oracle.adaln_modulate(bits(x), bits(sh), bits(sc), eps=1e-6, lib=lib)
    assert np.array_equal(y, np.broadcast_to(f64(sh).numpy()[:, None, :], y.shape))


def pin_adaln_unit_statistics(lib):
    D = 512
    x = rand_bf16((1, 4, D), seed=9, scale=3.0, loc=-2.0)
    zeros = torch.zeros((1, D), dtype=torch.bfloat16)
    eps = 1e-3
    y = oracle.adaln_modulate(bits(x), bits(zeros), bits(zeros), eps=eps, lib=lib)
    var = f64(x).numpy().var(axis=-1)
    assert np.allclose(y.mean(axis=-1), 0.0, atol=1e-13)
    assert np.allclose((y ** 2).mean(axis=-1), var / (var + eps), rtol=1e-12)


def pin_adaln_large_offset_cancellation(lib):
    D = 4096
    parity = np.arange(D) % 2 == 0
    x = b16(np.where(parity, 256.0, 258.0), (1, 1, D))
    zeros = b16(np.zeros(D), (1, D))
    y = oracle.adaln_modulate(x, zeros, zeros, eps=1e-6, lib=lib)[0, 0]
    assert close(y, np.where(parity, -1.0, 1.0) / math.sqrt(1.0 + 1e-6))


def pin_adaln_per_sample_vectors(lib):
    D = 16
    x = torch.zeros((2, 3, D), dtype=torch.bfloat16)
    x[:, :, : D // 2] = 1.0
    x[:, :, D // 2:] = -1.0
    sc = from_float(np.stack([np.zeros(D), np.ones(D)]))
    sh = from_float(np.stack([np.zeros(D), np.full(D, 5.0)]))
    y = oracle.adaln_modulate(bits(x), bits(sh), bits(sc), eps=1e-6, lib=lib)
    ln = np.where(np.arange(D) < D // 2, 1.0, -1.0) / math.sqrt(1.0 + 1e-6)
    assert close(y[0], np.broadcast_to(ln, (3, D)))
    assert close(y[1], np.broadcast_to(2.0 * ln + 5.0, (3, D)))


# --------------------------------------------------------------------------- gated residual

def pin_gated_residual_hand_cases(lib):
    for case in cases("gated_residual_hand.txt"):
        D = len(case["x"])
        x = b16([float(v) for v in case["x"]], (1, 1, D))
        y = b16([float(v) for v in case["y"]], (1, 1, D))
        g = b16([float(v) for v in case["gate"]], (1, D))
        out = oracle.gated_residual(x, y, g, lib=lib)[0, 0]
        assert close(out, values(case["out"]))


def pin_gated_residual_zero_gate_is_identity(lib):
    x = rand_bf16((2, 5, 40), seed=11)
    y = rand_bf16((2, 5, 40), seed=12)
    g = torch.zeros((2, 40), dtype=torch.bfloat16)
    assert np.array_equal(oracle.gated_residual(bits(x), bits(y), bits(g), lib=lib), f64(x).numpy())


def pin_gated_residual_unit_gate_is_plain_sum(lib):
    x = rand_bf16((1, 6, 24), seed=13)
    y = rand_bf16((1, 6, 24), seed=14)
    g = torch.ones((1, 24), dtype=torch.bfloat16)
    out = oracle.gated_residual(bits(x), bits(y), bits(g), lib=lib)
    assert np.array_equal(out, (f64(x) + f64(y)).numpy())  # exact: a bf16 sum fits in fp64


def pin_gated_residual_per_sample_gate(lib):
    D = 8
    x = torch.ones((2, 2, D), dtype=torch.bfloat16)
    y = torch.full((2, 2, D), 2.0, dtype=torch.bfloat16)
    g = from_float(np.stack([np.full(D, 0.5), np.full(D, -1.0)]))
    out = oracle.gated_residual(bits(x), bits(y), bits(g), lib=lib)
    assert np.all(out[0] == 2.0) and np.all(out[1] == -1.0)


# --------------------------------------------------------------------------- SwiGLU

def pin_swiglu_hand_cases(lib):
    for case in cases("swiglu_hand.txt"):
        a = [float(v) for v in case["a"]]
        b = [float(v) for v in case["b"]]
        out = oracle.swiglu(b16(a + b, (1, 2 * len(a))), lib=lib)[0]
        assert np.all(np.isfinite(out))
        assert close(out, values(case["out"])), out


def pin_swiglu_zero_input(lib):
    assert np.all(oracle.swiglu(np.zeros((3, 32), dtype=np.uint16), lib=lib) == 0.0)
    gate_zero = b16(np.concatenate([np.zeros((3, 16)), np.full((3, 16), 7.0)], axis=1), (3, 32))
    assert np.all(oracle.swiglu(gate_zero, lib=lib) == 0.0)


def pin_swiglu_matches_library_silu(lib):
    M, F = 5, 48
    inp = rand_bf16((M, 2 * F), seed=21, scale=4.0)
    x = f64(inp)
    ref = (Fn.silu(x[:, :F]) * x[:, F:]).numpy()
    assert close(oracle.swiglu(bits(inp), lib=lib), ref, rel=1e-14)


# --------------------------------------------------------------------------- RMSNorm

def pin_rmsnorm_hand_cases(lib):
    for case in cases("rmsnorm_hand.txt"):
        u = oracle.rmsnorm([float(x) for x in case["v"]], [float(x) for x in case["w"]],
                           eps=float(case["eps"][0]), lib=lib)
        assert close(u, values(case["u"])), u


def pin_rmsnorm_unit_rms_before_weight(lib):
    g = torch.Generator().manual_seed(31)
    v = torch.randn(128, generator=g, dtype=torch.float64) * 3.0
    w = 1.0 + 0.02 * torch.randn(128, generator=g, dtype=torch.float64)
    eps = 1e-6
    u = oracle.rmsnorm(v.numpy(), w.numpy(), eps=eps, lib=lib)
    ms = float((v ** 2).mean())
    assert math.isclose(float(np.mean((u / w.numpy()) ** 2)), ms / (ms + eps), rel_tol=1e-13)


def pin_rmsnorm_matches_library(lib):
    g = torch.Generator().manual_seed(32)
    v = torch.randn(64, generator=g, dtype=torch.float64)
    w = 1.0 + 0.02 * torch.randn(64, generator=g, dtype=torch.float64)
    ref = Fn.rms_norm(v, (64,), weight=w, eps=1e-6).numpy()
    assert close(oracle.rmsnorm(v.numpy(), w.numpy(), eps=1e-6, lib=lib), ref, rel=1e-13)


# --------------------------------------------------------------------------- RoPE

def pin_rope_hand_cases(lib):
    for case in cases("rope_hand.txt"):
        coord = tuple(int(c) for c in case["coord"])
        ch = int(case["ch"][0])
        u = np.zeros(64)
        u[ch], u[ch + 1] = (float(v) for v in case["in"])
        out = oracle.rope3d(u, BANDS, coord, lib=lib)
        expect = np.zeros(64)
        expect[ch], expect[ch + 1] = values(case["out"])
        assert close(out, expect, rel=1e-12, abs_=1e-13), (case, out[ch:ch + 2])


def pin_rope_frequency_tables(lib):
    """Recover each pair's frequency from the angle it turns (1, 0) by at coordinate 1."""
    for case in cases("rope_freq.txt"):
        d = int(case["d"][0])
        for j in range(d // 2):
            u = np.zeros(d + 4)
            u[2 * j] = 1.0
            out = oracle.rope3d(u, (d, 2, 2), (1, 0, 0), lib=lib)
            freq = math.atan2(out[2 * j + 1], out[2 * j])
            assert math.isclose(freq, evaluate(case["freq"][0], j=j), rel_tol=1e-12), (d, j)


def pin_rope_zero_position_is_identity(lib):
    u = torch.randn(64, generator=torch.Generator().manual_seed(41), dtype=torch.float64).numpy()
    assert np.array_equal(oracle.rope3d(u, BANDS, (0, 0, 0), lib=lib), u)


def pin_rope_preserves_pair_norms(lib):
    u = torch.randn(128, generator=torch.Generator().manual_seed(42), dtype=torch.float64).numpy()
    out = oracle.rope3d(u, (16, 56, 56), (30, 47, 83), lib=lib)
    assert np.allclose((u.reshape(-1, 2) ** 2).sum(1), (out.reshape(-1, 2) ** 2).sum(1), rtol=1e-12, atol=1e-12)
    assert not np.allclose(u, out)


def pin_rope_composes_additively(lib):
    u = torch.randn(64, generator=torch.Generator().manual_seed(43), dtype=torch.float64).numpy()
    p1, p2 = (3, 5, 7), (11, 2, 9)
    twice = oracle.rope3d(oracle.rope3d(u, BANDS, p1, lib=lib), BANDS, p2, lib=lib)
    once = oracle.rope3d(u, BANDS, tuple(a + b for a, b in zip(p1, p2)), lib=lib)
    assert close(twice, once, rel=1e-11, abs_=1e-12)


def pin_rope_inner_product_depends_on_offset_only(lib):
    g = torch.Generator().manual_seed(44)
    q = torch.randn(64, generator=g, dtype=torch.float64).numpy()
    k = torch.randn(64, generator=g, dtype=torch.float64).numpy()
    a = np.dot(oracle.rope3d(q, BANDS, (5, 9, 2), lib=lib), oracle.rope3d(k, BANDS, (2, 4, 1), lib=lib))
    b = np.dot(oracle.rope3d(q, BANDS, (13, 20, 40), lib=lib), oracle.rope3d(k, BANDS, (10, 15, 39), lib=lib))
    assert math.isclose(a, b, rel_tol=1e-11)


def pin_rope_bands_in_t_h_w_order(lib):
    edges = np.cumsum((0,) + BANDS)
    for axis in range(3):
        u = torch.randn(64, generator=torch.Generator().manual_seed(45 + axis), dtype=torch.float64).numpy()
        coord = [0, 0, 0]
        coord[axis] = 9
        out = oracle.rope3d(u, BANDS, tuple(coord), lib=lib)
        for band in range(3):
            lo, hi = edges[band], edges[band + 1]
            if band == axis:
                assert not np.allclose(out[lo:hi], u[lo:hi]), (axis, band)
            else:
                assert np.array_equal(out[lo:hi], u[lo:hi]), (axis, band)


def _complex_rope(u, bands, coord):
    """Independent composition: complex multiply by polar(1, angle) over adjacent pairs."""
    pieces, start = [], 0
    for d, p in zip(bands, coord):
        freq = 1e4 ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
        z = torch.view_as_complex(u[..., start:start + d].reshape(*u.shape[:-1], d // 2, 2).contiguous())
        ang = torch.as_tensor(p, dtype=torch.float64)[..., None] * freq
        z = z * torch.polar(torch.ones_like(ang), ang)
        pieces.append(torch.view_as_real(z).reshape(*u.shape[:-1], d))
        start += d
    return torch.cat(pieces, dim=-1)


def pin_rope_matches_complex_rotation(lib):
    bands = (16, 56, 56)
    u = torch.randn(128, generator=torch.Generator().manual_seed(46), dtype=torch.float64)
    coord = (17, 33, 61)
    out = oracle.rope3d(u.numpy(), bands, coord, lib=lib)
    assert close(out, _complex_rope(u, bands, coord).numpy(), rel=1e-12, abs_=1e-12)


# --------------------------------------------------------------------------- QK RMSNorm + RoPE (composed)

def _weights(Dh, seed):
    g = torch.Generator().manual_seed(seed)
    return (1.0 + 0.02 * torch.randn(Dh, generator=g)).to(torch.bfloat16)


def pin_qk_position_zero_equals_rmsnorm_times_weight(lib):
    B, N, H, Dh = 1, 1, 3, 64
    q = rand_bf16((B, N, H, Dh), seed=51)
    k = rand_bf16((B, N, H, Dh), seed=52)
    wq, wk = _weights(Dh, 53), _weights(Dh, 54)
    pos = np.zeros((1, 3), dtype=np.int32)
    qo, ko = oracle.qk_rmsnorm_rope3d(bits(q), bits(k), bits(wq), bits(wk), pos, BANDS, lib=lib)
    for h in range(H):
        assert np.array_equal(qo[0, 0, h], oracle.rmsnorm(f64(q)[0, 0, h].numpy(), f64(wq).numpy(), lib=lib))
        assert np.array_equal(ko[0, 0, h], oracle.rmsnorm(f64(k)[0, 0, h].numpy(), f64(wk).numpy(), lib=lib))


def pin_qk_heads_normalised_separately(lib):
    Dh = 64
    head = rand_bf16((Dh,), seed=55)
    q = torch.stack([head, (head.float() * 4.0).to(torch.bfloat16)]).reshape(1, 1, 2, Dh)
    w = torch.ones(Dh, dtype=torch.bfloat16)
    pos = np.array([[2, 3, 4]], dtype=np.int32)
    qo, _ = oracle.qk_rmsnorm_rope3d(bits(q), bits(q), bits(w), bits(w), pos, BANDS, eps=1e-30, lib=lib)
    assert close(qo[0, 0, 0], qo[0, 0, 1], rel=1e-12, abs_=1e-14)


def pin_qk_matches_library_composition(lib):
    """torch fp64 rms_norm then complex rotation, per token position and per tensor weight."""
    B, N, H, Dh = 2, 5, 4, 64
    q = rand_bf16((B, N, H, Dh), seed=61)
    k = rand_bf16((B, N, H, Dh), seed=62)
    wq, wk = _weights(Dh, 63), _weights(Dh, 64)
    pos = np.array([[0, 0, 0], [1, 2, 3], [4, 0, 1], [0, 3, 3], [479, 0, 0]], dtype=np.int32)
    qo, ko = oracle.qk_rmsnorm_rope3d(bits(q), bits(k), bits(wq), bits(wk), pos, BANDS, lib=lib)
    coord = tuple(torch.as_tensor(pos[:, a])[None, :, None] for a in range(3))

    def ref(v, w):
        return _complex_rope(Fn.rms_norm(f64(v), (Dh,), weight=f64(w), eps=1e-6), BANDS, coord).numpy()

    assert close(qo, ref(q, wq), rel=1e-11, abs_=1e-12)
    assert close(ko, ref(k, wk), rel=1e-11, abs_=1e-12)


# --------------------------------------------------------------------------- bf16 storage rounding

def pin_bf16_encode_hand_cases(lib):
    for case in cases("bf16_round_hand.txt"):
        value = evaluate(case["value"][0])
        assert oracle.bf16_encode(value, lib=lib) == int(case["bits"][0], 16), case


def pin_bf16_encode_matches_library_rounding(lib):
    g = torch.Generator().manual_seed(81)
    vals = torch.cat([torch.randn(2000, generator=g) * 3.0, torch.randn(500, generator=g) * 1e-30,
                      torch.randn(500, generator=g) * 1e30])
    ref = vals.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_encode(float(v), lib=lib) for v in vals.tolist()], dtype=np.uint16)
    assert np.array_equal(got, ref)


def pin_bf16_encode_round_trips(lib):
    for bits in list(range(0, 0x7F80, 97)) + [0x7F7F, 0x0001, 0x8001, 0xC049]:
        assert oracle.bf16_encode(oracle.bf16_decode(bits, lib=lib), lib=lib) == bits


# --------------------------------------------------------------------------- fused gated residual + AdaLN

def pin_residual_adaln_hand_cases(lib):
    zeros = b16([0.0] * 4, (1, 4))
    for case in cases("residual_adaln_hand.txt"):
        x = b16([evaluate(v) for v in case["x"]], (1, 1, 4))
        y = b16([evaluate(v) for v in case["y"]], (1, 1, 4))
        g = b16([evaluate(v) for v in case["gate"]], (1, 4))
        x_out, z = oracle.gated_residual_adaln(x, y, g, zeros, zeros, eps=1e-6, lib=lib)
        assert close(x_out[0, 0], values(case["x_out"])), case
        stored = b16(values(case["stored"]), (1, 1, 4))
        assert close(z, oracle.adaln_modulate(stored, zeros, zeros, eps=1e-6, lib=lib)), case
    x = b16([1, 2, 3, 4], (1, 1, 4))
    y = b16([2 ** -8, 0, 0, 0], (1, 1, 4))
    _, z = oracle.gated_residual_adaln(x, y, b16([1] * 4, (1, 4)), zeros, zeros, eps=1e-6, lib=lib)
    assert close(z[0, 0], [v / math.sqrt(1.25 + 1e-6) for v in (-1.5, -0.5, 0.5, 1.5)])


def pin_residual_adaln_is_the_pipeline(lib):
    """Special cases reducing to the pinned unfused ops: gate = 0 and y = 0."""
    B, N, D = 2, 5, 64
    x = rand_bf16((B, N, D), seed=91)
    y = rand_bf16((B, N, D), seed=92)
    sh = rand_bf16((B, D), seed=93, scale=0.1)
    sc = rand_bf16((B, D), seed=94, scale=0.1)
    zero_g = torch.zeros((B, D), dtype=torch.bfloat16)
    x_out, z = oracle.gated_residual_adaln(bits(x), bits(y), bits(zero_g), bits(sh), bits(sc), lib=lib)
    assert np.array_equal(x_out, f64(x).numpy())
    assert np.array_equal(z, oracle.adaln_modulate(bits(x), bits(sh), bits(sc), lib=lib))
    g = rand_bf16((B, D), seed=95, scale=0.1)
    zero_y = torch.zeros_like(y)
    x_out, z = oracle.gated_residual_adaln(bits(x), bits(zero_y), bits(g), bits(sh), bits(sc), lib=lib)
    assert np.array_equal(z, oracle.adaln_modulate(bits(x), bits(sh), bits(sc), lib=lib))
    x_out, _ = oracle.gated_residual_adaln(bits(x), bits(y), bits(g), bits(sh), bits(sc), lib=lib)
    assert np.array_equal(x_out, (f64(x) + f64(g)[:, None, :] * f64(y)).numpy())  # exact in fp64


# --------------------------------------------------------------------------- QK with memory layouts

def _qkv(B, N, H, Dh, seed, v_fill=None):
    """A fused [B,N,3,H,Dh] projection buffer; v is filled with NaN bits to catch stray reads."""
    qkv = rand_bf16((B, N, 3, H, Dh), seed=seed)
    if v_fill is not None:
        qkv[:, :, 2] = v_fill
    return qkv


def pin_qk_layout_plain_case_matches_qk(lib):
    B, N, H, Dh = 2, 5, 3, 64
    q = rand_bf16((B, N, H, Dh), seed=111)
    k = rand_bf16((B, N, H, Dh), seed=112)
    w1, w2 = _weights(Dh, 113), _weights(Dh, 114)
    pos = np.array([[t, t % 3, 2 * t + 1] for t in range(N)], dtype=np.int32)
    ref = oracle.qk_rmsnorm_rope3d(bits(q), bits(k), bits(w1), bits(w2), pos, BANDS, lib=lib)
    got = oracle.qk_rmsnorm_rope3d_layout(bits(q).ravel(), bits(k).ravel(), bits(w1), bits(w2), pos, BANDS,
                                          B, N, H, Dh, H * Dh, 0, lib=lib)
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


def pin_qk_layout_head_major_is_a_transpose(lib):
    """Brute force over a tiny case: every (b, n, h) head lands at ((b*H + h)*N + n)."""
    B, N, H, Dh = 2, 4, 3, 64
    q = rand_bf16((B, N, H, Dh), seed=121)
    k = rand_bf16((B, N, H, Dh), seed=122)
    w1, w2 = _weights(Dh, 123), _weights(Dh, 124)
    pos = np.array([[t, 2 * t, 3 * t] for t in range(N)], dtype=np.int32)
    tm = oracle.qk_rmsnorm_rope3d_layout(bits(q).ravel(), bits(k).ravel(), bits(w1), bits(w2), pos, BANDS,
                                         B, N, H, Dh, H * Dh, 0, lib=lib)
    hm = oracle.qk_rmsnorm_rope3d_layout(bits(q).ravel(), bits(k).ravel(), bits(w1), bits(w2), pos, BANDS,
                                         B, N, H, Dh, H * Dh, 1, lib=lib)
    for b in range(B):
        for n in range(N):
            for h in range(H):
                assert np.array_equal(hm[0][b, h, n], tm[0][b, n, h]) and np.array_equal(hm[1][b, h, n], tm[1][b, n, h])


def pin_qk_layout_reads_q_and_k_from_a_fused_qkv_buffer(lib):
    B, N, H, Dh = 2, 3, 2, 64
    nan_bits = torch.tensor(0x7FC0, dtype=torch.int16).view(torch.bfloat16)
    qkv = _qkv(B, N, H, Dh, seed=131, v_fill=nan_bits)
    flat = bits(qkv).ravel()
    w1, w2 = _weights(Dh, 132), _weights(Dh, 133)
    pos = np.array([[1, 2, 3], [4, 5, 6], [7, 8, 9]], dtype=np.int32)
    got = oracle.qk_rmsnorm_rope3d_layout(flat, flat[H * Dh:], bits(w1), bits(w2), pos, BANDS,
                                          B, N, H, Dh, 3 * H * Dh, 1, lib=lib)
    ref = oracle.qk_rmsnorm_rope3d(bits(qkv[:, :, 0].contiguous()), bits(qkv[:, :, 1].contiguous()),
                                   bits(w1), bits(w2), pos, BANDS, lib=lib)
    assert np.all(np.isfinite(got[0])) and np.all(np.isfinite(got[1]))
    assert np.array_equal(got[0], ref[0].transpose(0, 2, 1, 3)) and np.array_equal(got[1], ref[1].transpose(0, 2, 1, 3))


# --------------------------------------------------------------------------- Cache-DiT residual change

def pin_residual_change_hand_cases(lib):
    for case in cases("residual_change_hand.txt"):
        D = len(case["r"])
        r = b16([evaluate(v) for v in case["r"]], (1, 1, D))
        rc = b16([evaluate(v) for v in case["rc"]], (1, 1, D))
        out = oracle.residual_change(r, rc, lib=lib)[0]
        expect = [evaluate(case["num"][0]), evaluate(case["den"][0]), evaluate(case["ratio"][0])]
        assert out[0] == expect[0] and out[1] == expect[1], (case, out)
        assert out[2] == expect[2] or math.isclose(out[2], expect[2], rel_tol=1e-15), (case, out)


def pin_residual_change_matches_library_per_sample(lib):
    B, N, D = 3, 7, 40
    r = rand_bf16((B, N, D), seed=161)
    rc = rand_bf16((B, N, D), seed=162, scale=2.0)
    out = oracle.residual_change(bits(r), bits(rc), lib=lib)
    num = (f64(r) - f64(rc)).abs().sum(dim=(1, 2))
    den = f64(rc).abs().sum(dim=(1, 2))
    assert np.allclose(out[:, 0], num.numpy(), rtol=1e-14) and np.allclose(out[:, 1], den.numpy(), rtol=1e-14)
    assert np.allclose(out[:, 2], (num / den).numpy(), rtol=1e-14)
    # samples are separate: changing sample 1 leaves samples 0 and 2 alone
    r2 = r.clone()
    r2[1] += 1.0
    out2 = oracle.residual_change(bits(r2), bits(rc), lib=lib)
    assert np.array_equal(out2[[0, 2]], out[[0, 2]]) and out2[1, 0] != out[1, 0]


# --------------------------------------------------------------------------- SubBlock routing

def pin_subblock_pool_hand_cases(lib):
    for case in cases("subblock_pool_hand.txt"):
        block, N, H, Dh = (int(case[k][0]) for k in ("block", "N", "H", "Dh"))
        x = b16(values(case["x"]), (1, N, H, Dh))
        out = oracle.subblock_pool(x, block, lib=lib)
        nb = -(-N // block)
        assert out.shape == (1, H, nb, Dh), case
        assert close(out.reshape(-1), values(case["out"]), rel=1e-15), (case, out)


def pin_subblock_pool_matches_library_mean(lib):
    # numpy's mean over each block's token slice (its own summation order)
    B, N, H, Dh = 2, 150, 3, 8
    x = rand_bf16((B, N, H, Dh), seed=181)
    for block in (64, 7):
        out = oracle.subblock_pool(bits(x), block, lib=lib)
        xf = f64(x).numpy()
        nb = -(-N // block)
        assert out.shape == (B, H, nb, Dh)
        for i in range(nb):
            ref = xf[:, i * block:(i + 1) * block].mean(axis=1)  # [B, H, Dh]
            assert np.allclose(out[:, :, i], ref, rtol=1e-13, atol=1e-15), (block, i)


def pin_subblock_pool_invariants(lib):
    # a block of equal tokens pools to that token; a ramp pools to its midpoint;
    # changing sample 1 leaves sample 0 alone
    B, N, H, Dh, block = 2, 64 * 3, 2, 4, 64
    vals = np.zeros((B, N, H, Dh))
    for i in range(3):
        vals[:, i * block:(i + 1) * block] = (i + 1) * 0.5
    vals[1, :block, 1, 2] = np.arange(block) * 0.25  # ramp 0 .. 15.75, mean 7.875
    x = b16(vals.reshape(-1), (B, N, H, Dh))
    out = oracle.subblock_pool(x, block, lib=lib)
    assert np.all(out[0, :, 0] == 0.5) and np.all(out[0, :, 1] == 1.0) and np.all(out[0, :, 2] == 1.5)
    assert out[1, 1, 0, 2] == 7.875 and out[1, 0, 0, 2] == 0.5
    vals[1] += 1.0
    out2 = oracle.subblock_pool(b16(vals.reshape(-1), (B, N, H, Dh)), block, lib=lib)
    assert np.array_equal(out2[0], out[0]) and np.array_equal(out2[1], out[1] + 1.0)


def pin_subblock_scores_hand_cases(lib):
    for case in cases("subblock_scores_hand.txt"):
        nb, Dh = int(case["nb"][0]), int(case["Dh"][0])
        qp = np.array(values(case["qp"])).reshape(1, 1, nb, Dh)
        kp = np.array(values(case["kp"])).reshape(1, 1, nb, Dh)
        s = oracle.subblock_scores(qp, kp, lib=lib)
        assert s.reshape(-1).tolist() == values(case["s"]), (case, s)


def pin_subblock_scores_match_library(lib):
    # torch's own bf16 rounding of the means, then an fp64 matmul per (sample, head)
    g = torch.Generator().manual_seed(191)
    B, H, nb, Dh = 2, 3, 9, 16
    qp = torch.randn((B, H, nb, Dh), generator=g, dtype=torch.float64) * 0.3
    kp = torch.randn((B, H, nb, Dh), generator=g, dtype=torch.float64) * 0.3
    s = oracle.subblock_scores(qp.numpy(), kp.numpy(), lib=lib)
    qb = qp.to(torch.bfloat16).to(torch.float64)
    kb = kp.to(torch.bfloat16).to(torch.float64)
    ref = torch.matmul(qb, kb.transpose(-1, -2).contiguous())
    assert np.allclose(s, ref.numpy(), rtol=1e-13, atol=1e-15)
    # the rounding matters for these inputs: unrounded products differ
    assert not np.allclose(s, torch.matmul(qp, kp.transpose(-1, -2).contiguous()).numpy(), rtol=1e-6)


def pin_subblock_row_subset(lib):
    # scoring and routing a subset of query blocks gives those rows of the full result
    g = torch.Generator().manual_seed(193)
    qp = (torch.randn((1, 2, 11, 8), generator=g, dtype=torch.float64) * 0.3).numpy()
    kp = (torch.randn((1, 2, 11, 8), generator=g, dtype=torch.float64) * 0.3).numpy()
    rows = [0, 4, 10]
    full = oracle.subblock_scores(qp, kp, lib=lib)
    part = oracle.subblock_scores(qp[:, :, rows], kp, lib=lib)
    assert part.shape == (1, 2, 3, 11) and np.array_equal(part, full[:, :, rows])
    assert np.array_equal(oracle.subblock_topk(part, 4, lib=lib), oracle.subblock_topk(full, 4, lib=lib)[:, :, rows])


def pin_subblock_keep_cases(lib):
    for case in cases("subblock_keep_hand.txt"):
        nb, sparsity = int(case["nb"][0]), evaluate(case["sparsity"][0])
        assert oracle.subblock_keep(nb, sparsity, lib=lib) == int(case["keep"][0]), case
    for bad in (-0.1, 1.0, float("nan")):
        with pytest.raises(ValueError):
            oracle.subblock_keep(10, bad, lib=lib)


def pin_subblock_topk_hand_cases(lib):
    for case in cases("subblock_topk_hand.txt"):
        row = values(case["s"])
        keep = int(case["keep"][0])
        idx = oracle.subblock_topk(np.array(row).reshape(1, 1, 1, -1).repeat(len(row), axis=2), keep, lib=lib)
        for r in range(len(row)):
            assert idx[0, 0, r].tolist() == [int(v) for v in case["idx"]], (case, idx[0, 0, r])


def pin_subblock_topk_brute_force(lib):
    # numpy's stable lexsort on (score descending, index ascending); scores drawn
    # from a few values so that ties are common
    rng = np.random.default_rng(201)
    B, H, nb = 2, 2, 23
    s = rng.integers(-3, 4, size=(B, H, nb, nb)).astype(np.float64) * 0.5
    for keep in (0, 1, 5, 12, nb):
        idx = oracle.subblock_topk(s, keep, lib=lib)
        for b in range(B):
            for h in range(H):
                for i in range(nb):
                    order = np.lexsort((np.arange(nb), -s[b, h, i]))
                    assert idx[b, h, i].tolist() == sorted(order[:keep].tolist()), (keep, b, h, i)


def pin_subblock_route_structured(lib):
    # Query block i is made of tokens +-e_i (mean e_i exactly); key block j of
    # tokens c_j +- d (mean c_j), so score (i, j) = c_j[i] and the kept blocks
    # follow from the table c by hand.
    block, nb, Dh = 4, 4, 8
    c = np.array([[2.0, -1.0, 0.5, 3.0, 0, 0, 0, 0],   # key block 0
                  [1.0, 4.0, 0.5, -2.0, 0, 0, 0, 0],   # key block 1
                  [3.0, 0.0, 0.25, 1.0, 0, 0, 0, 0],   # key block 2
                  [-1.0, 2.0, 0.75, 3.0, 0, 0, 0, 0]])  # key block 3
    q = np.zeros((1, nb * block, 1, Dh))
    k = np.zeros((1, nb * block, 1, Dh))
    for i in range(nb):
        for t in range(block):
            sign = 1.0 if t % 2 == 0 else -1.0
            q[0, i * block + t, 0, i] = 1.0 + sign * 0.5
            k[0, i * block + t, 0] = c[i] + sign * 0.125
    qp, kp, s, idx = oracle.subblock_route(b16(q.reshape(-1), q.shape), b16(k.reshape(-1), k.shape), 0.5,
                                           block=block, lib=lib)
    assert np.array_equal(qp[0, 0], np.eye(nb, Dh)) and np.array_equal(kp[0, 0], c)
    assert np.array_equal(s[0, 0], c[:, :nb].T)
    # keep = 4 - floor(0.5 * 4) = 2 per query block: the two largest of c[:, i].
    # Query block 2 sees (0.5, 0.5, 0.25, 0.75): block 3, then the tie of blocks
    # 0 and 1 goes to the lower index.
    assert idx[0, 0].tolist() == [[0, 2], [1, 3], [0, 3], [0, 3]]


def pin_qk_pool_hand_cases(lib):
    for case in cases("qk_pool_hand.txt"):
        n_tok = int(case["tokens"][0])
        v = b16(values(case["v"]) * n_tok, (1, n_tok, 1, 2))
        w = b16(values(case["w"]))
        pos = np.zeros((n_tok, 3), dtype=np.int32)
        qo, ko, qp, kp = oracle.qk_rmsnorm_rope3d_pool(v, v, w, w, pos, (2, 0, 0), 1e4, 1e-6, lib=lib)
        assert close(qo[0, 0, 0], values(case["exact"]), rel=1e-15), (case, qo)
        assert qp.reshape(-1).tolist() == values(case["pooled"]), (case, qp)
        assert np.array_equal(qp, kp)


def pin_qk_pool_is_the_pipeline(lib):
    # the fused oracle equals QK, then the oracle's bf16 store, then block pooling
    B, N, H, Dh = 2, 130, 2, 64
    q = rand_bf16((B, N, H, Dh), seed=211)
    k = rand_bf16((B, N, H, Dh), seed=212, scale=3.0)
    wq, wk = _weights(Dh, 213), _weights(Dh, 214)
    pos = np.array([[n // 20, (n // 5) % 4, n % 5] for n in range(N)], dtype=np.int32)
    qo, ko, qp, kp = oracle.qk_rmsnorm_rope3d_pool(bits(q), bits(k), bits(wq), bits(wk), pos, BANDS, lib=lib)
    qr, kr = oracle.qk_rmsnorm_rope3d(bits(q), bits(k), bits(wq), bits(wk), pos, BANDS, lib=lib)
    assert np.array_equal(qo, qr) and np.array_equal(ko, kr)
    encode = np.vectorize(lambda x: oracle.bf16_encode(x, lib=lib), otypes=[np.uint16])
    assert np.array_equal(qp, oracle.subblock_pool(encode(qr), lib=lib))
    assert np.array_equal(kp, oracle.subblock_pool(encode(kr), lib=lib))
    assert not np.array_equal(qp, kp)


# --------------------------------------------------------------------------- argument checks and threading

def pin_rope_rejects_bad_bands(lib):
    for bands in [(15, 25, 24), (16, 24, 26)]:
        with pytest.raises(ValueError):
            oracle.rope3d(np.zeros(64), bands, (1, 1, 1), lib=lib)


def pin_threaded_calls_equal_serial(lib):
    x = rand_bf16((2, 37, 64), seed=71)
    sc = rand_bf16((2, 64), seed=72, scale=0.1)
    sh = rand_bf16((2, 64), seed=73, scale=0.1)
    a = oracle.adaln_modulate(bits(x), bits(sh), bits(sc), threads=1, lib=lib)
    b = oracle.adaln_modulate(bits(x), bits(sh), bits(sc), threads=5, lib=lib)
    assert np.array_equal(a, b)
    inp = rand_bf16((37, 96), seed=74)
    assert np.array_equal(oracle.swiglu(bits(inp), threads=1, lib=lib), oracle.swiglu(bits(inp), threads=4, lib=lib))
    y = rand_bf16((2, 37, 64), seed=75)
    assert np.array_equal(oracle.gated_residual(bits(x), bits(y), bits(sc), threads=1, lib=lib),
                          oracle.gated_residual(bits(x), bits(y), bits(sc), threads=3, lib=lib))
    q = rand_bf16((2, 9, 2, 64), seed=76)
    k = rand_bf16((2, 9, 2, 64), seed=77)
    w = _weights(64, 78)
    pos = np.array([[t, t % 3, 2 * t] for t in range(9)], dtype=np.int32)
    a = oracle.qk_rmsnorm_rope3d(bits(q), bits(k), bits(w), bits(sc[0]), pos, BANDS, threads=1, lib=lib)
    b = oracle.qk_rmsnorm_rope3d(bits(q), bits(k), bits(w), bits(sc[0]), pos, BANDS, threads=4, lib=lib)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


PINS = {name[4:]: fn for name, fn in sorted(globals().items()) if name.startswith("pin_") and callable(fn)}


@pytest.mark.parametrize("name", sorted(PINS))
def test_oracle_pin(oracle_lib, name):
    PINS[name](oracle_lib)
