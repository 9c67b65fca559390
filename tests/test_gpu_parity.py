"""Parity of the HIP kernels (through the C ABI) with the fp64 oracle.

Small and ragged shapes are compared on every element; the full-size
workloads (the shapes the benchmark launches, through the same entry points)
on sampled rows that the oracle recomputes one by one, plus properties that
hold at any size.  Positions (integer work) must match bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
import video_diffusion_transformer_dit_amd as dit
from parity_util import assert_close, to_f64
from synthetic_inputs import bits

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    dit.load_library()  # raises if libdit_ops.so is missing: no fallback path exists
    torch.cuda.synchronize()
    yield
    torch.cuda.synchronize()


def randn_bf16(shape, seed, scale=1.0, loc=0.0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV) * scale + loc).to(torch.bfloat16)


def weights(n, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return (1.0 + 0.02 * torch.randn(n, generator=g, device=DEV)).to(torch.bfloat16)


def sync():
    torch.cuda.synchronize()


# --------------------------------------------------------------------------- positions

@pytest.mark.parametrize("grid,extra", [((2, 4, 4), 0), ((3, 5, 7), 11), ((1, 1, 1), 0), ((0, 0, 0), 9),
                                        ((31, 24, 42), 0), ((31, 48, 84), 0), ((61, 48, 84), 480)])
def test_packed_positions_bit_exact(grid, extra):
    T, Hg, Wg = grid
    pos = dit.dit_packed_positions(T, Hg, Wg, extra, device=DEV)
    sync()
    ref = oracle.packed_positions(T, Hg, Wg, extra)
    assert np.array_equal(pos.cpu().numpy(), ref)


# --------------------------------------------------------------------------- tiny workload, every element

def test_tiny_workload_all_ops():
    wl = si.WORKLOADS["tiny"]
    ins = si.make_inputs(wl, device=DEV)
    pos = dit.dit_packed_positions(*wl.grid, wl.n_extra, device=DEV)
    y = dit.dit_adaln_modulate(ins["x_mod"], ins["shift"], ins["scale"], eps=wl.eps)
    out = dit.dit_gated_residual(ins["res_x"], ins["res_y"], ins["gate"])
    sw = dit.dit_swiglu(ins["swiglu_in"])
    qo, ko = dit.dit_qk_rmsnorm_rope3d(ins["q"], ins["k"], ins["wq"], ins["wk"], pos, wl.bands,
                                       theta=wl.theta, eps=wl.eps)
    sync()
    b = {k: bits(v) for k, v in ins.items()}
    pos_ref = oracle.packed_positions(*wl.grid, wl.n_extra)
    assert np.array_equal(pos.cpu().numpy(), pos_ref)
    assert_close(y, oracle.adaln_modulate(b["x_mod"], b["shift"], b["scale"], eps=wl.eps), "adaln")
    assert_close(out, oracle.gated_residual(b["res_x"], b["res_y"], b["gate"]), "residual")
    assert_close(sw, oracle.swiglu(b["swiglu_in"]), "swiglu")
    qr, kr = oracle.qk_rmsnorm_rope3d(b["q"], b["k"], b["wq"], b["wk"], pos_ref, wl.bands, wl.theta, wl.eps)
    assert_close(qo, qr, "q")
    assert_close(ko, kr, "k")


# --------------------------------------------------------------------------- AdaLN

ADALN_SHAPES = [(1, 33, 4096), (2, 1953, 4096), (1, 7, 8), (3, 5, 264), (1, 3, 8192), (2, 17, 4104),
                (1, 5, 256), (2, 3, 1000), (1, 1, 512), (1, 2, 520)]


@pytest.mark.parametrize("B,N,D", ADALN_SHAPES)
def test_adaln_shapes(B, N, D):
    x = randn_bf16((B, N, D), seed=B * 1000 + N + D)
    sh = randn_bf16((B, D), seed=11, scale=0.1)
    sc = randn_bf16((B, D), seed=12, scale=0.1)
    y = dit.dit_adaln_modulate(x, sh, sc)
    sync()
    assert_close(y, oracle.adaln_modulate(bits(x), bits(sh), bits(sc), threads=8), f"adaln {B}x{N}x{D}")


def test_adaln_hard_rows():
    D = 4096
    rows = []
    rows.append(torch.full((D,), 3.0))                                    # constant row: output = shift
    rows.append(torch.where(torch.arange(D) % 2 == 0, 256.0, 258.0))     # large offset, unit spread
    g = torch.Generator().manual_seed(5)
    heavy = torch.randn(D, generator=g)
    heavy[torch.randperm(D, generator=g)[: round(0.05 * D)]] *= 20.0
    rows.append(heavy)                                                   # 5% of channels x20
    rows.append(1000.0 + torch.randn(D, generator=g))                    # mean far from zero
    rows.append(torch.zeros(D))                                          # all zero
    rows.append(torch.randn(D, generator=g) * 1e-3)                      # tiny spread vs eps
    x = torch.stack(rows).reshape(1, -1, D).to(torch.bfloat16).to(DEV)
    sh = randn_bf16((1, D), seed=21, scale=0.1)
    sc = randn_bf16((1, D), seed=22, scale=0.1)
    y = dit.dit_adaln_modulate(x, sh, sc)
    sync()
    assert_close(y, oracle.adaln_modulate(bits(x), bits(sh), bits(sc)), "adaln hard rows")
    assert torch.equal(y[0, 0], sh[0]) and torch.equal(y[0, 4], sh[0])


def test_adaln_in_place_and_deterministic():
    x = randn_bf16((2, 257, 4096), seed=31)
    sh = randn_bf16((2, 4096), seed=32, scale=0.1)
    sc = randn_bf16((2, 4096), seed=33, scale=0.1)
    a = dit.dit_adaln_modulate(x, sh, sc)
    b = dit.dit_adaln_modulate(x, sh, sc)
    xi = x.clone()
    dit.dit_adaln_modulate(xi, sh, sc, y=xi)
    sync()
    assert torch.equal(a, b) and torch.equal(a, xi)


@pytest.mark.parametrize("N,D", [(5, 4096), (7, 1032), (3, 512), (9, 8192)])
def test_adaln_row_result_independent_of_batch_position(N, D):
    # Four rows per workgroup: with N % 4 != 0 some workgroups straddle two
    # samples, and their second-sample rows read the modulation vectors from
    # cache instead of the workgroup's staged copy.  Identical rows with
    # identical vectors must still give identical bits in every position.
    B = 3
    x = randn_bf16((B, N, D), seed=41 + N)
    x[1:] = x[0]
    sh = randn_bf16((1, D), seed=42, scale=0.1).expand(B, D).contiguous()
    sc = randn_bf16((1, D), seed=43, scale=0.1).expand(B, D).contiguous()
    y = dit.dit_adaln_modulate(x, sh, sc)
    ry = randn_bf16((B, N, D), seed=44 + N)
    ry[1:] = ry[0]
    g = randn_bf16((1, D), seed=45, scale=0.1).expand(B, D).contiguous()
    x_out, z = dit.dit_gated_residual_adaln(x, ry, g, sh, sc)
    sync()
    for b in range(1, B):
        assert torch.equal(y[b], y[0]), f"adaln sample {b} differs from sample 0"
        assert torch.equal(z[b], z[0]), f"fused z sample {b} differs from sample 0"
        assert torch.equal(x_out[b], x_out[0])
    assert_close(y, oracle.adaln_modulate(bits(x), bits(sh), bits(sc)), "adaln straddling samples")


# --------------------------------------------------------------------------- gated residual

RESIDUAL_SHAPES = [(1, 33, 4096), (2, 1953, 4096), (1, 7, 8), (3, 5, 264), (2, 3, 1000), (1, 2, 65536), (1, 9, 24),
                   (2, 5, 12288)]


@pytest.mark.parametrize("B,N,D", RESIDUAL_SHAPES)
def test_gated_residual_shapes(B, N, D):
    x = randn_bf16((B, N, D), seed=B + N + D)
    y = randn_bf16((B, N, D), seed=B + N + D + 1)
    g = randn_bf16((B, D), seed=41, scale=0.1)
    out = dit.dit_gated_residual(x, y, g)
    sync()
    assert_close(out, oracle.gated_residual(bits(x), bits(y), bits(g), threads=8), f"residual {B}x{N}x{D}")


def test_gated_residual_zero_gate_in_place_deterministic():
    x = randn_bf16((2, 100, 4096), seed=51)
    y = randn_bf16((2, 100, 4096), seed=52)
    g = randn_bf16((2, 4096), seed=53, scale=0.1)
    zero = torch.zeros_like(g)
    assert torch.equal(dit.dit_gated_residual(x, y, zero), x)
    a = dit.dit_gated_residual(x, y, g)
    b = dit.dit_gated_residual(x, y, g)
    xi, yi = x.clone(), y.clone()
    dit.dit_gated_residual(xi, y, g, out=xi)
    dit.dit_gated_residual(x, yi, g, out=yi)
    sync()
    assert torch.equal(a, b) and torch.equal(a, xi) and torch.equal(a, yi)


# --------------------------------------------------------------------------- fused gated residual + AdaLN

FUSED_SHAPES = [(1, 33, 4096), (2, 1953, 4096), (3, 5, 264), (2, 17, 4104), (1, 3, 8192), (1, 7, 8), (2, 3, 1000)]


def fused_inputs(B, N, D, seed):
    return (randn_bf16((B, N, D), seed=seed), randn_bf16((B, N, D), seed=seed + 1),
            randn_bf16((B, D), seed=seed + 2, scale=0.1), randn_bf16((B, D), seed=seed + 3, scale=0.1),
            randn_bf16((B, D), seed=seed + 4, scale=0.1))


@pytest.mark.parametrize("B,N,D", FUSED_SHAPES)
def test_gated_residual_adaln_shapes(B, N, D):
    x, y, g, sh, sc = fused_inputs(B, N, D, seed=B * 7 + N + D)
    x_out, z = dit.dit_gated_residual_adaln(x, y, g, sh, sc)
    sync()
    xr, zr = oracle.gated_residual_adaln(bits(x), bits(y), bits(g), bits(sh), bits(sc), threads=8)
    assert_close(x_out, xr, f"fused x_out {B}x{N}x{D}")
    assert_close(z, zr, f"fused z {B}x{N}x{D}")


@pytest.mark.parametrize("B,N,D", FUSED_SHAPES)
def test_gated_residual_adaln_equals_the_two_calls(B, N, D):
    """The fused kernel reproduces dit_gated_residual then dit_adaln_modulate bit for bit."""
    x, y, g, sh, sc = fused_inputs(B, N, D, seed=B * 11 + N + D)
    x_out, z = dit.dit_gated_residual_adaln(x, y, g, sh, sc)
    x_ref = dit.dit_gated_residual(x, y, g)
    z_ref = dit.dit_adaln_modulate(x_ref, sh, sc)
    sync()
    assert torch.equal(x_out, x_ref) and torch.equal(z, z_ref)


def test_gated_residual_adaln_in_place_and_deterministic():
    x, y, g, sh, sc = fused_inputs(2, 257, 4096, seed=101)
    a = dit.dit_gated_residual_adaln(x, y, g, sh, sc)
    b = dit.dit_gated_residual_adaln(x, y, g, sh, sc)
    xi, yi = x.clone(), y.clone()
    dit.dit_gated_residual_adaln(xi, yi, g, sh, sc, x_out=xi, z=yi)
    sync()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(a[0], xi) and torch.equal(a[1], yi)


def test_gated_residual_adaln_rounding_ties():
    """Rows whose residual lands exactly halfway between bf16 neighbours."""
    D = 4096
    x = torch.ones((1, 2, D), dtype=torch.bfloat16, device=DEV)
    x[..., 1::2] = 3.0
    y = torch.zeros_like(x)
    y[0, 0, 0::2] = 2.0 ** -8        # 1 + 2^-8 -> 1 (tie to even)
    y[0, 1, 0::2] = 3 * 2.0 ** -8    # 1 + 3*2^-8 -> 1 + 2^-6 (tie to even, up)
    g = torch.ones((1, D), dtype=torch.bfloat16, device=DEV)
    sh = torch.zeros_like(g)
    sc = torch.zeros_like(g)
    x_out, z = dit.dit_gated_residual_adaln(x, y, g, sh, sc)
    sync()
    assert torch.all(x_out[0, 0, 0::2] == 1.0) and torch.all(x_out[0, 1, 0::2] == 1.0 + 2.0 ** -6)
    xr, zr = oracle.gated_residual_adaln(bits(x), bits(y), bits(g), bits(sh), bits(sc))
    assert_close(z, zr, "fused z at rounding ties")


# --------------------------------------------------------------------------- Cache-DiT residual change

CHANGE_RTOL = 2e-6  # fp32 over 8 values per vector, fp64 above: relative error below 8 * 2^-24


def check_change(got, ref, what):
    got = got.cpu().numpy()
    assert got.shape == ref.shape, what
    for b in range(ref.shape[0]):
        for j in range(3):
            g, r = float(got[b, j]), float(ref[b, j])
            if math.isinf(r) or r == 0.0:
                assert g == r, (what, b, j, g, r)
            else:
                assert abs(g - r) <= CHANGE_RTOL * abs(r), (what, b, j, g, r, abs(g - r) / abs(r))


@pytest.mark.parametrize("B,N,D", [(1, 33, 4096), (2, 1953, 4096), (3, 5, 264), (1, 1, 8), (2, 257, 1000)])
def test_residual_change_shapes(B, N, D):
    r = randn_bf16((B, N, D), seed=B + N + D)
    rc = randn_bf16((B, N, D), seed=B + N + D + 1, scale=0.9)
    out = dit.dit_residual_change(r, rc)
    sync()
    check_change(out, oracle.residual_change(bits(r), bits(rc)), f"change {B}x{N}x{D}")


def test_residual_change_special_cases():
    rc = randn_bf16((2, 300, 4096), seed=171)
    zero = torch.zeros_like(rc)
    same = dit.dit_residual_change(rc, rc)
    double = dit.dit_residual_change((rc.float() * 2).to(torch.bfloat16), rc)
    from_zero = dit.dit_residual_change(rc, zero)
    both_zero = dit.dit_residual_change(zero, zero)
    empty = dit.dit_residual_change(rc[:, :0], rc[:, :0])
    sync()
    assert torch.all(same[:, 0] == 0) and torch.all(same[:, 2] == 0)
    assert torch.all(double[:, 2] == 1.0)  # |2c - c| and |c| take the same fp32 sums
    assert torch.all(torch.isinf(from_zero[:, 2])) and torch.all(both_zero == 0) and torch.all(empty == 0)


def test_residual_change_deterministic_and_workspace_reuse():
    r = randn_bf16((2, 5000, 4096), seed=181)
    rc = randn_bf16((2, 5000, 4096), seed=182)
    ws = torch.empty(dit.dit_residual_change_workspace_bytes(2, 5000, 4096), dtype=torch.uint8, device=DEV)
    ws.fill_(0xFF)  # stale contents must not matter
    a = dit.dit_residual_change(r, rc, workspace=ws)
    b = dit.dit_residual_change(r, rc, workspace=ws)
    c = dit.dit_residual_change(r[:1, :17], rc[:1, :17], workspace=ws)
    sync()
    assert torch.equal(a, b)
    check_change(c, oracle.residual_change(bits(r[:1, :17]), bits(rc[:1, :17])), "smaller call after larger")


# --------------------------------------------------------------------------- SwiGLU

SWIGLU_SHAPES = [(33, 16384), (7, 8), (5, 1000), (3, 16392), (64, 2048), (1, 8), (1953, 512), (2, 24), (5, 6144)]


@pytest.mark.parametrize("M,F", SWIGLU_SHAPES)
def test_swiglu_shapes(M, F):
    inp = randn_bf16((M, 2 * F), seed=M + F, scale=2.0)
    out = dit.dit_swiglu(inp)
    sync()
    assert_close(out, oracle.swiglu(bits(inp), threads=8), f"swiglu {M}x{F}")


def test_swiglu_saturation_and_hand_values():
    a = [1, -1, 2, 20, -20, 0, 100, -100, 0.5, 1000, -1000, 3e38, -3e38, 88, -88, 89, -89, 1e-3, -1e-3, 60]
    b = [2, 1, 0.5, 1, 1, 5, 1, 1, -3, 1, 1, 1, 1, 1, 1, 1, 1, 7, 7, -2]
    F = 24  # multiple of 8; pad the rest with zeros
    row_a = a + [0.0] * (F - len(a))
    row_b = b + [0.0] * (F - len(b))
    inp = torch.tensor([row_a + row_b], dtype=torch.float32).to(torch.bfloat16).to(DEV)
    out = dit.dit_swiglu(inp)
    sync()
    assert torch.isfinite(out.float()).all()
    assert_close(out, oracle.swiglu(bits(inp)), "swiglu saturation")


def test_swiglu_deterministic():
    inp = randn_bf16((300, 2 * 16384), seed=61, scale=3.0)
    a = dit.dit_swiglu(inp)
    b = dit.dit_swiglu(inp)
    sync()
    assert torch.equal(a, b)


# --------------------------------------------------------------------------- QK RMSNorm + RoPE

QK_SHAPES = [
    (1, 33, 32, 128, (16, 56, 56)),
    (2, 17, 4, 64, (16, 24, 24)),
    (1, 9, 3, 256, (64, 96, 96)),
    (1, 5, 2, 8, (2, 2, 4)),
    (1, 7, 5, 16, (4, 6, 6)),
    (1, 4, 7, 32, (8, 12, 12)),
    (1, 3, 1, 128, (128, 0, 0)),
    (2, 65, 32, 128, (16, 56, 56)),
    (1, 1, 48, 128, (16, 56, 56)),
    (1, 6, 128, 64, (16, 24, 24)),
]


def random_positions(N, seed, hi=480):
    g = torch.Generator().manual_seed(seed)
    pos = torch.randint(0, hi, (N, 3), generator=g, dtype=torch.int32)
    pos[0] = 0
    if N > 1:
        pos[-1] = torch.tensor([479, 0, 0], dtype=torch.int32)
    return pos


@pytest.mark.parametrize("B,N,H,Dh,bands", QK_SHAPES)
def test_qk_shapes(B, N, H, Dh, bands):
    q = randn_bf16((B, N, H, Dh), seed=N * H + Dh)
    k = randn_bf16((B, N, H, Dh), seed=N * H + Dh + 1)
    wq, wk = weights(Dh, 71), weights(Dh, 72)
    pos = random_positions(N, seed=N + H)
    qo, ko = dit.dit_qk_rmsnorm_rope3d(q, k, wq, wk, pos.to(DEV), bands)
    sync()
    qr, kr = oracle.qk_rmsnorm_rope3d(bits(q), bits(k), bits(wq), bits(wk), pos.numpy(), bands, threads=8)
    assert_close(qo, qr, f"q {B}x{N}x{H}x{Dh}")
    assert_close(ko, kr, f"k {B}x{N}x{H}x{Dh}")


QK_LAYOUT_SHAPES = [(1, 33, 32, 128, (16, 56, 56), 3), (2, 17, 4, 64, (16, 24, 24), 3), (1, 9, 3, 256, (64, 96, 96), 2),
                    (2, 7, 5, 16, (4, 6, 6), 4), (1, 5, 48, 128, (16, 56, 56), 3)]


@pytest.mark.parametrize("B,N,H,Dh,bands,parts", QK_LAYOUT_SHAPES)
@pytest.mark.parametrize("head_major", [True, False])
def test_qk_layout_fused_qkv(B, N, H, Dh, bands, parts, head_major):
    """q and k read out of a [B,N,parts*H*Dh] projection; outputs head- or token-major."""
    qkv = randn_bf16((B, N, parts * H * Dh), seed=N * H + Dh + parts)
    qkv[..., 2 * H * Dh:] = float("nan")  # anything past k (e.g. v) must not be read
    wq, wk = weights(Dh, 141), weights(Dh, 142)
    pos = random_positions(N, seed=N + 7)
    qo, ko = dit.dit_qk_rmsnorm_rope3d_layout(qkv, H, Dh, wq, wk, pos.to(DEV), bands, head_major=head_major)
    sync()
    flat = bits(qkv).ravel()
    qr, kr = oracle.qk_rmsnorm_rope3d_layout(flat, flat[H * Dh:], bits(wq), bits(wk), pos.numpy(), bands,
                                             B, N, H, Dh, parts * H * Dh, 1 if head_major else 0)
    assert_close(qo, qr, f"q layout {B}x{N}x{H}x{Dh} hm={head_major}")
    assert_close(ko, kr, f"k layout {B}x{N}x{H}x{Dh} hm={head_major}")


# (B, N, H, Dh, bands, extra values of padding after each head plane)
QK_PLANE_CASES = [(1, 33, 32, 128, (16, 56, 56), 64), (2, 17, 4, 64, (16, 24, 24), 8), (1, 130, 5, 16, (4, 6, 6), 2048),
                  (2, 65, 32, 128, (16, 56, 56), 128), (1, 7, 3, 256, (64, 96, 96), 0)]


def padded_head_major(B, H, N, Dh, pad):
    """[B,H,N,Dh] views into [B,H,N*Dh+pad] buffers pre-filled with NaN bits."""
    buf = torch.full((B, H, N * Dh + pad), float("nan"), dtype=torch.bfloat16, device=DEV)
    return buf, buf[..., :N * Dh].view(B, H, N, Dh)


@pytest.mark.parametrize("B,N,H,Dh,bands,pad", QK_PLANE_CASES)
@pytest.mark.parametrize("with_means", [False, True])
def test_qk_head_major_padded_planes(B, N, H, Dh, bands, pad, with_means):
    """Head planes pad apart: values as the oracle's head-major layout, padding never written."""
    qkv = randn_bf16((B, N, 3 * H * Dh), seed=N * H + Dh + pad)
    qkv[..., 2 * H * Dh:] = float("nan")
    wq, wk = weights(Dh, 161), weights(Dh, 162)
    pos = random_positions(N, seed=N + 9).to(DEV)
    qbuf, qv = padded_head_major(B, H, N, Dh, pad)
    kbuf, kv = padded_head_major(B, H, N, Dh, pad)
    if with_means:
        qo, ko, qp, kp = dit.dit_qk_rmsnorm_rope3d_pool(qkv, None, wq, wk, pos, bands, head_major=True, heads=(H, Dh),
                                                        q_out=qv, k_out=kv)
        packed = dit.dit_qk_rmsnorm_rope3d_pool(qkv, None, wq, wk, pos, bands, head_major=True, heads=(H, Dh))
    else:
        qo, ko = dit.dit_qk_rmsnorm_rope3d_layout(qkv, H, Dh, wq, wk, pos, bands, head_major=True, q_out=qv,
                                                  k_out=kv)
        packed = dit.dit_qk_rmsnorm_rope3d_layout(qkv, H, Dh, wq, wk, pos, bands, head_major=True)
    sync()
    assert qo.data_ptr() == qv.data_ptr() and ko.data_ptr() == kv.data_ptr()
    flat = bits(qkv).ravel()
    qr, kr = oracle.qk_rmsnorm_rope3d_layout(flat, flat[H * Dh:], bits(wq), bits(wk), pos.cpu().numpy(), bands,
                                             B, N, H, Dh, 3 * H * Dh, 1)
    assert_close(qv.contiguous(), qr, f"q padded {B}x{N}x{H}x{Dh}+{pad}")
    assert_close(kv.contiguous(), kr, f"k padded {B}x{N}x{H}x{Dh}+{pad}")
    # the same bits as the packed layout, and the padding untouched (still NaN bits)
    assert torch.equal(qv, packed[0]) and torch.equal(kv, packed[1])
    if with_means:
        assert torch.equal(qp, packed[2]) and torch.equal(kp, packed[3])
    for buf in (qbuf, kbuf):
        assert torch.isnan(buf[..., N * Dh:].float()).all(), "padding between head planes was written"


def test_qk_layout_plain_case_equals_qk():
    B, N, H, Dh = 2, 65, 32, 128
    q = randn_bf16((B, N, H, Dh), seed=151)
    k = randn_bf16((B, N, H, Dh), seed=152)
    wq, wk = weights(Dh, 153), weights(Dh, 154)
    pos = random_positions(N, seed=155).to(DEV)
    a = dit.dit_qk_rmsnorm_rope3d(q, k, wq, wk, pos, (16, 56, 56))
    qkv = torch.cat([q.reshape(B, N, -1), k.reshape(B, N, -1)], dim=-1).contiguous()
    b = dit.dit_qk_rmsnorm_rope3d_layout(qkv, H, Dh, wq, wk, pos, (16, 56, 56), head_major=False)
    c = dit.dit_qk_rmsnorm_rope3d_layout(qkv, H, Dh, wq, wk, pos, (16, 56, 56), head_major=True)
    sync()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(a[0].transpose(1, 2), c[0]) and torch.equal(a[1].transpose(1, 2), c[1])


def test_qk_heavy_tails_and_large_positions():
    B, N, H, Dh = 1, 64, 32, 128
    g = torch.Generator(device=DEV).manual_seed(81)
    qf = torch.randn((B, N, H * Dh), generator=g, device=DEV)
    kf = torch.randn((B, N, H * Dh), generator=g, device=DEV)
    heavy = torch.randperm(H * Dh, generator=torch.Generator().manual_seed(82))[:205].to(DEV)
    qf[..., heavy] *= 20.0
    kf[..., heavy] *= 20.0
    q = qf.reshape(B, N, H, Dh).to(torch.bfloat16)
    k = kf.reshape(B, N, H, Dh).to(torch.bfloat16)
    wq, wk = weights(Dh, 83), weights(Dh, 84)
    pos = torch.stack([torch.arange(N) * 7 + 30, torch.arange(N) % 48, 83 - torch.arange(N) % 84], 1).to(torch.int32)
    qo, ko = dit.dit_qk_rmsnorm_rope3d(q, k, wq, wk, pos.to(DEV), (16, 56, 56))
    sync()
    qr, kr = oracle.qk_rmsnorm_rope3d(bits(q), bits(k), bits(wq), bits(wk), pos.numpy(), (16, 56, 56))
    assert_close(qo, qr, "q heavy")
    assert_close(ko, kr, "k heavy")


def test_qk_in_place_and_deterministic():
    B, N, H, Dh = 2, 129, 32, 128
    q = randn_bf16((B, N, H, Dh), seed=91)
    k = randn_bf16((B, N, H, Dh), seed=92)
    wq, wk = weights(Dh, 93), weights(Dh, 94)
    pos = random_positions(N, seed=95).to(DEV)
    a = dit.dit_qk_rmsnorm_rope3d(q, k, wq, wk, pos, (16, 56, 56))
    b = dit.dit_qk_rmsnorm_rope3d(q, k, wq, wk, pos, (16, 56, 56))
    qi, ki = q.clone(), k.clone()
    dit.dit_qk_rmsnorm_rope3d(qi, ki, wq, wk, pos, (16, 56, 56), q_out=qi, k_out=ki)
    sync()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(a[0], qi) and torch.equal(a[1], ki)


def test_qk_position_zero_is_plain_rmsnorm():
    B, N, H, Dh = 1, 4, 8, 128
    q = randn_bf16((B, N, H, Dh), seed=96)
    w = weights(Dh, 97)
    pos = torch.zeros((N, 3), dtype=torch.int32, device=DEV)
    qo, _ = dit.dit_qk_rmsnorm_rope3d(q, q, w, w, pos, (16, 56, 56))
    sync()
    v = q.double().cpu()
    ref = v / torch.sqrt((v * v).mean(-1, keepdim=True) + 1e-6) * w.double().cpu()
    assert_close(qo, ref.numpy(), "rmsnorm at position 0")


# --------------------------------------------------------------------------- binding errors on the device

def test_binding_errors_raise_before_launch():
    x = torch.zeros((1, 4, 12), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros((1, 12), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(dit.DitError) as err:
        dit.dit_adaln_modulate(x, v, v)
    assert err.value.status == dit.DIT_ERR_SHAPE
    q = torch.zeros((1, 2, 1, 96), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((96,), dtype=torch.bfloat16, device=DEV)
    pos = torch.zeros((2, 3), dtype=torch.int32, device=DEV)
    with pytest.raises(dit.DitError):
        dit.dit_qk_rmsnorm_rope3d(q, q, w, w, pos, (32, 32, 32))
    sync()


# --------------------------------------------------------------------------- full-size workloads, sampled rows

def sample_rows(R, N, B, n_extra, seed, count=48):
    g = np.random.default_rng(seed)
    rows = set(g.choice(R, size=min(count, R), replace=False).tolist())
    rows |= {0, 1, R - 2, R - 1}
    for b in range(1, B):
        rows |= {b * N - 1, b * N}
    if n_extra:
        for b in range(B):
            rows |= {b * N + N - n_extra, b * N + N - 1, b * N + N - n_extra // 2}
    return sorted(r for r in rows if 0 <= r < R)


def contiguous_runs(rows):
    """Group sorted row indices into (start, length) runs."""
    runs, start, prev = [], rows[0], rows[0]
    for r in rows[1:]:
        if r != prev + 1:
            runs.append((start, prev - start + 1))
            start = r
        prev = r
    runs.append((start, prev - start + 1))
    return runs


@pytest.mark.parametrize("name", ["lowres", "full5s", "full10s", "batch2"])
def test_full_workload_sampled(name):
    wl = si.WORKLOADS[name]
    B, N, R = wl.B, wl.N, wl.R
    rows = sample_rows(R, N, B, wl.n_extra, seed=sum(map(ord, name)))
    print(f"[{name}] rows={R} sampled={len(rows)}", flush=True)

    pos = dit.dit_packed_positions(*wl.grid, wl.n_extra, device=DEV)
    pos_ref = oracle.packed_positions(*wl.grid, wl.n_extra)
    sync()
    assert np.array_equal(pos.cpu().numpy(), pos_ref)

    def row_of(t, r):
        return t.reshape(R, -1)[r]

    # AdaLN
    ins = si.op_inputs(wl, "adaln", device=DEV)
    y = dit.dit_adaln_modulate(ins["x_mod"], ins["shift"], ins["scale"], eps=wl.eps)
    sync()
    assert torch.isfinite(y).all()
    for r in rows:
        b = r // N
        ref = oracle.adaln_modulate(bits(row_of(ins["x_mod"], r)).reshape(1, 1, -1), bits(ins["shift"][b:b + 1]),
                                    bits(ins["scale"][b:b + 1]), eps=wl.eps)
        assert_close(row_of(y, r), ref.reshape(-1), f"{name} adaln row {r}")
    del ins, y

    # gated residual
    ins = si.op_inputs(wl, "residual", device=DEV)
    out = dit.dit_gated_residual(ins["res_x"], ins["res_y"], ins["gate"])
    sync()
    assert torch.isfinite(out).all()
    for r in rows:
        b = r // N
        ref = oracle.gated_residual(bits(row_of(ins["res_x"], r)).reshape(1, 1, -1),
                                    bits(row_of(ins["res_y"], r)).reshape(1, 1, -1), bits(ins["gate"][b:b + 1]))
        assert_close(row_of(out, r), ref.reshape(-1), f"{name} residual row {r}")
    del ins, out

    # Cache-DiT residual change over the whole packed sequence (the residual
    # inputs stand in for the current and cached boundary residuals)
    ins = si.make_inputs(wl, device=DEV, names=("res_x", "res_y"))
    stat = dit.dit_residual_change(ins["res_x"], ins["res_y"])
    sync()
    check_change(stat, oracle.residual_change(bits(ins["res_x"]), bits(ins["res_y"])), f"{name} residual change")
    del ins, stat

    # fused gated residual + AdaLN (residual inputs, AdaLN vectors)
    ins = si.make_inputs(wl, device=DEV, names=("res_x", "res_y", "gate", "shift", "scale"))
    x_out, z = dit.dit_gated_residual_adaln(ins["res_x"], ins["res_y"], ins["gate"], ins["shift"], ins["scale"],
                                            eps=wl.eps)
    sync()
    assert torch.isfinite(x_out).all() and torch.isfinite(z).all()
    for r in rows:
        b = r // N
        xr, zr = oracle.gated_residual_adaln(
            bits(row_of(ins["res_x"], r)).reshape(1, 1, -1), bits(row_of(ins["res_y"], r)).reshape(1, 1, -1),
            bits(ins["gate"][b:b + 1]), bits(ins["shift"][b:b + 1]), bits(ins["scale"][b:b + 1]), eps=wl.eps)
        assert_close(row_of(x_out, r), xr.reshape(-1), f"{name} fused x_out row {r}")
        assert_close(row_of(z, r), zr.reshape(-1), f"{name} fused z row {r}")
    del ins, x_out, z

    # SwiGLU (the largest tensors: check runs of rows at once)
    ins = si.op_inputs(wl, "swiglu", device=DEV)
    sw = dit.dit_swiglu(ins["swiglu_in"])
    sync()
    assert torch.isfinite(sw).all()
    for start, length in contiguous_runs(rows):
        ref = oracle.swiglu(bits(ins["swiglu_in"][start:start + length]), threads=8)
        assert_close(sw[start:start + length], ref, f"{name} swiglu rows {start}+{length}")
    del ins, sw
    torch.cuda.empty_cache()

    # QK RMSNorm + 3D RoPE
    ins = si.op_inputs(wl, "qk", device=DEV)
    qo, ko = dit.dit_qk_rmsnorm_rope3d(ins["q"], ins["k"], ins["wq"], ins["wk"], pos, wl.bands,
                                       theta=wl.theta, eps=wl.eps)
    sync()
    assert torch.isfinite(qo).all() and torch.isfinite(ko).all()
    qf, kf = ins["q"].reshape(R, wl.H, wl.Dh), ins["k"].reshape(R, wl.H, wl.Dh)
    qof, kof = qo.reshape(R, wl.H, wl.Dh), ko.reshape(R, wl.H, wl.Dh)
    for r in rows:
        n = r % N
        qr, kr = oracle.qk_rmsnorm_rope3d(bits(qf[r]).reshape(1, 1, wl.H, wl.Dh), bits(kf[r]).reshape(1, 1, wl.H, wl.Dh),
                                          bits(ins["wq"]), bits(ins["wk"]), pos_ref[n:n + 1], wl.bands, wl.theta, wl.eps)
        assert_close(qof[r], qr[0, 0], f"{name} q row {r}")
        assert_close(kof[r], kr[0, 0], f"{name} k row {r}")
    del qo, ko
    # The same op on a fused QKV projection buffer with head-major outputs.
    qkv = torch.cat([ins["q"].reshape(B, N, -1), ins["k"].reshape(B, N, -1),
                     ins["q"].reshape(B, N, -1)], dim=-1)  # [q | k | a stand-in for v]
    del ins["q"], ins["k"]
    torch.cuda.empty_cache()
    qo, ko = dit.dit_qk_rmsnorm_rope3d_layout(qkv, wl.H, wl.Dh, ins["wq"], ins["wk"], pos, wl.bands,
                                              head_major=True, theta=wl.theta, eps=wl.eps)
    sync()
    assert torch.isfinite(qo).all() and torch.isfinite(ko).all()
    S = qkv.shape[-1]
    qkv_rows = qkv.reshape(R, S)
    for r in rows[:24]:
        b, n = divmod(r, N)
        flat = bits(qkv_rows[r])
        qr, kr = oracle.qk_rmsnorm_rope3d_layout(flat, flat[wl.H * wl.Dh:], bits(ins["wq"]), bits(ins["wk"]),
                                                 pos_ref[n:n + 1], wl.bands, 1, 1, wl.H, wl.Dh, S, 1, wl.theta, wl.eps)
        assert_close(qo[b, :, n], qr[0, :, 0], f"{name} q head-major row {r}")
        assert_close(ko[b, :, n], kr[0, :, 0], f"{name} k head-major row {r}")
    # Every element: the head-major outputs are the token-major ones of the
    # same buffer, transposed (same arithmetic per element, another layout).
    qt, kt = dit.dit_qk_rmsnorm_rope3d_layout(qkv, wl.H, wl.Dh, ins["wq"], ins["wk"], pos, wl.bands,
                                              head_major=False, theta=wl.theta, eps=wl.eps)
    sync()
    assert torch.equal(qo.permute(0, 2, 1, 3), qt), f"{name} head-major q differs from token-major q transposed"
    assert torch.equal(ko.permute(0, 2, 1, 3), kt), f"{name} head-major k differs from token-major k transposed"
    del qt, kt
    del ins, qo, ko, qkv, qkv_rows
    torch.cuda.empty_cache()
    # Rows of a sample are the same computation for every sample: the same
    # inputs give the same outputs wherever they sit in the batch.
    if B > 1:
        x = si.op_inputs(wl, "adaln", device=DEV)
        x["x_mod"][1, :5] = x["x_mod"][0, :5]
        x["shift"][1] = x["shift"][0]
        x["scale"][1] = x["scale"][0]
        y = dit.dit_adaln_modulate(x["x_mod"], x["shift"], x["scale"], eps=wl.eps)
        sync()
        assert torch.equal(y[0, :5], y[1, :5])
        del x, y
    torch.cuda.empty_cache()
