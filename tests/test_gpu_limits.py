"""The chain's entry points at the largest sizes the C ABI accepts.

At 2^24 - 1 rows (the ABI's row limit) the one-row-per-wave kernels run
their largest grids, and the gated residual's grid is capped at 2^23 - 1
workgroups, so its workgroups loop over the remaining (row, segment) tiles.
The row width is the smallest allowed (8) so the tensors stay small.  A
second case puts SwiGLU past 2^24 tiles, where its grid is capped too; that
needs about 104 GB of device memory and is skipped when less is free.  Sampled
rows -- the first, the middle, those around the cap and the last -- are
checked against the fp64 oracle to the usual bound.
"""
import numpy as np
import pytest
import torch

import oracle
import video_diffusion_transformer_dit_amd as dit
from parity_util import assert_close
from synthetic_inputs import bits

pytestmark = pytest.mark.gpu

DEV = "cuda"
MAX_ROWS = (1 << 24) - 1


def randn_bf16(shape, seed, scale=1.0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV) * scale).to(torch.bfloat16)


def sampled(n, around=()):
    parts = [np.arange(0, 256), np.arange(n // 2 - 128, n // 2 + 128), np.arange(n - 256, n)]
    parts += [np.arange(a - 128, a + 128) for a in around]
    idx = np.unique(np.concatenate(parts))
    return idx[(idx >= 0) & (idx < n)]


def rows_of(t, idx, width):
    return t.reshape(-1, width).index_select(0, torch.as_tensor(idx, device=t.device))


@pytest.fixture(autouse=True)
def _release_memory():
    torch.cuda.empty_cache()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B", [1, 2])
def test_row_limit_streaming_ops(B):
    N = MAX_ROWS // B
    R, D = B * N, 8
    print(f"[limits] B={B} N={N} rows={R} D={D}", flush=True)
    x, y = randn_bf16((B, N, D), 1), randn_bf16((B, N, D), 2)
    shift, scale, gate = (randn_bf16((B, D), s, 0.1) for s in (3, 4, 5))
    sw_in = randn_bf16((R, 2 * D), 6, 2.0)

    y_ad = dit.dit_adaln_modulate(x, shift, scale)
    res = dit.dit_gated_residual(x, y, gate)  # R tiles > 2^23 - 1: workgroups loop
    x_out, z = dit.dit_gated_residual_adaln(x, y, gate, shift, scale)
    sw = dit.dit_swiglu(sw_in)
    torch.cuda.synchronize()

    idx = sampled(R, around=((1 << 23) - 1, 2 * ((1 << 23) - 1), N))
    hx, hy, hsw = bits(rows_of(x, idx, D)), bits(rows_of(y, idx, D)), bits(rows_of(sw_in, idx, 2 * D))
    samples = idx // N
    for b in range(B):
        sel = np.nonzero(samples == b)[0]
        n = sel.size
        xs, ys = hx[sel].reshape(1, n, D), hy[sel].reshape(1, n, D)
        sh, sc, g = bits(shift[b:b + 1]), bits(scale[b:b + 1]), bits(gate[b:b + 1])
        rows_b = idx[sel]
        assert_close(rows_of(y_ad, rows_b, D), oracle.adaln_modulate(xs, sh, sc).reshape(n, D), f"adaln b={b}")
        assert_close(rows_of(res, rows_b, D), oracle.gated_residual(xs, ys, g).reshape(n, D), f"residual b={b}")
        xo_ref, z_ref = oracle.gated_residual_adaln(xs, ys, g, sh, sc)
        assert_close(rows_of(x_out, rows_b, D), xo_ref.reshape(n, D), f"fused x_out b={b}")
        assert_close(rows_of(z, rows_b, D), z_ref.reshape(n, D), f"fused z b={b}")
    assert_close(rows_of(sw, idx, D), oracle.swiglu(hsw), "swiglu")


def test_row_limit_positions_and_qk():
    T, Hg, Wg, extra = 255, 256, 256, 65535
    N = T * Hg * Wg + extra
    assert N == MAX_ROWS
    H, Dh, bands = 1, 8, (2, 2, 4)
    print(f"[limits] positions and QK over N={N} tokens", flush=True)
    pos = dit.dit_packed_positions(T, Hg, Wg, extra)
    q, k = randn_bf16((1, N, H, Dh), 11), randn_bf16((1, N, H, Dh), 12)
    wq = (1 + 0.02 * randn_bf16((Dh,), 13).float()).to(torch.bfloat16)
    wk = (1 + 0.02 * randn_bf16((Dh,), 14).float()).to(torch.bfloat16)
    qo, ko = dit.dit_qk_rmsnorm_rope3d(q, k, wq, wk, pos, bands)
    qkv = torch.cat([q.reshape(1, N, H * Dh), k.reshape(1, N, H * Dh)], dim=2)
    qh, kh = dit.dit_qk_rmsnorm_rope3d_layout(qkv, H, Dh, wq, wk, pos, bands, head_major=True)
    torch.cuda.synchronize()

    idx = sampled(N, around=(T * Hg * Wg,))
    pos_ref = oracle.packed_positions(T, Hg, Wg, extra)
    t_idx = torch.as_tensor(idx, device=DEV)
    assert np.array_equal(pos.index_select(0, t_idx).cpu().numpy(), pos_ref[idx])
    hq = bits(rows_of(q, idx, H * Dh)).reshape(1, idx.size, H, Dh)
    hk = bits(rows_of(k, idx, H * Dh)).reshape(1, idx.size, H, Dh)
    q_ref, k_ref = oracle.qk_rmsnorm_rope3d(hq, hk, bits(wq), bits(wk), pos_ref[idx], bands)
    n = idx.size
    assert_close(rows_of(qo, idx, H * Dh), q_ref.reshape(n, H * Dh), "q token-major")
    assert_close(rows_of(ko, idx, H * Dh), k_ref.reshape(n, H * Dh), "k token-major")
    # head-major [1, H, N, Dh] with H = 1 holds the same rows
    assert_close(rows_of(qh, idx, Dh), q_ref.reshape(n, Dh), "q head-major")
    assert_close(rows_of(kh, idx, Dh), k_ref.reshape(n, Dh), "k head-major")


def test_swiglu_past_the_grid_cap():
    M, F = (1 << 23) + 8, 2056  # 257 vectors per output row: 5 segments of 64, 5 * (2^23 + 8) tiles
    need = M * 3 * F * 2
    free, _ = torch.cuda.mem_get_info()
    if free < need + (16 << 30):
        pytest.skip(f"needs {need / 1e9:.0f} GB of free device memory, {free / 1e9:.0f} GB free")
    print(f"[limits] swiglu M={M} F={F} ({need / 1e9:.0f} GB)", flush=True)
    inp = torch.empty((M, 2 * F), dtype=torch.bfloat16, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(21)
    step = 1 << 18  # 4 GB of fp32 draws at a time
    for r0 in range(0, M, step):
        r1 = min(M, r0 + step)
        inp[r0:r1].copy_((torch.randn((r1 - r0, 2 * F), generator=g, device=DEV) * 2.0).to(torch.bfloat16))
    out = dit.dit_swiglu(inp)
    torch.cuda.synchronize()
    # tiles from 2^24 - 1 on are a second tile of a workgroup (rows from (2^24 - 1) // 5 on), from
    # 2 * (2^24 - 1) on a third
    idx = sampled(M, around=(((1 << 24) - 1) // 5, 2 * ((1 << 24) - 1) // 5))
    assert_close(rows_of(out, idx, F), oracle.swiglu(bits(rows_of(inp, idx, 2 * F))), "swiglu past the cap")
    del inp, out


def test_width_limits_streaming_ops():
    W = 1 << 24  # the widest row SwiGLU, the gated residual and the residual change accept
    print(f"[limits] rows {W} wide", flush=True)
    sw_in = randn_bf16((2, 2 * W), 31, 2.0)
    sw = dit.dit_swiglu(sw_in)
    x, y = randn_bf16((1, 2, W), 32), randn_bf16((1, 2, W), 33)
    gate = randn_bf16((1, W), 34, 0.1)
    res = dit.dit_gated_residual(x, y, gate)
    change = dit.dit_residual_change(x, y)
    torch.cuda.synchronize()
    assert_close(sw, oracle.swiglu(bits(sw_in)), "swiglu 2^24 wide")
    assert_close(res, oracle.gated_residual(bits(x), bits(y), bits(gate)), "residual 2^24 wide")
    ref = oracle.residual_change(bits(x), bits(y))
    got = change.cpu().numpy()
    # fp32 sums over each 8-value vector, fp64 above: relative error below 8 * 2^-24
    assert np.allclose(got, ref, rtol=2e-6, atol=0.0), (got, ref)


@pytest.mark.parametrize("head_major", [False, True])
def test_head_row_limit_qk(head_major):
    B, N, H, Dh, bands = 1, 67, 256, 256, (64, 96, 96)  # H * Dh = 65536, the largest head row
    print(f"[limits] QK with H*Dh={H * Dh}, head_major={head_major}", flush=True)
    pos = dit.dit_packed_positions(1, 1, N - 3, 3)
    q, k = randn_bf16((B, N, H, Dh), 41), randn_bf16((B, N, H, Dh), 42)
    wq = (1 + 0.02 * randn_bf16((Dh,), 43).float()).to(torch.bfloat16)
    wk = (1 + 0.02 * randn_bf16((Dh,), 44).float()).to(torch.bfloat16)
    qo, ko = dit.dit_qk_rmsnorm_rope3d(q, k, wq, wk, pos, bands)
    qkv = torch.cat([q.reshape(B, N, H * Dh), k.reshape(B, N, H * Dh)], dim=2)
    ql, kl = dit.dit_qk_rmsnorm_rope3d_layout(qkv, H, Dh, wq, wk, pos, bands, head_major=head_major)
    qp_out, kp_out, qp, kp = dit.dit_qk_rmsnorm_rope3d_pool(q, k, wq, wk, pos, bands, head_major=head_major)
    torch.cuda.synchronize()
    pos_ref = oracle.packed_positions(1, 1, N - 3, 3)
    q_ref, k_ref = oracle.qk_rmsnorm_rope3d(bits(q), bits(k), bits(wq), bits(wk), pos_ref, bands)
    assert_close(qo, q_ref, "q")
    assert_close(ko, k_ref, "k")
    t = (lambda a: a.transpose(0, 2, 1, 3)) if head_major else (lambda a: a)
    assert_close(ql, t(q_ref), "q layout")
    assert_close(kl, t(k_ref), "k layout")
    # the fused pooling writes the same q', k' and the 64-token block means of the stored values
    assert torch.equal(qp_out, ql) and torch.equal(kp_out, kl)
    qo_tm = qp_out.permute(0, 2, 1, 3).contiguous() if head_major else qp_out
    ko_tm = kp_out.permute(0, 2, 1, 3).contiguous() if head_major else kp_out
    assert_close(qp, oracle.subblock_pool(bits(qo_tm)), "q block means")
    assert_close(kp, oracle.subblock_pool(bits(ko_tm)), "k block means")


def test_sample_limit():
    B = 65535  # the most samples a call accepts (samples index a grid dimension)
    print(f"[limits] B={B} samples", flush=True)
    from subblock_checks import pool_bound

    # routing on exact means (a 1/8 grid: every score is exact in fp32), 3 blocks of Dh 16 per sample
    rng = np.random.default_rng(7)
    qp = rng.integers(-8, 9, size=(B, 1, 3, 16)) / 8.0
    kp = rng.integers(-8, 9, size=(B, 1, 3, 16)) / 8.0
    kept, scores = dit.dit_subblock_route(torch.from_numpy(qp).float().to(DEV), torch.from_numpy(kp).float().to(DEV),
                                          keep=2)
    # block means over 65 tokens per sample (a ragged block of one token)
    q = randn_bf16((B, 65, 1, 16), 51)
    k = randn_bf16((B, 65, 1, 16), 52)
    qm, km = dit.dit_subblock_pool(q, k)
    # the residual change and AdaLN with one short row per sample
    r, rc = randn_bf16((B, 2, 8), 53), randn_bf16((B, 2, 8), 54, 0.9)
    change = dit.dit_residual_change(r, rc)
    x = randn_bf16((B, 1, 8), 55)
    shift, scale = randn_bf16((B, 8), 56, 0.1), randn_bf16((B, 8), 57, 0.1)
    y = dit.dit_adaln_modulate(x, shift, scale)
    torch.cuda.synchronize()

    s_ref = oracle.subblock_scores(qp, kp)
    assert np.array_equal(scores[..., :3].cpu().numpy().astype(np.float64), s_ref)
    assert np.array_equal(kept.cpu().numpy(), oracle.subblock_topk(s_ref, 2))
    for got, src in ((qm, q), (km, k)):
        ref = oracle.subblock_pool(bits(src))
        assert np.all(np.abs(got.cpu().numpy().astype(np.float64) - ref) <= pool_bound(bits(src), ref))
    ref = oracle.residual_change(bits(r), bits(rc))
    assert np.allclose(change.cpu().numpy(), ref, rtol=2e-6, atol=0.0)
    assert_close(y, oracle.adaln_modulate(bits(x), bits(shift), bits(scale), threads=8), "adaln")
