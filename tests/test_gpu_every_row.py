"""Every row of every workload against the fp64 oracle.

For each of the five workloads (the tiny case, the low-resolution stage, the
1344x768 5 s and 10 s sequences, and the heavy-tailed two-sample batch) each
op of the chain runs once over all R tokens through the C ABI, as the
benchmark launches it, and every output row is then checked against the
oracle, 1024 rows at a time: AdaLN modulate, gated residual, the fused
residual -> AdaLN (both outputs), SwiGLU, and QK RMSNorm + 3D RoPE (q' and k').
QK is also run from a fused QKV buffer into head-major outputs, which must be
the token-major outputs transposed, bit for bit.  The bound is the
per-element |gpu - oracle| <= 1e-2 + 8e-3 |oracle| of the other parity tests;
each test prints the rows it checked and the worst |err| / bound.
"""
import os
import time

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
import video_diffusion_transformer_dit_amd as dit
from parity_util import worst_ratio_threaded
from synthetic_inputs import bits

pytestmark = pytest.mark.gpu

DEV = "cuda"
CHUNK = 1024
THREADS = max(1, min(16, os.cpu_count() or 1))  # the host share of one GPU


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    dit.load_library()  # raises if libdit_ops.so is missing: no fallback path exists
    torch.cuda.synchronize()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def host_rows(t, R, r0, r1):
    """Rows r0..r1-1 of a [R, ...] view as raw bf16 bits on the host."""
    return bits(t.reshape(R, -1)[r0:r1])


def gpu_rows(t, R, r0, r1):
    """The same rows of a GPU output, widened exactly to fp32 on the host."""
    return t.reshape(R, -1)[r0:r1].float().cpu().numpy()


def sample_runs(r0, r1, N):
    """Split rows r0..r1-1 into runs that stay inside one sample: (b, first row, end row)."""
    r = r0
    while r < r1:
        b = r // N
        end = min(r1, (b + 1) * N)
        yield b, r, end
        r = end


class Worst:
    def __init__(self):
        self.ratio = {}
        self.rows = 0

    def add(self, what, gpu, ref):
        self.ratio[what] = max(self.ratio.get(what, 0.0), worst_ratio_threaded(gpu, ref, THREADS))

    def report(self, name, op, R, t0):
        text = ", ".join(f"{k} {v:.4f}" for k, v in self.ratio.items())
        print(f"[every-row] {name} {op}: rows checked {self.rows} of {R}; worst |err|/bound: {text} "
              f"({time.perf_counter() - t0:.1f} s)", flush=True)
        assert self.rows == R
        bad = {k: v for k, v in self.ratio.items() if not v <= 1.0}
        assert not bad, f"{name} {op}: outside the bound: {bad}"


WORKLOADS = ("tiny", "lowres", "full5s", "full10s", "batch2")


@pytest.mark.parametrize("name", WORKLOADS)
def test_every_row_adaln(name):
    wl = si.WORKLOADS[name]
    R, N = wl.R, wl.N
    print(f"[every-row] {name} adaln: {R} rows", flush=True)
    t0 = time.perf_counter()
    ins = si.op_inputs(wl, "adaln", device=DEV)
    y = dit.dit_adaln_modulate(ins["x_mod"], ins["shift"], ins["scale"], eps=wl.eps)
    torch.cuda.synchronize()
    shift, scale = bits(ins["shift"]), bits(ins["scale"])
    w = Worst()
    for c0 in range(0, R, CHUNK):
        for b, r0, r1 in sample_runs(c0, min(R, c0 + CHUNK), N):
            n = r1 - r0
            ref = oracle.adaln_modulate(host_rows(ins["x_mod"], R, r0, r1).reshape(1, n, -1), shift[b:b + 1],
                                        scale[b:b + 1], eps=wl.eps, threads=THREADS)
            w.add("y", gpu_rows(y, R, r0, r1), ref.reshape(n, -1))
            w.rows += n
    w.report(name, "adaln", R, t0)


@pytest.mark.parametrize("name", WORKLOADS)
def test_every_row_gated_residual(name):
    wl = si.WORKLOADS[name]
    R, N = wl.R, wl.N
    print(f"[every-row] {name} residual: {R} rows", flush=True)
    t0 = time.perf_counter()
    ins = si.op_inputs(wl, "residual", device=DEV)
    out = dit.dit_gated_residual(ins["res_x"], ins["res_y"], ins["gate"])
    torch.cuda.synchronize()
    gate = bits(ins["gate"])
    w = Worst()
    for c0 in range(0, R, CHUNK):
        for b, r0, r1 in sample_runs(c0, min(R, c0 + CHUNK), N):
            n = r1 - r0
            ref = oracle.gated_residual(host_rows(ins["res_x"], R, r0, r1).reshape(1, n, -1),
                                        host_rows(ins["res_y"], R, r0, r1).reshape(1, n, -1), gate[b:b + 1],
                                        threads=THREADS)
            w.add("out", gpu_rows(out, R, r0, r1), ref.reshape(n, -1))
            w.rows += n
    w.report(name, "residual", R, t0)


@pytest.mark.parametrize("name", WORKLOADS)
def test_every_row_fused_residual_adaln(name):
    wl = si.WORKLOADS[name]
    R, N = wl.R, wl.N
    print(f"[every-row] {name} fused residual->adaln: {R} rows", flush=True)
    t0 = time.perf_counter()
    ins = si.make_inputs(wl, device=DEV, names=("res_x", "res_y", "gate", "shift", "scale"))
    x_out, z = dit.dit_gated_residual_adaln(ins["res_x"], ins["res_y"], ins["gate"], ins["shift"], ins["scale"],
                                            eps=wl.eps)
    torch.cuda.synchronize()
    gate, shift, scale = bits(ins["gate"]), bits(ins["shift"]), bits(ins["scale"])
    w = Worst()
    for c0 in range(0, R, CHUNK):
        for b, r0, r1 in sample_runs(c0, min(R, c0 + CHUNK), N):
            n = r1 - r0
            xr, zr = oracle.gated_residual_adaln(host_rows(ins["res_x"], R, r0, r1).reshape(1, n, -1),
                                                 host_rows(ins["res_y"], R, r0, r1).reshape(1, n, -1),
                                                 gate[b:b + 1], shift[b:b + 1], scale[b:b + 1], eps=wl.eps,
                                                 threads=THREADS)
            w.add("x_out", gpu_rows(x_out, R, r0, r1), xr.reshape(n, -1))
            w.add("z", gpu_rows(z, R, r0, r1), zr.reshape(n, -1))
            w.rows += n
    w.report(name, "fused residual->adaln", R, t0)


@pytest.mark.parametrize("name", WORKLOADS)
def test_every_row_swiglu(name):
    wl = si.WORKLOADS[name]
    R = wl.R
    print(f"[every-row] {name} swiglu: {R} rows", flush=True)
    t0 = time.perf_counter()
    ins = si.op_inputs(wl, "swiglu", device=DEV)
    sw = dit.dit_swiglu(ins["swiglu_in"])
    torch.cuda.synchronize()
    w = Worst()
    for r0 in range(0, R, CHUNK):
        r1 = min(R, r0 + CHUNK)
        ref = oracle.swiglu(host_rows(ins["swiglu_in"], R, r0, r1), threads=THREADS)
        w.add("out", gpu_rows(sw, R, r0, r1), ref)
        w.rows += r1 - r0
    w.report(name, "swiglu", R, t0)


@pytest.mark.parametrize("name", WORKLOADS)
def test_every_row_qk(name):
    wl = si.WORKLOADS[name]
    B, R, N, H, Dh = wl.B, wl.R, wl.N, wl.H, wl.Dh
    print(f"[every-row] {name} qk: {R} rows", flush=True)
    t0 = time.perf_counter()
    pos = dit.dit_packed_positions(*wl.grid, wl.n_extra, device=DEV)
    pos_ref = oracle.packed_positions(*wl.grid, wl.n_extra)
    ins = si.op_inputs(wl, "qk", device=DEV)
    qo, ko = dit.dit_qk_rmsnorm_rope3d(ins["q"], ins["k"], ins["wq"], ins["wk"], pos, wl.bands, theta=wl.theta,
                                       eps=wl.eps)
    torch.cuda.synchronize()
    assert np.array_equal(pos.cpu().numpy(), pos_ref), "positions differ from the oracle"
    wq, wk = bits(ins["wq"]), bits(ins["wk"])
    w = Worst()
    for c0 in range(0, R, CHUNK):
        for b, r0, r1 in sample_runs(c0, min(R, c0 + CHUNK), N):
            n = r1 - r0
            n0 = r0 - b * N
            qr, kr = oracle.qk_rmsnorm_rope3d(host_rows(ins["q"], R, r0, r1).reshape(1, n, H, Dh),
                                              host_rows(ins["k"], R, r0, r1).reshape(1, n, H, Dh), wq, wk,
                                              pos_ref[n0:n0 + n], wl.bands, wl.theta, wl.eps, threads=THREADS)
            w.add("q'", gpu_rows(qo, R, r0, r1), qr.reshape(n, -1))
            w.add("k'", gpu_rows(ko, R, r0, r1), kr.reshape(n, -1))
            w.rows += n
    # From a fused QKV buffer into head-major outputs: the same values, transposed.
    HD = H * Dh
    qkv = torch.empty((B, N, 3 * HD), dtype=torch.bfloat16, device=DEV)
    qkv[..., :HD].copy_(ins["q"].reshape(B, N, HD))
    qkv[..., HD:2 * HD].copy_(ins["k"].reshape(B, N, HD))
    qkv[..., 2 * HD:].copy_(ins["q"].reshape(B, N, HD))  # a stand-in for v
    del ins["q"], ins["k"]
    qh, kh = dit.dit_qk_rmsnorm_rope3d_layout(qkv, H, Dh, ins["wq"], ins["wk"], pos, wl.bands, head_major=True,
                                              theta=wl.theta, eps=wl.eps)
    torch.cuda.synchronize()
    assert torch.equal(qh.permute(0, 2, 1, 3), qo), f"{name}: head-major q' is not token-major q' transposed"
    assert torch.equal(kh.permute(0, 2, 1, 3), ko), f"{name}: head-major k' is not token-major k' transposed"
    w.report(name, "qk", R, t0)
