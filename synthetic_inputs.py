"""Seeded synthetic inputs for the fused DiT non-GEMM operator chain.

This module only draws random tensors of the right shapes and distributions.
It holds none of the operators' arithmetic, and it does not build token
positions (the HIP library and the oracle each build those themselves).  It is
shared by the tests, the smoke check and the benchmark, and feeds the HIP path
and the oracle the same bytes.

Workloads (shapes follow the latent grids of 1344x768 video at 24 fps, 5 s and
10 s, and the half-resolution first stage of a two-stage schedule; the text the
shapes come from names the model, resolution, frame rate and clip lengths but
prints no tensor shapes, so the grid arithmetic assumes 16x spatial and 4x
temporal latent compression):

  tiny     B=1, grid 2x4x4 (32 tokens), D=256, 4 heads x 64 (bands 16/24/24), F=512
  lowres   B=1, grid 31x24x42 (31,248 tokens), D=4096, 32 x 128 (16/56/56), F=16384
  full5s   B=1, grid 31x48x84 (124,992 tokens), same widths
  full10s  B=1, grid 61x48x84 (245,952 tokens) + 480 temporal-only extra tokens
  batch2   B=2, grid 31x48x84 per sample, heavy-tailed activations

Distributions: activations N(0, 1); AdaLN shift/scale and residual gate
N(0, 0.1) per sample; RMSNorm weights 1 + N(0, 0.02).  All are drawn in fp32
and rounded to bf16 by torch's round-to-nearest-even cast.  For heavy-tailed
workloads a seeded 5% subset of each activation tensor's last-dimension
channels is multiplied by 20 before the cast (the same subset for every row and
sample).

Every tensor has its own generator seeded from (seed, tensor index), so any
subset of tensors can be drawn and each is reproducible on its own.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

TENSOR_ORDER = (
    "x_mod", "shift", "scale",          # AdaLN modulate
    "res_x", "res_y", "gate",           # gated residual
    "swiglu_in",                        # SwiGLU
    "q", "k", "wq", "wk",               # QK RMSNorm + RoPE
)

OP_TENSORS = {
    "adaln": ("x_mod", "shift", "scale"),
    "residual": ("res_x", "res_y", "gate"),
    "swiglu": ("swiglu_in",),
    "qk": ("q", "k", "wq", "wk"),
}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    grid: tuple  # (T, Hg, Wg) latent grid of the video tokens
    n_extra: int  # temporal-only tokens appended after the video grid
    D: int  # hidden width (= H * Dh)
    H: int
    Dh: int
    bands: tuple  # RoPE band widths (t, h, w)
    F: int  # SwiGLU output width (input is 2F)
    heavy_tail: bool = False
    theta: float = 1e4
    eps: float = 1e-6
    description: str = ""

    @property
    def N(self) -> int:
        T, Hg, Wg = self.grid
        return T * Hg * Wg + self.n_extra

    @property
    def R(self) -> int:
        return self.B * self.N

    def shapes(self) -> dict:
        B, N, D, R = self.B, self.N, self.D, self.R
        return {
            "x_mod": (B, N, D), "shift": (B, D), "scale": (B, D),
            "res_x": (B, N, D), "res_y": (B, N, D), "gate": (B, D),
            "swiglu_in": (R, 2 * self.F),
            "q": (B, N, self.H, self.Dh), "k": (B, N, self.H, self.Dh),
            "wq": (self.Dh,), "wk": (self.Dh,),
        }


WORKLOADS = {
    "tiny": Workload("tiny", 1, (2, 4, 4), 0, 256, 4, 64, (16, 24, 24), 512,
                     description="tiny: B=1, grid 2x4x4 (32 tokens), hidden 256, 4x64 heads, SwiGLU 2x512->512"),
    "lowres": Workload("lowres", 1, (31, 24, 42), 0, 4096, 32, 128, (16, 56, 56), 16384,
                       description="low-res stage: B=1, grid 31x24x42 (31,248 tokens), hidden 4096, "
                                   "32x128 heads, SwiGLU 2x16384->16384"),
    "full5s": Workload("full5s", 1, (31, 48, 84), 0, 4096, 32, 128, (16, 56, 56), 16384,
                       description="1344x768 5 s: B=1, grid 31x48x84 (124,992 tokens), hidden 4096, "
                                   "32x128 heads, SwiGLU 2x16384->16384"),
    "full10s": Workload("full10s", 1, (61, 48, 84), 480, 4096, 32, 128, (16, 56, 56), 16384,
                        description="1344x768 10 s packed: B=1, grid 61x48x84 (245,952 tokens) + 480 "
                                    "temporal-only tokens, hidden 4096, 32x128 heads, SwiGLU 2x16384->16384"),
    "batch2": Workload("batch2", 2, (31, 48, 84), 0, 4096, 32, 128, (16, 56, 56), 16384, heavy_tail=True,
                       description="two-sample 1344x768 5 s: B=2 x 124,992 tokens, heavy-tailed activations, "
                                   "hidden 4096, 32x128 heads, SwiGLU 2x16384->16384"),
}

_HEAVY = ("x_mod", "res_x", "res_y", "swiglu_in", "q", "k")
_MOD = ("shift", "scale", "gate")
_WEIGHTS = ("wq", "wk")

# Elements drawn per fp32 chunk, to bound the temporary fp32 memory.
_CHUNK_ELEMS = 1 << 27


def _generator(device, seed: int, index: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + index)
    return g


def heavy_channels(wl: Workload, name: str, seed: int = 0) -> torch.Tensor | None:
    """Seeded subset (5% of the last dimension) of channels scaled x20, or None."""
    if not wl.heavy_tail or name not in _HEAVY:
        return None
    shape = wl.shapes()[name]
    C = shape[-1] if name != "q" and name != "k" else wl.H * wl.Dh
    g = _generator("cpu", seed + 7, TENSOR_ORDER.index(name))
    count = round(0.05 * C)
    return torch.randperm(C, generator=g)[:count].sort().values


def _draw(wl: Workload, name: str, device, seed: int) -> torch.Tensor:
    shape = wl.shapes()[name]
    g = _generator(device, seed, TENSOR_ORDER.index(name))
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    if name in _MOD:
        out.copy_((torch.randn(shape, generator=g, device=device) * 0.1).to(torch.bfloat16))
        return out
    if name in _WEIGHTS:
        out.copy_((1.0 + 0.02 * torch.randn(shape, generator=g, device=device)).to(torch.bfloat16))
        return out
    heavy = heavy_channels(wl, name, seed)
    if heavy is not None:
        heavy = heavy.to(device)
    flat = out.view(-1, shape[-1]) if name not in ("q", "k") else out.view(-1, wl.H * wl.Dh)
    rows, cols = flat.shape
    step = max(1, _CHUNK_ELEMS // cols)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        chunk = torch.randn((r1 - r0, cols), generator=g, device=device)
        if heavy is not None:
            chunk[:, heavy] *= 20.0
        flat[r0:r1].copy_(chunk.to(torch.bfloat16))
        del chunk
    return out


def make_inputs(wl: Workload | str, device="cpu", seed: int = 0, names=None) -> dict:
    """Draw the named input tensors (default: all) of a workload as bf16 tensors on ``device``."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    names = TENSOR_ORDER if names is None else tuple(names)
    unknown = set(names) - set(TENSOR_ORDER)
    if unknown:
        raise KeyError(f"unknown input tensors: {sorted(unknown)}")
    return {n: _draw(wl, n, device, seed) for n in names}


def op_inputs(wl: Workload | str, op: str, device="cpu", seed: int = 0) -> dict:
    """Inputs of one op ('adaln', 'residual', 'swiglu' or 'qk')."""
    return make_inputs(wl, device, seed, OP_TENSORS[op])


def correlated_heads(shape, seed: int = 0, run: int = 48, device="cpu") -> torch.Tensor:
    """bf16 [B, N, H, Dh] head vectors with local correlation along the sequence.

    Each token is 0.5 * N(0, 1) noise plus an offset N(0, 1) shared by the
    ``run`` consecutive tokens it falls in (per sample and head), the way
    neighbouring video tokens resemble each other.  Runs are not aligned to any
    block size the consumer uses.
    """
    B, N, H, Dh = shape
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + 101)
    runs = -(-N // run) if N else 0
    offset = torch.randn((B, runs, H, Dh), generator=g, device=device)
    noise = torch.randn((B, N, H, Dh), generator=g, device=device) * 0.5
    return (noise + offset.repeat_interleave(run, dim=1)[:, :N]).to(torch.bfloat16)


def bits(t: torch.Tensor):
    """Raw bf16 bit patterns of a tensor as a host numpy uint16 array."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view("uint16")


def from_float(values, device="cpu") -> torch.Tensor:
    """bf16 tensor from Python/numpy floats (round-to-nearest-even)."""
    return torch.as_tensor(values, dtype=torch.float32, device=device).to(torch.bfloat16)
