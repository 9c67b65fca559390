"""ctypes binding of libdit_ops.so: argument marshalling only.

Every function here has the name of the C entry point it calls, takes torch
tensors that already live on a HIP device, checks that they are bf16 (int32
for positions), contiguous and on one device, reads the sizes from their
shapes, and passes raw device pointers plus the current torch stream to the
library.  All arithmetic runs in the library's HIP kernels; there is no other
code path.  If the library is not built, the first call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdit_ops.so")

DIT_OK, DIT_ERR_NULL, DIT_ERR_SHAPE, DIT_ERR_ALIGN, DIT_ERR_ARG, DIT_ERR_HIP, DIT_ERR_SCRATCH = range(7)

# Every entry point the header declares, with its ctypes signature.
_I64, _I32, _F32, _P = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
SIGNATURES = {
    "dit_status_str": ([ctypes.c_int], ctypes.c_char_p),
    "dit_abi_version": ([], ctypes.c_int),
    "dit_adaln_modulate": ([_P, _P, _P, _P, _I64, _I64, _I64, _F32, _P], ctypes.c_int),
    "dit_gated_residual": ([_P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "dit_swiglu": ([_P, _P, _I64, _I64, _P], ctypes.c_int),
    "dit_qk_rmsnorm_rope3d": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I32, _I32, _I32, _F32, _F32, _P],
                              ctypes.c_int),
    "dit_qk_rmsnorm_rope3d_layout": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I32, _I64, _I32,
                                      _I32, _I32, _F32, _F32, _P], ctypes.c_int),
    "dit_gated_residual_adaln": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _F32, _P], ctypes.c_int),
    "dit_residual_change": ([_P, _P, _P, _P, _I64, _I64, _I64, _I64, _P], ctypes.c_int),
    "dit_residual_change_workspace_bytes": ([_I64, _I64, _I64], ctypes.c_int64),
    "dit_residual_change_noalloc": ([_P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "dit_subblock_keep": ([_I64, ctypes.c_double], ctypes.c_int64),
    "dit_subblock_scores_ld": ([_I64], ctypes.c_int64),
    "dit_subblock_pool": ([_P, _P, _P, _P, _I64, _I64, _I64, _I64, _I32, _P], ctypes.c_int),
    "dit_subblock_route": ([_P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P], ctypes.c_int),
    "dit_qk_rmsnorm_rope3d_pool": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I32, _I64,
                                    _I32, _I32, _I32, _F32, _F32, _P], ctypes.c_int),
    "dit_packed_positions": ([_P, _I64, _I64, _I64, _I64, _P], ctypes.c_int),
    "dit_copy16": ([_P, _P, _I64, _P], ctypes.c_int),
    "dit_stream_pattern": ([_I32, _P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
}

_lib = None


class DitError(RuntimeError):
    """A library call returned a status other than DIT_OK."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {dit_status_str(status)}")


def load_library(path: str = LIB_PATH):
    """Load libdit_ops.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m video_diffusion_transformer_dit_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (args, res) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if path == LIB_PATH:
        _lib = lib
    return lib


def dit_status_str(status: int) -> str:
    return load_library().dit_status_str(int(status)).decode()


def dit_abi_version() -> int:
    return load_library().dit_abi_version()


def _check(fn: str, status: int):
    if status != DIT_OK:
        raise DitError(fn, status)


def _tensor(t, name: str, dtype=torch.bfloat16, ndim: int | None = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    return t


def _shape(t, name: str, shape: tuple):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _same_device(*ts):
    devs = {t.device for t in ts}
    if len(devs) != 1:
        raise ValueError(f"all tensors must be on one device, got {sorted(map(str, devs))}")
    return ts[0].device


def _stream(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if isinstance(stream, torch.cuda.Stream) else int(stream)


def dit_adaln_modulate(x, shift, scale, y=None, eps: float = 1e-6, stream=None):
    """y = LayerNorm(x) * (1 + scale[b]) + shift[b]; x [B,N,D], shift/scale [B,D]. Returns y."""
    _tensor(x, "x", ndim=3)
    B, N, D = x.shape
    _shape(_tensor(shift, "shift"), "shift", (B, D))
    _shape(_tensor(scale, "scale"), "scale", (B, D))
    y = torch.empty_like(x) if y is None else y
    _shape(_tensor(y, "y"), "y", (B, N, D))
    dev = _same_device(x, shift, scale, y)
    with torch.cuda.device(dev):
        _check("dit_adaln_modulate", load_library().dit_adaln_modulate(
            x.data_ptr(), shift.data_ptr(), scale.data_ptr(), y.data_ptr(), B, N, D, float(eps), _stream(stream, dev)))
    return y


def dit_gated_residual(x, y, gate, out=None, stream=None):
    """out = x + gate[b] * y; x, y [B,N,D], gate [B,D]. Returns out."""
    _tensor(x, "x", ndim=3)
    B, N, D = x.shape
    _shape(_tensor(y, "y"), "y", (B, N, D))
    _shape(_tensor(gate, "gate"), "gate", (B, D))
    out = torch.empty_like(x) if out is None else out
    _shape(_tensor(out, "out"), "out", (B, N, D))
    dev = _same_device(x, y, gate, out)
    with torch.cuda.device(dev):
        _check("dit_gated_residual", load_library().dit_gated_residual(
            x.data_ptr(), y.data_ptr(), gate.data_ptr(), out.data_ptr(), B, N, D, _stream(stream, dev)))
    return out


def dit_gated_residual_adaln(x, y, gate, shift, scale, x_out=None, z=None, eps: float = 1e-6, stream=None):
    """x_out = x + gate[b]*y (bf16); z = LayerNorm(x_out)*(1+scale[b]) + shift[b]. Returns (x_out, z)."""
    _tensor(x, "x", ndim=3)
    B, N, D = x.shape
    _shape(_tensor(y, "y"), "y", (B, N, D))
    for t, name in ((gate, "gate"), (shift, "shift"), (scale, "scale")):
        _shape(_tensor(t, name), name, (B, D))
    x_out = torch.empty_like(x) if x_out is None else x_out
    z = torch.empty_like(x) if z is None else z
    _shape(_tensor(x_out, "x_out"), "x_out", (B, N, D))
    _shape(_tensor(z, "z"), "z", (B, N, D))
    dev = _same_device(x, y, gate, shift, scale, x_out, z)
    with torch.cuda.device(dev):
        _check("dit_gated_residual_adaln", load_library().dit_gated_residual_adaln(
            x.data_ptr(), y.data_ptr(), gate.data_ptr(), shift.data_ptr(), scale.data_ptr(), x_out.data_ptr(),
            z.data_ptr(), B, N, D, float(eps), _stream(stream, dev)))
    return x_out, z


def dit_swiglu(inp, out=None, stream=None):
    """out[r, j] = silu(inp[r, j]) * inp[r, F + j]; inp [M, 2F] -> out [M, F]. Returns out."""
    _tensor(inp, "inp", ndim=2)
    M, twoF = inp.shape
    if twoF % 2:
        raise ValueError(f"inp's last dimension must be even, got {twoF}")
    F = twoF // 2
    out = torch.empty((M, F), dtype=inp.dtype, device=inp.device) if out is None else out
    _shape(_tensor(out, "out"), "out", (M, F))
    dev = _same_device(inp, out)
    with torch.cuda.device(dev):
        _check("dit_swiglu", load_library().dit_swiglu(inp.data_ptr(), out.data_ptr(), M, F, _stream(stream, dev)))
    return out


def dit_qk_rmsnorm_rope3d(q, k, wq, wk, pos, bands, q_out=None, k_out=None, theta: float = 1e4,
                          eps: float = 1e-6, stream=None):
    """Per-head RMSNorm then 3D RoPE of q and k [B,N,H,Dh]; wq/wk [Dh]; pos [N,3] int32.

    ``bands`` = (d_t, d_h, d_w).  Returns (q_out, k_out).
    """
    _tensor(q, "q", ndim=4)
    B, N, H, Dh = q.shape
    _shape(_tensor(k, "k"), "k", (B, N, H, Dh))
    _shape(_tensor(wq, "wq"), "wq", (Dh,))
    _shape(_tensor(wk, "wk"), "wk", (Dh,))
    _shape(_tensor(pos, "pos", dtype=torch.int32), "pos", (N, 3))
    q_out = torch.empty_like(q) if q_out is None else q_out
    k_out = torch.empty_like(k) if k_out is None else k_out
    _shape(_tensor(q_out, "q_out"), "q_out", (B, N, H, Dh))
    _shape(_tensor(k_out, "k_out"), "k_out", (B, N, H, Dh))
    d_t, d_h, d_w = (int(b) for b in bands)
    dev = _same_device(q, k, wq, wk, pos, q_out, k_out)
    with torch.cuda.device(dev):
        _check("dit_qk_rmsnorm_rope3d", load_library().dit_qk_rmsnorm_rope3d(
            q.data_ptr(), k.data_ptr(), q_out.data_ptr(), k_out.data_ptr(), wq.data_ptr(), wk.data_ptr(),
            pos.data_ptr(), B, N, H, Dh, d_t, d_h, d_w, float(theta), float(eps), _stream(stream, dev)))
    return q_out, k_out


DIT_QK_TOKEN_MAJOR, DIT_QK_HEAD_MAJOR = 0, 1


def _qk_outputs(q_out, k_out, shape, head_major: bool, plane_stride, device):
    """Output tensors of a QK entry point and their head-plane stride argument (0 = packed).

    Token-major outputs are contiguous [B,N,H,Dh].  Head-major outputs are [B,H,N,Dh] views whose head
    planes may sit ``P`` elements apart (strides (H*P, P, Dh, 1), P >= N*Dh), e.g. slices of a [B,H,P]
    buffer; given ``plane_stride`` and no outputs, such buffers are allocated and their views returned.
    """
    B, A, C, Dh = shape  # head-major: A = H, C = N
    if plane_stride is not None and not head_major:
        raise ValueError("plane_stride applies to head-major outputs only")
    if plane_stride and (plane_stride < C * Dh or plane_stride % 8):
        raise ValueError(f"plane_stride must be 0 or a multiple of 8 >= N*Dh = {C * Dh}, got {plane_stride}")
    outs = []
    for t, name in ((q_out, "q_out"), (k_out, "k_out")):
        if t is None:
            if head_major and plane_stride:
                t = torch.empty((B, A, int(plane_stride)), dtype=torch.bfloat16, device=device)[..., :C * Dh]
                t = t.view(B, A, C, Dh)
            else:
                t = torch.empty(shape, dtype=torch.bfloat16, device=device)
        outs.append(t)
    planes = set()
    for t, name in zip(outs, ("q_out", "k_out")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.device.type != "cuda":
            raise TypeError(f"{name} must be a bf16 tensor on a HIP device")
        _shape(t, name, shape)
        if t.is_contiguous():
            planes.add(0)
            continue
        st = t.stride()
        if not head_major or st[3] != 1 or st[2] != Dh or st[1] < C * Dh or st[1] % 8 or st[0] != A * st[1]:
            raise ValueError(f"{name} must be contiguous, or head-major with strides (H*P, P, Dh, 1), P >= N*Dh "
                             f"a multiple of 8; got strides {st}")
        planes.add(st[1])
    if len(planes) != 1:
        raise ValueError("q_out and k_out must have the same head-plane stride")
    P = planes.pop()
    return outs[0], outs[1], (0 if P == C * Dh else P)


def dit_qk_rmsnorm_rope3d_layout(qkv, H: int, Dh: int, wq, wk, pos, bands, head_major: bool = True,
                                 q_out=None, k_out=None, plane_stride=None, theta: float = 1e4, eps: float = 1e-6,
                                 stream=None):
    """Per-head RMSNorm + 3D RoPE of the q and k parts of a fused projection ``qkv`` [B,N,S] whose last
    dimension holds q at [0, H*Dh) and k at [H*Dh, 2*H*Dh) (S >= 2*H*Dh, e.g. 3*H*Dh with v after k).

    Outputs are head-major [B,H,N,Dh] (or token-major [B,N,H,Dh] with ``head_major=False``).  Head-major
    outputs may have padded head planes: pass views with strides (H*P, P, Dh, 1), or ``plane_stride=P``
    to allocate them.  Returns (q_out, k_out).
    """
    _tensor(qkv, "qkv", ndim=3)
    B, N, S = qkv.shape
    if S < 2 * H * Dh:
        raise ValueError(f"qkv's last dimension {S} cannot hold q and k of {H}x{Dh}")
    _shape(_tensor(wq, "wq"), "wq", (Dh,))
    _shape(_tensor(wk, "wk"), "wk", (Dh,))
    _shape(_tensor(pos, "pos", dtype=torch.int32), "pos", (N, 3))
    shape = (B, H, N, Dh) if head_major else (B, N, H, Dh)
    q_out, k_out, plane = _qk_outputs(q_out, k_out, shape, head_major, plane_stride, qkv.device)
    d_t, d_h, d_w = (int(b) for b in bands)
    dev = _same_device(qkv, wq, wk, pos, q_out, k_out)
    k_ptr = qkv.data_ptr() + H * Dh * qkv.element_size()
    with torch.cuda.device(dev):
        _check("dit_qk_rmsnorm_rope3d_layout", load_library().dit_qk_rmsnorm_rope3d_layout(
            qkv.data_ptr(), k_ptr, q_out.data_ptr(), k_out.data_ptr(), wq.data_ptr(), wk.data_ptr(), pos.data_ptr(),
            B, N, H, Dh, S, DIT_QK_HEAD_MAJOR if head_major else DIT_QK_TOKEN_MAJOR, plane, d_t, d_h, d_w,
            float(theta), float(eps), _stream(stream, dev)))
    return q_out, k_out


def dit_residual_change_workspace_bytes(B: int, N: int, D: int) -> int:
    return load_library().dit_residual_change_workspace_bytes(B, N, D)


def dit_residual_change(r, r_cached, out=None, workspace=None, stream=None):
    """Per sample (sum |r - r_cached|, sum |r_cached|, ratio) as a [B, 3] float64 device tensor.

    ``workspace`` (optional) is a device tensor of at least dit_residual_change_workspace_bytes bytes.
    """
    _tensor(r, "r", ndim=3)
    B, N, D = r.shape
    _shape(_tensor(r_cached, "r_cached"), "r_cached", (B, N, D))
    out = torch.empty((B, 3), dtype=torch.float64, device=r.device) if out is None else out
    _shape(_tensor(out, "out", dtype=torch.float64), "out", (B, 3))
    need = dit_residual_change_workspace_bytes(B, N, D)
    if need < 0:
        raise ValueError(f"unsupported sizes {(B, N, D)}")
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=r.device)
    if not isinstance(workspace, torch.Tensor) or not workspace.is_contiguous() or workspace.device != r.device:
        raise ValueError("workspace must be a contiguous tensor on the same device")
    nbytes = workspace.numel() * workspace.element_size()
    dev = _same_device(r, r_cached, out)
    with torch.cuda.device(dev):
        _check("dit_residual_change", load_library().dit_residual_change(
            r.data_ptr(), r_cached.data_ptr(), out.data_ptr(), workspace.data_ptr(), nbytes, B, N, D,
            _stream(stream, dev)))
    return out


def dit_residual_change_noalloc(r, r_cached, out, stream=None):
    """dit_residual_change with its partials in the library's static scratch array: no workspace, no allocation.

    ``out`` is a caller-owned [B, 3] float64 device tensor (this wrapper allocates nothing either).  Calls that
    overlap in time on one GPU share the scratch array and race; calls ordered on one stream are safe.
    """
    _tensor(r, "r", ndim=3)
    B, N, D = r.shape
    _shape(_tensor(r_cached, "r_cached"), "r_cached", (B, N, D))
    _shape(_tensor(out, "out", dtype=torch.float64), "out", (B, 3))
    dev = _same_device(r, r_cached, out)
    with torch.cuda.device(dev):
        _check("dit_residual_change_noalloc", load_library().dit_residual_change_noalloc(
            r.data_ptr(), r_cached.data_ptr(), out.data_ptr(), B, N, D, _stream(stream, dev)))
    return out


DIT_SUBBLOCK_TOKENS = 64


def dit_subblock_keep(nb: int, sparsity: float) -> int:
    """Key blocks kept per query block: nb - floor(sparsity * nb), at least 1."""
    keep = load_library().dit_subblock_keep(int(nb), float(sparsity))
    if keep < 0:
        raise ValueError(f"sparsity must be in [0, 1) and nb >= 0, got nb={nb}, sparsity={sparsity}")
    return keep


def dit_subblock_scores_ld(nb: int) -> int:
    ld = load_library().dit_subblock_scores_ld(int(nb))
    if ld < 0:
        raise ValueError(f"unsupported block count {nb}")
    return ld


def dit_subblock_pool(q, k, head_major: bool = False, q_pooled=None, k_pooled=None, stream=None):
    """Means of each 64-token block of q' and k' -> (q_pooled, k_pooled) fp32 [B,H,nb,Dh].

    q, k are bf16 [B,N,H,Dh] (or [B,H,N,Dh] with ``head_major=True``); nb = ceil(N/64).
    """
    _tensor(q, "q", ndim=4)
    if head_major:
        B, H, N, Dh = q.shape
    else:
        B, N, H, Dh = q.shape
    _shape(_tensor(k, "k"), "k", tuple(q.shape))
    nb = -(-N // DIT_SUBBLOCK_TOKENS)
    shape = (B, H, nb, Dh)
    q_pooled = torch.empty(shape, dtype=torch.float32, device=q.device) if q_pooled is None else q_pooled
    k_pooled = torch.empty(shape, dtype=torch.float32, device=q.device) if k_pooled is None else k_pooled
    _shape(_tensor(q_pooled, "q_pooled", dtype=torch.float32), "q_pooled", shape)
    _shape(_tensor(k_pooled, "k_pooled", dtype=torch.float32), "k_pooled", shape)
    dev = _same_device(q, k, q_pooled, k_pooled)
    with torch.cuda.device(dev):
        _check("dit_subblock_pool", load_library().dit_subblock_pool(
            q.data_ptr(), k.data_ptr(), q_pooled.data_ptr(), k_pooled.data_ptr(), B, N, H, Dh,
            DIT_QK_HEAD_MAJOR if head_major else DIT_QK_TOKEN_MAJOR, _stream(stream, dev)))
    return q_pooled, k_pooled


def dit_qk_rmsnorm_rope3d_pool(q, k, wq, wk, pos, bands, head_major: bool = False, q_out=None, k_out=None,
                               q_pooled=None, k_pooled=None, heads=None, plane_stride=None, theta: float = 1e4,
                               eps: float = 1e-6, stream=None):
    """QK RMSNorm + 3D RoPE plus the 64-token block means of its stored outputs.

    Inputs: q, k bf16 [B,N,H,Dh]; or, with ``k=None`` and ``heads=(H, Dh)``, q is a fused projection
    [B,N,S] holding q at [0, H*Dh) and k at [H*Dh, 2*H*Dh) of each token.  Outputs q', k' are
    [B,N,H,Dh], or [B,H,N,Dh] with ``head_major=True`` (head planes optionally padded apart, as for
    dit_qk_rmsnorm_rope3d_layout); the means are fp32 [B,H,nb,Dh], nb = ceil(N/64).
    Returns (q_out, k_out, q_pooled, k_pooled).
    """
    if k is None:
        _tensor(q, "qkv", ndim=3)
        if heads is None:
            raise ValueError("a fused projection needs heads=(H, Dh)")
        B, N, S = q.shape
        H, Dh = (int(v) for v in heads)
        if S < 2 * H * Dh:
            raise ValueError(f"the projection's last dimension {S} cannot hold q and k of {H}x{Dh}")
        stride, q_ptr, k_ptr, src = S, q.data_ptr(), q.data_ptr() + H * Dh * q.element_size(), (q,)
    else:
        _tensor(q, "q", ndim=4)
        B, N, H, Dh = q.shape
        _shape(_tensor(k, "k"), "k", (B, N, H, Dh))
        stride, q_ptr, k_ptr, src = H * Dh, q.data_ptr(), k.data_ptr(), (q, k)
    _shape(_tensor(wq, "wq"), "wq", (Dh,))
    _shape(_tensor(wk, "wk"), "wk", (Dh,))
    _shape(_tensor(pos, "pos", dtype=torch.int32), "pos", (N, 3))
    shape = (B, H, N, Dh) if head_major else (B, N, H, Dh)
    q_out, k_out, plane = _qk_outputs(q_out, k_out, shape, head_major, plane_stride, q.device)
    nb = -(-N // DIT_SUBBLOCK_TOKENS)
    pshape = (B, H, nb, Dh)
    q_pooled = torch.empty(pshape, dtype=torch.float32, device=q.device) if q_pooled is None else q_pooled
    k_pooled = torch.empty(pshape, dtype=torch.float32, device=q.device) if k_pooled is None else k_pooled
    _shape(_tensor(q_pooled, "q_pooled", dtype=torch.float32), "q_pooled", pshape)
    _shape(_tensor(k_pooled, "k_pooled", dtype=torch.float32), "k_pooled", pshape)
    d_t, d_h, d_w = (int(b) for b in bands)
    dev = _same_device(*src, wq, wk, pos, q_out, k_out, q_pooled, k_pooled)
    with torch.cuda.device(dev):
        _check("dit_qk_rmsnorm_rope3d_pool", load_library().dit_qk_rmsnorm_rope3d_pool(
            q_ptr, k_ptr, q_out.data_ptr(), k_out.data_ptr(), wq.data_ptr(), wk.data_ptr(), pos.data_ptr(),
            q_pooled.data_ptr(), k_pooled.data_ptr(), B, N, H, Dh, stride,
            DIT_QK_HEAD_MAJOR if head_major else DIT_QK_TOKEN_MAJOR, plane, d_t, d_h, d_w, float(theta), float(eps),
            _stream(stream, dev)))
    return q_out, k_out, q_pooled, k_pooled


def dit_subblock_route(q_pooled, k_pooled, sparsity: float | None = None, keep: int | None = None, scores=None,
                       kept=None, write_scores: bool = True, stream=None):
    """Block scores and kept key blocks from pooled q', k' fp32 [B,H,nb,Dh].

    Give ``sparsity`` (share of key blocks dropped) or ``keep`` (count kept).  Returns (kept, scores):
    kept int32 [B,H,nb,keep] ascending per query block; scores fp32 [B,H,nb,ld] whose first nb
    columns hold the scores (ld = dit_subblock_scores_ld(nb)).  With ``write_scores=False`` no score
    matrix is written (the library keeps the scores on chip) and scores is None.
    """
    _tensor(q_pooled, "q_pooled", dtype=torch.float32, ndim=4)
    B, H, nb, Dh = q_pooled.shape
    _shape(_tensor(k_pooled, "k_pooled", dtype=torch.float32), "k_pooled", (B, H, nb, Dh))
    if (sparsity is None) == (keep is None):
        raise ValueError("give exactly one of sparsity and keep")
    keep = dit_subblock_keep(nb, sparsity) if keep is None else int(keep)
    ld = dit_subblock_scores_ld(nb)
    if write_scores:
        scores = torch.empty((B, H, nb, ld), dtype=torch.float32, device=q_pooled.device) if scores is None \
            else scores
        _shape(_tensor(scores, "scores", dtype=torch.float32), "scores", (B, H, nb, ld))
    elif scores is not None:
        raise ValueError("scores given with write_scores=False")
    kept = torch.empty((B, H, nb, keep), dtype=torch.int32, device=q_pooled.device) if kept is None else kept
    _shape(_tensor(kept, "kept", dtype=torch.int32), "kept", (B, H, nb, keep))
    dev = _same_device(q_pooled, k_pooled, kept, *((scores,) if scores is not None else ()))
    with torch.cuda.device(dev):
        _check("dit_subblock_route", load_library().dit_subblock_route(
            q_pooled.data_ptr(), k_pooled.data_ptr(), scores.data_ptr() if scores is not None else None,
            kept.data_ptr(), B, H, nb, Dh, keep, _stream(stream, dev)))
    return kept, scores


def dit_packed_positions(T: int, Hg: int, Wg: int, n_extra: int = 0, pos=None, device=None, stream=None):
    """[T*Hg*Wg + n_extra, 3] int32 (t, h, w) coordinates of a packed sequence, built on the device."""
    n = T * Hg * Wg + n_extra
    if pos is None:
        pos = torch.empty((n, 3), dtype=torch.int32, device=device if device is not None else "cuda")
    _shape(_tensor(pos, "pos", dtype=torch.int32), "pos", (n, 3))
    dev = pos.device
    with torch.cuda.device(dev):
        _check("dit_packed_positions", load_library().dit_packed_positions(
            pos.data_ptr(), T, Hg, Wg, n_extra, _stream(stream, dev)))
    return pos


def dit_copy16(src, dst, stream=None):
    """dst = src (bytewise), both contiguous device tensors of the same byte size (a multiple of 16)."""
    for t, name in ((src, "src"), (dst, "dst")):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst differ in size")
    dev = _same_device(src, dst)
    with torch.cuda.device(dev):
        _check("dit_copy16", load_library().dit_copy16(src.data_ptr(), dst.data_ptr(), nbytes, _stream(stream, dev)))
    return dst


DIT_STREAM_READ, DIT_STREAM_WRITE, DIT_STREAM_SPLIT_ROWS, DIT_STREAM_TWO_IN, DIT_STREAM_ROW_GROUP, \
    DIT_STREAM_ROW_GROUP_2X2, DIT_STREAM_HEAD_MAJOR, DIT_STREAM_SCORE_TILES, DIT_STREAM_TOPK_ROWS = range(9)


def dit_stream_pattern(kind: int, rows: int, row_bytes: int, in0=None, in1=None, out0=None, out1=None, heads: int = 0,
                       stream=None):
    """Access-pattern stream (measurement only): the traffic of one of the chain's kernels with no arithmetic.

    Tensors are contiguous device tensors of any dtype holding at least the bytes the pattern touches
    (see dit_ops.h); unused ones may be None.  For DIT_STREAM_SCORE_TILES and DIT_STREAM_TOPK_ROWS `heads` is the block count n.
    """
    split = kind == DIT_STREAM_SPLIT_ROWS
    means = rows * 512 if kind == DIT_STREAM_SCORE_TILES else None  # [rows][128] fp32 query / key means
    need = {"in0": means or rows * row_bytes * (2 if split else 1), "in1": means or rows * row_bytes,
            "out0": 16 if kind == DIT_STREAM_READ else rows * row_bytes, "out1": rows * row_bytes}
    if kind == DIT_STREAM_TOPK_ROWS and heads > 0:
        need["out0"] = rows * (-(-heads // 4)) * 4  # [rows][ceil(n / 4)] int32
    ptrs, devs = {}, []
    for name, t in (("in0", in0), ("in1", in1), ("out0", out0), ("out1", out1)):
        if t is None:
            ptrs[name] = None
            continue
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
        if t.numel() * t.element_size() < need[name]:
            raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, the pattern touches {need[name]}")
        ptrs[name] = t.data_ptr()
        devs.append(t)
    dev = _same_device(*devs)
    with torch.cuda.device(dev):
        _check("dit_stream_pattern", load_library().dit_stream_pattern(
            int(kind), ptrs["in0"], ptrs["in1"], ptrs["out0"], ptrs["out1"], int(rows), int(row_bytes), int(heads),
            _stream(stream, dev)))
