"""fp64 CPU oracle for the fused DiT non-GEMM operator chain.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library and never imports it; the product package never imports
this one.

The arithmetic lives in ``dit_oracle.c`` (plain C, double precision, serial
loops, built with ``-O2 -ffp-contract=off`` and no fast-math).  This module only
marshals numpy arrays into it: it decodes nothing, rounds nothing and reorders
nothing.  With ``threads=1`` (the default) each op is one call of its C function over
the whole tensor.  With more threads the rows are split into contiguous chunks,
each handed to the same C function on its own thread (ctypes releases the
GIL); every row is still computed by the same serial code.

Inputs are raw bf16 bit patterns as ``numpy.uint16`` arrays (C-contiguous);
outputs are unrounded ``numpy.float64`` arrays.
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle_dit.so")
SOURCE = os.path.join(_HERE, "dit_oracle.c")

# Compiler command for the oracle (plain C, no fast-math, no FMA contraction).
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]

_c_i64 = ctypes.c_int64
_c_i32 = ctypes.c_int32
_c_dbl = ctypes.c_double
_c_p = ctypes.c_void_p

_lib = None


def build(out_path: str = LIB_PATH, source: str = SOURCE, cc: str = "gcc") -> str:
    """Compile the oracle shared library with the plain C compiler."""
    import subprocess

    cmd = [cc, *CFLAGS, "-o", out_path, source, "-lm"]
    subprocess.run(cmd, check=True)
    return out_path


def _bind(lib):
    lib.dit_oracle_bf16_decode.argtypes = [ctypes.c_uint16]
    lib.dit_oracle_bf16_decode.restype = _c_dbl
    lib.dit_oracle_bf16_encode.argtypes = [_c_dbl]
    lib.dit_oracle_bf16_encode.restype = ctypes.c_uint16
    lib.dit_oracle_gated_residual_adaln.argtypes = [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                                    _c_i64, _c_i64, _c_i64, _c_dbl]
    lib.dit_oracle_gated_residual_adaln.restype = ctypes.c_int
    lib.dit_oracle_packed_positions.argtypes = [_c_p, _c_i64, _c_i64, _c_i64, _c_i64]
    lib.dit_oracle_packed_positions.restype = _c_i64
    lib.dit_oracle_adaln_modulate.argtypes = [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_dbl]
    lib.dit_oracle_adaln_modulate.restype = ctypes.c_int
    lib.dit_oracle_gated_residual.argtypes = [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64]
    lib.dit_oracle_gated_residual.restype = ctypes.c_int
    lib.dit_oracle_swiglu.argtypes = [_c_p, _c_p, _c_i64, _c_i64]
    lib.dit_oracle_swiglu.restype = ctypes.c_int
    lib.dit_oracle_rmsnorm.argtypes = [_c_p, _c_p, _c_p, _c_i64, _c_dbl]
    lib.dit_oracle_rmsnorm.restype = ctypes.c_int
    lib.dit_oracle_rope3d.argtypes = [_c_p, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_dbl]
    lib.dit_oracle_rope3d.restype = ctypes.c_int
    lib.dit_oracle_qk_rmsnorm_rope3d.argtypes = [
        _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
        _c_i64, _c_i64, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_dbl, _c_dbl,
    ]
    lib.dit_oracle_qk_rmsnorm_rope3d.restype = ctypes.c_int
    lib.dit_oracle_qk_rmsnorm_rope3d_layout.argtypes = [
        _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
        _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_dbl, _c_dbl,
    ]
    lib.dit_oracle_qk_rmsnorm_rope3d_layout.restype = ctypes.c_int
    lib.dit_oracle_residual_change.argtypes = [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64]
    lib.dit_oracle_residual_change.restype = ctypes.c_int
    lib.dit_oracle_subblock_pool.argtypes = [_c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64]
    lib.dit_oracle_subblock_pool.restype = ctypes.c_int
    lib.dit_oracle_subblock_scores.argtypes = [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64]
    lib.dit_oracle_subblock_scores.restype = ctypes.c_int
    lib.dit_oracle_subblock_keep.argtypes = [_c_i64, _c_dbl]
    lib.dit_oracle_subblock_keep.restype = _c_i64
    lib.dit_oracle_subblock_topk.argtypes = [_c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64]
    lib.dit_oracle_subblock_topk.restype = ctypes.c_int
    lib.dit_oracle_qk_rmsnorm_rope3d_pool.argtypes = [
        _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
        _c_i64, _c_i64, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_dbl, _c_dbl, _c_i64,
    ]
    lib.dit_oracle_qk_rmsnorm_rope3d_pool.restype = ctypes.c_int
    return lib


def load(path: str | None = None):
    """Load (building first if absent) the oracle library.

    With ``path`` given, loads that file and returns it without caching, so a
    test can run the same checks against another build of the oracle.
    """
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = _bind(ctypes.CDLL(LIB_PATH))
    return _lib


def _ptr(a: np.ndarray, offset_elems: int = 0) -> int:
    return a.ctypes.data + offset_elems * a.itemsize


def _bits(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"oracle inputs are raw bf16 bits (uint16), got {a.dtype}")
    return a


def _check(status: int, what: str):
    if status != 0:
        raise ValueError(f"oracle rejected the arguments of {what}")


def _chunks(n: int, threads: int):
    threads = max(1, min(threads, n)) if n > 0 else 1
    step = -(-n // threads) if n > 0 else 0
    return [(s, min(n, s + step)) for s in range(0, n, step)] if n > 0 else []


def _run(jobs, threads: int):
    if threads <= 1 or len(jobs) <= 1:
        for job in jobs:
            job()
        return
    with ThreadPoolExecutor(max_workers=threads) as pool:
        for fut in [pool.submit(job) for job in jobs]:
            fut.result()


def bf16_decode(bits: int, lib=None) -> float:
    return (lib or load()).dit_oracle_bf16_decode(int(bits))


def bf16_encode(value: float, lib=None) -> int:
    """Bit pattern of the bf16 nearest to ``value`` (ties to even)."""
    return int((lib or load()).dit_oracle_bf16_encode(float(value)))


def packed_positions(T: int, Hg: int, Wg: int, n_extra: int = 0, lib=None) -> np.ndarray:
    """[N, 3] int32 token coordinates of a packed sequence (video grid, then extra tokens)."""
    lib = lib or load()
    n = T * Hg * Wg + n_extra
    pos = np.zeros((n, 3), dtype=np.int32)
    written = lib.dit_oracle_packed_positions(_ptr(pos), T, Hg, Wg, n_extra)
    if written != n:
        raise ValueError("oracle rejected the arguments of packed_positions")
    return pos


def adaln_modulate(x, shift, scale, eps: float = 1e-6, threads: int = 1, lib=None) -> np.ndarray:
    """x [B,N,D], shift/scale [B,D] (bf16 bits) -> y [B,N,D] float64."""
    lib = lib or load()
    x, shift, scale = _bits(x), _bits(shift), _bits(scale)
    B, N, D = x.shape
    assert shift.shape == (B, D) and scale.shape == (B, D)
    y = np.empty((B, N, D), dtype=np.float64)
    if threads <= 1:
        _check(lib.dit_oracle_adaln_modulate(_ptr(x), _ptr(shift), _ptr(scale), _ptr(y), B, N, D, eps),
               "adaln_modulate")
        return y
    jobs = []
    for b in range(B):
        for lo, hi in _chunks(N, threads):
            row0 = b * N + lo

            def job(b=b, lo=lo, hi=hi, row0=row0):
                _check(lib.dit_oracle_adaln_modulate(
                    _ptr(x, row0 * D), _ptr(shift, b * D), _ptr(scale, b * D),
                    _ptr(y, row0 * D), 1, hi - lo, D, eps), "adaln_modulate")
            jobs.append(job)
    _run(jobs, threads)
    return y


def gated_residual(x, y, gate, threads: int = 1, lib=None) -> np.ndarray:
    """x, y [B,N,D], gate [B,D] (bf16 bits) -> out [B,N,D] float64."""
    lib = lib or load()
    x, y, gate = _bits(x), _bits(y), _bits(gate)
    B, N, D = x.shape
    assert y.shape == x.shape and gate.shape == (B, D)
    out = np.empty((B, N, D), dtype=np.float64)
    if threads <= 1:
        _check(lib.dit_oracle_gated_residual(_ptr(x), _ptr(y), _ptr(gate), _ptr(out), B, N, D), "gated_residual")
        return out
    jobs = []
    for b in range(B):
        for lo, hi in _chunks(N, threads):
            row0 = b * N + lo

            def job(b=b, lo=lo, hi=hi, row0=row0):
                _check(lib.dit_oracle_gated_residual(
                    _ptr(x, row0 * D), _ptr(y, row0 * D), _ptr(gate, b * D),
                    _ptr(out, row0 * D), 1, hi - lo, D), "gated_residual")
            jobs.append(job)
    _run(jobs, threads)
    return out


def gated_residual_adaln(x, y, gate, shift, scale, eps: float = 1e-6, threads: int = 1, lib=None):
    """x, y [B,N,D], gate/shift/scale [B,D] (bf16 bits) -> (x_out, z) [B,N,D] float64.

    x_out = x + gate*y (unrounded); z = AdaLN of x_out as stored in bf16.
    """
    lib = lib or load()
    x, y, gate, shift, scale = _bits(x), _bits(y), _bits(gate), _bits(shift), _bits(scale)
    B, N, D = x.shape
    assert y.shape == x.shape and gate.shape == shift.shape == scale.shape == (B, D)
    x_out = np.empty((B, N, D), dtype=np.float64)
    z = np.empty((B, N, D), dtype=np.float64)
    if threads <= 1:
        _check(lib.dit_oracle_gated_residual_adaln(_ptr(x), _ptr(y), _ptr(gate), _ptr(shift), _ptr(scale),
                                                   _ptr(x_out), _ptr(z), B, N, D, eps), "gated_residual_adaln")
        return x_out, z
    jobs = []
    for b in range(B):
        for lo, hi in _chunks(N, threads):
            row0 = b * N + lo

            def job(b=b, lo=lo, hi=hi, row0=row0):
                _check(lib.dit_oracle_gated_residual_adaln(
                    _ptr(x, row0 * D), _ptr(y, row0 * D), _ptr(gate, b * D), _ptr(shift, b * D),
                    _ptr(scale, b * D), _ptr(x_out, row0 * D), _ptr(z, row0 * D), 1, hi - lo, D, eps),
                    "gated_residual_adaln")
            jobs.append(job)
    _run(jobs, threads)
    return x_out, z


def swiglu(inp, threads: int = 1, lib=None) -> np.ndarray:
    """inp [M, 2F] (bf16 bits) -> out [M, F] float64."""
    lib = lib or load()
    inp = _bits(inp)
    M, twoF = inp.shape
    assert twoF % 2 == 0
    F = twoF // 2
    out = np.empty((M, F), dtype=np.float64)
    jobs = []
    for lo, hi in _chunks(M, threads):
        def job(lo=lo, hi=hi):
            _check(lib.dit_oracle_swiglu(_ptr(inp, lo * twoF), _ptr(out, lo * F), hi - lo, F), "swiglu")
        jobs.append(job)
    _run(jobs, threads)
    return out


def rmsnorm(v, w, eps: float = 1e-6, lib=None) -> np.ndarray:
    """One head vector (float64) -> v / sqrt(mean(v^2)+eps) * w."""
    lib = lib or load()
    v = np.ascontiguousarray(v, dtype=np.float64)
    w = np.ascontiguousarray(w, dtype=np.float64)
    u = np.empty_like(v)
    _check(lib.dit_oracle_rmsnorm(_ptr(v), _ptr(w), _ptr(u), v.size, eps), "rmsnorm")
    return u


def rope3d(u, bands, coord, theta: float = 1e4, lib=None) -> np.ndarray:
    """Rotate one head vector (float64) by the 3D rotary embedding at integer coord (t,h,w)."""
    lib = lib or load()
    out = np.array(u, dtype=np.float64, copy=True)
    d_t, d_h, d_w = (int(b) for b in bands)
    p_t, p_h, p_w = (int(c) for c in coord)
    _check(lib.dit_oracle_rope3d(_ptr(out), out.size, d_t, d_h, d_w, p_t, p_h, p_w, theta), "rope3d")
    return out


def qk_rmsnorm_rope3d(q, k, wq, wk, pos, bands, theta: float = 1e4, eps: float = 1e-6,
                      threads: int = 1, lib=None):
    """q, k [B,N,H,Dh], wq/wk [Dh] (bf16 bits), pos [N,3] int32 -> (q', k') float64."""
    lib = lib or load()
    q, k, wq, wk = _bits(q), _bits(k), _bits(wq), _bits(wk)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    B, N, H, Dh = q.shape
    assert k.shape == q.shape and wq.shape == (Dh,) and wk.shape == (Dh,) and pos.shape == (N, 3)
    d_t, d_h, d_w = (int(b) for b in bands)
    qo = np.empty(q.shape, dtype=np.float64)
    ko = np.empty(k.shape, dtype=np.float64)
    row = H * Dh
    if threads <= 1:
        _check(lib.dit_oracle_qk_rmsnorm_rope3d(
            _ptr(q), _ptr(k), _ptr(wq), _ptr(wk), _ptr(pos), _ptr(qo), _ptr(ko), B, N, H, Dh,
            d_t, d_h, d_w, theta, eps), "qk_rmsnorm_rope3d")
        return qo, ko
    jobs = []
    for b in range(B):
        for lo, hi in _chunks(N, threads):
            r0 = b * N + lo

            def job(lo=lo, hi=hi, r0=r0):
                _check(lib.dit_oracle_qk_rmsnorm_rope3d(
                    _ptr(q, r0 * row), _ptr(k, r0 * row), _ptr(wq), _ptr(wk), _ptr(pos, lo * 3),
                    _ptr(qo, r0 * row), _ptr(ko, r0 * row), 1, hi - lo, H, Dh,
                    d_t, d_h, d_w, theta, eps), "qk_rmsnorm_rope3d")
            jobs.append(job)
    _run(jobs, threads)
    return qo, ko


def qk_rmsnorm_rope3d_layout(q, k, wq, wk, pos, bands, B, N, H, Dh, in_stride, out_layout,
                             theta: float = 1e4, eps: float = 1e-6, lib=None):
    """Strided q/k input (flat bf16 bits, token stride ``in_stride`` elements) -> (q', k') float64.

    Output shape [B,N,H,Dh] for out_layout 0, [B,H,N,Dh] for out_layout 1.  ``q`` and ``k`` are flat
    arrays that may be views into one buffer (e.g. q = qkv, k = qkv[H*Dh:]); their first element is
    token 0's head 0.
    """
    lib = lib or load()
    q, k, wq, wk = _bits(q), _bits(k), _bits(wq), _bits(wk)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    need = ((B * N - 1) * in_stride + H * Dh) if B * N else 0
    assert q.size >= need and k.size >= need and pos.shape == (N, 3)
    shape = (B, N, H, Dh) if out_layout == 0 else (B, H, N, Dh)
    qo = np.empty(shape, dtype=np.float64)
    ko = np.empty(shape, dtype=np.float64)
    d_t, d_h, d_w = (int(b) for b in bands)
    _check(lib.dit_oracle_qk_rmsnorm_rope3d_layout(
        _ptr(q), _ptr(k), _ptr(wq), _ptr(wk), _ptr(pos), _ptr(qo), _ptr(ko), B, N, H, Dh, in_stride,
        out_layout, d_t, d_h, d_w, theta, eps), "qk_rmsnorm_rope3d_layout")
    return qo, ko


def residual_change(r, r_cached, lib=None) -> np.ndarray:
    """r, r_cached [B,N,D] (bf16 bits) -> [B,3] float64: (sum |r-rc|, sum |rc|, ratio) per sample."""
    lib = lib or load()
    r, r_cached = _bits(r), _bits(r_cached)
    B, N, D = r.shape
    assert r_cached.shape == r.shape
    out = np.empty((B, 3), dtype=np.float64)
    _check(lib.dit_oracle_residual_change(_ptr(r), _ptr(r_cached), _ptr(out), B, N, D), "residual_change")
    return out



# --------------------------------------------------------------------------- SubBlock routing

SUBBLOCK_TOKENS = 64  # tokens per SubBlock attention block


def subblock_pool(x, block: int = SUBBLOCK_TOKENS, lib=None) -> np.ndarray:
    """x [B,N,H,Dh] (bf16 bits, token-major) -> [B,H,nb,Dh] float64 block means, nb = ceil(N/block)."""
    lib = lib or load()
    x = _bits(x)
    B, N, H, Dh = x.shape
    nb = -(-N // block)
    out = np.empty((B, H, nb, Dh), dtype=np.float64)
    _check(lib.dit_oracle_subblock_pool(_ptr(x), _ptr(out), B, N, H, Dh, block), "subblock_pool")
    return out


def subblock_scores(qp, kp, lib=None) -> np.ndarray:
    """Pooled means qp [B,H,nq,Dh], kp [B,H,nk,Dh] float64 -> scores [B,H,nq,nk].

    The means are rounded to bf16 before the products.  ``qp`` may hold any
    selection of query blocks (e.g. a sample of rows); every key block is scored.
    """
    lib = lib or load()
    qp = np.ascontiguousarray(qp, dtype=np.float64)
    kp = np.ascontiguousarray(kp, dtype=np.float64)
    assert qp.ndim == 4 and kp.ndim == 4 and qp.shape[:2] == kp.shape[:2] and qp.shape[3] == kp.shape[3]
    B, H, nq, Dh = qp.shape
    nk = kp.shape[2]
    s = np.empty((B, H, nq, nk), dtype=np.float64)
    _check(lib.dit_oracle_subblock_scores(_ptr(qp), _ptr(kp), _ptr(s), B, H, nq, nk, Dh), "subblock_scores")
    return s


def subblock_keep(nb: int, sparsity: float, lib=None) -> int:
    """Key blocks kept per query block for a sparsity (fraction of blocks that may be dropped)."""
    lib = lib or load()
    keep = lib.dit_oracle_subblock_keep(nb, sparsity)
    _check(0 if keep >= 0 else -1, "subblock_keep")
    return int(keep)


def subblock_topk(s, keep: int, lib=None) -> np.ndarray:
    """Scores [B,H,nq,nb] float64 -> kept key blocks [B,H,nq,keep] int32, ascending per query block."""
    lib = lib or load()
    s = np.ascontiguousarray(s, dtype=np.float64)
    B, H, nq, nb = s.shape
    idx = np.empty((B, H, nq, keep), dtype=np.int32)
    _check(lib.dit_oracle_subblock_topk(_ptr(s), _ptr(idx), B, H, nq, nb, keep), "subblock_topk")
    return idx


def subblock_route(q, k, sparsity: float, block: int = SUBBLOCK_TOKENS, lib=None):
    """q', k' [B,N,H,Dh] (bf16 bits) -> (qp, kp, scores, kept indices) of SubBlock routing."""
    lib = lib or load()
    qp = subblock_pool(q, block, lib=lib)
    kp = subblock_pool(k, block, lib=lib)
    s = subblock_scores(qp, kp, lib=lib)
    idx = subblock_topk(s, subblock_keep(qp.shape[2], sparsity, lib=lib), lib=lib)
    return qp, kp, s, idx


def qk_rmsnorm_rope3d_pool(q, k, wq, wk, pos, bands, theta: float = 1e4, eps: float = 1e-6,
                           block: int = SUBBLOCK_TOKENS, lib=None):
    """QK RMSNorm + 3D RoPE and the block means of its bf16-stored outputs.

    q, k [B,N,H,Dh], wq/wk [Dh] (bf16 bits), pos [N,3] -> (q', k' [B,N,H,Dh], q_pooled, k_pooled [B,H,nb,Dh]).
    """
    lib = lib or load()
    q, k, wq, wk = _bits(q), _bits(k), _bits(wq), _bits(wk)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    B, N, H, Dh = q.shape
    assert k.shape == q.shape and wq.shape == (Dh,) and wk.shape == (Dh,) and pos.shape == (N, 3)
    nb = -(-N // block)
    qo = np.empty(q.shape, dtype=np.float64)
    ko = np.empty(k.shape, dtype=np.float64)
    qp = np.empty((B, H, nb, Dh), dtype=np.float64)
    kp = np.empty((B, H, nb, Dh), dtype=np.float64)
    d_t, d_h, d_w = (int(b) for b in bands)
    _check(lib.dit_oracle_qk_rmsnorm_rope3d_pool(
        _ptr(q), _ptr(k), _ptr(wq), _ptr(wk), _ptr(pos), _ptr(qo), _ptr(ko), _ptr(qp), _ptr(kp),
        B, N, H, Dh, d_t, d_h, d_w, theta, eps, block), "qk_rmsnorm_rope3d_pool")
    return qo, ko, qp, kp
