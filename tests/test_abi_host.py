"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every entry point include/dit_ops.h declares,
and reject invalid arguments with the documented status codes.  Every call
here fails validation (or is a zero-row no-op), so no HIP call is made and no
pointer is dereferenced; the pointers are fake aligned addresses.
"""
import ctypes
import math
import os
import re

import pytest

import video_diffusion_transformer_dit_amd as dit
from video_diffusion_transformer_dit_amd import (DIT_ERR_ALIGN, DIT_ERR_ARG, DIT_ERR_NULL, DIT_ERR_SHAPE, DIT_OK)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dit_ops.h")

P = 0x100000  # fake 16-byte-aligned device addresses, never dereferenced
Q = 0x200000
R = 0x300000
S = 0x400000
T = 0x500000
U = 0x600000
V = 0x700000


@pytest.fixture(scope="module")
def lib():
    import torch

    if torch.cuda.is_available():
        # A wrong expectation in this file would launch a kernel on fake
        # addresses; on a machine with a device that would fault it, so these
        # checks run only where no device is visible.
        pytest.skip("fake-pointer validation checks run only without a HIP device")
    if not os.path.exists(dit.LIB_PATH):
        from video_diffusion_transformer_dit_amd import build

        build.build()
    return dit.load_library()


def declared_functions():
    with open(HEADER, encoding="utf-8") as fh:
        text = fh.read()
    return set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(dit_\w+)\s*\(", text, flags=re.M))


def test_header_and_binding_agree():
    names = declared_functions()
    assert names == set(dit.SIGNATURES), names ^ set(dit.SIGNATURES)


def declared_signatures():
    """name -> (parameter ctypes, result ctypes) parsed from the header's declarations."""
    with open(HEADER, encoding="utf-8") as fh:
        text = re.sub(r"/\*.*?\*/", " ", fh.read(), flags=re.S)

    def ctype(decl):
        decl = decl.strip()
        if "*" in decl:
            return ctypes.c_char_p if re.match(r"const\s+char\s*\*", decl) else ctypes.c_void_p
        base = decl.split()[0] if decl.split()[0] != "const" else decl.split()[1]
        return {"int64_t": ctypes.c_int64, "int32_t": ctypes.c_int32, "int": ctypes.c_int, "float": ctypes.c_float,
                "double": ctypes.c_double, "dit_status": ctypes.c_int}[base]

    out = {}
    for m in re.finditer(r"^\s*((?:const\s+)?\w+\s*\*?)\s*(dit_\w+)\s*\(([^;]*?)\)\s*;", text, flags=re.M):
        ret, name, params = m.groups()
        params = params.strip()
        args = [] if params in ("", "void") else [ctype(p) for p in params.split(",")]
        out[name] = (args, ctype(ret))
    return out


def test_binding_signatures_match_header():
    # a parameter added to, dropped from or retyped in a declaration without
    # the same change in the ctypes table would pass wrong arguments silently
    decl = declared_signatures()
    assert set(decl) == set(dit.SIGNATURES)
    for name, (args, res) in dit.SIGNATURES.items():
        want_args, want_res = decl[name]
        assert [a.__name__ for a in args] == [a.__name__ for a in want_args], name
        assert res.__name__ == want_res.__name__, name


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_abi_version_matches_header(lib):
    with open(HEADER, encoding="utf-8") as fh:
        version = int(re.search(r"#define DIT_ABI_VERSION (\d+)", fh.read()).group(1))
    assert dit.dit_abi_version() == version


def test_status_strings(lib):
    for code in range(7):
        assert dit.dit_status_str(code).startswith(("DIT_OK", "DIT_ERR_"))
    assert dit.dit_status_str(99) == "unknown dit_status"


def adaln(lib, x=P, sh=Q, sc=R, y=S, B=1, N=4, D=4096, eps=1e-6):
    return lib.dit_adaln_modulate(x, sh, sc, y, B, N, D, eps, None)


def test_adaln_validation(lib):
    assert adaln(lib, B=-1) == DIT_ERR_ARG
    assert adaln(lib, B=1 << 40, N=1 << 40) == DIT_ERR_ARG
    assert adaln(lib, N=(1 << 24) + 1) == DIT_ERR_ARG
    assert adaln(lib, D=12) == DIT_ERR_SHAPE
    assert adaln(lib, D=0) == DIT_ERR_SHAPE
    assert adaln(lib, D=8200) == DIT_ERR_SHAPE
    assert adaln(lib, eps=0.0) == DIT_ERR_ARG
    assert adaln(lib, eps=math.nan) == DIT_ERR_ARG
    assert adaln(lib, eps=math.inf) == DIT_ERR_ARG
    assert adaln(lib, x=0) == DIT_ERR_NULL
    assert adaln(lib, y=0) == DIT_ERR_NULL
    assert adaln(lib, x=P + 2) == DIT_ERR_ALIGN
    assert adaln(lib, sc=R + 8) == DIT_ERR_ALIGN
    assert adaln(lib, y=P + 16) == DIT_ERR_ARG  # partial overlap with x
    assert adaln(lib, y=Q) == DIT_ERR_ARG  # output over the shift vector
    assert adaln(lib, x=0, sh=0, sc=0, y=0, N=0) == DIT_OK  # zero rows: no-op
    assert adaln(lib, N=0, D=12) == DIT_ERR_SHAPE  # shapes still checked


def test_gated_residual_validation(lib):
    f = lib.dit_gated_residual
    assert f(P, Q, R, S, 1, -3, 4096, None) == DIT_ERR_ARG
    assert f(P, Q, R, S, 1, 3, 4100, None) == DIT_ERR_SHAPE
    assert f(P, 0, R, S, 1, 3, 4096, None) == DIT_ERR_NULL
    assert f(P, Q, R + 4, S, 1, 3, 4096, None) == DIT_ERR_ALIGN
    assert f(P, Q, R, Q + 32, 1, 3, 4096, None) == DIT_ERR_ARG  # partial overlap with y
    assert f(P, Q, R, R, 1, 3, 4096, None) == DIT_ERR_ARG  # output over the gate
    assert f(0, 0, 0, 0, 0, 3, 4096, None) == DIT_OK
    # rows x ceil(D / 512) tiles (64 vectors each) must fit the 32-bit tile counter with the 2^23 - 1
    # workgroup grid: refused as an argument, before any launch
    wide = 1 << 24  # 32768 segments per row
    assert f(P, 0, R, S, 1, (2 ** 32 - 2 ** 23) // 32768, wide, None) == DIT_ERR_NULL  # exactly at the limit
    assert f(P, Q, R, S, 1, (2 ** 32 - 2 ** 23) // 32768 + 1, wide, None) == DIT_ERR_ARG
    assert f(P, Q, R, S, 1, (1 << 24) - 1, wide, None) == DIT_ERR_ARG


def test_gated_residual_adaln_validation(lib):
    W = 0x800000
    X = 0x900000

    def f(x=P, y=Q, g=R, sh=S, sc=T, xo=U, z=V, B=1, N=3, D=4096, eps=1e-6):
        return lib.dit_gated_residual_adaln(x, y, g, sh, sc, xo, z, B, N, D, eps, None)

    assert f(N=-1) == DIT_ERR_ARG
    assert f(D=8200) == DIT_ERR_SHAPE
    assert f(D=20) == DIT_ERR_SHAPE
    assert f(eps=0.0) == DIT_ERR_ARG
    assert f(sh=0) == DIT_ERR_NULL
    assert f(z=V + 4) == DIT_ERR_ALIGN
    assert f(xo=P + 32) == DIT_ERR_ARG  # partial overlap with x
    assert f(xo=Q) == DIT_ERR_ARG  # x_out over y
    assert f(z=P) == DIT_ERR_ARG  # z over x
    assert f(z=U) == DIT_ERR_ARG  # both outputs in one buffer
    assert f(xo=R) == DIT_ERR_ARG  # x_out over the gate
    assert f(z=T) == DIT_ERR_ARG  # z over scale
    assert f(x=0, y=0, g=0, sh=0, sc=0, xo=0, z=0, B=0) == DIT_OK
    assert f(xo=W, z=X, N=0) == DIT_OK


def test_swiglu_validation(lib):
    f = lib.dit_swiglu
    assert f(P, Q, -1, 16384, None) == DIT_ERR_ARG
    assert f(P, Q, (1 << 24) + 1, 16384, None) == DIT_ERR_ARG
    assert f(P, Q, 4, 0, None) == DIT_ERR_SHAPE
    assert f(P, Q, 4, 1001, None) == DIT_ERR_SHAPE
    assert f(0, Q, 4, 16384, None) == DIT_ERR_NULL
    assert f(P, Q + 2, 4, 16384, None) == DIT_ERR_ALIGN
    assert f(P, P + 4 * 16384, 4, 16384, None) == DIT_ERR_ARG  # output inside the input
    assert f(0, 0, 0, 16384, None) == DIT_OK
    # M x ceil(F / 512) tiles (64 vectors each) must fit the 32-bit tile counter with the 2^24 - 1
    # workgroup grid: refused as an argument, before any launch
    wide = 1 << 24  # 32768 segments per row
    assert f(0, Q, (2 ** 32 - 2 ** 24) // 32768, wide, None) == DIT_ERR_NULL  # exactly at the limit
    assert f(P, Q, (2 ** 32 - 2 ** 24) // 32768 + 1, wide, None) == DIT_ERR_ARG
    assert f(P, Q, (1 << 24) - 1, wide, None) == DIT_ERR_ARG


def qk(lib, q=P, k=Q, qo=R, ko=S, wq=T, wk=U, pos=V, B=1, N=8, H=32, Dh=128, bands=(16, 56, 56),
       theta=1e4, eps=1e-6):
    return lib.dit_qk_rmsnorm_rope3d(q, k, qo, ko, wq, wk, pos, B, N, H, Dh, *bands, theta, eps, None)


def test_qk_validation(lib):
    assert qk(lib, N=-1) == DIT_ERR_ARG
    assert qk(lib, Dh=96, bands=(32, 32, 32)) == DIT_ERR_SHAPE
    assert qk(lib, Dh=512, bands=(128, 192, 192)) == DIT_ERR_SHAPE
    assert qk(lib, H=0) == DIT_ERR_SHAPE
    assert qk(lib, H=1024) == DIT_ERR_SHAPE  # H*Dh beyond 65536
    assert qk(lib, bands=(15, 57, 56)) == DIT_ERR_SHAPE
    assert qk(lib, bands=(16, 56, 58)) == DIT_ERR_SHAPE
    assert qk(lib, bands=(-2, 74, 56)) == DIT_ERR_SHAPE
    assert qk(lib, theta=1.0) == DIT_ERR_ARG
    assert qk(lib, theta=math.inf) == DIT_ERR_ARG
    assert qk(lib, eps=-1e-6) == DIT_ERR_ARG
    assert qk(lib, pos=0) == DIT_ERR_NULL
    assert qk(lib, wk=0) == DIT_ERR_NULL
    assert qk(lib, pos=V + 2) == DIT_ERR_ALIGN
    assert qk(lib, wq=T + 8) == DIT_ERR_ALIGN
    assert qk(lib, qo=P + 64) == DIT_ERR_ARG  # partial overlap with q
    assert qk(lib, qo=Q) == DIT_ERR_ARG  # q output over k
    assert qk(lib, ko=R) == DIT_ERR_ARG  # both outputs in one buffer
    assert qk(lib, ko=V) == DIT_ERR_ARG  # k output over the positions
    assert qk(lib, q=0, k=0, qo=0, ko=0, wq=0, wk=0, pos=0, B=0) == DIT_OK


def test_qk_layout_validation(lib):
    def f(q=P, k=P + 256, qo=R, ko=S, wq=T, wk=U, pos=V, B=1, N=8, H=32, Dh=128, stride=3 * 4096, layout=1,
          plane=0, bands=(16, 56, 56), theta=1e4, eps=1e-6):
        return lib.dit_qk_rmsnorm_rope3d_layout(q, k, qo, ko, wq, wk, pos, B, N, H, Dh, stride, layout, plane,
                                                *bands, theta, eps, None)

    assert f(stride=-8) == DIT_ERR_ARG
    assert f(layout=2) == DIT_ERR_ARG
    assert f(stride=4100) == DIT_ERR_SHAPE  # not a multiple of 8
    assert f(stride=4088) == DIT_ERR_SHAPE  # shorter than one token's heads
    assert f(Dh=96, bands=(32, 32, 32)) == DIT_ERR_SHAPE
    assert f(qo=P) == DIT_ERR_ARG  # head-major output over the fused input
    assert f(qo=P + 3 * 4096 * 2 * 3) == DIT_ERR_ARG  # inside the strided input's extent
    assert f(ko=R + 64) == DIT_ERR_ARG  # the two outputs overlap
    assert f(layout=0, stride=4096, qo=P + 64, k=Q) == DIT_ERR_ARG  # token-major, q_out partly over q
    assert f(pos=0) == DIT_ERR_NULL
    assert f(q=P + 8) == DIT_ERR_ALIGN
    assert f(q=0, k=0, qo=0, ko=0, wq=0, wk=0, pos=0, N=0) == DIT_OK
    # head-plane stride: 0 (packed) or a multiple of 8 >= N*Dh = 1024; token-major outputs take only 0
    assert f(plane=-8) == DIT_ERR_ARG
    assert f(plane=1016, pos=0) == DIT_ERR_SHAPE  # shorter than a plane
    assert f(plane=1028, pos=0) == DIT_ERR_SHAPE  # not a multiple of 8
    assert f(plane=1024, pos=0) == DIT_ERR_NULL and f(plane=1024 + 2048, pos=0) == DIT_ERR_NULL
    assert f(plane=(1 << 40) + 8) == DIT_ERR_ARG  # past the stride limit
    assert f(layout=0, stride=4096, plane=4096) == DIT_ERR_ARG
    assert f(B=1 << 16, N=1, plane=1 << 40) == DIT_ERR_ARG  # the whole output past 2^62 bytes
    # the padded extent counts for overlaps: 32 planes of 1024 + 1024 padding values = 32 * 4 KiB - 2 KiB bytes
    assert f(plane=2048, ko=R + 31 * 4096 + 2048 - 16) == DIT_ERR_ARG
    assert f(plane=2048, ko=R + 31 * 4096 + 2048, pos=0) == DIT_ERR_NULL
    assert f(plane=2048, q=0, k=0, qo=0, ko=0, wq=0, wk=0, pos=0, N=0) == DIT_OK


def test_residual_change_validation(lib):
    ws = lib.dit_residual_change_workspace_bytes
    assert ws(1, 124992, 4096) == 16 * ((124992 * 512 + 2047) // 2048)
    assert ws(2, 3, 8) == 2 * 16
    assert ws(1, 0, 8) == 0
    assert ws(-1, 4, 8) == -1 and ws(1, 4, 12) == -1 and ws(70000, 4, 8) == -1
    # at most 2^22 - 1 tiles of 2048 vectors per sample (1024-thread workgroups: < 2^32 work-items)
    assert ws(1, 8_388_606, 8192) == 16 * 4_194_303
    assert ws(1, 8_388_607, 8192) == -1

    def f(r=P, rc=Q, out=R, w=S, wb=1 << 20, B=1, N=4, D=4096):
        return lib.dit_residual_change(r, rc, out, w, wb, B, N, D, None)

    assert f(B=-1) == DIT_ERR_ARG
    assert f(N=8_388_607, D=8192) == DIT_ERR_ARG  # 4,194,304 tiles
    assert f(D=12) == DIT_ERR_SHAPE
    assert f(wb=0) == DIT_ERR_ARG  # workspace too small
    assert f(out=0) == DIT_ERR_NULL
    assert f(w=0) == DIT_ERR_NULL
    assert f(out=R + 4) == DIT_ERR_ALIGN
    assert f(w=S + 8) == DIT_ERR_ALIGN
    assert f(out=P + 64) == DIT_ERR_ARG  # output inside r
    assert f(w=Q) == DIT_ERR_ARG  # workspace over r_cached
    assert f(r=0, rc=0, out=0, w=0, B=0) == DIT_OK


def test_residual_change_noalloc_validation(lib):
    from video_diffusion_transformer_dit_amd import DIT_ERR_SCRATCH

    def f(r=P, rc=Q, out=R, B=1, N=4, D=4096):
        return lib.dit_residual_change_noalloc(r, rc, out, B, N, D, None)

    # capacity 131,072 partials: B * ceil(N * D / 16384) of them
    tiles_10s = (246_432 * 4096 // 8 + 2047) // 2048
    assert tiles_10s == 61_608 and 2 * ((124_992 * 512 + 2047) // 2048) == 62_496  # the shipped workloads fit
    assert f(N=524_288, D=4096, r=0) == DIT_ERR_NULL  # 524,288 tokens of width 4096 fill it exactly
    assert f(N=524_289, D=4096) == DIT_ERR_SCRATCH
    assert f(B=2, N=524_288, D=4096) == DIT_ERR_SCRATCH  # 2 x 131,072 partials
    assert f(B=1, N=262_145, D=8192) == DIT_ERR_SCRATCH  # one partial more than the capacity
    assert f(B=1, N=262_144, D=8192, out=0) == DIT_ERR_NULL  # exactly the capacity
    assert f(B=-1) == DIT_ERR_ARG
    assert f(B=70_000) == DIT_ERR_ARG
    assert f(N=8_388_607, D=8192) == DIT_ERR_ARG  # past the per-sample tile limit, before the capacity check
    assert f(D=12) == DIT_ERR_SHAPE
    assert f(out=0) == DIT_ERR_NULL
    assert f(r=0) == DIT_ERR_NULL
    assert f(out=R + 4) == DIT_ERR_ALIGN
    assert f(rc=Q + 8) == DIT_ERR_ALIGN
    assert f(out=P + 64) == DIT_ERR_ARG  # output inside r
    assert f(out=Q + 8) == DIT_ERR_ARG  # output inside r_cached
    assert f(r=0, rc=0, out=0, B=0) == DIT_OK
    assert f(B=2, N=524_288, D=4096, r=0, rc=0, out=0) == DIT_ERR_SCRATCH  # capacity before pointers


def test_subblock_keep_and_ld(lib):
    keep = lib.dit_subblock_keep
    assert keep(1953, 0.75) == 489 and keep(3914, 0.8) == 783 and keep(7, 0.5) == 4
    assert keep(10, 0.0) == 10 and keep(100, 0.999) == 1 and keep(0, 0.75) == 0
    assert keep(-1, 0.5) == -1 and keep(10, 1.0) == -1 and keep(10, -0.1) == -1 and keep(10, math.nan) == -1
    ld = lib.dit_subblock_scores_ld
    assert ld(1953) == 1984 and ld(32) == 32 and ld(1) == 32 and ld(0) == 0 and ld(4096) == 4096
    assert ld(4097) == -1 and ld(-1) == -1


def test_subblock_pool_validation(lib):
    # B=1, N=128, H=2, Dh=16: inputs 8 KiB each, outputs 2*2*16 floats
    def f(q=P, k=Q, qp=R, kp=S, B=1, N=128, H=2, Dh=16, layout=0):
        return lib.dit_subblock_pool(q, k, qp, kp, B, N, H, Dh, layout, None)

    assert f(B=-1, qp=0) == DIT_ERR_ARG
    assert f(N=4096 * 64 + 1, qp=0) == DIT_ERR_ARG  # more than 4096 blocks
    assert f(B=70000, qp=0) == DIT_ERR_ARG
    assert f(layout=2) == DIT_ERR_ARG
    assert f(Dh=8) == DIT_ERR_SHAPE and f(Dh=48) == DIT_ERR_SHAPE and f(Dh=512) == DIT_ERR_SHAPE
    assert f(H=0) == DIT_ERR_SHAPE and f(H=4096, Dh=32) == DIT_ERR_SHAPE  # H*Dh beyond 65536
    assert f(qp=0) == DIT_ERR_NULL and f(k=0) == DIT_ERR_NULL
    assert f(q=P + 8) == DIT_ERR_ALIGN and f(kp=S + 4) == DIT_ERR_ALIGN
    assert f(qp=P + 64) == DIT_ERR_ARG  # output inside q
    assert f(kp=Q + 4096) == DIT_ERR_ARG  # output inside k
    assert f(kp=R + 128) == DIT_ERR_ARG  # outputs overlap
    assert f(q=0, k=0, qp=0, kp=0, N=0) == DIT_OK
    assert f(q=0, k=0, qp=0, kp=0, B=0) == DIT_OK


def test_qk_pool_validation(lib):
    # B=1, N=128, H=2, Dh=16 (bands 4/6/6): q, k 8 KiB each, pooled 2*2*16 floats
    def f(q=P, k=Q, qo=R, ko=S, wq=T, wk=T + 64, pos=U, qp=V, kp=V + 4096, B=1, N=128, H=2, Dh=16, stride=32,
          layout=0, plane=0, bands=(4, 6, 6), theta=1e4, eps=1e-6):
        return lib.dit_qk_rmsnorm_rope3d_pool(q, k, qo, ko, wq, wk, pos, qp, kp, B, N, H, Dh, stride, layout, plane,
                                              *bands, theta, eps, None)

    assert f(B=-1, qp=0) == DIT_ERR_ARG
    assert f(N=4096 * 64 + 1, qp=0) == DIT_ERR_ARG
    assert f(Dh=8, bands=(2, 2, 4), qp=0) == DIT_ERR_SHAPE  # pooling needs Dh >= 16
    assert f(bands=(4, 6, 4), qp=0) == DIT_ERR_SHAPE and f(bands=(5, 5, 6), qp=0) == DIT_ERR_SHAPE
    assert f(eps=0.0, qp=0) == DIT_ERR_ARG and f(theta=1.0, qp=0) == DIT_ERR_ARG
    assert f(qp=0) == DIT_ERR_NULL and f(pos=0) == DIT_ERR_NULL
    assert f(kp=V + 4) == DIT_ERR_ALIGN and f(q=P + 8) == DIT_ERR_ALIGN
    assert f(qp=P + 64) == DIT_ERR_ARG  # pooled q over q
    assert f(kp=V + 64) == DIT_ERR_ARG  # the two pooled outputs overlap
    assert f(kp=R) == DIT_ERR_ARG  # pooled k over q_out
    assert f(qo=P + 16) == DIT_ERR_ARG  # q_out partly over q
    assert f(ko=P) == DIT_ERR_ARG  # k_out over q
    assert f(stride=24, qp=0) == DIT_ERR_SHAPE  # stride below H*Dh
    assert f(stride=36, qp=0) == DIT_ERR_SHAPE  # stride not a multiple of 8
    assert f(layout=2, qp=0) == DIT_ERR_ARG
    assert f(layout=1, qo=P) == DIT_ERR_ARG  # head-major output over its own input is not in place
    assert f(stride=96, qo=P + 64 * 200, k=P + 64) == DIT_ERR_ARG  # inside the strided input's extent
    assert f(q=0, k=0, qo=0, ko=0, wq=0, wk=0, pos=0, qp=0, kp=0, N=0) == DIT_OK
    # head-plane stride (N*Dh = 2048 values per plane)
    assert f(plane=2048) == DIT_ERR_ARG  # token-major output with a plane stride
    assert f(layout=1, plane=2040, qp=0) == DIT_ERR_SHAPE
    assert f(layout=1, plane=2052, qp=0) == DIT_ERR_SHAPE
    assert f(layout=1, plane=4096, qp=0) == DIT_ERR_NULL
    assert f(layout=1, plane=4096, ko=R + 4096 * 2 + 2048 * 2 - 16) == DIT_ERR_ARG  # k_out inside q_out's extent


def test_subblock_route_validation(lib):
    # B=1, H=2, nb=5, Dh=16: pooled 640 B each, scores 2*5*8 floats, kept 2*5*keep ints
    def f(qp=P, kp=Q, sc=R, kept=S, B=1, H=2, nb=5, Dh=16, keep=2):
        return lib.dit_subblock_route(qp, kp, sc, kept, B, H, nb, Dh, keep, None)

    assert f(B=-1, sc=0) == DIT_ERR_ARG
    assert f(nb=4097, sc=0) == DIT_ERR_ARG
    assert f(keep=-1) == DIT_ERR_ARG
    assert f(keep=6) == DIT_ERR_ARG  # more than nb
    assert f(Dh=8) == DIT_ERR_SHAPE and f(Dh=100) == DIT_ERR_SHAPE and f(H=0) == DIT_ERR_SHAPE
    assert f(kept=0) == DIT_ERR_NULL and f(qp=0) == DIT_ERR_NULL
    # no score matrix (scores and selection fused): kept is still required, and checked for overlaps
    assert f(sc=0, kept=0) == DIT_ERR_NULL and f(sc=0, kp=0) == DIT_ERR_NULL
    assert f(sc=0, kept=P + 64) == DIT_ERR_ARG and f(sc=0, kept=S + 2) == DIT_ERR_ALIGN
    assert f(sc=0, keep=0, qp=0, kp=0, kept=0) == DIT_OK  # neither output: a no-op
    assert f(sc=0, keep=6) == DIT_ERR_ARG
    assert f(qp=P + 4) == DIT_ERR_ALIGN and f(sc=R + 8) == DIT_ERR_ALIGN and f(kept=S + 2) == DIT_ERR_ALIGN
    assert f(sc=P + 64) == DIT_ERR_ARG  # scores over q_pooled
    assert f(kept=R + 16) == DIT_ERR_ARG  # kept over scores
    assert f(kept=Q) == DIT_ERR_ARG  # kept over k_pooled
    assert f(qp=0, kp=0, sc=0, kept=0, nb=0, keep=0) == DIT_OK
    assert f(qp=0, kp=0, sc=0, kept=0, B=0) == DIT_OK


def test_positions_validation(lib):
    f = lib.dit_packed_positions
    assert f(P, -1, 4, 4, 0, None) == DIT_ERR_ARG
    assert f(P, 2, 4, 4, -1, None) == DIT_ERR_ARG
    assert f(P, 1 << 12, 1 << 12, 2, 0, None) == DIT_ERR_ARG  # 2^25 tokens
    assert f(P, 1 << 40, 1 << 40, 1 << 40, 0, None) == DIT_ERR_ARG  # overflow
    assert f(0, 2, 4, 4, 0, None) == DIT_ERR_NULL
    assert f(P + 2, 2, 4, 4, 0, None) == DIT_ERR_ALIGN
    assert f(0, 0, 4, 4, 0, None) == DIT_OK


def test_copy_validation(lib):
    f = lib.dit_copy16
    assert f(P, Q, -16, None) == DIT_ERR_ARG
    assert f(P, Q, 17, None) == DIT_ERR_SHAPE
    assert f(0, Q, 16, None) == DIT_ERR_NULL
    assert f(P + 8, Q, 16, None) == DIT_ERR_ALIGN
    assert f(P, P + 16, 64, None) == DIT_ERR_ARG
    assert f(0, 0, 0, None) == DIT_OK


def test_stream_pattern_validation(lib):
    from video_diffusion_transformer_dit_amd import (DIT_STREAM_HEAD_MAJOR, DIT_STREAM_READ, DIT_STREAM_ROW_GROUP,
                                                     DIT_STREAM_ROW_GROUP_2X2, DIT_STREAM_SCORE_TILES,
                                                     DIT_STREAM_SPLIT_ROWS, DIT_STREAM_TOPK_ROWS, DIT_STREAM_TWO_IN,
                                                     DIT_STREAM_WRITE)

    def f(kind=DIT_STREAM_TWO_IN, a=P, b=Q, o=R, o2=S, rows=4, width=8192, heads=0):
        return lib.dit_stream_pattern(kind, a, b, o, o2, rows, width, heads, None)

    assert f(kind=9) == DIT_ERR_ARG and f(kind=-1) == DIT_ERR_ARG
    assert f(rows=-1) == DIT_ERR_ARG and f(rows=1 << 24) == DIT_ERR_ARG
    assert f(width=8) == DIT_ERR_SHAPE and f(width=8200) == DIT_ERR_SHAPE and f(width=0) == DIT_ERR_SHAPE
    assert f(kind=DIT_STREAM_ROW_GROUP, width=16400) == DIT_ERR_SHAPE  # row-group rows up to 16 KiB
    assert f(kind=DIT_STREAM_HEAD_MAJOR, heads=0) == DIT_ERR_SHAPE
    assert f(kind=DIT_STREAM_HEAD_MAJOR, width=8192, heads=3) == DIT_ERR_SHAPE  # 512 vectors over 3 heads
    assert f(kind=DIT_STREAM_HEAD_MAJOR, width=96 * 16, heads=32) == DIT_ERR_SHAPE  # 3 vectors per head
    assert f(kind=DIT_STREAM_HEAD_MAJOR, rows=(1 << 23), width=8192, heads=32) == DIT_ERR_ARG  # 2^24 workgroups
    assert f(kind=DIT_STREAM_SPLIT_ROWS, rows=(1 << 24) - 1, width=1 << 25) == DIT_ERR_ARG  # tile counter
    assert f(kind=DIT_STREAM_TWO_IN, rows=(1 << 24) - 1, width=1 << 25) == DIT_ERR_ARG
    assert f(b=0) == DIT_ERR_NULL and f(o=0) == DIT_ERR_NULL
    assert f(kind=DIT_STREAM_ROW_GROUP_2X2, o2=0) == DIT_ERR_NULL
    assert f(kind=DIT_STREAM_WRITE, a=0, b=0, o2=0, o=P + 8) == DIT_ERR_ALIGN
    assert f(o=Q + 16) == DIT_ERR_ARG  # output inside in1
    assert f(kind=DIT_STREAM_SPLIT_ROWS, o=P + 4 * 8192 + 16) == DIT_ERR_ARG  # inside the doubled input rows
    assert f(kind=DIT_STREAM_ROW_GROUP_2X2, o2=R + 64) == DIT_ERR_ARG  # the two outputs overlap
    assert f(kind=DIT_STREAM_READ, o=P + 4 * 8192 - 16) == DIT_ERR_ARG  # sink inside the input
    assert f(rows=0, a=0, b=0, o=0, o2=0) == DIT_OK

    def st(**kw):  # block-score tiles: heads = n blocks, rows = planes * n
        args = dict(kind=DIT_STREAM_SCORE_TILES, rows=8, width=16, heads=4, o2=0)
        args.update(kw)
        return f(**args)

    assert st(heads=0) == DIT_ERR_SHAPE
    assert st(rows=10) == DIT_ERR_SHAPE  # not a whole number of planes
    assert st(heads=8, width=16) == DIT_ERR_SHAPE  # 8 columns need 32 bytes per row
    assert st(rows=1 << 23, heads=1 << 23, width=1 << 25) == DIT_ERR_ARG  # 2^32 tiles
    assert st(b=0) == DIT_ERR_NULL  # both means are read
    assert st(o=P + 8 * 512 - 16) == DIT_ERR_ARG  # output inside the [rows][128] fp32 query means
    assert st(rows=0, a=0, b=0, o=0) == DIT_OK

    def tk(**kw):  # top-k rows: heads = n blocks, rows = planes * n, keep = ceil(n / 4) words out per row
        args = dict(kind=DIT_STREAM_TOPK_ROWS, rows=8, width=16, heads=4, b=0, o2=0)
        args.update(kw)
        return f(**args)

    assert tk(heads=0) == DIT_ERR_SHAPE and tk(heads=4097, rows=4097, width=16400) == DIT_ERR_SHAPE
    assert tk(rows=10) == DIT_ERR_SHAPE  # not a whole number of planes
    assert tk(heads=8, width=16) == DIT_ERR_SHAPE  # 8 scores need 32 bytes per row
    assert tk(rows=65536 * 2, heads=2) == DIT_ERR_ARG  # 65536 planes: past the grid's y limit
    assert tk(a=0) == DIT_ERR_NULL
    assert tk(o=P + 8 * 16 - 16) == DIT_ERR_ARG  # kept words inside the scores
    assert tk(rows=0, a=0, o=0) == DIT_OK


def test_binding_rejects_host_tensors():
    import torch

    x = torch.zeros((1, 2, 8), dtype=torch.bfloat16)
    v = torch.zeros((1, 8), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        dit.dit_adaln_modulate(x, v, v)
    with pytest.raises(TypeError):
        dit.dit_adaln_modulate(x.float(), v, v)
