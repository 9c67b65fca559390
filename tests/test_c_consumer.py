"""The C ABI used from a plain C program (host only).

A small C99 program includes include/dit_ops.h, links libdit_ops.so and calls
the entry points that make no HIP call: the version and status strings, the
SubBlock size helpers, and argument validation with fake pointers (every
call below fails validation or is a zero-row no-op, so nothing is launched).
This checks that the header is valid C, that the symbols resolve at link
time from C, and that the documented status codes come back through the C
calling convention, not only through ctypes.
"""
import os
import shutil
import subprocess

import pytest

import video_diffusion_transformer_dit_amd as dit

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CC = shutil.which("gcc") or shutil.which("cc")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "dit_ops.h"

#define CHECK(cond) do { if (!(cond)) { printf("FAIL line %d: %s\n", __LINE__, #cond); return 1; } } while (0)

int main(void)
{
    dit_bf16 *p = (dit_bf16 *)(uintptr_t)0x100000; /* aligned, never dereferenced */
    dit_bf16 *q = (dit_bf16 *)(uintptr_t)0x200000;
    dit_bf16 *r = (dit_bf16 *)(uintptr_t)0x300000;
    dit_bf16 *s = (dit_bf16 *)(uintptr_t)0x400000;
    CHECK(dit_abi_version() == DIT_ABI_VERSION);
    CHECK(strlen(dit_status_str(DIT_OK)) > 0);
    CHECK(dit_status_str(12345) != NULL);
    CHECK(dit_subblock_keep(1953, 0.75) == 1953 - 1464);
    CHECK(dit_subblock_keep(-1, 0.5) == -1);
    CHECK(dit_subblock_scores_ld(1953) == 1984);
    /* validation before any HIP call */
    CHECK(dit_adaln_modulate(NULL, q, r, s, 1, 4, 4096, 1e-6f, NULL) == DIT_ERR_NULL);
    CHECK(dit_adaln_modulate(p, q, r, s, 1, 4, 4100, 1e-6f, NULL) == DIT_ERR_SHAPE);
    CHECK(dit_adaln_modulate(p, q, r, s, 1, 4, 4096, 0.0f, NULL) == DIT_ERR_ARG);
    CHECK(dit_gated_residual(p, q, r, (dit_bf16 *)((char *)s + 2), 1, 4, 4096, NULL) == DIT_ERR_ALIGN);
    CHECK(dit_swiglu(p, q, 4, 12, NULL) == DIT_ERR_SHAPE);
    CHECK(dit_qk_rmsnorm_rope3d(p, q, r, s, p, q, (const int32_t *)r, 1, 4, 32, 128, 16, 56, 58, 1e4f, 1e-6f,
                                NULL) == DIT_ERR_SHAPE);
    /* zero rows: a no-op that succeeds */
    CHECK(dit_adaln_modulate(p, q, r, s, 1, 0, 4096, 1e-6f, NULL) == DIT_OK);
    CHECK(dit_swiglu(p, q, 0, 16384, NULL) == DIT_OK);
    printf("ok\n");
    return 0;
}
"""


@pytest.mark.skipif(CC is None, reason="no C compiler")
def test_c_program_links_and_validates(tmp_path):
    import torch

    if torch.cuda.is_available():
        pytest.skip("fake-pointer validation checks run only without a HIP device")
    if not os.path.exists(dit.LIB_PATH):
        from video_diffusion_transformer_dit_amd import build

        build.build()
    src = tmp_path / "consumer.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "consumer"
    libdir = os.path.dirname(dit.LIB_PATH)
    cmd = [CC, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", f"-I{os.path.join(ROOT, 'include')}",
           str(src), "-o", str(exe), f"-L{libdir}", "-l:libdit_ops.so", f"-Wl,-rpath,{libdir}"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
