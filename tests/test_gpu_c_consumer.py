"""The library driven from a plain C program on the GPU, with no Python or torch
in the process.

A C99 program built with gcc against include/dit_ops.h and the HIP runtime's
C API allocates device memory, copies seeded bf16 inputs in, calls
dit_swiglu and dit_adaln_modulate on a stream of its own, copies the results
back and checks every element against the C oracle (liboracle_dit.so) within
|err| <= 1e-2 + 8e-3 |ref|.  This shows the C ABI is complete on its own:
torch is plumbing for the Python binding, not a dependency of the library.
"""
import os
import re
import shutil
import subprocess

import pytest

import oracle
import video_diffusion_transformer_dit_amd as dit

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CC = shutil.which("gcc") or shutil.which("cc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

PROGRAM = r"""
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <hip/hip_runtime_api.h>
#include "dit_ops.h"

/* the oracle's entry points (oracle/dit_oracle.c) */
double dit_oracle_bf16_decode(uint16_t bits);
int dit_oracle_swiglu(const uint16_t *in, double *out, int64_t M, int64_t F);
int dit_oracle_adaln_modulate(const uint16_t *x, const uint16_t *shift, const uint16_t *scale, double *y,
                              int64_t B, int64_t N, int64_t D, double eps);

/* seeded inputs: xorshift64, a sum of twelve uniforms (about normal), rounded to bf16 bits */
static uint64_t state = 0x9e3779b97f4a7c15ull;
static double uniform(void)
{
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (double)(state >> 11) / 9007199254740992.0;
}
static uint16_t draw(double sigma)
{
    double v = 0.0;
    for (int i = 0; i < 12; ++i)
        v += uniform();
    float f = (float)((v - 6.0) * sigma);
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static double worst_ratio(const uint16_t *got, const double *ref, size_t n)
{
    double w = 0.0;
    for (size_t i = 0; i < n; ++i) {
        const double r = fabs(dit_oracle_bf16_decode(got[i]) - ref[i]) / (1e-2 + 8e-3 * fabs(ref[i]));
        if (!(r <= w))
            w = r; /* a NaN sticks */
    }
    return w;
}

#define HIPCHECK(x)                                                                                                \
    do {                                                                                                           \
        hipError_t e_ = (x);                                                                                       \
        if (e_ != hipSuccess) {                                                                                    \
            printf("HIP error %d at line %d\n", (int)e_, __LINE__);                                               \
            return 2;                                                                                              \
        }                                                                                                          \
    } while (0)

int main(void)
{
    int ndev = 0;
    HIPCHECK(hipGetDeviceCount(&ndev));
    if (ndev < 1) {
        printf("no device\n");
        return 3;
    }
    hipStream_t st;
    HIPCHECK(hipStreamCreate(&st));

    /* SwiGLU: 37 rows of [a | b], F = 1000 */
    const int64_t M = 37, F = 1000;
    const size_t nin = (size_t)(M * 2 * F), nout = (size_t)(M * F);
    uint16_t *h_in = malloc(nin * 2), *h_out = malloc(nout * 2);
    double *ref = malloc(nout * sizeof(double));
    for (size_t i = 0; i < nin; ++i)
        h_in[i] = draw(1.0);
    void *d_in, *d_out;
    HIPCHECK(hipMalloc(&d_in, nin * 2));
    HIPCHECK(hipMalloc(&d_out, nout * 2));
    HIPCHECK(hipMemcpy(d_in, h_in, nin * 2, hipMemcpyHostToDevice));
    int rc = dit_swiglu(d_in, d_out, M, F, st);
    if (rc != DIT_OK) {
        printf("dit_swiglu: %s\n", dit_status_str(rc));
        return 1;
    }
    HIPCHECK(hipStreamSynchronize(st));
    HIPCHECK(hipMemcpy(h_out, d_out, nout * 2, hipMemcpyDeviceToHost));
    if (dit_oracle_swiglu(h_in, ref, M, F) != 0)
        return 4;
    const double w_swiglu = worst_ratio(h_out, ref, nout);

    /* AdaLN: two samples of 5 rows, D = 264 (ragged against the 16-value thread slices) */
    const int64_t B = 2, N = 5, D = 264;
    const size_t nx = (size_t)(B * N * D), nv = (size_t)(B * D);
    uint16_t *h_x = malloc(nx * 2), *h_sh = malloc(nv * 2), *h_sc = malloc(nv * 2), *h_y = malloc(nx * 2);
    double *ref_y = malloc(nx * sizeof(double));
    for (size_t i = 0; i < nx; ++i)
        h_x[i] = draw(1.0);
    for (size_t i = 0; i < nv; ++i) {
        h_sh[i] = draw(0.1);
        h_sc[i] = draw(0.1);
    }
    void *d_x, *d_sh, *d_sc, *d_y;
    HIPCHECK(hipMalloc(&d_x, nx * 2));
    HIPCHECK(hipMalloc(&d_sh, nv * 2));
    HIPCHECK(hipMalloc(&d_sc, nv * 2));
    HIPCHECK(hipMalloc(&d_y, nx * 2));
    HIPCHECK(hipMemcpy(d_x, h_x, nx * 2, hipMemcpyHostToDevice));
    HIPCHECK(hipMemcpy(d_sh, h_sh, nv * 2, hipMemcpyHostToDevice));
    HIPCHECK(hipMemcpy(d_sc, h_sc, nv * 2, hipMemcpyHostToDevice));
    rc = dit_adaln_modulate(d_x, d_sh, d_sc, d_y, B, N, D, 1e-6f, st);
    if (rc != DIT_OK) {
        printf("dit_adaln_modulate: %s\n", dit_status_str(rc));
        return 1;
    }
    HIPCHECK(hipStreamSynchronize(st));
    HIPCHECK(hipMemcpy(h_y, d_y, nx * 2, hipMemcpyDeviceToHost));
    if (dit_oracle_adaln_modulate(h_x, h_sh, h_sc, ref_y, B, N, D, 1e-6) != 0)
        return 4;
    const double w_adaln = worst_ratio(h_y, ref_y, nx);

    printf("worst swiglu %.4f adaln %.4f\n", w_swiglu, w_adaln);
    HIPCHECK(hipFree(d_in));
    HIPCHECK(hipFree(d_out));
    HIPCHECK(hipFree(d_x));
    HIPCHECK(hipFree(d_sh));
    HIPCHECK(hipFree(d_sc));
    HIPCHECK(hipFree(d_y));
    HIPCHECK(hipStreamDestroy(st));
    free(h_in), free(h_out), free(ref), free(h_x), free(h_sh), free(h_sc), free(h_y), free(ref_y);
    return (w_swiglu <= 1.0 && w_adaln <= 1.0) ? 0 : 1;
}
"""


@pytest.mark.skipif(CC is None, reason="no C compiler")
def test_c_program_runs_the_library_on_the_gpu(tmp_path):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    assert os.path.exists(dit.LIB_PATH), "libdit_ops.so is not built"
    oracle.load()  # builds liboracle_dit.so if it is absent
    src = tmp_path / "gpu_consumer.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "gpu_consumer"
    libdir, odir = os.path.dirname(dit.LIB_PATH), os.path.dirname(oracle.LIB_PATH)
    cmd = [CC, "-std=c99", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{os.path.join(ROCM, 'include')}",
           f"-I{os.path.join(ROOT, 'include')}", str(src), "-o", str(exe),
           f"-L{libdir}", "-l:libdit_ops.so", f"-Wl,-rpath,{libdir}",
           f"-L{odir}", "-l:liboracle_dit.so", f"-Wl,-rpath,{odir}",
           f"-L{os.path.join(ROCM, 'lib')}", "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    print("running", exe, flush=True)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(run.stdout, flush=True)
    assert run.returncode == 0, run.stdout + run.stderr[-2000:]
    m = re.search(r"worst swiglu ([0-9.]+) adaln ([0-9.]+)", run.stdout)
    assert m and float(m.group(1)) <= 1.0 and float(m.group(2)) <= 1.0, run.stdout
