"""The C ABI end to end from plain C on the GPU: a C99 program (gcc, HIP's C runtime API for device
memory) fills q, k, v, dO with closed-form values, calls la2_forward and la2_backward through
include/la2.h and checks the results on the host, with no C++, Python or torch in between.

Inputs (fp32, B = 1, H = 2, T = 1000, d = d_v = 64, tile 64, so the chains are split into segments):
q_t = k_t = e_0, v_t = 1, do_t = 1/64, lam = 1/2 for both heads.  By the token recurrence
  o_t = (2 - 2^-t) 1,  dq_t = (2 - 2^-t) e_0,  dk_t = c_t e_0,  dv_t = c_t / 64 1,
with c_t = 2 - 2^-(T-1-t).  Bar: max|err| <= 1e-5 max|ref| per tensor, as for every fp32 case.
"""
import os
import shutil
import subprocess

import pytest

from causal_linear_attention_amd import binding

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#define __HIP_PLATFORM_AMD__ 1
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include "la2.h"

#define B 1
#define H 2
#define T 1000
#define D 64

static double worst(const float *x, int n, double (*ref)(int t, int j)) {
    double w = 0.0;
    for (int i = 0; i < n; ++i) {
        const int t = (i / D) % T, j = i % D;
        const double e = fabs((double)x[i] - ref(t, j));
        if (!(e <= w)) w = e;   /* NaN propagates */
    }
    return w;
}
static double r_o(int t, int j) { (void)j; return 2.0 - ldexp(1.0, -t); }
static double r_dq(int t, int j) { return j == 0 ? 2.0 - ldexp(1.0, -t) : 0.0; }
static double r_dk(int t, int j) { return j == 0 ? 2.0 - ldexp(1.0, -(T - 1 - t)) : 0.0; }
static double r_dv(int t, int j) { (void)j; return (2.0 - ldexp(1.0, -(T - 1 - t))) / D; }

#define CHECK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("hip %d at %s\n", (int)e_, #x); return 2; } } while (0)

int main(void) {
    const size_t n = (size_t)B * H * T * D, bytes = n * sizeof(float);
    float *hq = malloc(bytes), *hv = malloc(bytes), *hdo = malloc(bytes), *hout = malloc(bytes);
    for (size_t i = 0; i < n; ++i) {
        hq[i] = (i % D) == 0 ? 1.0f : 0.0f;
        hv[i] = 1.0f;
        hdo[i] = 1.0f / D;
    }
    const float hdecay[H] = {0.5f, 0.5f};
    float *q, *k, *v, *o, *dout, *dq, *dk, *dv, *decay;
    void *ws;
    const size_t wsb = la2_workspace_bytes(B, H, T, D, D, 64, LA2_F32, 1);
    CHECK(hipMalloc((void **)&q, bytes)); CHECK(hipMalloc((void **)&k, bytes)); CHECK(hipMalloc((void **)&v, bytes));
    CHECK(hipMalloc((void **)&o, bytes)); CHECK(hipMalloc((void **)&dout, bytes)); CHECK(hipMalloc((void **)&dq, bytes));
    CHECK(hipMalloc((void **)&dk, bytes)); CHECK(hipMalloc((void **)&dv, bytes));
    CHECK(hipMalloc((void **)&decay, sizeof hdecay)); CHECK(hipMalloc(&ws, wsb > 0 ? wsb : 16));
    CHECK(hipMemcpy(q, hq, bytes, hipMemcpyHostToDevice)); CHECK(hipMemcpy(k, hq, bytes, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(v, hv, bytes, hipMemcpyHostToDevice)); CHECK(hipMemcpy(dout, hdo, bytes, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(decay, hdecay, sizeof hdecay, hipMemcpyHostToDevice));
    int st = la2_forward(q, k, v, decay, o, B, H, T, D, D, 64, LA2_F32, ws, wsb, NULL);
    if (st != LA2_OK) { printf("la2_forward: %s\n", la2_status_string(st)); return 3; }
    st = la2_backward(q, k, v, decay, dout, dq, dk, dv, B, H, T, D, D, 64, LA2_F32, ws, wsb, NULL);
    if (st != LA2_OK) { printf("la2_backward: %s\n", la2_status_string(st)); return 3; }
    CHECK(hipDeviceSynchronize());
    CHECK(hipMemcpy(hout, o, bytes, hipMemcpyDeviceToHost));
    printf("o %.3e\n", worst(hout, (int)n, r_o) / 2.0);
    CHECK(hipMemcpy(hout, dq, bytes, hipMemcpyDeviceToHost));
    printf("dq %.3e\n", worst(hout, (int)n, r_dq) / 2.0);
    CHECK(hipMemcpy(hout, dk, bytes, hipMemcpyDeviceToHost));
    printf("dk %.3e\n", worst(hout, (int)n, r_dk) / 2.0);
    CHECK(hipMemcpy(hout, dv, bytes, hipMemcpyDeviceToHost));
    printf("dv %.3e\n", worst(hout, (int)n, r_dv) / (2.0 / D));
    hipFree(q); hipFree(k); hipFree(v); hipFree(o); hipFree(dout); hipFree(dq); hipFree(dk); hipFree(dv);
    hipFree(decay); hipFree(ws);
    free(hq); free(hv); free(hdo); free(hout);
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_plain_c_program_on_the_gpu(tmp_path):
    binding.load_library()
    src = tmp_path / "la2_c_gpu.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "la2_c_gpu"
    libdir = os.path.dirname(binding.LIB_PATH)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", f"-I{os.path.join(ROOT, 'include')}",
           f"-I{rocm}/include", str(src), f"-L{libdir}", "-lla2", f"-L{rocm}/lib", "-lamdhip64", "-lm",
           f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{rocm}/lib", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    print("running the C program: fp32, B=1, H=2, T=1000, d=d_v=64, tile 64, lam=1/2", flush=True)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(run.stdout, run.stderr, flush=True)
    assert run.returncode == 0, run.stdout
    errs = dict(line.split(" ", 1) for line in run.stdout.strip().splitlines())
    for name in ("o", "dq", "dk", "dv"):
        assert float(errs[name]) <= 1e-5, (name, errs[name])
