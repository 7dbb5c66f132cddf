"""The whole routed forward through the C ABI from a plain C program: no
Python, no torch.  A C99 caller built by gcc allocates device memory with
the HIP runtime, runs moe_make_row_id_map, moe_permute and moe_unpermute on
the default stream, and compares the results bit for bit with the CPU
oracle's, which it links as well (test infrastructure)."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_PROGRAM = r"""
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include "moe_perm.h"

/* the oracle (test infrastructure), declared here as it exports them */
int oracle_row_id_map(const int32_t *topk_idx, int T, int k, int E, int32_t *map,
                      int32_t *offsets);
int oracle_permute(const uint16_t *x, const float *probs, const int32_t *topk_idx,
                   const int32_t *map, int T, int H, int k, int E, uint16_t *out,
                   float *out_probs);
int oracle_unpermute(const uint16_t *in, const float *probs, const int32_t *topk_idx,
                     const int32_t *map, int T, int H, int k, int E, int64_t n_rows,
                     uint16_t *out);

#define CHECK(x) do { if ((x) != 0) { printf("fail: %s\n", #x); return 1; } } while (0)

int main(void) {
    const int T = 300, H = 136, E = 12, k = 3, n = T * k;
    int32_t *idx = malloc(sizeof(int32_t) * n);
    uint16_t *x = malloc(2 * (size_t)T * H), *P = malloc(2 * (size_t)n * H);
    float *p = malloc(sizeof(float) * n);
    uint32_t s = 12345u;
    for (int t = 0; t < T; t++) {
        int e0 = t % E;                 /* three distinct experts per token */
        idx[t * k] = e0;
        idx[t * k + 1] = (e0 + 1 + t / E % (E - 2)) % E;
        idx[t * k + 2] = (e0 + E - 1) % E;
        for (int j = 0; j < k; j++) {
            s = s * 1664525u + 1013904223u;
            p[t * k + j] = (float)(s >> 8) / 16777216.0f;
        }
    }
    for (size_t i = 0; i < (size_t)T * H; i++) {
        s = s * 1664525u + 1013904223u;
        x[i] = (uint16_t)(0x3C00u + (s >> 24)) ^ (uint16_t)((s >> 16) & 0x8000u);
    }
    for (size_t i = 0; i < (size_t)n * H; i++) {
        s = s * 1664525u + 1013904223u;
        P[i] = (uint16_t)(0x3E00u + (s >> 25)) ^ (uint16_t)((s >> 15) & 0x8000u);
    }
    void *d_idx, *d_x, *d_p, *d_map, *d_off, *d_ws, *d_out, *d_outp, *d_P, *d_y, *d_st;
    size_t ws = moe_make_row_id_map_workspace_bytes(T, k, E);
    CHECK(hipMalloc(&d_idx, sizeof(int32_t) * n));
    CHECK(hipMalloc(&d_x, 2 * (size_t)T * H));
    CHECK(hipMalloc(&d_p, sizeof(float) * n));
    CHECK(hipMalloc(&d_map, sizeof(int32_t) * (size_t)E * T));
    CHECK(hipMalloc(&d_off, sizeof(int32_t) * (E + 1)));
    CHECK(hipMalloc(&d_ws, ws));
    CHECK(hipMalloc(&d_out, 2 * (size_t)n * H));
    CHECK(hipMalloc(&d_outp, sizeof(float) * n));
    CHECK(hipMalloc(&d_P, 2 * (size_t)n * H));
    CHECK(hipMalloc(&d_y, 2 * (size_t)T * H));
    CHECK(hipMalloc(&d_st, sizeof(int32_t)));
    CHECK(hipMemset(d_st, 0, sizeof(int32_t)));
    CHECK(hipMemcpy(d_idx, idx, sizeof(int32_t) * n, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(d_x, x, 2 * (size_t)T * H, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(d_p, p, sizeof(float) * n, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(d_P, P, 2 * (size_t)n * H, hipMemcpyHostToDevice));

    CHECK(moe_make_row_id_map(d_idx, T, k, E, d_map, d_off, d_st, d_ws, ws, 0));
    CHECK(moe_permute(d_x, d_p, d_idx, d_map, T, H, k, E, n, d_out, d_outp, d_st, 0));
    CHECK(moe_unpermute(d_P, d_p, d_idx, d_map, T, H, k, E, n, d_y, d_st, 0));
    CHECK(hipDeviceSynchronize());

    int32_t *map = malloc(sizeof(int32_t) * (size_t)E * T), *off = malloc(sizeof(int32_t) * (E + 1));
    int32_t *rmap = malloc(sizeof(int32_t) * (size_t)E * T), *roff = malloc(sizeof(int32_t) * (E + 1));
    uint16_t *out = malloc(2 * (size_t)n * H), *rout = malloc(2 * (size_t)n * H);
    uint16_t *y = malloc(2 * (size_t)T * H), *ry = malloc(2 * (size_t)T * H);
    float *outp = malloc(sizeof(float) * n), *routp = malloc(sizeof(float) * n);
    int32_t st;
    CHECK(hipMemcpy(map, d_map, sizeof(int32_t) * (size_t)E * T, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(off, d_off, sizeof(int32_t) * (E + 1), hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(out, d_out, 2 * (size_t)n * H, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(outp, d_outp, sizeof(float) * n, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(y, d_y, 2 * (size_t)T * H, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(&st, d_st, sizeof(int32_t), hipMemcpyDeviceToHost));

    CHECK(oracle_row_id_map(idx, T, k, E, rmap, roff));
    CHECK(oracle_permute(x, p, idx, rmap, T, H, k, E, rout, routp));
    CHECK(oracle_unpermute(P, p, idx, rmap, T, H, k, E, n, ry));
    CHECK(st);
    CHECK(memcmp(map, rmap, sizeof(int32_t) * (size_t)E * T));
    CHECK(memcmp(off, roff, sizeof(int32_t) * (E + 1)));
    CHECK(memcmp(out, rout, 2 * (size_t)n * H));
    CHECK(memcmp(outp, routp, sizeof(float) * n));
    CHECK(memcmp(y, ry, 2 * (size_t)T * H));
    printf("c caller ok\n");
    return 0;
}
"""


def test_c_caller_routed_forward(tmp_path):
    print("[gpu-case] plain C caller: row map, permute, unpermute", flush=True)
    src = tmp_path / "caller.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "caller"
    libdir = os.path.join(ROOT, "unpermute_moe_make_amd")
    oradir = os.path.join(ROOT, "oracle")
    if not os.path.exists(os.path.join(oradir, "liboracle.so")):
        import oracle
        oracle.build()
    subprocess.check_call([
        "gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
        "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", str(src),
        "-L", libdir, "-lmoeperm", "-L", oradir, "-loracle", "-L", "/opt/rocm/lib",
        "-lamdhip64", "-Wl,-rpath," + libdir + ":" + oradir + ":/opt/rocm/lib", "-o", str(exe)])
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and "c caller ok" in out.stdout, out.stdout + out.stderr
