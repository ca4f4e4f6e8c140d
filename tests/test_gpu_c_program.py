"""The C ABI used from plain C, with no Python or torch in the process: a
C99 program allocates device memory with the HIP runtime, calls
frn_reduce_residual_rmsnorm, frn_reduce_sandwich_norm and
frn_moe_finalize_reduce_norm (with a workspace at T=64, so on the split-row
finalize, and without one) on the default stream, and compares every output bit with the CPU oracle's C entry point
(oracle_boundary in oracle/frn_oracle.c), which it links as test
infrastructure.  Inputs: BF16 bit patterns with exponents in [2^-9, 2^1]
and random mantissas from a xorshift generator, FP32 gammas in [0.5, 1.5)."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "tp_reduction_rmsnorm_amd")
ORACLE_DIR = os.path.join(ROOT, "oracle")
ROCM = "/opt/rocm"

PROGRAM = r"""
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <hip/hip_runtime_api.h>
#include "fused_reduce_norm.h"

/* the oracle's C entry point (test infrastructure) */
int oracle_boundary(const uint16_t* const* src, const uint16_t* const* shared, int32_t R,
                    const float* w, const int32_t* idx, int32_t k, int64_t num_rows,
                    int32_t epilogue, int32_t split, const uint16_t* x, const float* g1,
                    const float* g2, float eps, int64_t T, int64_t H, uint16_t* y,
                    uint16_t* xout, uint16_t* u, const void* dbg, int32_t nthreads);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next(void) {
    state ^= state << 13; state ^= state >> 7; state ^= state << 17;
    return (uint32_t)(state >> 16);
}
static uint16_t bf16_bits(void) {
    const uint32_t r = next();
    return (uint16_t)((r & 0x807Fu) | ((118u + (r >> 8) % 10u) << 7));
}

#define CHECK(c) do { if ((c) != hipSuccess) { printf("HIP error at %d\n", __LINE__); return 2; } } while (0)

static int run(int sandwich, int32_t R, int64_t T, int64_t H) {
    const size_t n = (size_t)T * (size_t)H, bytes = n * 2;
    uint16_t* hp[16]; void* dp[16];
    uint16_t* hx = malloc(bytes); uint16_t* hy = malloc(bytes); uint16_t* hxo = malloc(bytes);
    uint16_t* ry = malloc(bytes); uint16_t* rxo = malloc(bytes);
    float* g1 = malloc((size_t)H * 4); float* g2 = malloc((size_t)H * 4);
    void *dx, *dy, *dxo; float *dg1, *dg2;
    for (int r = 0; r < R; ++r) {
        hp[r] = malloc(bytes);
        for (size_t i = 0; i < n; ++i) hp[r][i] = bf16_bits();
        CHECK(hipMalloc(&dp[r], bytes));
        CHECK(hipMemcpy(dp[r], hp[r], bytes, hipMemcpyHostToDevice));
    }
    for (size_t i = 0; i < n; ++i) hx[i] = bf16_bits();
    for (int64_t i = 0; i < H; ++i) {
        g1[i] = 0.5f + (float)(next() % 4096u) / 4096.0f;
        g2[i] = 0.5f + (float)(next() % 4096u) / 4096.0f;
    }
    CHECK(hipMalloc(&dx, bytes)); CHECK(hipMalloc(&dy, bytes)); CHECK(hipMalloc(&dxo, bytes));
    CHECK(hipMalloc((void**)&dg1, (size_t)H * 4)); CHECK(hipMalloc((void**)&dg2, (size_t)H * 4));
    CHECK(hipMemcpy(dx, hx, bytes, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dg1, g1, (size_t)H * 4, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dg2, g2, (size_t)H * 4, hipMemcpyHostToDevice));
    const float eps = 1e-6f;
    frn_status st = sandwich
        ? frn_reduce_sandwich_norm((const void* const*)dp, R, dx, dg1, dg2, eps, T, H, dy, dxo,
                                   NULL, 0, NULL)
        : frn_reduce_residual_rmsnorm((const void* const*)dp, R, dx, dg1, eps, T, H, dy, dxo,
                                      NULL, 0, NULL);
    if (st != FRN_OK) { printf("call failed: %s\n", frn_last_error()); return 3; }
    CHECK(hipDeviceSynchronize());
    CHECK(hipMemcpy(hy, dy, bytes, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(hxo, dxo, bytes, hipMemcpyDeviceToHost));
    if (oracle_boundary((const uint16_t* const*)hp, NULL, R, NULL, NULL, 0, 0, sandwich ? 1 : 0,
                        0, hx, g1, sandwich ? g2 : NULL, eps, T, H, ry, rxo, NULL, NULL, 8) != 0) {
        printf("oracle failed\n"); return 4;
    }
    size_t dy_n = 0, dx_n = 0;
    for (size_t i = 0; i < n; ++i) { dy_n += hy[i] != ry[i]; dx_n += hxo[i] != rxo[i]; }
    printf("%s R=%d T=%lld H=%lld: %zu of %zu out and %zu residual_out elements differ\n",
           sandwich ? "sandwich" : "rmsnorm", R, (long long)T, (long long)H, dy_n, n, dx_n);
    for (int r = 0; r < R; ++r) { hipFree(dp[r]); free(hp[r]); }
    hipFree(dx); hipFree(dy); hipFree(dxo); hipFree(dg1); hipFree(dg2);
    free(hx); free(hy); free(hxo); free(ry); free(rxo); free(g1); free(g2);
    return (dy_n || dx_n) ? 1 : 0;
}

/* MoE finalize folded in: R ranks of T*k expert rows, a shared-expert row
   per rank and token, the same routing on every rank (a random permutation
   of the rows), weights normalised per token; with a workspace where the
   call takes the split-row finalize */
static int run_moe(int32_t R, int32_t k, int64_t T, int64_t H, int use_ws) {
    const int64_t rows = T * k;
    const size_t n = (size_t)T * (size_t)H, bytes = n * 2, ebytes = (size_t)rows * (size_t)H * 2;
    uint16_t *he[16], *hs[16]; void *de[16], *ds[16];
    float* w = malloc((size_t)rows * 4); int32_t* idx = malloc((size_t)rows * 4);
    uint16_t* hx = malloc(bytes); uint16_t* hy = malloc(bytes); uint16_t* hxo = malloc(bytes);
    uint16_t* ry = malloc(bytes); uint16_t* rxo = malloc(bytes); float* g = malloc((size_t)H * 4);
    void *dx, *dy, *dxo, *dws = NULL, *dw, *didx; float* dg;
    for (int r = 0; r < R; ++r) {
        he[r] = malloc(ebytes); hs[r] = malloc(bytes);
        for (size_t i = 0; i < (size_t)rows * (size_t)H; ++i) he[r][i] = bf16_bits();
        for (size_t i = 0; i < n; ++i) hs[r][i] = bf16_bits();
        CHECK(hipMalloc(&de[r], ebytes)); CHECK(hipMalloc(&ds[r], bytes));
        CHECK(hipMemcpy(de[r], he[r], ebytes, hipMemcpyHostToDevice));
        CHECK(hipMemcpy(ds[r], hs[r], bytes, hipMemcpyHostToDevice));
    }
    for (int64_t i = 0; i < rows; ++i) idx[i] = (int32_t)i;
    for (int64_t i = rows - 1; i > 0; --i) {
        const int64_t j = (int64_t)(next() % (uint32_t)(i + 1));
        const int32_t t = idx[i]; idx[i] = idx[j]; idx[j] = t;
    }
    for (int64_t t = 0; t < T; ++t) {
        float sum = 0.0f;
        for (int j = 0; j < k; ++j) sum += (w[t * k + j] = 1.0f + (float)(next() % 1024u));
        for (int j = 0; j < k; ++j) w[t * k + j] /= sum;
    }
    for (size_t i = 0; i < n; ++i) hx[i] = bf16_bits();
    for (int64_t i = 0; i < H; ++i) g[i] = 0.5f + (float)(next() % 4096u) / 4096.0f;
    CHECK(hipMalloc(&dx, bytes)); CHECK(hipMalloc(&dy, bytes)); CHECK(hipMalloc(&dxo, bytes));
    CHECK(hipMalloc(&dw, (size_t)rows * 4)); CHECK(hipMalloc(&didx, (size_t)rows * 4));
    CHECK(hipMalloc((void**)&dg, (size_t)H * 4));
    CHECK(hipMemcpy(dx, hx, bytes, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dw, w, (size_t)rows * 4, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(didx, idx, (size_t)rows * 4, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dg, g, (size_t)H * 4, hipMemcpyHostToDevice));
    const size_t wsb = use_ws ? frn_workspace_bytes(T, H, R, k) : 0;
    if (wsb) CHECK(hipMalloc(&dws, wsb));
    const float eps = 1e-6f;
    frn_status st = frn_moe_finalize_reduce_norm((const void* const*)de, (const void* const*)ds, R,
                                                 (const float*)dw, (const int32_t*)didx, k, rows,
                                                 FRN_EPI_RMSNORM, dx, dg, NULL, eps, T, H, dy, dxo,
                                                 dws, wsb, NULL);
    if (st != FRN_OK) { printf("call failed: %s\n", frn_last_error()); return 3; }
    CHECK(hipDeviceSynchronize());
    CHECK(hipMemcpy(hy, dy, bytes, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(hxo, dxo, bytes, hipMemcpyDeviceToHost));
    if (oracle_boundary((const uint16_t* const*)he, (const uint16_t* const*)hs, R, w, idx, k, rows,
                        0, 0, hx, g, NULL, eps, T, H, ry, rxo, NULL, NULL, 8) != 0) {
        printf("oracle failed\n"); return 4;
    }
    size_t dy_n = 0, dx_n = 0;
    for (size_t i = 0; i < n; ++i) { dy_n += hy[i] != ry[i]; dx_n += hxo[i] != rxo[i]; }
    printf("moe R=%d k=%d T=%lld H=%lld%s: %zu of %zu out and %zu residual_out elements differ\n",
           R, k, (long long)T, (long long)H, wsb ? " (split-row finalize)" : "", dy_n, n, dx_n);
    for (int r = 0; r < R; ++r) { hipFree(de[r]); hipFree(ds[r]); free(he[r]); free(hs[r]); }
    hipFree(dx); hipFree(dy); hipFree(dxo); hipFree(dw); hipFree(didx); hipFree(dg);
    if (dws) hipFree(dws);
    free(w); free(idx); free(hx); free(hy); free(hxo); free(ry); free(rxo); free(g);
    return (dy_n || dx_n) ? 1 : 0;
}

int main(void) {
    int rc = 0;
    rc |= run(0, 2, 300, 4096);    /* several workgroups per CU, ragged count */
    rc |= run(1, 4, 300, 5120);
    rc |= run(1, 4, 1000, 5120);   /* four vectors per lane */
    rc |= run(0, 1, 2048, 7168);   /* the row-pipelined kernel */
    rc |= run_moe(8, 10, 64, 6144, 1);
    rc |= run_moe(8, 10, 300, 6144, 0);
    return rc;
}
"""


def test_c_program_matches_the_oracle(tmp_path):
    src = tmp_path / "frn_c_parity.c"
    src.write_text(PROGRAM)
    exe = str(tmp_path / "frn_c_parity")
    cc = subprocess.run(["gcc", "-std=c99", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                         "-I", os.path.join(ROOT, "include"), "-I", f"{ROCM}/include",
                         str(src), "-o", exe,
                         "-L", LIBDIR, "-lfused_reduce_norm", f"-Wl,-rpath,{LIBDIR}",
                         "-L", ORACLE_DIR, "-loracle_frn", f"-Wl,-rpath,{ORACLE_DIR}",
                         "-L", f"{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"],
                        capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(run.stdout)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.count(": 0 of") == 6
