"""The header is plain C: a C99 program includes it, links the library and
calls the entry points that need no GPU (CPU only)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "tp_reduction_rmsnorm_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "fused_reduce_norm.h"

static int fails = 0;
#define EXPECT(c) do { if (!(c)) { printf("FAILED: %s\n", #c); ++fails; } } while (0)

int main(void) {
    const void* parts[2] = {(const void*)0x100000, (const void*)0x200000};
    int32_t th = 0, vec = 0;
    EXPECT(strcmp(frn_version(), FRN_VERSION_STRING) == 0);
    EXPECT(frn_query(4, 0, 4096, 5120, FRN_EPI_SANDWICH) == FRN_OK);
    EXPECT(frn_query(FRN_MAX_R + 1, 0, 8, 512, FRN_EPI_RMSNORM) == FRN_ERR_UNSUPPORTED);
    EXPECT(frn_query(2, 0, FRN_MAX_T + 1LL, 512, FRN_EPI_RMSNORM) == FRN_ERR_UNSUPPORTED);
    EXPECT(frn_query(0, 0, 8, 512, FRN_EPI_RMSNORM) == FRN_ERR_INVALID);
    EXPECT(frn_workspace_bytes(64, 6144, 8, 10) == (size_t)64 * 6144 * 4 + 64 * 12 * 8);
    EXPECT(frn_workspace_bytes(64, 6144, 8, 0) == 0);
    EXPECT(frn_launch_shape(8, 10, 1024, 6144, FRN_EPI_RMSNORM | FRN_SHAPE_EP, &th, &vec) == FRN_OK);
    EXPECT(th == 768 && vec == 1);
    EXPECT(frn_split_rows(8, 10, 16, 6144, FRN_EPI_RMSNORM | FRN_SHAPE_EP) == 1);
    EXPECT(frn_split_rows(8, 10, 96, 6144, FRN_EPI_RMSNORM | FRN_SHAPE_EP) == 0);
    EXPECT(frn_split_rows(8, 10, 96, 6144, FRN_EPI_RMSNORM) == 1);
    /* a rejected call names its reason and launches nothing */
    EXPECT(frn_reduce_residual_rmsnorm(parts, 2, NULL, NULL, 1e-6f, 4, 64, NULL, NULL, NULL, 0,
                                       NULL) == FRN_ERR_INVALID);
    EXPECT(strlen(frn_last_error()) > 0);
    EXPECT(frn_moe_finalize_reduce_norm_noalloc(parts, NULL, 2, NULL, NULL, 3, 12, FRN_EPI_RMSNORM,
                                                NULL, NULL, NULL, 1e-6f, 0, 64, NULL, NULL,
                                                NULL) == FRN_OK);
    EXPECT(FRN_NOALLOC_SCRATCH_BYTES == 17825792u);
    EXPECT(strcmp(frn_status_string(FRN_OK), "") != 0);
    /* T == 0 is a no-op once the sizes are valid */
    EXPECT(frn_reduce_sandwich_norm(parts, 2, NULL, NULL, NULL, 1e-6f, 0, 64, NULL, NULL, NULL, 0,
                                    NULL) == FRN_OK);
    printf("%d failures\n", fails);
    return fails != 0;
}
"""


def test_header_compiles_as_c99_and_links(tmp_path):
    lib = os.path.join(LIBDIR, "libfused_reduce_norm.so")
    if not os.path.exists(lib):
        import __graft_entry__
        __graft_entry__.hip_build_module().build()
    src = tmp_path / "use_frn.c"
    src.write_text(PROGRAM)
    exe = str(tmp_path / "use_frn")
    cc = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                         "-I", os.path.join(ROOT, "include"), str(src), "-o", exe,
                         "-L", LIBDIR, "-lfused_reduce_norm", f"-Wl,-rpath,{LIBDIR}"],
                        capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
