"""Test configuration: the ``gpu`` marker and import paths.

Tests marked ``gpu`` run the HIP library on an MI355X.  Without a GPU they
fail loudly instead of skipping, so a GPU run can never turn green by
skipping its parity checks; a CPU run deselects them with ``-m "not gpu"``.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


@pytest.fixture(scope="session", autouse=True)
def built_library():
    """Build the HIP library once if nothing is built yet (a fresh checkout);
    a library already in the tree is used as it is."""
    lib = os.path.join(ROOT, "tp_reduction_rmsnorm_amd", "libfused_reduce_norm.so")
    if not os.path.exists(lib):
        import __graft_entry__
        __graft_entry__.hip_build_module().build()
    return lib


def pytest_runtest_setup(item):
    if item.get_closest_marker("gpu") is not None:
        import torch
        if not torch.cuda.is_available():
            pytest.fail("GPU test selected but no GPU is visible", pytrace=False)


def pytest_terminal_summary(terminalreporter):
    try:
        from tests import parity
    except Exception:
        return
    if not parity.REPORT:
        return
    terminalreporter.section("GPU vs oracle parity (BF16 ulp)")
    for s in parity.REPORT:
        terminalreporter.write_line(
            f"{s['case']:<58} n={s['n']:>10} max_ulp={s['max_ulp']} "
            f"1ulp={s['n_1ulp']} >1ulp={s['n_over']} max_abs={s['max_abs']:.3g}")
