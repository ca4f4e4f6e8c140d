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
