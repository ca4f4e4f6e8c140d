"""Element-by-element comparison of BF16 outputs, GPU against the oracle.

The bar (from the method's own precision: BF16 outputs of FP32 arithmetic)
is at most one BF16 ulp per element, with NaN matching NaN.  Both sides run
the same operation sequence, so the only expected source of a difference is
the order of the FP64 sum of squares: the GPU adds per lane, then across
lanes and waves, the oracle adds in index order.  After rounding the mean
square to FP32 the two agree except when the FP64 value lies within about
H * 2^-53 of an FP32 rounding boundary (roughly H * 2^-28 of rows); only
then can an output move by one ulp.  So the tests also require at least
99.9% of elements to be bit-identical, which any real arithmetic slip
(a contraction, a different order, a wrong rounding) would break.

Every comparison is recorded; the summary (max ulp, counts, max-abs error)
is printed at the end of the test run and, if FRN_PARITY_REPORT names a
file, written there as JSON lines.
"""
from __future__ import annotations

import json
import os
from typing import Dict, List

import numpy as np

REPORT: List[Dict] = []


def _ord(b: np.ndarray) -> np.ndarray:
    b = b.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def _is_nan(b: np.ndarray) -> np.ndarray:
    b = b.astype(np.int64)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)


def _val(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def _max_abs(got: np.ndarray, want: np.ndarray) -> float:
    """Largest |got - want| over elements finite on both sides (an infinity
    on both sides is compared by its ulp distance, which is 0 or large)."""
    g = _val(got).astype(np.float64)
    w = _val(want).astype(np.float64)
    ok = np.isfinite(g) & np.isfinite(w)
    return float(np.max(np.abs(g[ok] - w[ok]))) if np.any(ok) else 0.0


def compare(name: str, got: np.ndarray, want: np.ndarray, min_exact: float = 0.999) -> Dict:
    got = np.ascontiguousarray(got, dtype=np.uint16)
    want = np.ascontiguousarray(want, dtype=np.uint16)
    assert got.shape == want.shape, f"{name}: shape {got.shape} vs {want.shape}"
    gn, wn = _is_nan(got), _is_nan(want)
    nan_mismatch = int(np.count_nonzero(gn != wn))
    fin = ~(gn | wn)
    d = np.abs(_ord(got[fin]) - _ord(want[fin]))
    n = int(got.size)
    stats = dict(
        case=name, n=n,
        max_ulp=int(d.max()) if d.size else 0,
        n_exact=int(np.count_nonzero(d == 0)) + int(np.count_nonzero(gn & wn)),
        n_1ulp=int(np.count_nonzero(d == 1)),
        n_over=int(np.count_nonzero(d > 1)),
        nan_mismatch=nan_mismatch,
        max_abs=_max_abs(got[fin], want[fin]),
    )
    REPORT.append(stats)
    path = os.environ.get("FRN_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(stats) + "\n")
    assert nan_mismatch == 0, f"{name}: NaN positions differ ({nan_mismatch})"
    assert stats["max_ulp"] <= 1, f"{name}: {stats}"
    if n:
        assert stats["n_exact"] >= min_exact * n, f"{name}: too few bit-exact: {stats}"
    return stats
