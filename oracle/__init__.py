"""Plain CPU oracle of the fused reduce + norm boundary.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
(``tp_reduction_rmsnorm_amd``) never imports it and shares no code with it.

The arithmetic lives in ``frn_oracle.c`` (plain C, built with
``gcc -O2 -ffp-contract=off``); this module only compiles it, marshals numpy
arrays through ctypes and returns numpy arrays.  BF16 tensors travel as
``uint16`` bit patterns.

What each call computes, and the passages it follows:

* ``boundary(...)``: vLLM PR #62366, sections "Overview"/"Claims"/"Details":
  optional per-rank MoE top-k finalize rounded to BF16, FP32 reduction over
  the R partials, then residual add + RMSNorm or the FP32 norm -> residual
  add -> norm sandwich, FP32 math uncontracted; SGLang PR #34134 first commit
  message: the finalize includes the shared-expert add.
* ``split=True``: the large-batch path of vLLM PR #62366 "Claims": the
  reduction alone produces a BF16 tensor, the boundary kernel runs after it.
* ``ep_boundary(...)``: the expert-parallel deferral that vLLM PR #62366
  names in "Overview" and "Details" (tokens replicated on every rank,
  TP = 1, EP > 1): each rank finalizes only the top-k slots of its own
  experts (a negative row index marks another rank's slot), may or may not
  hold a shared-expert row, rounds to BF16, and the R partials then take the
  same reduction and epilogue.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "frn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_frn.so")

EPI_RMSNORM = 0
EPI_SANDWICH = 1
EPI_NONE = 2

_lib = None


GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
             "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra", "-Werror"]


def compile_source(src: str, out: str, werror: bool = True) -> str:
    """Compile an oracle source file into a shared library at ``out``."""
    tmp = out + f".tmp{os.getpid()}"
    flags = GCC_FLAGS if werror else [f for f in GCC_FLAGS if f != "-Werror"] + ["-w"]
    subprocess.run(["gcc", *flags, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    return compile_source(_SRC, _LIB)


class _Debug(ctypes.Structure):
    _fields_ = [("s", ctypes.c_void_p), ("a", ctypes.c_void_p),
                ("h", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("r1", ctypes.c_void_p), ("r2", ctypes.c_void_p),
                ("ss1", ctypes.c_void_p), ("ss2", ctypes.c_void_p),
                ("p", ctypes.c_void_p), ("u", ctypes.c_void_p)]


def _bind(lib):
    P = ctypes.c_void_p
    lib.oracle_boundary.restype = ctypes.c_int
    lib.oracle_boundary.argtypes = [
        P, P, ctypes.c_int32, P, P, ctypes.c_int32, ctypes.c_int64,
        ctypes.c_int32, ctypes.c_int32, P, P, P, ctypes.c_float,
        ctypes.c_int64, ctypes.c_int64, P, P, P, P, ctypes.c_int32]
    lib.oracle_ep_boundary.restype = ctypes.c_int
    lib.oracle_ep_boundary.argtypes = [
        P, P, ctypes.c_int32, P, P, ctypes.c_int32, P,
        ctypes.c_int32, ctypes.c_int32, P, P, P, ctypes.c_float,
        ctypes.c_int64, ctypes.c_int64, P, P, P, P, ctypes.c_int32]
    lib.oracle_bf16_to_f32.restype = ctypes.c_float
    lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
    lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.oracle_bf16_to_f32_array.restype = None
    lib.oracle_bf16_to_f32_array.argtypes = [P, P, ctypes.c_int64]
    lib.oracle_f32_to_bf16_array.restype = None
    lib.oracle_f32_to_bf16_array.argtypes = [P, P, ctypes.c_int64]
    lib.oracle_inv_rms.restype = ctypes.c_float
    lib.oracle_inv_rms.argtypes = [P, ctypes.c_int64, ctypes.c_float, P]
    return lib


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


_override = None


class use_library:
    """Context manager: route this module's calls through another build of
    the oracle source (the pin tests use it to show that a planted mistake
    is caught)."""

    def __init__(self, so_path: str):
        self.lib = _bind(ctypes.CDLL(so_path))

    def __enter__(self):
        global _override
        self._prev = _override
        _override = self.lib
        return self

    def __exit__(self, *exc):
        global _override
        _override = self._prev
        return False


def _active():
    return _override if _override is not None else _load()


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    b = _c(bits, np.uint16)
    out = np.empty(b.shape, np.float32)
    _active().oracle_bf16_to_f32_array(_ptr(b), _ptr(out), b.size)
    return out


def f32_to_bf16(vals: np.ndarray) -> np.ndarray:
    v = _c(vals, np.float32)
    out = np.empty(v.shape, np.uint16)
    _active().oracle_f32_to_bf16_array(_ptr(v), _ptr(out), v.size)
    return out


def inv_rms(x: np.ndarray, eps: float):
    """Inverse RMS of one FP32 row; returns (rinv, FP64 sum of squares)."""
    x = _c(x, np.float32)
    ss = np.zeros(1, np.float64)
    r = _active().oracle_inv_rms(_ptr(x), x.size, ctypes.c_float(eps), _ptr(ss))
    return np.float32(r), float(ss[0])


@dataclass
class Result:
    y: Optional[np.ndarray]      # [T,H] uint16 (BF16 normed output)
    xout: Optional[np.ndarray]   # [T,H] uint16 (BF16 new residual)
    u: Optional[np.ndarray]      # [T,H] uint16 (BF16 reduced sum, split pass 1)
    s: Optional[np.ndarray] = None    # [T,H] f32 reduced sum
    a: Optional[np.ndarray] = None    # [T,H] f32 first-norm output (sandwich)
    h: Optional[np.ndarray] = None    # [T,H] f32 new residual before rounding
    y32: Optional[np.ndarray] = None  # [T,H] f32 output before rounding
    r1: Optional[np.ndarray] = None   # [T] f32
    r2: Optional[np.ndarray] = None   # [T] f32
    ss1: Optional[np.ndarray] = None  # [T] f64
    ss2: Optional[np.ndarray] = None  # [T] f64
    p: Optional[np.ndarray] = None    # [R,T,H] uint16 finalized partials


def _outputs(T, H, R, epilogue, split, finalize, debug):
    """Output arrays and, with debug, the debug block for one oracle call."""
    if epilogue == EPI_NONE:
        y = xout = None
        u = np.zeros((T, H), np.uint16)
    else:
        y = np.zeros((T, H), np.uint16)
        xout = np.zeros((T, H), np.uint16)
        u = None
    res = Result(y=y, xout=xout, u=u)
    dbg = None
    if debug:
        res.s = np.zeros((T, H), np.float32)
        res.a = np.zeros((T, H), np.float32)
        res.h = np.zeros((T, H), np.float32)
        res.y32 = np.zeros((T, H), np.float32)
        res.r1 = np.zeros(T, np.float32)
        res.r2 = np.zeros(T, np.float32)
        res.ss1 = np.zeros(T, np.float64)
        res.ss2 = np.zeros(T, np.float64)
        res.p = np.zeros((R, T, H), np.uint16) if finalize else None
        res.u = np.zeros((T, H), np.uint16) if u is None else u
        dbg = _Debug(_ptr(res.s), _ptr(res.a), _ptr(res.h), _ptr(res.y32),
                     _ptr(res.r1), _ptr(res.r2), _ptr(res.ss1), _ptr(res.ss2),
                     _ptr(res.p), _ptr(res.u) if (split or epilogue == EPI_NONE) else None)
    return res, y, xout, u, dbg


def _finish(res, rc, name, debug, split, epilogue):
    if rc != 0:
        raise ValueError(f"{name} rejected its arguments")
    if debug and not (split or epilogue == EPI_NONE):
        res.u = None
    return res


def _dbg_ptr(dbg):
    return ctypes.cast(ctypes.pointer(dbg), ctypes.c_void_p) if dbg is not None else None


def boundary(src: Sequence[np.ndarray], *, residual=None, gamma1=None, gamma2=None,
             eps: float = 1e-6, epilogue: int = EPI_RMSNORM, split: bool = False,
             topk_w=None, topk_idx=None, shared: Optional[Sequence[np.ndarray]] = None,
             T: Optional[int] = None, H: Optional[int] = None, debug: bool = False,
             nthreads: int = 1) -> Result:
    """Run the oracle.

    src: R arrays of BF16 bits, the partials [T,H] (no finalize) or the expert
    output buffers [num_rows,H] (finalize, when topk_w/topk_idx are given).
    """
    lib = _active()
    R = len(src)
    srcs = [_c(a, np.uint16) for a in src]
    finalize = topk_w is not None
    if finalize:
        w = _c(topk_w, np.float32)
        idx = _c(topk_idx, np.int32)
        T = w.shape[0] if T is None else T
        k = w.shape[1]
        H = srcs[0].shape[1]
        num_rows = srcs[0].shape[0]
    else:
        w = idx = None
        k = 0
        T, H = srcs[0].shape
        num_rows = 0
    sh = [_c(a, np.uint16) for a in shared] if shared is not None else None
    src_arr = (ctypes.c_void_p * R)(*[a.ctypes.data for a in srcs])
    sh_arr = (ctypes.c_void_p * R)(*[a.ctypes.data for a in sh]) if sh else None
    x = _c(residual, np.uint16) if residual is not None else None
    g1 = _c(gamma1, np.float32) if gamma1 is not None else None
    g2 = _c(gamma2, np.float32) if gamma2 is not None else None
    res, y, xout, u, dbg = _outputs(T, H, R, epilogue, split, finalize, debug)
    rc = lib.oracle_boundary(
        ctypes.cast(src_arr, ctypes.c_void_p),
        ctypes.cast(sh_arr, ctypes.c_void_p) if sh_arr is not None else None,
        R, _ptr(w), _ptr(idx), k, num_rows, epilogue, int(bool(split)),
        _ptr(x), _ptr(g1), _ptr(g2), ctypes.c_float(eps), T, H,
        _ptr(y), _ptr(xout), _ptr(u), _dbg_ptr(dbg), nthreads)
    return _finish(res, rc, "oracle_boundary", debug, split, epilogue)


def ep_boundary(expert_rows: Sequence[Optional[np.ndarray]], *, topk_w, topk_rows,
                residual=None, gamma1=None, gamma2=None, eps: float = 1e-6,
                epilogue: int = EPI_RMSNORM, split: bool = False,
                shared: Optional[Sequence[Optional[np.ndarray]]] = None,
                num_rows: Optional[Sequence[int]] = None, H: Optional[int] = None,
                debug: bool = False, nthreads: int = 1) -> Result:
    """Run the oracle with the expert-parallel finalize.

    expert_rows: R arrays of BF16 bits [num_rows_r, H] (None for a rank with
    no rows); topk_w: [T,k] float32, the same for every rank; topk_rows: R
    int32 arrays [T,k], row of that rank's buffer or negative for another
    rank's slot; shared: None, or R entries each [T,H] BF16 bits or None.
    """
    lib = _active()
    R = len(expert_rows)
    w = _c(topk_w, np.float32)
    T, k = w.shape
    rows = [None if e is None else _c(e, np.uint16) for e in expert_rows]
    if H is None:
        H = next(e.shape[1] for e in rows if e is not None)
    nr = [0 if e is None else e.shape[0] for e in rows] if num_rows is None else list(num_rows)
    nr_arr = np.asarray(nr, np.int64)
    idx = [_c(i, np.int32) for i in topk_rows]
    if len(idx) != R or any(i.shape != (T, k) for i in idx):
        raise ValueError("topk_rows must hold R arrays of shape [T,k]")
    src_arr = (ctypes.c_void_p * R)(*[None if e is None else e.ctypes.data for e in rows])
    idx_arr = (ctypes.c_void_p * R)(*[i.ctypes.data for i in idx])
    sh = None if shared is None else [None if a is None else _c(a, np.uint16) for a in shared]
    sh_arr = (ctypes.c_void_p * R)(*[None if a is None else a.ctypes.data for a in sh]) \
        if sh is not None else None
    x = _c(residual, np.uint16) if residual is not None else None
    g1 = _c(gamma1, np.float32) if gamma1 is not None else None
    g2 = _c(gamma2, np.float32) if gamma2 is not None else None
    res, y, xout, u, dbg = _outputs(T, H, R, epilogue, split, True, debug)
    rc = lib.oracle_ep_boundary(
        ctypes.cast(src_arr, ctypes.c_void_p),
        ctypes.cast(sh_arr, ctypes.c_void_p) if sh_arr is not None else None,
        R, _ptr(w), ctypes.cast(idx_arr, ctypes.c_void_p), k, _ptr(nr_arr), epilogue,
        int(bool(split)), _ptr(x), _ptr(g1), _ptr(g2), ctypes.c_float(eps), T, H,
        _ptr(y), _ptr(xout), _ptr(u), _dbg_ptr(dbg), nthreads)
    return _finish(res, rc, "oracle_ep_boundary", debug, split, epilogue)
