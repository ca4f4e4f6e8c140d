"""Python binding of the fused reduce + norm boundary for MI355X (gfx950).

A thin ctypes layer over ``libfused_reduce_norm.so`` (the C ABI declared in
``include/fused_reduce_norm.h``).  It only checks tensor dtypes, devices and
layouts, passes raw device pointers and the current HIP stream, and turns
status codes into exceptions.  Every step of the computation runs in the
library's HIP kernels; there is no CPU or PyTorch fallback.  If the library
is missing the import fails.

Function names are the C entry points without their ``frn_`` prefix:

* ``reduce_residual_rmsnorm``    FP32 sum of R BF16 partials + residual + RMSNorm
* ``reduce_sandwich_norm``       FP32 sum + norm(gamma1) + residual + norm(gamma2)
* ``moe_finalize_reduce_norm``   top-k finalize (+ shared expert) per rank,
                                 rounded to BF16, then either epilogue
* ``moe_finalize_reduce_norm_noalloc``  the same for callers that cannot
                                 allocate: no workspace argument, scratch
                                 from the library's own device array
* ``reduce_bf16``, ``moe_finalize_reduce_bf16``  split path, pass 1
* ``split_reduce_norm``          both passes of the split path
* ``moe_finalize``               the per-rank finalize alone (materialized)
* ``ep_moe_finalize_reduce_norm``, ``ep_moe_finalize``  the same with
                                 expert-parallel routing (each rank owns
                                 some experts; per-rank row indices)
* ``query``, ``workspace_bytes``, ``version``
* ``set_launch_table``, ``launch_shape``, ``split_rows``,
  ``launch_pipelined``           tuned launch shapes, the split-row finalize
                                 choice and the row-pipelined kernel choice
                                 (tune.py)
* ``boundary``                   fused or split by a token threshold, and
                                 the materialized finalize when a fused
                                 finalize call declines (Python-side
                                 policies over the calls above)

Every call returns its outputs.  A declined call raises
``FusedReduceNormUnsupported``; it never returns unreduced data.  (The pages
record a bug where a declined fused call silently skipped the owed
reduction: SGLang PR #34134, second commit message.)
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Sequence, Tuple, Union

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfused_reduce_norm.so")

SHAPE_EP = 16  # FRN_SHAPE_EP

FRN_OK = 0
FRN_ERR_INVALID = 1
FRN_ERR_UNSUPPORTED = 2
FRN_ERR_HIP = 3
EPI_RMSNORM = 0
EPI_SANDWICH = 1
MAX_R = 16
MAX_K = 16
MAX_H = 16384
NOALLOC_SCRATCH_BYTES = 17 << 20  # FRN_NOALLOC_SCRATCH_BYTES


class FusedReduceNormError(RuntimeError):
    """The library returned FRN_ERR_HIP."""


class FusedReduceNormUnsupported(RuntimeError):
    """The call is outside what the library serves (FRN_ERR_UNSUPPORTED).
    The caller must take another path that still performs the reduction."""


if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python tp_reduction_rmsnorm_amd/build.py` "
        "(or __graft_entry__.build()); there is no fallback path")

_lib = ctypes.CDLL(LIB_PATH)
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F32 = ctypes.c_float
_SZ = ctypes.c_size_t


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_c_rms = _sig("frn_reduce_residual_rmsnorm", ctypes.c_int,
              [_P, _I32, _P, _P, _F32, _I64, _I64, _P, _P, _P, _SZ, _P])
_c_sandwich = _sig("frn_reduce_sandwich_norm", ctypes.c_int,
                   [_P, _I32, _P, _P, _P, _F32, _I64, _I64, _P, _P, _P, _SZ, _P])
_c_moe = _sig("frn_moe_finalize_reduce_norm", ctypes.c_int,
              [_P, _P, _I32, _P, _P, _I32, _I64, _I32, _P, _P, _P, _F32, _I64, _I64,
               _P, _P, _P, _SZ, _P])
_c_moe_noalloc = _sig("frn_moe_finalize_reduce_norm_noalloc", ctypes.c_int,
                      [_P, _P, _I32, _P, _P, _I32, _I64, _I32, _P, _P, _P, _F32, _I64, _I64,
                       _P, _P, _P])
_c_reduce_bf16 = _sig("frn_reduce_bf16", ctypes.c_int, [_P, _I32, _I64, _I64, _P, _P])
_c_moe_bf16 = _sig("frn_moe_finalize_reduce_bf16", ctypes.c_int,
                   [_P, _P, _I32, _P, _P, _I32, _I64, _I64, _I64, _P, _P])
_c_split = _sig("frn_split_reduce_norm", ctypes.c_int,
                [_P, _P, _I32, _P, _P, _I32, _I64, _I32, _P, _P, _P, _F32, _I64, _I64,
                 _P, _P, _P, _P])
_c_finalize = _sig("frn_moe_finalize", ctypes.c_int,
                   [_P, _P, _I32, _P, _P, _I32, _I64, _I64, _I64, _P, _P])
_c_ep_moe = _sig("frn_ep_moe_finalize_reduce_norm", ctypes.c_int,
                 [_P, _P, _I32, _P, _P, _I32, _P, _I32, _P, _P, _P, _F32, _I64, _I64,
                  _P, _P, _P, _SZ, _P])
_c_ep_finalize = _sig("frn_ep_moe_finalize", ctypes.c_int,
                      [_P, _P, _I32, _P, _P, _I32, _P, _I64, _I64, _P, _P])
_c_query = _sig("frn_query", ctypes.c_int, [_I32, _I32, _I64, _I64, _I32])
_c_set_table = _sig("frn_set_launch_table", ctypes.c_int, [ctypes.c_char_p])
_c_shape = _sig("frn_launch_shape", ctypes.c_int,
                [_I32, _I32, _I64, _I64, _I32, ctypes.POINTER(_I32), ctypes.POINTER(_I32)])
_c_ws = _sig("frn_workspace_bytes", _SZ, [_I64, _I64, _I32, _I32])
_c_split_rows = _sig("frn_split_rows", _I32, [_I32, _I32, _I64, _I64, _I32])
_c_pipelined = _sig("frn_launch_pipelined", _I32, [_I32, _I32, _I64, _I64, _I32])
_c_status = _sig("frn_status_string", ctypes.c_char_p, [ctypes.c_int])
_c_last = _sig("frn_last_error", ctypes.c_char_p, [])
_c_version = _sig("frn_version", ctypes.c_char_p, [])

C_FUNCTIONS = ("frn_reduce_residual_rmsnorm", "frn_reduce_sandwich_norm",
               "frn_moe_finalize_reduce_norm", "frn_moe_finalize_reduce_norm_noalloc",
               "frn_reduce_bf16",
               "frn_moe_finalize_reduce_bf16", "frn_split_reduce_norm", "frn_moe_finalize",
               "frn_ep_moe_finalize_reduce_norm", "frn_ep_moe_finalize",
               "frn_query", "frn_set_launch_table", "frn_launch_shape",
               "frn_workspace_bytes", "frn_split_rows", "frn_launch_pipelined",
               "frn_status_string", "frn_last_error", "frn_version")


def version() -> str:
    return _c_version().decode()


def _check(status: int) -> None:
    if status == FRN_OK:
        return
    text = _c_last().decode() or _c_status(status).decode()
    if status == FRN_ERR_UNSUPPORTED:
        raise FusedReduceNormUnsupported(text)
    if status == FRN_ERR_INVALID:
        raise ValueError(text)
    raise FusedReduceNormError(text)


def query(R: int, k: int, T: int, H: int, epilogue: int = EPI_RMSNORM) -> bool:
    """True if a call with these sizes is served (no launch)."""
    st = _c_query(R, k, T, H, epilogue)
    if st == FRN_ERR_INVALID:
        _check(st)
    return st == FRN_OK


def workspace_bytes(max_T: int, H: int, R: int, k: int = 0) -> int:
    """Bytes of the optional workspace of the finalize calls for up to max_T
    tokens: the split-row finalize's T x H FP32 rows and T x ceil(H / 512)
    FP64 sums of squares, for the largest T it is taken at (0: never)."""
    return int(_c_ws(max_T, H, R, k))


EPI_SUM = 2  # split pass 1, for launch tables and launch_shape


def set_launch_table(text: Optional[str]) -> None:
    """Load tuned launch rules ('H R k epilogue Tmin Tmax vec' per line, vec
    1 | 2 | 4 | split | fused), or None to restore the built-in rules.
    Raises ValueError on bad text."""
    _WS_NEED.clear()
    _check(_c_set_table(None if text is None else text.encode()))


def launch_shape(R: int, k: int, T: int, H: int, epilogue: int = EPI_RMSNORM, *,
                 ep: bool = False):
    """(lanes per workgroup, vectors per lane) the call would use -- of the
    row-pipelined kernel where it takes that (``launch_pipelined``), else of
    the one-row kernel; ``ep=True`` for an ``ep_moe_finalize_reduce_norm``
    call."""
    th, v = _I32(), _I32()
    _check(_c_shape(R, k, T, H, epilogue | (SHAPE_EP if ep else 0), ctypes.byref(th),
                    ctypes.byref(v)))
    return th.value, v.value


def split_rows(R: int, k: int, T: int, H: int, epilogue: int = EPI_RMSNORM, *,
               ep: bool = False) -> bool:
    """True if a finalize call of these sizes that is given a large enough
    workspace takes the split-row finalize (no launch)."""
    return bool(_c_split_rows(R, k, T, H, epilogue | (SHAPE_EP if ep else 0)))


def launch_pipelined(R: int, k: int, T: int, H: int, epilogue: int = EPI_RMSNORM) -> bool:
    """True if a call of these sizes (no finalize) runs the row-pipelined
    kernel -- one workgroup per compute unit walking the rows, the next
    row's loads in flight during the current row's epilogue -- rather than
    one workgroup per row (no launch)."""
    return bool(_c_pipelined(R, k, T, H, epilogue))


# ---------------------------------------------------------------- helpers --- #

TensorList = Union[torch.Tensor, Sequence[torch.Tensor]]


def _as_list(x: TensorList, what: str):
    if isinstance(x, torch.Tensor):
        if x.dim() != 3:
            raise ValueError(f"{what}: a stacked tensor must be [R, rows, H]")
        return list(x.unbind(0))
    return list(x)


def _need(t: torch.Tensor, what: str, dtype, dim: int, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype} (got {t.dtype})")
    if t.dim() != dim:
        raise ValueError(f"{what} must have {dim} dims (got {tuple(t.shape)})")
    if not t.is_cuda:
        raise ValueError(f"{what} must be on the GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{what} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")


def _ptr_array(ts):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def _ptr_array_opt(ts):
    """Like _ptr_array; None entries and empty tensors pass NULL."""
    return (ctypes.c_void_p * len(ts))(
        *[None if t is None or t.numel() == 0 else t.data_ptr() for t in ts])


def _stream(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ------------------------------------------------- the eager call's fast path --- #
# An eager call of a few tokens takes a few microseconds on the GPU, so the
# binding's own host time matters there.  The hot entry points first run one
# cheap test per tensor (the same conditions as _need, read without building
# device or shape objects); only if a test fails do they take the detailed
# checks, which raise with the reason.  Pointer arrays go into a per-thread
# C array that the library copies during the call, and the current stream's
# handle is read directly.

_BF16, _FP32, _INT32 = torch.bfloat16, torch.float32, torch.int32

try:
    _raw_current_stream = torch._C._cuda_getCurrentRawStream
except AttributeError:  # a torch without it: the public (slower) route
    def _raw_current_stream(index):
        return torch.cuda.current_stream(index).cuda_stream


def _stream_handle(stream, index: int) -> int:
    if stream is None:
        return _raw_current_stream(index)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _fits(t, dtype, index: int, shape) -> bool:
    """What _need checks, plus the shape, for a tensor expected on device
    `index`."""
    return (isinstance(t, torch.Tensor) and t.dtype is dtype and t.is_cuda and
            t.get_device() == index and t.shape == shape and t.is_contiguous())


_TLS = threading.local()


def _host_ptrs(ptrs, slot: int) -> int:
    """Address of a C array holding the device pointers `ptrs`: one of the
    calling thread's own arrays (slot 0, 1, 2), valid until the thread's
    next call; the library copies the pointers during the call."""
    arrs = getattr(_TLS, "arrs", None)
    if arrs is None:
        arrs = _TLS.arrs = [(ctypes.c_void_p * MAX_R)() for _ in range(3)]
    if len(ptrs) > MAX_R:  # declined by the library; pass them all the same
        a = (ctypes.c_void_p * len(ptrs))(*ptrs)
        _TLS.big = a
    else:
        a = arrs[slot]
        a[:len(ptrs)] = ptrs
    return ctypes.addressof(a)


def _fast_outputs(out, residual_out, shape, index, device_of):
    """(out, residual_out) when given ones fit or none are given (allocated
    like the first partial), else None."""
    if out is None:
        out = torch.empty(shape, dtype=_BF16, device=device_of.device)
    elif not _fits(out, _BF16, index, shape):
        return None
    if residual_out is None:
        residual_out = torch.empty(shape, dtype=_BF16, device=device_of.device)
    elif not _fits(residual_out, _BF16, index, shape):
        return None
    return out, residual_out


def _fast_reduce(ps, residual, gammas, out, residual_out):
    """(index, T, H, out, residual_out) if the operands of a reduction pass
    the cheap tests, else None."""
    if not ps or not isinstance(ps[0], torch.Tensor):
        return None
    p0 = ps[0]
    index = p0.get_device()
    shape = p0.shape
    if index < 0 or len(shape) != 2:
        return None
    for p in ps:
        if not _fits(p, _BF16, index, shape):
            return None
    if not _fits(residual, _BF16, index, shape):
        return None
    gshape = shape[1:]
    for g in gammas:
        if not _fits(g, _FP32, index, gshape):
            return None
    outs = _fast_outputs(out, residual_out, shape, index, p0)
    if outs is None:
        return None
    return (index, shape[0], shape[1]) + outs


def _fast_moe(es, topk_weights, topk_rows, residual, gamma1, gamma2, epilogue, shared, out,
              residual_out):
    """(index, T, H, k, num_rows, out, residual_out) if the operands of a
    finalize call pass the cheap tests, else None."""
    if not es or not isinstance(es[0], torch.Tensor) or not isinstance(residual, torch.Tensor):
        return None
    e0 = es[0]
    index = e0.get_device()
    eshape = e0.shape
    shape = residual.shape
    if index < 0 or len(eshape) != 2 or len(shape) != 2 or eshape[1] != shape[1]:
        return None
    for e in es:
        if not _fits(e, _BF16, index, eshape):
            return None
    if not _fits(residual, _BF16, index, shape):
        return None
    if not isinstance(topk_weights, torch.Tensor) or topk_weights.dim() != 2:
        return None
    kshape = topk_weights.shape
    if kshape[0] != shape[0] or not _fits(topk_weights, _FP32, index, kshape) or \
            not _fits(topk_rows, _INT32, index, kshape):
        return None
    gshape = shape[1:]
    if not _fits(gamma1, _FP32, index, gshape):
        return None
    if epilogue == EPI_SANDWICH and not _fits(gamma2, _FP32, index, gshape):
        return None
    if shared is not None:
        if len(shared) != len(es):
            return None
        for t in shared:
            if not _fits(t, _BF16, index, shape):
                return None
    outs = _fast_outputs(out, residual_out, shape, index, e0)
    if outs is None:
        return None
    return (index, shape[0], shape[1], kshape[1], eshape[0]) + outs


def _listed(x):
    return x if type(x) in (list, tuple) else _as_list(x, "tensors")


def _outputs(T, H, device, out, residual_out):
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=device)
    else:
        _need(out, "out", torch.bfloat16, 2, device)
    if residual_out is None:
        residual_out = torch.empty((T, H), dtype=torch.bfloat16, device=device)
    else:
        _need(residual_out, "residual_out", torch.bfloat16, 2, device)
    if tuple(out.shape) != (T, H) or tuple(residual_out.shape) != (T, H):
        raise ValueError("out and residual_out must be [T, H]")
    return out, residual_out


# Automatic workspaces per (device, stream): every buffer ever handed out is
# kept until the process ends, because a HIP graph captured with one keeps
# its address; a larger need allocates a new buffer (at least twice the last
# one, so there are few) instead of freeing the old.
_AUTO_WS = {}

# Automatic workspace bytes per call shape (0: the call takes no split-row
# finalize); cleared whenever set_launch_table loads a table.
_WS_NEED = {}


def _workspace(workspace, T=0, H=0, R=0, k=0, device=None, stream=None,
               epilogue=EPI_RMSNORM, ep=False):
    """(pointer, bytes) of the workspace argument.  ``"auto"``: a buffer
    kept per (device, stream) of the call and grown on demand (it holds
    nothing between calls), passed only to a call that takes the split-row
    finalize.  Calls on one stream run in order, so they can share it; graphs
    captured on one stream share it too and must not be replayed
    concurrently (give those explicit workspaces).  ``None``: none."""
    if workspace is None:
        return None, 0
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be a tensor, None or 'auto'")
        key = (R, k, T, H, epilogue, ep)
        need = _WS_NEED.get(key)
        if need is None:
            use = k > 0 and split_rows(R, k, T, H, epilogue, ep=ep)
            need = _WS_NEED[key] = workspace_bytes(T, H, R, k) if use else 0
        if need == 0:
            return None, 0
        index = device if isinstance(device, int) else device.index
        kept = _AUTO_WS.setdefault((index, stream), [])
        if not kept or kept[-1].numel() < need:
            size = max(need, 2 * kept[-1].numel()) if kept else need
            kept.append(torch.empty(size, dtype=torch.uint8, device=device))
        ws = kept[-1]
        return ws.data_ptr(), ws.numel()
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def _check_partials(partials: TensorList, residual: Optional[torch.Tensor]):
    ps = _as_list(partials, "partials")
    if not ps:
        raise ValueError("need at least one partial")
    device = ps[0].device
    for i, p in enumerate(ps):
        _need(p, f"partials[{i}]", torch.bfloat16, 2, device)
        if p.shape != ps[0].shape:
            raise ValueError("all partials must have the same [T, H] shape")
    T, H = ps[0].shape
    if residual is not None:
        _need(residual, "residual", torch.bfloat16, 2, device)
        if tuple(residual.shape) != (T, H):
            raise ValueError("residual must be [T, H] like the partials")
    return ps, T, H, device


def _check_gamma(g, H, device, what):
    _need(g, what, torch.float32, 1, device)
    if g.shape[0] != H:
        raise ValueError(f"{what} must have H={H} entries")


def _check_finalize(expert_rows, topk_weights, topk_rows, shared):
    es = _as_list(expert_rows, "expert_rows")
    if not es:
        raise ValueError("need at least one expert-row buffer")
    device = es[0].device
    for i, e in enumerate(es):
        _need(e, f"expert_rows[{i}]", torch.bfloat16, 2, device)
        if e.shape != es[0].shape:
            raise ValueError("all expert-row buffers must have the same shape")
    num_rows, H = es[0].shape
    _need(topk_weights, "topk_weights", torch.float32, 2, device)
    _need(topk_rows, "topk_rows", torch.int32, 2, device)
    T, k = topk_weights.shape
    if tuple(topk_rows.shape) != (T, k):
        raise ValueError("topk_rows must have the shape of topk_weights [T, k]")
    sh = None
    if shared is not None:
        sh = _as_list(shared, "shared")
        if len(sh) != len(es):
            raise ValueError("shared must give one [T, H] tensor per rank")
        for i, s in enumerate(sh):
            _need(s, f"shared[{i}]", torch.bfloat16, 2, device)
            if tuple(s.shape) != (T, H):
                raise ValueError("shared tensors must be [T, H]")
    return es, sh, T, H, k, num_rows, device


# ------------------------------------------------------------- entry points --- #

def reduce_residual_rmsnorm(partials: TensorList, residual: torch.Tensor, gamma: torch.Tensor,
                            eps: float = 1e-6, *, out=None, residual_out=None,
                            workspace=None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """h = sum(partials) + residual (FP32); returns (bf16(norm(h) * gamma), bf16(h)).
    Pass ``residual_out=residual`` to update the residual stream in place."""
    if residual is None:
        raise ValueError("residual is required: this boundary always adds the residual")
    ps = _listed(partials)
    fast = _fast_reduce(ps, residual, (gamma,), out, residual_out)
    if fast is None:  # the detailed checks: they raise, or allocate what is missing
        ps, T, H, device = _check_partials(partials, residual)
        _check_gamma(gamma, H, device, "gamma")
        out, residual_out = _outputs(T, H, device, out, residual_out)
        index = device.index
    else:
        index, T, H, out, residual_out = fast
    ws, wsb = _workspace(workspace)
    _check(_c_rms(_host_ptrs([p.data_ptr() for p in ps], 0), len(ps), residual.data_ptr(),
                  gamma.data_ptr(), eps, T, H, out.data_ptr(), residual_out.data_ptr(), ws, wsb,
                  _stream_handle(stream, index)))
    return out, residual_out


def reduce_sandwich_norm(partials: TensorList, residual: torch.Tensor, gamma1: torch.Tensor,
                         gamma2: torch.Tensor, eps: float = 1e-6, *, out=None,
                         residual_out=None, workspace=None,
                         stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """a = norm(sum(partials)) * gamma1; h = a + residual (FP32);
    returns (bf16(norm(h) * gamma2), bf16(h))."""
    if residual is None:
        raise ValueError("residual is required: this boundary always adds the residual")
    ps = _listed(partials)
    fast = _fast_reduce(ps, residual, (gamma1, gamma2), out, residual_out)
    if fast is None:  # the detailed checks: they raise, or allocate what is missing
        ps, T, H, device = _check_partials(partials, residual)
        _check_gamma(gamma1, H, device, "gamma1")
        _check_gamma(gamma2, H, device, "gamma2")
        out, residual_out = _outputs(T, H, device, out, residual_out)
        index = device.index
    else:
        index, T, H, out, residual_out = fast
    ws, wsb = _workspace(workspace)
    _check(_c_sandwich(_host_ptrs([p.data_ptr() for p in ps], 0), len(ps), residual.data_ptr(),
                       gamma1.data_ptr(), gamma2.data_ptr(), eps, T, H, out.data_ptr(),
                       residual_out.data_ptr(), ws, wsb, _stream_handle(stream, index)))
    return out, residual_out


def _check_moe_epilogue(residual, gamma1, gamma2, epilogue, T, H, device):
    if residual is None:
        raise ValueError("residual is required: this boundary always adds the residual")
    _need(residual, "residual", torch.bfloat16, 2, device)
    if tuple(residual.shape) != (T, H):
        raise ValueError("residual must be [T, H]")
    _check_gamma(gamma1, H, device, "gamma1")
    if epilogue == EPI_SANDWICH:
        if gamma2 is None:
            raise ValueError("the sandwich epilogue needs gamma2")
        _check_gamma(gamma2, H, device, "gamma2")


def moe_finalize_reduce_norm(expert_rows: TensorList, topk_weights: torch.Tensor,
                             topk_rows: torch.Tensor, residual: torch.Tensor,
                             gamma1: torch.Tensor, gamma2: Optional[torch.Tensor] = None,
                             eps: float = 1e-6, *, shared: Optional[TensorList] = None,
                             epilogue: int = EPI_RMSNORM, out=None, residual_out=None,
                             workspace="auto", stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per rank r: P_r = bf16(sum_j w[t,j] * E_r[rows[t,j]] (+ shared_r[t])); then
    the epilogue on sum_r P_r.  Returns (out, residual_out).  ``workspace``:
    "auto" (a buffer kept per device and stream, passed where ``split_rows``
    holds: small T), None (never), or a uint8 GPU tensor of at least
    ``workspace_bytes(T, H, R, k)`` bytes, 256-byte aligned."""
    if residual is None:
        raise ValueError("residual is required: this boundary always adds the residual")
    es = _listed(expert_rows)
    sh = _listed(shared) if shared is not None else None
    fast = _fast_moe(es, topk_weights, topk_rows, residual, gamma1, gamma2, epilogue, sh, out,
                     residual_out)
    if fast is None:  # the detailed checks: they raise, or allocate what is missing
        es, sh, T, H, k, num_rows, device = _check_finalize(expert_rows, topk_weights,
                                                            topk_rows, shared)
        _check_moe_epilogue(residual, gamma1, gamma2, epilogue, T, H, device)
        out, residual_out = _outputs(T, H, device, out, residual_out)
        index = device.index
    else:
        index, T, H, k, num_rows, out, residual_out = fast
    st = _stream_handle(stream, index)
    ws, wsb = _workspace(workspace, T, H, len(es), k, index, st, epilogue)
    _check(_c_moe(_host_ptrs([e.data_ptr() for e in es], 0),
                  _host_ptrs([t.data_ptr() for t in sh], 1) if sh is not None else None,
                  len(es), topk_weights.data_ptr(), topk_rows.data_ptr(), k, num_rows, epilogue,
                  residual.data_ptr(), gamma1.data_ptr(),
                  gamma2.data_ptr() if gamma2 is not None else None, eps, T, H,
                  out.data_ptr(), residual_out.data_ptr(), ws, wsb, st))
    return out, residual_out


def moe_finalize_reduce_norm_noalloc(expert_rows: TensorList, topk_weights: torch.Tensor,
                                     topk_rows: torch.Tensor, residual: torch.Tensor,
                                     gamma1: torch.Tensor,
                                     gamma2: Optional[torch.Tensor] = None, eps: float = 1e-6,
                                     *, out: torch.Tensor, residual_out: torch.Tensor,
                                     shared: Optional[TensorList] = None,
                                     epilogue: int = EPI_RMSNORM,
                                     stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """``moe_finalize_reduce_norm`` for callers that cannot allocate: the
    outputs are the caller's (``out`` and ``residual_out`` are required) and
    the split-row finalize's FP32 rank sums go to the library's own scratch
    array on the GPU (``NOALLOC_SCRATCH_BYTES``, enough for the largest
    split-row call), so neither this function nor the C call allocates.
    Calls that may overlap in time on one GPU share that array and race:
    serialise them."""
    if out is None or residual_out is None:
        raise ValueError("out and residual_out are required: this call allocates nothing")
    es = _listed(expert_rows)
    sh = _listed(shared) if shared is not None else None
    fast = _fast_moe(es, topk_weights, topk_rows, residual, gamma1, gamma2, epilogue, sh, out,
                     residual_out)
    if fast is None:  # the detailed checks: they raise
        es, sh, T, H, k, num_rows, device = _check_finalize(expert_rows, topk_weights,
                                                            topk_rows, shared)
        _check_moe_epilogue(residual, gamma1, gamma2, epilogue, T, H, device)
        out, residual_out = _outputs(T, H, device, out, residual_out)
        index = device.index
    else:
        index, T, H, k, num_rows, out, residual_out = fast
    _check(_c_moe_noalloc(_host_ptrs([e.data_ptr() for e in es], 0),
                          _host_ptrs([t.data_ptr() for t in sh], 1) if sh is not None else None,
                          len(es), topk_weights.data_ptr(), topk_rows.data_ptr(), k, num_rows,
                          epilogue, residual.data_ptr(), gamma1.data_ptr(),
                          gamma2.data_ptr() if gamma2 is not None else None, eps, T, H,
                          out.data_ptr(), residual_out.data_ptr(),
                          _stream_handle(stream, index)))
    return out, residual_out


def reduce_bf16(partials: TensorList, *, out=None, stream=None) -> torch.Tensor:
    """Split path, pass 1: bf16(sum_r partials[r]) (FP32 sum)."""
    ps, T, H, device = _check_partials(partials, None)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=device)
    else:
        _need(out, "out", torch.bfloat16, 2, device)
    arr = _ptr_array(ps)
    _check(_c_reduce_bf16(ctypes.cast(arr, _P), len(ps), T, H, out.data_ptr(),
                          _stream(stream, device)))
    return out


def moe_finalize_reduce_bf16(expert_rows: TensorList, topk_weights: torch.Tensor,
                             topk_rows: torch.Tensor, *, shared: Optional[TensorList] = None,
                             out=None, stream=None) -> torch.Tensor:
    """Split path, pass 1 with the finalize: bf16(sum_r P_r)."""
    es, sh, T, H, k, num_rows, device = _check_finalize(expert_rows, topk_weights, topk_rows,
                                                        shared)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=device)
    else:
        _need(out, "out", torch.bfloat16, 2, device)
    earr = _ptr_array(es)
    sarr = _ptr_array(sh) if sh is not None else None
    _check(_c_moe_bf16(ctypes.cast(earr, _P), ctypes.cast(sarr, _P) if sarr is not None else None,
                       len(es), topk_weights.data_ptr(), topk_rows.data_ptr(), k, num_rows, T, H,
                       out.data_ptr(), _stream(stream, device)))
    return out


def moe_finalize(expert_rows: TensorList, topk_weights: torch.Tensor, topk_rows: torch.Tensor,
                 *, shared: Optional[TensorList] = None, out=None, stream=None):
    """The per-rank finalize alone: returns R BF16 tensors [T, H],
    P_r = bf16(sum_j w[t,j] * E_r[rows[t,j]] (+ shared_r[t])).  Reducing them
    with ``reduce_residual_rmsnorm`` / ``reduce_sandwich_norm`` reproduces the
    fused ``moe_finalize_reduce_norm`` bit for bit."""
    es, sh, T, H, k, num_rows, device = _check_finalize(expert_rows, topk_weights, topk_rows,
                                                        shared)
    R = len(es)
    if out is None:
        out = [torch.empty((T, H), dtype=torch.bfloat16, device=device) for _ in range(R)]
    else:
        out = _as_list(out, "out")
        if len(out) != R:
            raise ValueError("out must give one [T, H] tensor per rank")
        for i, o in enumerate(out):
            _need(o, f"out[{i}]", torch.bfloat16, 2, device)
            if tuple(o.shape) != (T, H):
                raise ValueError("out tensors must be [T, H]")
    earr = _ptr_array(es)
    sarr = _ptr_array(sh) if sh is not None else None
    oarr = _ptr_array(out)
    _check(_c_finalize(ctypes.cast(earr, _P), ctypes.cast(sarr, _P) if sarr is not None else None,
                       R, topk_weights.data_ptr(), topk_rows.data_ptr(), k, num_rows, T, H,
                       ctypes.cast(oarr, _P), _stream(stream, device)))
    return out


def _check_ep(expert_rows, topk_weights, topk_rows, shared, H=None):
    """Expert-parallel operands: R expert buffers [num_rows_r, H] (None or
    0 rows for a rank without rows), weights [T,k] shared by every rank, R
    int32 index arrays [T,k], and shared: None or R entries each None or
    [T,H]."""
    es = list(expert_rows)
    if not es:
        raise ValueError("need at least one expert-row buffer")
    _need(topk_weights, "topk_weights", torch.float32, 2, topk_weights.device)
    device = topk_weights.device
    T, k = topk_weights.shape
    for i, e in enumerate(es):
        if e is not None:
            _need(e, f"expert_rows[{i}]", torch.bfloat16, 2, device)
            if H is None:
                H = e.shape[1]
            elif e.shape[1] != H:
                raise ValueError("all expert-row buffers must have H columns")
    rows = list(topk_rows) if not isinstance(topk_rows, torch.Tensor) else None
    if rows is None or len(rows) != len(es):
        raise ValueError("topk_rows must give one [T, k] int32 tensor per rank")
    for i, r in enumerate(rows):
        _need(r, f"topk_rows[{i}]", torch.int32, 2, device)
        if tuple(r.shape) != (T, k):
            raise ValueError("every topk_rows tensor must have the shape of topk_weights")
    sh = None
    if shared is not None:
        sh = list(shared)
        if len(sh) != len(es):
            raise ValueError("shared must give one entry (a [T, H] tensor or None) per rank")
        for i, s in enumerate(sh):
            if s is None:
                continue
            _need(s, f"shared[{i}]", torch.bfloat16, 2, device)
            if H is None:
                H = s.shape[1]
            if tuple(s.shape) != (T, H):
                raise ValueError("shared tensors must be [T, H]")
    if H is None:
        raise ValueError("H is unknown: no expert buffer or shared tensor gives it")
    num_rows = [0 if e is None else int(e.shape[0]) for e in es]
    return es, sh, rows, T, H, k, num_rows, device


def ep_moe_finalize_reduce_norm(expert_rows: Sequence[Optional[torch.Tensor]],
                                topk_weights: torch.Tensor, topk_rows: TensorList,
                                residual: torch.Tensor, gamma1: torch.Tensor,
                                gamma2: Optional[torch.Tensor] = None, eps: float = 1e-6, *,
                                shared: Optional[Sequence[Optional[torch.Tensor]]] = None,
                                epilogue: int = EPI_RMSNORM, out=None, residual_out=None,
                                workspace="auto", stream=None):
    """Expert-parallel finalize, then the epilogue: per rank r,
    P_r = bf16(sum over j with topk_rows[r][t,j] >= 0 of w[t,j] * E_r[row]
    (+ shared[r][t] if given)); a negative index marks another rank's slot.
    Returns (out, residual_out).  ``workspace`` as in
    ``moe_finalize_reduce_norm``."""
    if residual is None:
        raise ValueError("residual is required: this boundary always adds the residual")
    es, sh, rows, T, H, k, num_rows, device = _check_ep(
        expert_rows, topk_weights, topk_rows, shared,
        H=residual.shape[1] if residual.dim() == 2 else None)
    _need(residual, "residual", torch.bfloat16, 2, device)
    if tuple(residual.shape) != (T, H):
        raise ValueError("residual must be [T, H]")
    _check_gamma(gamma1, H, device, "gamma1")
    if epilogue == EPI_SANDWICH:
        if gamma2 is None:
            raise ValueError("the sandwich epilogue needs gamma2")
        _check_gamma(gamma2, H, device, "gamma2")
    out, residual_out = _outputs(T, H, device, out, residual_out)
    st = _stream(stream, device)
    R = len(es)
    ws, wsb = _workspace(workspace, T, H, R, k, device, st, epilogue, ep=True)
    earr = _ptr_array_opt(es)
    sarr = _ptr_array_opt(sh) if sh is not None else None
    rarr = _ptr_array(rows)
    nrows = (ctypes.c_int64 * R)(*num_rows)
    _check(_c_ep_moe(ctypes.cast(earr, _P), ctypes.cast(sarr, _P) if sarr is not None else None,
                     R, topk_weights.data_ptr(), ctypes.cast(rarr, _P), k,
                     ctypes.cast(nrows, _P), epilogue, residual.data_ptr(), gamma1.data_ptr(),
                     gamma2.data_ptr() if gamma2 is not None else None, eps, T, H,
                     out.data_ptr(), residual_out.data_ptr(), ws, wsb, st))
    return out, residual_out


def ep_moe_finalize(expert_rows: Sequence[Optional[torch.Tensor]], topk_weights: torch.Tensor,
                    topk_rows: TensorList, *, H: Optional[int] = None,
                    shared: Optional[Sequence[Optional[torch.Tensor]]] = None, out=None,
                    stream=None):
    """The expert-parallel finalize alone: returns R BF16 tensors [T, H]
    (P_r as in ``ep_moe_finalize_reduce_norm``)."""
    es, sh, rows, T, H, k, num_rows, device = _check_ep(expert_rows, topk_weights, topk_rows,
                                                        shared, H=H)
    R = len(es)
    if out is None:
        out = [torch.empty((T, H), dtype=torch.bfloat16, device=device) for _ in range(R)]
    else:
        out = _as_list(out, "out")
        if len(out) != R:
            raise ValueError("out must give one [T, H] tensor per rank")
        for i, o in enumerate(out):
            _need(o, f"out[{i}]", torch.bfloat16, 2, device)
            if tuple(o.shape) != (T, H):
                raise ValueError("out tensors must be [T, H]")
    earr = _ptr_array_opt(es)
    sarr = _ptr_array_opt(sh) if sh is not None else None
    rarr = _ptr_array(rows)
    nrows = (ctypes.c_int64 * R)(*num_rows)
    oarr = _ptr_array(out)
    _check(_c_ep_finalize(ctypes.cast(earr, _P),
                          ctypes.cast(sarr, _P) if sarr is not None else None, R,
                          topk_weights.data_ptr(), ctypes.cast(rarr, _P), k,
                          ctypes.cast(nrows, _P), T, H, ctypes.cast(oarr, _P),
                          _stream(stream, device)))
    return out


def split_reduce_norm(src: TensorList, residual: torch.Tensor, gamma1: torch.Tensor,
                      gamma2: Optional[torch.Tensor] = None, eps: float = 1e-6, *,
                      topk_weights=None, topk_rows=None, shared=None,
                      epilogue: int = EPI_RMSNORM, scratch=None, out=None, residual_out=None,
                      stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Both passes of the split path.  Without topk_weights, src are the
    partials; with them, src are the expert-row buffers."""
    if residual is None:
        raise ValueError("residual is required: this boundary always adds the residual")
    if topk_weights is not None:
        es, sh, T, H, k, num_rows, device = _check_finalize(src, topk_weights, topk_rows, shared)
        w_ptr, r_ptr = topk_weights.data_ptr(), topk_rows.data_ptr()
    else:
        es, T, H, device = _check_partials(src, residual)
        sh, k, num_rows, w_ptr, r_ptr = None, 0, 0, None, None
    _need(residual, "residual", torch.bfloat16, 2, device)
    _check_gamma(gamma1, H, device, "gamma1")
    if epilogue == EPI_SANDWICH:
        if gamma2 is None:
            raise ValueError("the sandwich epilogue needs gamma2")
        _check_gamma(gamma2, H, device, "gamma2")
    if scratch is None:
        scratch = torch.empty((T, H), dtype=torch.bfloat16, device=device)
    else:
        _need(scratch, "scratch", torch.bfloat16, 2, device)
    out, residual_out = _outputs(T, H, device, out, residual_out)
    earr = _ptr_array(es)
    sarr = _ptr_array(sh) if sh is not None else None
    _check(_c_split(ctypes.cast(earr, _P), ctypes.cast(sarr, _P) if sarr is not None else None,
                    len(es), w_ptr, r_ptr, k, num_rows, epilogue, residual.data_ptr(),
                    gamma1.data_ptr(), gamma2.data_ptr() if gamma2 is not None else None, eps,
                    T, H, scratch.data_ptr(), out.data_ptr(), residual_out.data_ptr(),
                    _stream(stream, device)))
    return out, residual_out


def boundary(src: TensorList, residual: torch.Tensor, gamma1: torch.Tensor,
             gamma2: Optional[torch.Tensor] = None, eps: float = 1e-6, *,
             topk_weights=None, topk_rows=None, shared=None, epilogue: int = EPI_RMSNORM,
             max_fused_tokens: Optional[int] = None, workspace="auto",
             on_decline: str = "raise", out=None, residual_out=None,
             stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """The layer boundary with a large-batch threshold, the analogue of the
    pages' maximum fused batch size (SGLang PR #34134, first commit message:
    a 16k-token prefill chunk is above it and takes another path).  Calls of
    up to ``max_fused_tokens`` tokens (None: every call) run the fused
    kernel; larger ones the split path (reduce -- with the finalize when
    topk_weights are given -- to a BF16 tensor, then the boundary kernel),
    which rounds the sum to BF16 once more.  Measured on MI355X the fused
    kernel is the faster one at every size tried (split/fused 1.05 at
    H=7168, T=4096 and 16384), hence the default.  src: partials, or the
    expert-row buffers when topk_weights/topk_rows are given.

    ``on_decline``: what a declined fused finalize call does.  "raise"
    raises ``FusedReduceNormUnsupported``.  "materialize" follows the pages'
    rule that a deferred finalize reaching a path that does not fuse it is
    materialized in place (SGLang PR #34134, first and second commit
    messages): the per-rank finalize runs alone (``moe_finalize``) and the R
    BF16 partials take the plain reduction and epilogue -- the same result,
    bit for bit, as the fused call.  That serves declines the fused call
    alone makes (a workspace that is misaligned or too small); if the
    materialized path declines too, it raises.  Never returns unreduced
    data."""
    if on_decline not in ("raise", "materialize"):
        raise ValueError("on_decline must be 'raise' or 'materialize'")
    T = (topk_weights.shape[0] if topk_weights is not None
         else _as_list(src, "src")[0].shape[0])
    if max_fused_tokens is not None and T > max_fused_tokens:
        return split_reduce_norm(src, residual, gamma1, gamma2, eps, topk_weights=topk_weights,
                                 topk_rows=topk_rows, shared=shared, epilogue=epilogue,
                                 out=out, residual_out=residual_out, stream=stream)
    if topk_weights is not None:
        try:
            return moe_finalize_reduce_norm(src, topk_weights, topk_rows, residual, gamma1,
                                            gamma2, eps, shared=shared, epilogue=epilogue,
                                            out=out, residual_out=residual_out,
                                            workspace=workspace, stream=stream)
        except FusedReduceNormUnsupported:
            if on_decline != "materialize":
                raise
        parts = moe_finalize(src, topk_weights, topk_rows, shared=shared, stream=stream)
        src = parts
    if epilogue == EPI_SANDWICH:
        return reduce_sandwich_norm(src, residual, gamma1, gamma2, eps, out=out,
                                    residual_out=residual_out, stream=stream)
    return reduce_residual_rmsnorm(src, residual, gamma1, eps, out=out,
                                   residual_out=residual_out, stream=stream)
