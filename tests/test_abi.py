"""The C ABI on the CPU: the library loads, exports every entry point the
header declares, and rejects bad arguments before launching anything.

No call here reaches a kernel launch: every call is either rejected by the
argument checks or has T == 0 (which returns before any HIP call).  The
pointers are fake, 16-byte-aligned integers; the library never dereferences
host-side device pointers.
"""
import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fused_reduce_norm.h")
LIB = os.path.join(ROOT, "tp_reduction_rmsnorm_amd", "libfused_reduce_norm.so")

OK, INVALID, UNSUPPORTED, HIP = 0, 1, 2, 3
P = ctypes.c_void_p


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__.hip_build_module().build()
    L = ctypes.CDLL(LIB)
    L.frn_reduce_residual_rmsnorm.argtypes = [P, ctypes.c_int32, P, P, ctypes.c_float,
                                              ctypes.c_int64, ctypes.c_int64, P, P, P,
                                              ctypes.c_size_t, P]
    L.frn_reduce_sandwich_norm.argtypes = [P, ctypes.c_int32, P, P, P, ctypes.c_float,
                                           ctypes.c_int64, ctypes.c_int64, P, P, P,
                                           ctypes.c_size_t, P]
    L.frn_moe_finalize_reduce_norm.argtypes = [P, P, ctypes.c_int32, P, P, ctypes.c_int32,
                                               ctypes.c_int64, ctypes.c_int32, P, P, P,
                                               ctypes.c_float, ctypes.c_int64, ctypes.c_int64,
                                               P, P, P, ctypes.c_size_t, P]
    L.frn_reduce_bf16.argtypes = [P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, P, P]
    L.frn_split_reduce_norm.argtypes = [P, P, ctypes.c_int32, P, P, ctypes.c_int32,
                                        ctypes.c_int64, ctypes.c_int32, P, P, P, ctypes.c_float,
                                        ctypes.c_int64, ctypes.c_int64, P, P, P, P]
    L.frn_query.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                            ctypes.c_int32]
    L.frn_status_string.restype = ctypes.c_char_p
    L.frn_last_error.restype = ctypes.c_char_p
    L.frn_version.restype = ctypes.c_char_p
    L.frn_workspace_bytes.restype = ctypes.c_size_t
    L.frn_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                      ctypes.c_int32]
    return L


def declared_functions():
    text = open(HEADER).read()
    pattern = r"^\s*(?:const char\*|frn_status|size_t|int32_t)\s+(frn_\w+)\("
    return sorted(set(re.findall(pattern, text, re.M)))


def test_header_declares_the_boundary_calls():
    names = declared_functions()
    for want in ("frn_reduce_residual_rmsnorm", "frn_reduce_sandwich_norm",
                 "frn_moe_finalize_reduce_norm", "frn_reduce_bf16",
                 "frn_moe_finalize_reduce_bf16", "frn_split_reduce_norm", "frn_query",
                 "frn_workspace_bytes", "frn_status_string", "frn_last_error", "frn_version"):
        assert want in names


def test_library_exports_exactly_the_declared_symbols():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = sorted({l.split()[-1] for l in out.splitlines() if " T " in l and
                       l.split()[-1].startswith("frn_")})
    assert exported == declared_functions()


def test_every_declared_symbol_resolves(lib):
    for name in declared_functions():
        assert getattr(lib, name) is not None


def test_python_binding_names_match_the_c_entry_points():
    import tp_reduction_rmsnorm_amd as frn
    assert sorted(frn.C_FUNCTIONS) == declared_functions()
    for name in frn.C_FUNCTIONS:
        if name not in ("frn_status_string", "frn_last_error"):
            assert hasattr(frn, name[len("frn_"):]), name
    # every C entry point has its own ctypes handle (none rebound by another)
    bound = sorted(getattr(frn, a).__name__ for a in dir(frn) if a.startswith("_c_"))
    assert bound == sorted(frn.C_FUNCTIONS)


def test_version_and_status_strings(lib):
    assert lib.frn_version() == b"0.1.0"
    for s in (OK, INVALID, UNSUPPORTED, HIP):
        assert lib.frn_status_string(s).startswith(b"FRN_")


# fake device addresses, 16-byte aligned and far apart
BASE = 1 << 40
def addr(i, off=0):
    return BASE + i * (1 << 32) + off


def ptrs(*xs):
    return ctypes.cast((ctypes.c_void_p * len(xs))(*xs), P)


TUNED_INC = os.path.join(ROOT, "tp_reduction_rmsnorm_amd", "csrc", "frn_tuned_mi355x.inc")
HAND_FITTED = "* * * * 0 * builtin\n"   # every call: the hand-fitted rule


def split_ws(T, H):
    """The split-row finalize's workspace: T x H FP32 rows, then T x S FP64
    sums of squares (S = 64-vector slices of a row)."""
    return T * H * 4 + T * (-(-(H // 8) // 64)) * 8


@pytest.fixture
def hand_fitted():
    """Every call under the hand-fitted rule for the test's duration."""
    import tp_reduction_rmsnorm_amd as frn
    frn.set_launch_table(HAND_FITTED)
    yield
    frn.set_launch_table(None)


def tuned_table_text():
    """The launch table compiled into the library (the raw string in
    frn_tuned_mi355x.inc)."""
    text = open(TUNED_INC).read()
    return text.split('R"FRN_TABLE(\n', 1)[1].split(')FRN_TABLE"', 1)[0]


def tuned_rules():
    return [l.split() for l in tuned_table_text().splitlines()
            if l.strip() and not l.lstrip().startswith("#")]


def call_rms(lib, R=2, T=4, H=64, eps=1e-6, parts=None, residual=None, gamma=None,
             out=None, rout=None):
    parts = ptrs(*[addr(10 + r) for r in range(R)]) if parts is None else parts
    return lib.frn_reduce_residual_rmsnorm(
        parts, R, addr(1) if residual is None else residual, addr(2) if gamma is None else gamma,
        eps, T, H, addr(3) if out is None else out, addr(4) if rout is None else rout,
        None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(R=0), INVALID),
    (dict(R=17), UNSUPPORTED),
    (dict(T=-1), INVALID),
    (dict(H=0), INVALID),
    (dict(H=12), UNSUPPORTED),
    (dict(H=16392), UNSUPPORTED),
    (dict(T=4194304), UNSUPPORTED),               # FRN_MAX_T + 1
    (dict(eps=float("nan")), INVALID),
    (dict(eps=-1e-6), INVALID),
    (dict(eps=float("inf")), INVALID),
    (dict(residual=0), INVALID),
    (dict(gamma=0), INVALID),
    (dict(out=0), INVALID),
    (dict(rout=0), INVALID),
    (dict(out=addr(3, 8)), UNSUPPORTED),          # 8-byte aligned only
    (dict(gamma=addr(2, 4)), UNSUPPORTED),
    (dict(out=addr(10, 64)), INVALID),            # out overlaps partial 0
    (dict(rout=addr(3, 128)), INVALID),           # residual_out overlaps out
    (dict(out=addr(1)), INVALID),                 # out aliases residual_in
])
def test_rmsnorm_rejects(lib, kw, status):
    assert call_rms(lib, **kw) == status
    assert lib.frn_last_error() != b""


def test_null_partial_and_misaligned_partial(lib):
    assert call_rms(lib, parts=ptrs(addr(10), 0)) == INVALID
    assert call_rms(lib, parts=ptrs(addr(10), addr(11, 2))) == UNSUPPORTED
    assert lib.frn_reduce_residual_rmsnorm(None, 2, addr(1), addr(2), 1e-6, 4, 64, addr(3),
                                           addr(4), None, 0, None) == INVALID


def test_zero_tokens_is_a_no_op(lib):
    # T == 0 returns before any HIP call, so this is safe without a GPU
    assert call_rms(lib, T=0) == OK
    assert lib.frn_last_error() == b""


def test_sandwich_needs_gamma2(lib):
    parts = ptrs(addr(10), addr(11))
    st = lib.frn_reduce_sandwich_norm(parts, 2, addr(1), addr(2), None, 1e-6, 4, 64, addr(3),
                                      addr(4), None, 0, None)
    assert st == INVALID


def call_moe(lib, R=2, k=3, T=4, H=64, num_rows=12, epilogue=0, shared=True, w=None, rows=None):
    src = ptrs(*[addr(10 + r) for r in range(R)])
    sh = ptrs(*[addr(30 + r) for r in range(R)]) if shared else None
    return lib.frn_moe_finalize_reduce_norm(
        src, sh, R, addr(5) if w is None else w, addr(6) if rows is None else rows, k, num_rows,
        epilogue, addr(1), addr(2), addr(7), 1e-6, T, H, addr(3), addr(4), None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), INVALID),
    (dict(k=17), UNSUPPORTED),
    (dict(T=4194304), UNSUPPORTED),
    (dict(num_rows=0), INVALID),
    (dict(epilogue=7), INVALID),
    (dict(w=0), INVALID),
    (dict(rows=0), INVALID),
    (dict(rows=addr(6, 2)), UNSUPPORTED),
    (dict(w=addr(3)), INVALID),   # out overlaps the weights
])
def test_moe_rejects(lib, kw, status):
    assert call_moe(lib, **kw) == status


def test_moe_zero_tokens_is_a_no_op(lib):
    assert call_moe(lib, T=0) == OK


def call_moe_noalloc(lib, R=2, k=3, T=4, H=64, num_rows=12, epilogue=0, shared=True, w=None,
                     rows=None):
    lib.frn_moe_finalize_reduce_norm_noalloc.argtypes = [
        P, P, ctypes.c_int32, P, P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, P, P, P,
        ctypes.c_float, ctypes.c_int64, ctypes.c_int64, P, P, P]
    src = ptrs(*[addr(10 + r) for r in range(R)])
    sh = ptrs(*[addr(30 + r) for r in range(R)]) if shared else None
    return lib.frn_moe_finalize_reduce_norm_noalloc(
        src, sh, R, addr(5) if w is None else w, addr(6) if rows is None else rows, k, num_rows,
        epilogue, addr(1), addr(2), addr(7), 1e-6, T, H, addr(3), addr(4), None)


def noalloc_scratch_bytes():
    m = re.search(r"#define FRN_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    return int(m.group(1)) << int(m.group(2))


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), INVALID),
    (dict(k=17), UNSUPPORTED),
    (dict(T=4194304), UNSUPPORTED),
    (dict(num_rows=0), INVALID),
    (dict(epilogue=7), INVALID),
    (dict(w=0), INVALID),
    (dict(rows=0), INVALID),
    (dict(rows=addr(6, 2)), UNSUPPORTED),
    (dict(w=addr(3)), INVALID),   # out overlaps the weights
    (dict(H=68), UNSUPPORTED),
])
def test_noalloc_rejects_like_the_workspace_call(lib, kw, status):
    assert call_moe_noalloc(lib, **kw) == status
    assert call_moe(lib, **kw) == status


def test_noalloc_zero_tokens_is_a_no_op(lib):
    assert call_moe_noalloc(lib, T=0) == OK


def test_noalloc_scratch_covers_every_split_row_call(lib):
    """The scratch array holds the workspace of the largest call the
    split-row finalize takes (256 tokens of H=16384: FP32 rows and FP64
    slice sums), so the no-allocation entry point never declines for its
    size."""
    import tp_reduction_rmsnorm_amd as frn
    cap = noalloc_scratch_bytes()
    assert cap == frn.NOALLOC_SCRATCH_BYTES == 17 << 20
    assert split_ws(256, 16384) == 256 * 16384 * 4 + 256 * 32 * 8 <= cap
    frn.set_launch_table("* * * * 0 * split\n")   # split wherever the library allows
    try:
        R, k, H, T = 16, 16, 16384, 256
        assert frn.split_rows(R, k, T, H) and not frn.split_rows(R, k, T + 1, H)
        assert lib.frn_workspace_bytes(100000, H, R, k) == split_ws(T, H) <= cap
    finally:
        frn.set_launch_table(None)
    assert lib.frn_workspace_bytes(100000, 6144, 8, 10) <= cap


def call_ep(lib, R=2, k=3, T=4, H=64, num_rows=(12, 12), epilogue=0, src=None, shared=None,
            rows=None, w=None, nr_ptr=True, outs=None):
    lib.frn_ep_moe_finalize_reduce_norm.argtypes = [
        P, P, ctypes.c_int32, P, P, ctypes.c_int32, P, ctypes.c_int32, P, P, P, ctypes.c_float,
        ctypes.c_int64, ctypes.c_int64, P, P, P, ctypes.c_size_t, P]
    src = ptrs(*[addr(10 + r) for r in range(R)]) if src is None else src
    rows = ptrs(*[addr(40 + r) for r in range(R)]) if rows is None else rows
    nr = (ctypes.c_int64 * len(num_rows))(*num_rows)
    return lib.frn_ep_moe_finalize_reduce_norm(
        src, shared, R, addr(5) if w is None else w, rows, k,
        ctypes.cast(nr, P) if nr_ptr else None, epilogue, addr(1), addr(2), addr(7), 1e-6, T,
        H, addr(3), addr(4), None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), INVALID),
    (dict(k=17), UNSUPPORTED),
    (dict(epilogue=7), INVALID),
    (dict(num_rows=(12, -1)), INVALID),
    (dict(nr_ptr=False), INVALID),
    (dict(rows=0), INVALID),                                  # no index-array list
    (dict(rows=ptrs(addr(40), 0)), INVALID),                  # one index array missing
    (dict(rows=ptrs(addr(40), addr(41, 2))), UNSUPPORTED),    # misaligned index array
    (dict(src=ptrs(addr(10), 0)), INVALID),                   # rank with rows but no buffer
    (dict(w=addr(3)), INVALID),                               # out overlaps the weights
    (dict(rows=ptrs(addr(40), addr(3))), INVALID),            # out overlaps an index array
    (dict(shared=ptrs(0, addr(3))), INVALID),                 # out overlaps a shared row
    (dict(H=68), UNSUPPORTED),
])
def test_ep_rejects(lib, kw, status):
    assert call_ep(lib, **kw) == status


def test_ep_accepts_ranks_without_rows_or_shared_rows(lib):
    # Rank 1 owns no rows (NULL buffer) and holds no shared row (NULL entry).
    # With T > 0 every check runs; the overlap planted on the weights stops
    # the call before any launch, after those two entries were accepted.
    src = ptrs(addr(10), 0)
    st = call_ep(lib, num_rows=(12, 0), src=src, shared=ptrs(addr(30), 0), w=addr(3))
    assert st == INVALID and b"overlaps" in lib.frn_last_error()
    assert call_ep(lib, T=0) == OK


def test_ep_standalone_finalize_rejects(lib):
    lib.frn_ep_moe_finalize.argtypes = [P, P, ctypes.c_int32, P, P, ctypes.c_int32, P,
                                        ctypes.c_int64, ctypes.c_int64, P, P]
    src = ptrs(addr(10), addr(11))
    rows = ptrs(addr(40), addr(41))
    nr = (ctypes.c_int64 * 2)(12, 12)
    args = (src, None, 2, addr(5), rows, 3, ctypes.cast(nr, P))
    assert lib.frn_ep_moe_finalize(*args, 0, 64, ptrs(addr(20), addr(21)), None) == OK
    assert lib.frn_ep_moe_finalize(*args, 4, 64, None, None) == INVALID
    assert lib.frn_ep_moe_finalize(*args, 4, 64, ptrs(addr(20), addr(10)), None) == INVALID
    assert lib.frn_ep_moe_finalize(*args, 4, 64, ptrs(addr(20), addr(40)), None) == INVALID
    assert lib.frn_ep_moe_finalize(src, None, 2, addr(5), rows, 3, None, 4, 64,
                                   ptrs(addr(20), addr(21)), None) == INVALID


def test_split_scratch_must_not_alias(lib):
    src = ptrs(addr(10), addr(11))
    st = lib.frn_split_reduce_norm(src, None, 2, None, None, 0, 0, 0, addr(1), addr(2), None,
                                   1e-6, 4, 64, addr(3), addr(3), addr(4), None)
    assert st == INVALID
    st = lib.frn_split_reduce_norm(src, None, 2, None, None, 0, 0, 0, addr(1), addr(2), None,
                                   1e-6, 4, 64, addr(11), addr(3), addr(4), None)
    assert st == INVALID
    st = lib.frn_split_reduce_norm(src, None, 2, None, None, 0, 0, 0, addr(1), addr(2), None,
                                   1e-6, 0, 64, addr(20), addr(3), addr(4), None)
    assert st == OK


def test_pass1_rejects(lib):
    src = ptrs(addr(10), addr(11))
    assert lib.frn_reduce_bf16(src, 2, 4, 64, 0, None) == INVALID
    assert lib.frn_reduce_bf16(src, 2, 4, 64, addr(10, 16), None) == INVALID
    assert lib.frn_reduce_bf16(src, 2, 0, 64, addr(20), None) == OK


def test_workspace_bytes(lib):
    lib.frn_set_launch_table.argtypes = [ctypes.c_char_p]
    assert lib.frn_set_launch_table(HAND_FITTED.encode()) == OK
    try:
        assert lib.frn_workspace_bytes(8, 6144, 8, 10) == split_ws(8, 6144)   # FP32 sums
        # covers the largest T either routing splits at: R=8 H=6144 -> 128 (TP)
        assert lib.frn_workspace_bytes(5000, 6144, 8, 10) == split_ws(128, 6144)
        assert lib.frn_workspace_bytes(5000, 4096, 2, 4) == split_ws(64, 4096)   # EP only
        assert lib.frn_workspace_bytes(64, 5120, 4, 0) == 0      # no finalize: none used
        assert lib.frn_workspace_bytes(64, 5124, 4, 2) == 0      # unsupported H
        assert lib.frn_workspace_bytes(0, 5120, 4, 2) == 0
        assert lib.frn_workspace_bytes(8, 5120, 4, 17) == 0      # k beyond FRN_MAX_K
        # the size covers the compiled-in table's split rules too
        assert lib.frn_workspace_bytes(5000, 7168, 2, 8) == split_ws(max(
            [64] + [int(r[5]) for r in tuned_rules()
                    if r[:3] == ["7168", "2", "8"] and r[6] == "split"]), 7168)
    finally:
        lib.frn_set_launch_table(None)


def test_split_rows_builtin_rule():
    """The hand-fitted choice of the split-row finalize at its measured
    edges (a 'builtin' rule turns the compiled-in table off)."""
    import tp_reduction_rmsnorm_amd as frn
    S, EP = frn.EPI_SANDWICH, True
    frn.set_launch_table(HAND_FITTED)
    cases = [  # R, k, H, ep, T, expected
        (8, 10, 6144, False, 1, True), (8, 10, 6144, False, 128, True),
        (8, 10, 6144, False, 129, False), (8, 10, 6144, False, 256, False),
        (1, 8, 7168, False, 1, False),
        (2, 8, 7168, False, 64, True), (2, 8, 7168, False, 65, False),
        (2, 16, 5120, False, 96, True), (2, 16, 5120, False, 97, False),
        (2, 4, 4096, False, 1, False), (4, 8, 2048, False, 256, True),
        (4, 8, 2048, False, 257, False), (16, 8, 4096, False, 192, True),
        (16, 8, 4096, False, 193, False), (3, 8, 7168, False, 96, True),
        (3, 8, 7168, False, 97, False), (4, 8, 5120, False, 128, True),
        (4, 8, 5120, False, 129, False), (4, 8, 8192, False, 96, True),
        (4, 8, 8192, False, 97, False), (8, 2, 6144, False, 192, True),
        (8, 2, 6144, False, 193, False),
        (8, 10, 6144, EP, 64, True), (8, 10, 6144, EP, 65, False),
        (8, 4, 6144, EP, 32, True), (8, 4, 6144, EP, 33, False),
        (2, 10, 6144, EP, 64, True), (2, 10, 6144, EP, 65, False),
        (4, 8, 7168, EP, 64, True), (4, 8, 7168, EP, 65, False),
        (16, 8, 4096, EP, 128, True), (16, 8, 4096, EP, 129, False),
        (16, 8, 7168, EP, 96, True), (16, 8, 7168, EP, 97, False),
        (8, 8, 2048, EP, 256, True), (8, 8, 2048, EP, 257, False),
        (16, 8, 7168, False, 128, True), (16, 8, 7168, False, 129, False),
        (8, 6, 3072, False, 224, True), (8, 6, 3072, False, 225, False),
        (8, 10, 5120, False, 128, True), (8, 10, 5120, False, 129, False),
        (16, 6, 3072, EP, 128, True), (16, 6, 3072, EP, 129, False),
    ]
    try:
        for R, k, H, ep, T, want in cases:
            assert frn.split_rows(R, k, T, H, ep=ep) is want, (R, k, H, ep, T)
            assert frn.split_rows(R, k, T, H, S, ep=ep) is want, (R, k, H, ep, T)
        assert not frn.split_rows(8, 0, 8, 6144)                 # no finalize
        assert not frn.split_rows(8, 10, 0, 6144)                # empty call
        assert not frn.split_rows(8, 10, 8, 6148)                # unsupported H
        assert not frn.split_rows(8, 10, 8, 6144, frn.EPI_SUM)   # split pass 1: no workspace
    finally:
        frn.set_launch_table(None)


def test_split_rows_is_covered_by_workspace_bytes(lib):
    """Over a grid of shapes and both routings: the calls that take the
    split-row finalize form a prefix of T, and frn_workspace_bytes for a
    larger max_T covers every one of them."""
    import tp_reduction_rmsnorm_amd as frn
    frn.set_launch_table(None)
    for R in (1, 2, 3, 4, 8, 9, 16):
        for H in (8, 520, 2048, 2056, 4096, 6144, 16384):
            for k in (1, 4, 8, 16):
                cap_bytes = lib.frn_workspace_bytes(100000, H, R, k)
                for ep in (False, True):
                    seen_fused = False
                    for T in list(range(1, 200, 7)) + [256, 257, 1000]:
                        split = frn.split_rows(R, k, T, H, ep=ep)
                        assert not (split and seen_fused), (R, H, k, ep, T)
                        seen_fused |= not split
                        if split:
                            assert split_ws(T, H) <= cap_bytes, (R, H, k, ep, T)


def test_launch_table_split_and_fused_rules(lib):
    """split / fused rules override the built-in choice, leave the vec
    rules alone, never split above 256 tokens, and widen the workspace size
    to what they route to the split-row finalize."""
    import tp_reduction_rmsnorm_amd as frn
    try:
        frn.set_launch_table(None)
        base = frn.launch_shape(8, 10, 200, 6144, ep=True)
        frn.set_launch_table("6144 8 10 ep-rmsnorm 0 200 split\n"
                             "6144 8 10 rmsnorm 0 * fused\n"
                             "* * * * 0 * split\n")
        assert frn.split_rows(8, 10, 200, 6144, ep=True)
        assert frn.split_rows(8, 10, 201, 6144, ep=True)                # the '*' split rule
        assert not frn.split_rows(8, 10, 8, 6144)                       # fused rule first
        assert frn.split_rows(8, 10, 8, 6144, frn.EPI_SANDWICH)         # sandwich: '*' rule
        assert not frn.split_rows(8, 10, 257, 6144, ep=True)            # never above 256
        assert frn.launch_shape(8, 10, 200, 6144, ep=True) == base      # vec rules untouched
        assert lib.frn_workspace_bytes(5000, 6144, 8, 10) == split_ws(256, 6144)
        frn.set_launch_table("6144 8 10 * 0 * fused\n")
        assert not frn.split_rows(8, 10, 1, 6144)
        assert not frn.split_rows(8, 10, 1, 6144, ep=True)
        assert lib.frn_workspace_bytes(5000, 6144, 8, 10) == split_ws(128, 6144)  # built-in
        for bad in ("6144 8 10 rmsnorm 0 * splits", "6144 8 10 rmsnorm 0 * 3"):
            with pytest.raises(ValueError):
                frn.set_launch_table(bad)
    finally:
        frn.set_launch_table(None)


def test_misaligned_or_overlapping_workspace_rejected(lib):
    need = lib.frn_workspace_bytes(4, 64, 2, 3)
    src = ptrs(addr(10), addr(11))
    sh = ptrs(addr(30), addr(31))
    def moe(ws, wsb):
        return lib.frn_moe_finalize_reduce_norm(src, sh, 2, addr(5), addr(6), 3, 12, 0, addr(1),
                                                addr(2), None, 1e-6, 4, 64, addr(3), addr(4),
                                                ws, wsb, None)
    import tp_reduction_rmsnorm_amd as frn
    lib.frn_set_launch_table.argtypes = [ctypes.c_char_p]
    try:
        # The built-in rule keeps R=2, H*k=192 on the one-row kernel, whose
        # calls ignore the workspace (not called here: it would launch); a
        # table routes it to the split-row finalize, which checks it.
        assert not frn.split_rows(2, 3, 4, 64)
        assert lib.frn_set_launch_table(b"* * * * 0 * split\n") == OK
        assert frn.split_rows(2, 3, 4, 64)
        assert moe(addr(40, 16), need) == UNSUPPORTED   # not 256-byte aligned
        assert moe(addr(40), need - 1) == UNSUPPORTED   # too small for the split-row mode
        assert b"smaller than" in lib.frn_last_error()
        assert moe(addr(10), need) == INVALID           # overlaps expert rows of rank 0
        assert moe(addr(3), need) == INVALID            # overlaps out
    finally:
        lib.frn_set_launch_table(None)


def test_standalone_finalize_rejects(lib):
    lib.frn_moe_finalize.argtypes = [P, P, ctypes.c_int32, P, P, ctypes.c_int32, ctypes.c_int64,
                                     ctypes.c_int64, ctypes.c_int64, P, P]
    src = ptrs(addr(10), addr(11))
    outs = ptrs(addr(20), addr(21))
    ok_args = (src, None, 2, addr(5), addr(6), 3, 12, 4, 64)
    assert lib.frn_moe_finalize(*ok_args[:-2], 0, 64, outs, None) == OK        # T = 0
    assert lib.frn_moe_finalize(src, None, 2, addr(5), addr(6), 0, 12, 4, 64, outs, None) == INVALID
    assert lib.frn_moe_finalize(*ok_args, None, None) == INVALID                 # no outputs
    assert lib.frn_moe_finalize(*ok_args, ptrs(addr(20), 0), None) == INVALID
    assert lib.frn_moe_finalize(*ok_args, ptrs(addr(20), addr(20, 64)), None) == INVALID  # overlap
    assert lib.frn_moe_finalize(*ok_args, ptrs(addr(20), addr(10)), None) == INVALID      # aliases E_0
    assert lib.frn_moe_finalize(*ok_args, ptrs(addr(20), addr(21, 8)), None) == UNSUPPORTED
    assert lib.frn_moe_finalize(src, None, 2, addr(5), addr(6), 3, 12, 4, 68, outs, None) == UNSUPPORTED


def test_query(lib):
    assert lib.frn_query(4, 0, 1024, 5120, 1) == OK
    assert lib.frn_query(8, 10, 64, 6144, 0) == OK
    assert lib.frn_query(2, 8, 16384, 7168, 0) == OK
    assert lib.frn_query(4, 0, 1024, 5124, 1) == UNSUPPORTED
    assert lib.frn_query(0, 0, 1024, 5120, 1) == INVALID
    assert lib.frn_query(20, 0, 1024, 5120, 1) == UNSUPPORTED
    assert lib.frn_query(4, 0, 1 << 31, 5120, 1) == UNSUPPORTED


DECLINE_SCRIPT = r"""
import ctypes, sys
sys.path.insert(0, {root!r})
L = ctypes.CDLL({lib!r})
L.frn_query.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32]
assert L.frn_query(4, 0, 1024, 5120, 1) == 2
import tp_reduction_rmsnorm_amd as frn
assert frn.query(4, 0, 1024, 5120, 1) is False
print("declined")
"""


def test_forced_decline_env():
    code = DECLINE_SCRIPT.format(root=ROOT, lib=LIB)
    env = dict(os.environ, FRN_FORCE_DECLINE="1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr
    assert "declined" in r.stdout


def test_python_layer_raises_on_decline_and_never_returns_inputs(monkeypatch):
    """The binding turns FRN_ERR_UNSUPPORTED into an exception (it cannot
    hand back unreduced data), using a stand-in for the C call."""
    import tp_reduction_rmsnorm_amd as frn
    with pytest.raises(frn.FusedReduceNormUnsupported):
        frn._check(UNSUPPORTED)
    with pytest.raises(ValueError):
        frn._check(INVALID)
    with pytest.raises(frn.FusedReduceNormError):
        frn._check(HIP)
    frn._check(OK)


def test_boundary_materializes_a_declined_finalize_or_raises(monkeypatch):
    """boundary()'s decline policy, with stand-ins for the library calls:
    'raise' re-raises; 'materialize' runs the standalone finalize and reduces
    its R partials; a decline the materialized path makes too still raises,
    so no unreduced data is ever returned."""
    import torch
    import tp_reduction_rmsnorm_amd as frn
    calls = []

    def fused_declines(*a, **k):
        calls.append("fused")
        raise frn.FusedReduceNormUnsupported("workspace is not 256-byte aligned")

    def finalize(src, w, rows, shared=None, stream=None):
        calls.append(("finalize", tuple(src), shared))
        return ["P0", "P1"]

    def reduce(parts, residual, gamma, eps, out=None, residual_out=None, stream=None):
        calls.append(("reduce", tuple(parts), residual))
        return "y", "x"

    monkeypatch.setattr(frn, "moe_finalize_reduce_norm", fused_declines)
    monkeypatch.setattr(frn, "moe_finalize", finalize)
    monkeypatch.setattr(frn, "reduce_residual_rmsnorm", reduce)
    w = torch.zeros(3, 2)
    args = (["E0", "E1"], "res", "g")
    kw = dict(topk_weights=w, topk_rows="idx", shared=["S0", "S1"])
    with pytest.raises(frn.FusedReduceNormUnsupported):
        frn.boundary(*args, **kw)
    assert frn.boundary(*args, **kw, on_decline="materialize") == ("y", "x")
    assert calls == ["fused", "fused", ("finalize", ("E0", "E1"), ["S0", "S1"]),
                     ("reduce", ("P0", "P1"), "res")]

    def finalize_declines(*a, **k):
        raise frn.FusedReduceNormUnsupported("R=17 exceeds 16")

    monkeypatch.setattr(frn, "moe_finalize", finalize_declines)
    with pytest.raises(frn.FusedReduceNormUnsupported, match="exceeds"):
        frn.boundary(*args, **kw, on_decline="materialize")
    with pytest.raises(ValueError):
        frn.boundary(*args, **kw, on_decline="skip")


def test_python_layer_requires_gpu_tensors():
    import torch
    import tp_reduction_rmsnorm_amd as frn
    p = torch.zeros(4, 64, dtype=torch.bfloat16)
    g = torch.ones(64)
    with pytest.raises(ValueError, match="GPU"):
        frn.reduce_residual_rmsnorm([p, p], p, g)
    with pytest.raises(ValueError, match="residual is required"):
        frn.reduce_residual_rmsnorm([p, p], None, g)
    with pytest.raises(TypeError):
        frn.reduce_residual_rmsnorm([p.float()], p, g)


# ------------------------------------------------------- launch tables --- #

def test_launch_shape_builtin_rule(hand_fitted):
    import tp_reduction_rmsnorm_amd as frn
    S = frn.EPI_SANDWICH
    assert frn.launch_shape(4, 0, 1, 5120, S) == (640, 1)      # small T: one vector ...
    assert frn.launch_shape(8, 0, 200, 6144, 0) == (768, 1)    # ... up to 896 lanes
    assert frn.launch_shape(2, 0, 256, 7168, 0) == (896, 1)
    assert frn.launch_shape(8, 0, 8, 8192, S) == (512, 2)
    assert frn.launch_shape(4, 0, 512, 5120, S) == (320, 2)    # T <= 512: two below 1024 vectors
    assert frn.launch_shape(8, 0, 512, 8192, S) == (256, 4)
    assert frn.launch_shape(4, 0, 1024, 5120, S) == (192, 4)   # mid T: four vectors
    assert frn.launch_shape(4, 0, 4096, 5120, S) == (320, 2)   # large T
    assert frn.launch_shape(8, 0, 4096, 8192, S) == (256, 4)   # long rows: four up to 4096
    assert frn.launch_shape(8, 0, 16384, 8192, S) == (1024, 1)  # beyond 4096: one vector
    assert frn.launch_shape(2, 0, 16384, 16384, 0) == (1024, 2)  # ... up to 1024 lanes
    assert frn.launch_shape(2, 0, 16384, 7168, frn.EPI_SUM) == (448, 2)  # not split pass 1
    assert frn.launch_shape(2, 8, 4096, 7168, 0) == (896, 1)   # finalize: one vector
    assert frn.launch_shape(2, 8, 1024, 7168, 0) == (448, 2)   # ... two at mid T for R <= 2
    assert frn.launch_shape(8, 10, 512, 6144, 0) == (384, 2)   # ... and up to 512 above
    assert frn.launch_shape(8, 10, 1024, 6144, 0) == (768, 1)
    assert frn.launch_shape(2, 8, 1024, 7168, frn.EPI_SUM) == (448, 2)
    assert frn.launch_shape(2, 8, 2048, 7168, frn.EPI_SUM) == (896, 1)
    assert frn.launch_shape(2, 0, 1024, 7168, frn.EPI_SUM) == (448, 2)  # no 4 in pass 1
    assert frn.launch_shape(2, 0, 8, 16384, S) == (1024, 2)
    # expert-parallel finalize: one vector per lane, two for 256 < T <= 512
    assert frn.launch_shape(8, 10, 1024, 6144, 0, ep=True) == (768, 1)
    assert frn.launch_shape(8, 10, 512, 6144, 0, ep=True) == (384, 2)
    assert frn.launch_shape(8, 10, 64, 6144, 0, ep=True) == (768, 1)
    assert frn.launch_shape(2, 4, 64, 16384, S, ep=True) == (1024, 2)
    with pytest.raises(ValueError):
        frn.launch_shape(8, 0, 1024, 6144, 0, ep=True)      # no finalize
    with pytest.raises(ValueError):
        frn.launch_shape(8, 10, 1024, 6144, frn.EPI_SUM, ep=True)


def test_pipelined_builtin_rule(hand_fitted):
    """Under the hand-fitted rule, calls without finalize take the
    row-pipelined kernel (one workgroup per CU walking the rows) from
    T = 1536 where it serves them."""
    import tp_reduction_rmsnorm_amd as frn
    S, N = frn.EPI_SANDWICH, frn.EPI_RMSNORM
    assert frn.launch_pipelined(4, 0, 4096, 5120, S)
    assert frn.launch_shape(4, 0, 4096, 5120, S) == (320, 2)
    assert frn.launch_pipelined(4, 0, 1536, 5120, S)
    assert not frn.launch_pipelined(4, 0, 1535, 5120, S)       # below the measured crossover
    assert frn.launch_shape(4, 0, 1535, 5120, S) == (320, 2)   # one-row kernel, two vectors
    assert frn.launch_pipelined(1, 0, 16384, 7168, N)          # split pass 2
    assert frn.launch_shape(1, 0, 16384, 7168, N) == (448, 2)
    assert not frn.launch_pipelined(2, 0, 16384, 7168, N)      # residual + RMSNorm R = 2: T <= 4096
    assert frn.launch_pipelined(2, 0, 4096, 7168, N)
    assert frn.launch_shape(2, 0, 4096, 7168, N) == (896, 1)
    assert frn.launch_pipelined(2, 0, 1536, 8192, N)           # ... 512 to 1024 vectors, one each
    assert frn.launch_shape(2, 0, 1536, 8192, N) == (1024, 1)
    assert not frn.launch_pipelined(2, 0, 1535, 8192, N)
    assert not frn.launch_pipelined(2, 0, 4096, 2048, N)       # 256 vectors
    assert not frn.launch_pipelined(3, 0, 4096, 6144, N)       # residual + RMSNorm: R <= 2
    assert frn.launch_pipelined(2, 0, 2048, 6144, S)           # the sandwich at R = 2
    assert frn.launch_pipelined(3, 0, 2048, 6144, S)           # 768 vectors, R = 3
    assert frn.launch_shape(3, 0, 2048, 6144, S) == (384, 2)
    assert frn.launch_pipelined(4, 0, 4096, 6144, S)           # R >= 3, 768+ vectors: up to 4096
    assert not frn.launch_pipelined(4, 0, 4097, 6144, S)
    assert frn.launch_shape(4, 0, 8192, 6144, S) == (768, 1)
    assert frn.launch_pipelined(2, 0, 16384, 6144, S)          # R = 2: all T
    assert frn.launch_pipelined(4, 0, 16384, 5120, S)          # 640 vectors: all T
    assert not frn.launch_pipelined(4, 0, 4096, 8192, S)       # 1024 vectors: one row per group
    assert not frn.launch_pipelined(4, 0, 4096, 4096, S)       # 512 vectors: the same
    assert frn.launch_pipelined(2, 0, 4096, 4096, N)           # except residual + RMSNorm at R = 2
    assert not frn.launch_pipelined(8, 0, 4096, 8192, S)       # R > 4
    assert not frn.launch_pipelined(4, 10, 4096, 6144, N)      # finalize
    assert not frn.launch_pipelined(4, 0, 4096, 5128, S)       # 641 vectors: idle lanes
    assert not frn.launch_pipelined(2, 0, 4096, 16384, N)      # more lanes than it takes
    assert not frn.launch_pipelined(4, 0, 4096, 5120, frn.EPI_SUM)   # split pass 1
    assert not frn.launch_pipelined(0, 0, 4096, 5120, S)       # malformed sizes: no
    assert not frn.launch_pipelined(4, 0, 4096, 5124, S)


def test_launch_table_pipelined_rules():
    import tp_reduction_rmsnorm_amd as frn
    S, N = frn.EPI_SANDWICH, frn.EPI_RMSNORM
    try:
        frn.set_launch_table(None)
        base = frn.launch_shape(8, 0, 4096, 8192, S)
        frn.set_launch_table("5120 4 0 sandwich 0 * p1\n")
        assert frn.launch_pipelined(4, 0, 8, 5120, S)
        assert frn.launch_shape(4, 0, 8, 5120, S) == (640, 1)
        frn.set_launch_table("5120 4 0 sandwich 0 * 4\n")        # a numeric rule: one row
        assert not frn.launch_pipelined(4, 0, 4096, 5120, S)
        assert frn.launch_shape(4, 0, 4096, 5120, S) == (192, 4)
        frn.set_launch_table("* * * * 0 * p2\n")
        assert frn.launch_pipelined(2, 0, 8, 1024, N)              # 128 vectors: 64 lanes
        assert frn.launch_shape(2, 0, 8, 1024, N) == (64, 2)
        assert not frn.launch_pipelined(8, 0, 4096, 8192, S)       # does not fit: skipped
        assert frn.launch_shape(8, 0, 4096, 8192, S) == base        # the compiled-in rule
        assert not frn.launch_pipelined(2, 0, 8, 520, N)           # 65 vectors: skipped
        assert not frn.launch_pipelined(4, 10, 8, 6144, N)         # finalize: skipped
        for bad in ("5120 4 0 sandwich 0 * p3\n", "5120 4 0 sandwich 0 * p\n",
                    "5120 4 0 sandwich 0 * P2\n"):
            with pytest.raises(ValueError):
                frn.set_launch_table(bad)
    finally:
        frn.set_launch_table(None)


def test_launch_table_expert_parallel_rules():
    import tp_reduction_rmsnorm_amd as frn
    try:
        frn.set_launch_table("6144 8 10 ep-rmsnorm 0 * 2\n6144 8 10 rmsnorm 0 * 1\n")
        assert frn.launch_shape(8, 10, 4096, 6144, 0, ep=True) == (384, 2)
        assert frn.launch_shape(8, 10, 4096, 6144, 0) == (768, 1)
        frn.set_launch_table("* * * ep-* 0 * 2\n")
        assert frn.launch_shape(8, 10, 64, 6144, frn.EPI_SANDWICH, ep=True) == (384, 2)
        assert frn.launch_shape(8, 10, 4096, 6144, 0) == (768, 1)   # TP: built-in rule
        frn.set_launch_table("* * * * 0 * 2\n")                    # '*' matches both
        assert frn.launch_shape(8, 10, 4096, 6144, 0, ep=True) == (384, 2)
        for bad in ("6144 8 10 ep-sum 0 * 1\n", "6144 8 10 ep 0 * 1\n", "1 1 1 ep-x 0 * 1\n"):
            with pytest.raises(ValueError):
                frn.set_launch_table(bad)
    finally:
        frn.set_launch_table(None)


def test_launch_table_overrides_and_restores():
    import tp_reduction_rmsnorm_amd as frn
    try:
        frn.set_launch_table("""
            # comment line
            5120 4 0 sandwich 1000 5000 1   # exact shape, T range
            * * 0 * 0 * 4                   # any shape without finalize
            * * * * 0 * 2
        """)
        S = frn.EPI_SANDWICH
        assert frn.launch_shape(4, 0, 4096, 5120, S) == (640, 1)
        assert frn.launch_shape(4, 0, 8, 5120, S) == (192, 4)      # second rule
        assert frn.launch_shape(8, 0, 8, 8192, S) == (256, 4)
        # vec 4 does not fit a finalize or pass 1: the next fitting rule decides
        assert frn.launch_shape(8, 10, 8, 6144, 0) == (384, 2)
        assert frn.launch_shape(2, 0, 8, 7168, frn.EPI_SUM) == (448, 2)
        # a rule that would need more than 1024 lanes is skipped
        frn.set_launch_table("* * * * 0 * 1")
        assert frn.launch_shape(2, 0, 8, 16384, S) == (1024, 2)
        with pytest.raises(ValueError, match="line 2"):
            frn.set_launch_table("* * * * 0 * 1\n5120 4 0 sandwich 1 2 3\n")
        assert frn.launch_shape(4, 0, 8, 5120, S) == (640, 1)      # unchanged by the failure
    finally:
        frn.set_launch_table(None)
    assert frn.launch_shape(4, 0, 4096, 5120, frn.EPI_SANDWICH) == (320, 2)


ENV_TABLE_SCRIPT = r"""
import sys
sys.path.insert(0, {root!r})
import tp_reduction_rmsnorm_amd as frn
print(frn.launch_shape(4, 0, 4096, 5120, frn.EPI_SANDWICH))
"""  # built-in rule: (320, 2)


def test_launch_table_from_environment(tmp_path):
    table = tmp_path / "table.txt"
    table.write_text("5120 4 0 sandwich 0 * 1\n")
    env = dict(os.environ, FRN_LAUNCH_TABLE=str(table))
    r = subprocess.run([sys.executable, "-c", ENV_TABLE_SCRIPT.format(root=ROOT)], env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "(640, 1)"
    table.write_text("not a table\n")
    r = subprocess.run([sys.executable, "-c", ENV_TABLE_SCRIPT.format(root=ROOT)], env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "(320, 2)"
    assert "launch table line 1" in r.stderr


def test_tuner_merges_rules():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "frn_tune", os.path.join(ROOT, "tp_reduction_rmsnorm_amd", "tune.py"))
    tune = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(tune)
    rows = [(1, 1, {}), (8, 1, {}), (64, 2, {}), (1024, 4, {}), (4096, 2, {})]
    assert tune.rules_for(5120, 4, 0, "sandwich", rows) == [
        "5120 4 0 sandwich 0 8 1", "5120 4 0 sandwich 9 64 2",
        "5120 4 0 sandwich 65 1024 4", "5120 4 0 sandwich 1025 * 2"]
    split = [(1, "split", {}), (16, "split", {}), (32, "fused", {}), (256, "fused", {})]
    lines = tune.rules_for(6144, 8, 10, "ep-rmsnorm", split, last="256")
    assert lines == ["6144 8 10 ep-rmsnorm 0 16 split", "6144 8 10 ep-rmsnorm 17 256 fused"]
    rows = [(1024, "4", {}), (2048, "p2", {}), (4096, "p2", {})]
    piped = tune.rules_for(5120, 4, 0, "sandwich", rows)
    assert piped == ["5120 4 0 sandwich 0 1024 4", "5120 4 0 sandwich 1025 * p2"]
    import tp_reduction_rmsnorm_amd as frn
    try:
        frn.set_launch_table("\n".join(lines))   # the tuner's output parses
        assert frn.split_rows(8, 10, 16, 6144, ep=True)
        assert not frn.split_rows(8, 10, 17, 6144, ep=True)
        frn.set_launch_table("\n".join(piped))
        assert frn.launch_pipelined(4, 0, 1025, 5120, frn.EPI_SANDWICH)
        assert not frn.launch_pipelined(4, 0, 1024, 5120, frn.EPI_SANDWICH)
        # what the tuner times is what a call of that size takes under the rule
        for choice, ok in (("1", True), ("4", True), ("p1", True), ("p2", True)):
            frn.set_launch_table(f"5120 4 0 sandwich 4096 4096 {choice}")
            assert tune.fits(5120, 4, 0, "sandwich", 4096, choice) == ok
        for choice in ("p1", "p2"):                 # R = 8 or a finalize: not served
            frn.set_launch_table(f"* * * * 0 * {choice}")
            assert not tune.fits(8192, 8, 0, "sandwich", 4096, choice)
            assert not tune.fits(6144, 8, 10, "rmsnorm", 4096, choice)
            assert not tune.fits(6144, 8, 10, "ep-rmsnorm", 4096, choice)
    finally:
        frn.set_launch_table(None)


def test_launch_table_is_thread_safe():
    """Threads replacing the table while others ask for shapes: no crash, and
    every answer is one of the shapes some table gives."""
    import threading
    import tp_reduction_rmsnorm_amd as frn
    tables = ["5120 4 0 sandwich 0 * 1\n", "5120 4 0 sandwich 0 * 2\n", None]
    allowed = {(640, 1), (320, 2)}
    seen, errors = set(), []

    def setter():
        try:
            for i in range(300):
                frn.set_launch_table(tables[i % 3])
        except Exception as e:  # pragma: no cover - reported below
            errors.append(e)

    def reader():
        try:
            for _ in range(300):
                seen.add(frn.launch_shape(4, 0, 4096, 5120, frn.EPI_SANDWICH))
        except Exception as e:  # pragma: no cover
            errors.append(e)

    th = [threading.Thread(target=setter) for _ in range(2)] + \
         [threading.Thread(target=reader) for _ in range(4)]
    try:
        for t in th:
            t.start()
        for t in th:
            t.join()
    finally:
        frn.set_launch_table(None)
    assert not errors, errors
    assert seen and seen <= allowed, seen


def test_builtin_launch_shapes_always_fit():
    """Over every H, R, k, epilogue and a spread of T: at most 1024 lanes, a
    multiple of 64, enough lanes for the row, and four vectors never with a
    finalize or in split pass 1."""
    import tp_reduction_rmsnorm_amd as frn
    frn.set_launch_table(None)
    for H in list(range(8, 16385, 8 * 97)) + [8, 512, 5120, 6144, 7168, 8192, 16384]:
        nvec = H // 8
        for R in (1, 2, 8, 16):
            for k in (0, 1, 10, 16):
                for epi in (frn.EPI_RMSNORM, frn.EPI_SANDWICH, frn.EPI_SUM):
                    for ep in ((False, True) if k and epi != frn.EPI_SUM else (False,)):
                        for T in (1, 8, 256, 257, 1024, 1025, 2048, 4096, 4097, 16384):
                            th, v = frn.launch_shape(R, k, T, H, epi, ep=ep)
                            assert th % 64 == 0 and 64 <= th <= 1024, (H, R, k, epi, T, th)
                            assert th * v >= nvec, (H, R, k, epi, T, th, v)
                            assert th - 64 < -(-nvec // v), (H, R, k, epi, T, th, v)
                            assert v in (1, 2, 4)
                            if k or epi == frn.EPI_SUM:
                                assert v != 4, (H, R, k, epi, T)


def test_compiled_in_table_decides_its_shapes_by_default():
    """With no caller table and no environment variable, every rule of the
    table compiled into the library decides its shapes: at each range's
    first and last T, launch_shape / launch_pipelined / split_rows give what
    the table says (the edges are read from the table, which a re-tune may
    move).  The text also loads as a caller table."""
    import tp_reduction_rmsnorm_amd as frn
    frn.set_launch_table(tuned_table_text())           # it parses
    frn.set_launch_table(None)                         # the defaults
    assert os.environ.get("FRN_LAUNCH_TABLE") is None
    epis = {"rmsnorm": frn.EPI_RMSNORM, "sandwich": frn.EPI_SANDWICH, "sum": frn.EPI_SUM}
    rules = tuned_rules()
    assert len({tuple(r[:4]) for r in rules}) >= 20     # the twenty tuned shapes
    seen = set()
    for H, R, k, epi, lo, hi, v in rules:
        H, R, k = int(H), int(R), int(k)
        ep = epi.startswith("ep-")
        e = epis[epi.replace("ep-", "")]
        ts = [max(int(lo), 1)] + ([int(hi)] if hi != "*" else [])
        for T in ts:
            if (H, R, k, epi, T, v in ("split", "fused")) in seen:
                continue                            # an earlier rule decides this T
            seen.add((H, R, k, epi, T, v in ("split", "fused")))
            if v in ("split", "fused"):
                assert frn.split_rows(R, k, T, H, e, ep=ep) == (v == "split"), (H, R, k, epi, T)
            elif v in ("p1", "p2"):
                assert frn.launch_pipelined(R, k, T, H, e), (H, R, k, epi, T)
                assert frn.launch_shape(R, k, T, H, e)[1] == int(v[1])
            else:
                assert not ep and frn.launch_shape(R, k, T, H, e)[1] == int(v) or \
                    ep and frn.launch_shape(R, k, T, H, e, ep=True)[1] == int(v), (H, R, k, epi, T)
                if k == 0 and epi != "sum":
                    assert not frn.launch_pipelined(R, k, T, H, e), (H, R, k, epi, T)


def test_compiled_in_table_file_is_what_the_tuner_writes():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "frn_tune", os.path.join(ROOT, "tp_reduction_rmsnorm_amd", "tune.py"))
    tune = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(tune)
    assert tune.as_inc(tuned_table_text()) == open(TUNED_INC).read()


def test_caller_table_and_builtin_rule_override_the_compiled_in_table():
    import tp_reduction_rmsnorm_amd as frn
    S = frn.EPI_SANDWICH
    rules = tuned_rules()
    # the measured table sends the headline call (T=4096) to the row-pipelined kernel
    assert any(r[:4] == ["5120", "4", "0", "sandwich"] and int(r[4]) <= 4096 and
               (r[5] == "*" or int(r[5]) >= 4096) and r[6] in ("p1", "p2") for r in rules)
    try:
        frn.set_launch_table(None)
        assert frn.launch_pipelined(4, 0, 4096, 5120, S)
        frn.set_launch_table("5120 4 0 sandwich 4000 5000 4\n")   # a caller rule wins
        assert not frn.launch_pipelined(4, 0, 4096, 5120, S)
        assert frn.launch_shape(4, 0, 4096, 5120, S) == (192, 4)
        assert frn.launch_pipelined(4, 0, 8192, 5120, S)          # outside it: the table
        frn.set_launch_table("5120 4 0 sandwich 0 1200 builtin\n")
        assert not frn.launch_pipelined(4, 0, 1100, 5120, S)      # hand-fitted: not below 1536
        assert frn.launch_pipelined(4, 0, 1300, 5120, S)          # the table again
        frn.set_launch_table("6144 8 10 rmsnorm 0 256 builtin\n")
        assert frn.split_rows(8, 10, 128, 6144) and not frn.split_rows(8, 10, 129, 6144)
    finally:
        frn.set_launch_table(None)


def test_shipped_launch_table_parses_and_routes():
    """The measured table, loaded as a caller table, routes its split /
    fused rules and its row-pipelined rules as it says."""
    import tp_reduction_rmsnorm_amd as frn
    text = tuned_table_text()
    rules = tuned_rules()
    epis = {"rmsnorm": frn.EPI_RMSNORM, "sandwich": frn.EPI_SANDWICH}
    try:
        frn.set_launch_table(text)
        splits = [r for r in rules if r[6] == "split"]
        assert splits, "the table has split rules"
        for H, R, k, epi, lo, hi, _ in splits:
            ep = epi.startswith("ep-")
            H, R, k, hi = int(H), int(R), int(k), int(hi)
            assert frn.split_rows(R, k, hi, H, epis[epi.replace("ep-", "")], ep=ep)
            assert not frn.split_rows(R, k, hi + 1, H, epis[epi.replace("ep-", "")], ep=ep)
        piped = [r for r in rules if r[6] in ("p1", "p2")]
        assert piped, "the table has row-pipelined rules"
        for H, R, k, epi, lo, hi, v in piped:
            H, R, k, lo = int(H), int(R), int(k), max(int(lo), 1)
            assert frn.launch_pipelined(R, k, lo, H, epis[epi])
            assert frn.launch_shape(R, k, lo, H, epis[epi])[1] == int(v[1])
    finally:
        frn.set_launch_table(None)


