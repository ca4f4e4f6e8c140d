"""GPU test of frn_moe_finalize_reduce_norm_noalloc, called through the C ABI
(via the binding): the MoE finalize + reduce + norm call whose split-row
scratch is the library's own device array instead of a caller workspace.

Two calls in a row, the second with a smaller input, both taking the
split-row finalize (so both use the array, and the second runs on what the
first left there): each output equals, bit for bit, that of the workspace
entry point frn_moe_finalize_reduce_norm on the same inputs, and both equal
the oracle.  A call above the split-row range (no scratch used), the
largest split-row call at the largest H (R=16, H=16384), and the call
captured in a HIP graph and replayed with new data are checked too.
"""
import pytest
import torch

import workloads
from tests import parity
from tests.test_gpu_parity import DEV, frn, log, oracle_ref, to_dev

pytestmark = pytest.mark.gpu


def _epi(m, d):
    return m.EPI_SANDWICH if d.epilogue == "sandwich" else m.EPI_RMSNORM


def _noalloc(d):
    m = frn()
    out = torch.full((d.T, d.H), 7.0, dtype=torch.bfloat16, device=DEV)
    rout = torch.full((d.T, d.H), 7.0, dtype=torch.bfloat16, device=DEV)
    m.moe_finalize_reduce_norm_noalloc(d.expert_rows, d.topk_w, d.topk_idx, d.residual,
                                       d.gamma1, d.gamma2, d.eps, out=out, residual_out=rout,
                                       shared=d.shared, epilogue=_epi(m, d))
    return out, rout


def _with_workspace(d):
    m = frn()
    ws = torch.empty(m.workspace_bytes(d.T, d.H, d.R, d.k), dtype=torch.uint8, device=DEV)
    return m.moe_finalize_reduce_norm(d.expert_rows, d.topk_w, d.topk_idx, d.residual,
                                      d.gamma1, d.gamma2, d.eps, shared=d.shared,
                                      epilogue=_epi(m, d), workspace=ws)


def _same(name, got, want):
    torch.cuda.synchronize()
    parity.compare(name, workloads.bits(got), workloads.bits(want), min_exact=1.0)


# (R, T, H, k, epilogue): the MoE finalize workload at T=64, then the same
# shape at T=8; a sandwich pair at another shape; each pair large then small.
PAIRS = [
    ((8, 64, 6144, 10, "rmsnorm"), (8, 8, 6144, 10, "rmsnorm")),
    ((4, 40, 2048, 3, "sandwich"), (4, 5, 2048, 3, "sandwich")),
]


@pytest.mark.parametrize("pair", PAIRS, ids=["moe_h6144_r8_k10", "sandwich_h2048_r4_k3"])
def test_noalloc_matches_workspace_call_twice(pair):
    m = frn()
    for i, (R, T, H, k, epi) in enumerate(pair):
        assert m.split_rows(R, k, T, H, m.EPI_SANDWICH if epi == "sandwich" else m.EPI_RMSNORM)
        assert m.workspace_bytes(T, H, R, k) <= m.NOALLOC_SCRATCH_BYTES
        log(f"noalloc call {i}: R={R} T={T} H={H} k={k} {epi}")
        inp = workloads.make(R, T, H, k=k, shared=True, epilogue=epi, seed=900 + 10 * i + R)
        d = to_dev(inp)
        y, x = _noalloc(d)
        yw, xw = _with_workspace(d)
        _same(f"noalloc call {i} T={T} out vs workspace call", y, yw)
        _same(f"noalloc call {i} T={T} residual_out vs workspace call", x, xw)
        ref = oracle_ref(inp)
        parity.compare(f"noalloc call {i} T={T} out vs oracle", workloads.bits(y), ref.y)
        parity.compare(f"noalloc call {i} T={T} residual_out vs oracle", workloads.bits(x),
                       ref.xout)


def test_noalloc_without_split_rows_and_at_the_largest_h():
    m = frn()
    # above the split-row range: the one-row kernel, no scratch
    R, T, H, k = 2, 300, 520, 2
    assert not m.split_rows(R, k, T, H)
    inp = workloads.make(R, T, H, k=k, shared=True, seed=977)
    d = to_dev(inp)
    log(f"noalloc call without scratch: R={R} T={T} H={H} k={k}")
    y, x = _noalloc(d)
    yw, xw = _with_workspace(d)
    _same("noalloc one-row out vs workspace call", y, yw)
    _same("noalloc one-row residual_out vs workspace call", x, xw)
    # sixteen ranks at H=16384: the split-row finalize's workspace (FP32 rows
    # and FP64 slice sums) does not grow with R
    R, T, H, k = 16, 64, 16384, 2
    assert m.split_rows(R, k, T, H) and m.workspace_bytes(T, H, R, k) <= m.NOALLOC_SCRATCH_BYTES
    inp = workloads.make(R, T, H, k=k, shared=True, seed=979)
    d = to_dev(inp)
    log(f"noalloc call at the largest H: R={R} T={T} H={H} k={k}")
    y, x = _noalloc(d)
    yw, xw = _with_workspace(d)
    _same("noalloc R=16 H=16384 out vs workspace call", y, yw)
    _same("noalloc R=16 H=16384 residual_out vs workspace call", x, xw)
    ref = oracle_ref(inp)
    parity.compare("noalloc R=16 H=16384 out vs oracle", workloads.bits(y), ref.y)
    parity.compare("noalloc R=16 H=16384 residual_out vs oracle", workloads.bits(x), ref.xout)


def test_noalloc_under_graph_capture():
    """The callers this entry point is for: a HIP graph captures it (after
    one eager call on the device, which looks up the array's address) and is
    replayed four times with new data copied into the captured inputs and
    eager work between the replays; every replay matches the oracle, and
    the workspace entry point bit for bit."""
    m = frn()
    R, T, H, k = 8, 16, 6144, 10
    assert m.split_rows(R, k, T, H)
    base = to_dev(workloads.make(R, T, H, k=k, shared=True, seed=1200))
    out = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    rout = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)

    def call():
        m.moe_finalize_reduce_norm_noalloc(base.expert_rows, base.topk_w, base.topk_idx,
                                           base.residual, base.gamma1, None, base.eps,
                                           out=out, residual_out=rout, shared=base.shared)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    log("noalloc graph capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        new = workloads.make(R, T, H, k=k, shared=True, seed=1300 + rep)
        for dst, src in zip(base.expert_rows + base.shared, new.expert_rows + new.shared):
            dst.copy_(src.to(DEV))
        base.topk_w.copy_(new.topk_w.to(DEV))
        base.topk_idx.copy_(new.topk_idx.to(DEV))
        base.residual.copy_(new.residual.to(DEV))
        base.gamma1.copy_(new.gamma1.to(DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = oracle_ref(new)
        parity.compare(f"noalloc graph replay {rep} out", workloads.bits(out), ref.y)
        parity.compare(f"noalloc graph replay {rep} residual_out", workloads.bits(rout),
                       ref.xout)
        yw, xw = _with_workspace(to_dev(new))
        _same(f"noalloc graph replay {rep} out vs workspace call", out, yw)
        _same(f"noalloc graph replay {rep} residual_out vs workspace call", rout, xw)
