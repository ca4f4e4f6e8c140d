"""GPU parity of the expert-parallel finalize (per-rank routing: each rank
owns a share of the experts, a negative row index marks another rank's slot)
against the CPU oracle, through the C ABI (via the Python binding).

Moderate sizes run whole batches through the oracle, through the split-row
finalize (where the built-in rule takes it, and at every T <= 256 when a
launch table forces it) and the one-row kernel; the full-size
workload (H=6144, top-10 of 256 experts over 8 ranks, T=4096) runs in the
launch configuration the benchmark times and the oracle recomputes sampled
rows.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import parity

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def frn():
    import tp_reduction_rmsnorm_amd as m
    return m


def log(msg):
    print(msg, flush=True)


def dev(inp):
    mv = lambda t: None if t is None else t.to(DEV)
    ml = lambda ts: None if ts is None else [mv(t) for t in ts]
    out = workloads.Inputs(R=inp.R, T=inp.T, H=inp.H, epilogue=inp.epilogue,
                           residual=mv(inp.residual), gamma1=mv(inp.gamma1),
                           gamma2=mv(inp.gamma2), eps=inp.eps, k=inp.k,
                           expert_rows=ml(inp.expert_rows), shared=ml(inp.shared),
                           topk_w=mv(inp.topk_w), topk_idx=mv(inp.topk_idx))
    out.ep_rows = ml(inp.ep_rows)
    return out


def epi(inp, m):
    return m.EPI_SANDWICH if inp.epilogue == "sandwich" else m.EPI_RMSNORM


def oracle_ep(inp, debug=False):
    return oracle.ep_boundary(
        [workloads.bits(e) for e in inp.expert_rows], topk_w=workloads.f32(inp.topk_w),
        topk_rows=[r.cpu().numpy() for r in inp.ep_rows], residual=workloads.bits(inp.residual),
        gamma1=workloads.f32(inp.gamma1),
        gamma2=workloads.f32(inp.gamma2) if inp.gamma2 is not None else None, eps=inp.eps,
        epilogue=oracle.EPI_SANDWICH if inp.epilogue == "sandwich" else oracle.EPI_RMSNORM,
        shared=None if inp.shared is None else
        [None if s is None else workloads.bits(s) for s in inp.shared],
        num_rows=[e.shape[0] for e in inp.expert_rows], H=inp.H, debug=debug, nthreads=8)


def gpu_ep(d, **kw):
    m = frn()
    return m.ep_moe_finalize_reduce_norm(d.expert_rows, d.topk_w, d.ep_rows, d.residual,
                                         d.gamma1, d.gamma2, d.eps, shared=d.shared,
                                         epilogue=epi(d, m), **kw)


def same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


# (R, T, H, epilogue, k, experts, shared_rank)
CASES = [
    (8, 8, 6144, "rmsnorm", 10, 256, 0),      # the workload at decode sizes
    (8, 64, 6144, "rmsnorm", 10, 256, 0),
    (8, 300, 6144, "rmsnorm", 10, 256, 0),    # above the split-row range
    (8, 33, 6144, "sandwich", 10, 256, 3),
    (4, 37, 5128, "sandwich", 4, 16, 2),      # ragged: 641 vectors
    (2, 5, 520, "rmsnorm", 8, 8, None),       # few experts: ranks own many slots, no shared
    (16, 6, 2048, "sandwich", 16, 64, 15),    # maximum R and k
    (3, 1100, 1032, "rmsnorm", 6, 12, 1),     # T > 1024, ragged
    (2, 3, 16384, "rmsnorm", 3, 4, 0),        # maximum H
    (1, 9, 4096, "rmsnorm", 5, 32, 0),        # one rank owns every expert
]


def cid(c):
    R, T, H, e, k, E, s = c
    return f"R{R}_T{T}_H{H}_{e}_k{k}_of{E}_shared{s}"


@pytest.mark.parametrize("case", CASES, ids=[cid(c) for c in CASES])
@pytest.mark.parametrize("workspace", ["auto", None, "forced-split"])
def test_ep_fused_matches_oracle(case, workspace):
    """"auto": the built-in choice; None: the one-row kernel; "forced-split":
    a launch table routes every T <= 256 to the split-row finalize."""
    R, T, H, e, k, E, s = case
    m = frn()
    log(f"ep fused {cid(case)} workspace={workspace}")
    inp = workloads.make_ep(R, T, H, k=k, experts=E, epilogue=e, shared_rank=s,
                            seed=5000 + R * 7 + T * 13 + H)
    d = dev(inp)
    if workspace == "forced-split":
        try:
            m.set_launch_table("* * * * 0 * split\n")
            assert m.split_rows(R, k, T, H, epi(d, m), ep=True) == (T <= 256)
            y, x = gpu_ep(d, workspace="auto")
        finally:
            m.set_launch_table(None)
    else:
        y, x = gpu_ep(d, workspace=workspace)
    torch.cuda.synchronize()
    ref = oracle_ep(inp)
    parity.compare(f"ep {cid(case)} ws={workspace} out", workloads.bits(y), ref.y)
    parity.compare(f"ep {cid(case)} ws={workspace} residual_out", workloads.bits(x), ref.xout)


@pytest.mark.parametrize("side", [0, 1])
def test_ep_at_the_split_row_edge(side):
    """Either side of the split-row edge the library applies to the
    expert-parallel workload (R=8, H=6144, k=10; read from the library, as a
    re-tune may move it): automatic workspace, one-row kernel and oracle
    agree bit for bit."""
    m = frn()
    edge = max(t for t in range(1, 257) if m.split_rows(8, 10, t, 6144, ep=True))
    T = edge + side
    assert m.split_rows(8, 10, T, 6144, ep=True) == (side == 0)
    log(f"ep split-row edge {edge}: T={T}")
    inp = workloads.make_ep(8, T, 6144, k=10, experts=256, shared_rank=0, seed=6400 + T)
    d = dev(inp)
    y, x = gpu_ep(d)
    y2, x2 = gpu_ep(d, workspace=None)
    torch.cuda.synchronize()
    assert same(y, y2) and same(x, x2)
    ref = oracle_ep(inp)
    parity.compare(f"ep edge T={T} out", workloads.bits(y), ref.y)
    parity.compare(f"ep edge T={T} residual_out", workloads.bits(x), ref.xout)


@pytest.mark.parametrize("case", CASES[:2] + CASES[4:7], ids=[cid(c) for c in CASES[:2] + CASES[4:7]])
def test_ep_standalone_finalize_matches_oracle(case):
    R, T, H, e, k, E, s = case
    log(f"ep standalone finalize {cid(case)}")
    inp = workloads.make_ep(R, T, H, k=k, experts=E, epilogue=e, shared_rank=s, seed=6000 + T)
    d = dev(inp)
    parts = frn().ep_moe_finalize(d.expert_rows, d.topk_w, d.ep_rows, H=H, shared=d.shared)
    torch.cuda.synchronize()
    ref = oracle_ep(inp, debug=True)
    for r in range(R):
        parity.compare(f"ep finalize {cid(case)} rank {r}", workloads.bits(parts[r]), ref.p[r],
                       min_exact=1.0)


def test_ep_fused_equals_materialized_and_one_rank_equals_tp():
    m = frn()
    for T in (24, 300):
        inp = dev(workloads.make_ep(8, T, 6144, k=10, experts=256, shared_rank=0, seed=77 + T))
        y, x = gpu_ep(inp)
        parts = m.ep_moe_finalize(inp.expert_rows, inp.topk_w, inp.ep_rows, H=6144,
                                  shared=inp.shared)
        y2, x2 = m.reduce_residual_rmsnorm(parts, inp.residual, inp.gamma1, inp.eps)
        torch.cuda.synchronize()
        assert same(y, y2) and same(x, x2), T
    # one rank owning every slot: the TP finalize call, bit for bit
    for T in (24, 300):
        inp = dev(workloads.make(1, T, 6144, k=10, shared=True, seed=88 + T))
        y, x = m.moe_finalize_reduce_norm(inp.expert_rows, inp.topk_w, inp.topk_idx,
                                          inp.residual, inp.gamma1, shared=inp.shared)
        y2, x2 = m.ep_moe_finalize_reduce_norm(inp.expert_rows, inp.topk_w, [inp.topk_idx],
                                               inp.residual, inp.gamma1, shared=inp.shared)
        torch.cuda.synchronize()
        assert same(y, y2) and same(x, x2), T


def test_ep_rank_without_rows_and_index_past_buffer():
    """A rank with no rows at all (no buffer) contributes +0; an index at or
    past a rank's row count reads as NaN for that token only, with no memory
    access."""
    m = frn()
    inp = workloads.make_ep(3, 6, 256, k=4, experts=12, shared_rank=0, seed=91)
    # rank 2 loses its buffer; its slots now belong to no rank
    inp.ep_rows[2][:] = -1
    inp.expert_rows[2] = torch.empty((0, 256), dtype=torch.bfloat16)
    ref = oracle_ep(inp)
    d = dev(inp)
    d.expert_rows[2] = None
    y, x = gpu_ep(d, workspace=None)
    torch.cuda.synchronize()
    parity.compare("ep rank without rows out", workloads.bits(y), ref.y, min_exact=1.0)
    parity.compare("ep rank without rows residual_out", workloads.bits(x), ref.xout,
                   min_exact=1.0)
    bad = [r.clone() for r in d.ep_rows]
    t_bad = 3
    j = int(torch.nonzero(bad[0][t_bad] < 0)[0])
    for r in bad:
        r[t_bad, j] = -1
    bad[1][t_bad, j] = d.expert_rows[1].shape[0]   # one past rank 1's buffer
    for ws in ("auto", None):
        y, x = m.ep_moe_finalize_reduce_norm(d.expert_rows, d.topk_w, bad, d.residual,
                                             d.gamma1, shared=d.shared, workspace=ws)
        torch.cuda.synchronize()
        yf = y.float().cpu()
        assert torch.isnan(yf[t_bad]).all(), ws
        keep = [t for t in range(6) if t != t_bad]
        assert torch.isfinite(yf[keep]).all(), ws


def _sub_ep(d, rows):
    """Host copy of the sampled token rows: each rank's buffer keeps only
    the rows those tokens use, with the indices renumbered."""
    ri = torch.as_tensor(rows, device=DEV)
    cpu = lambda t: t.index_select(0, ri).cpu()
    sub = workloads.Inputs(R=d.R, T=len(rows), H=d.H, epilogue=d.epilogue,
                           residual=cpu(d.residual), gamma1=d.gamma1.cpu(),
                           gamma2=d.gamma2.cpu() if d.gamma2 is not None else None,
                           eps=d.eps, k=d.k, topk_w=cpu(d.topk_w))
    sub.expert_rows, sub.ep_rows = [], []
    for r in range(d.R):
        idx = d.ep_rows[r].index_select(0, ri).cpu()           # [S,k]
        own = idx >= 0
        new = torch.full_like(idx, -1)
        new[own] = torch.arange(int(own.sum()), dtype=torch.int32)
        src = d.expert_rows[r]
        used = idx[own].long().to(DEV)
        sub.expert_rows.append(src.index_select(0, used).cpu() if used.numel() else
                               torch.empty((0, d.H), dtype=torch.bfloat16))
        sub.ep_rows.append(new)
    sub.shared = None if d.shared is None else [None if s is None else cpu(s) for s in d.shared]
    return sub


@pytest.mark.parametrize("T", [64, 1024, 4096, 16384])
def test_ep_full_size_sampled_rows(T):
    log(f"ep full size T={T}")
    d = workloads.make_workload(6, T, device=DEV)
    y, x = gpu_ep(d)
    torch.cuda.synchronize()
    g = np.random.default_rng(T)
    rows = np.array(sorted(set(range(min(8, T))) | set(range(max(0, T - 8), T)) |
                           set(int(r) for r in g.choice(T, size=min(48, T), replace=False))))
    ri = torch.as_tensor(rows, device=DEV)
    ref = oracle_ep(_sub_ep(d, rows))
    parity.compare(f"ep full T={T} out (rows sampled)", workloads.bits(y.index_select(0, ri)),
                   ref.y)
    parity.compare(f"ep full T={T} residual_out (rows sampled)",
                   workloads.bits(x.index_select(0, ri)), ref.xout)
    assert torch.isfinite(y.float()).all() and torch.isfinite(x.float()).all()


@pytest.mark.parametrize("T,workspace", [(24, "auto"), (300, None)])
def test_ep_graph_capture_and_replay_with_new_data(T, workspace):
    """Capture the expert-parallel call in a HIP graph and replay it with new
    row values, weights, shared rows and residual copied in between (the
    routing keeps its shape), checking every replay against the oracle."""
    m = frn()
    log(f"ep graph T={T} workspace={workspace}")
    assert m.split_rows(8, 6, T, 2048, m.EPI_SANDWICH, ep=True) == (workspace == "auto")
    host = workloads.make_ep(8, T, 2048, k=6, experts=32, epilogue="sandwich", shared_rank=2,
                             seed=321 + T)
    d = dev(host)
    out = torch.empty(T, 2048, dtype=torch.bfloat16, device=DEV)
    rout = torch.empty(T, 2048, dtype=torch.bfloat16, device=DEV)

    def call():
        m.ep_moe_finalize_reduce_norm(d.expert_rows, d.topk_w, d.ep_rows, d.residual, d.gamma1,
                                      d.gamma2, d.eps, shared=d.shared, epilogue=m.EPI_SANDWICH,
                                      out=out, residual_out=rout, workspace=workspace)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    gen = torch.Generator().manual_seed(999 + T)
    rnd = lambda t: torch.randn(t.shape, generator=gen).to(t.dtype)
    for rep in range(4):
        for r in range(8):
            if host.expert_rows[r].numel():
                host.expert_rows[r] = rnd(host.expert_rows[r])
                d.expert_rows[r].copy_(host.expert_rows[r].to(DEV))
        host.shared[2] = rnd(host.shared[2])
        d.shared[2].copy_(host.shared[2].to(DEV))
        host.topk_w = torch.softmax(torch.randn(host.topk_w.shape, generator=gen), -1)
        d.topk_w.copy_(host.topk_w.to(DEV))
        host.residual = rnd(host.residual)
        d.residual.copy_(host.residual.to(DEV))
        torch.sum(d.residual.float()).item()   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = oracle_ep(host)
        parity.compare(f"ep graph T={T} replay {rep} out", workloads.bits(out), ref.y)
        parity.compare(f"ep graph T={T} replay {rep} residual_out", workloads.bits(rout), ref.xout)


@pytest.mark.parametrize("vec", [1, 2])
def test_ep_results_do_not_depend_on_launch_shape(vec):
    """The expert-parallel kernel forced to one or two vectors per lane
    through a launch table gives the same bits."""
    m = frn()
    inp = workloads.make_ep(4, 300, 2056, k=5, experts=16, epilogue="sandwich", shared_rank=3,
                            seed=4242)
    d = dev(inp)
    try:
        m.set_launch_table(f"* * * ep-* 0 * {vec}\n")
        assert m.launch_shape(4, 5, 300, 2056, m.EPI_SANDWICH, ep=True)[1] == vec
        y, x = gpu_ep(d, workspace=None)
        torch.cuda.synchronize()
    finally:
        m.set_launch_table(None)
    ref = oracle_ep(inp)
    parity.compare(f"ep vec={vec} out", workloads.bits(y), ref.y, min_exact=1.0)
    parity.compare(f"ep vec={vec} residual_out", workloads.bits(x), ref.xout, min_exact=1.0)
