"""GPU parity of the row-pipelined kernel against the CPU oracle.

The row-pipelined kernel launches one workgroup per compute unit.  Each
workgroup walks the rows b, b + G, b + 2G, ..., holds the gamma rows in
LDS, and loads the next row while the current row runs its epilogue.  The
built-in rule takes it at T >= 1536.  Here launch-table rules (p1 / p2)
force it at sizes the oracle finishes in seconds, with T chosen so that
workgroups take different numbers of rows, and T below the CU count.  The
full-size sandwich workload (H=5120 R=4 T=4096), which takes it by the
built-in rule, is covered by the sampled-row test in test_gpu_parity.py and
compared here against the one-row kernel, bit for bit, on every row.
"""
import pytest
import torch

import workloads
from tests.test_gpu_parity import DEV, check, gpu_fused, log, oracle_ref, to_dev

pytestmark = pytest.mark.gpu


def frn():
    import tp_reduction_rmsnorm_amd as m
    return m


def epi_code(m, epi):
    return m.EPI_SANDWICH if epi == "sandwich" else m.EPI_RMSNORM


# (R, T, H, epilogue, vectors per lane)
PIPE_CASES = [
    (4, 600, 5120, "sandwich", 2),   # the sandwich workload's rows, 2-3 rows per workgroup
    (4, 257, 5120, "sandwich", 1),   # one workgroup takes two rows, the rest one
    (1, 300, 7168, "rmsnorm", 2),    # split pass 2's rows
    (2, 513, 1024, "rmsnorm", 1),
    (3, 300, 4096, "sandwich", 2),   # R = 3
    (4, 5, 8192, "sandwich", 2),     # T below the CU count; gamma rows fill 64 KiB of LDS
    (2, 1, 512, "rmsnorm", 1),       # one row of one wave
    (1, 1600, 512, "sandwich", 1),   # six or seven rows per workgroup
    (2, 700, 1024, "sandwich", 2),   # 64 lanes, two vectors each
    (4, 256, 6144, "rmsnorm", 2),    # T equal to the CU count: one row per workgroup, R = 4
    (3, 1537, 6144, "sandwich", 1),  # the built-in rule's first T, one vector per lane
]


def case_id(c):
    R, T, H, epi, v = c
    return f"R{R}_T{T}_H{H}_{epi}_p{v}"


@pytest.mark.parametrize("case", PIPE_CASES, ids=[case_id(c) for c in PIPE_CASES])
def test_pipelined_matches_oracle(case):
    R, T, H, epi, v = case
    m = frn()
    try:
        m.set_launch_table(f"{H} {R} 0 {epi} 0 * p{v}")
        assert m.launch_pipelined(R, 0, T, H, epi_code(m, epi))
        assert m.launch_shape(R, 0, T, H, epi_code(m, epi)) == (H // 8 // v, v)
        log(f"pipelined {case_id(case)}")
        inp = workloads.make(R, T, H, epilogue=epi, sigma=0.5, seed=5000 + R * 7 + T * 13 + H)
        y, x = gpu_fused(to_dev(inp))
        check(f"pipelined {case_id(case)}", y, x, oracle_ref(inp))
    finally:
        m.set_launch_table(None)


def test_pipelined_in_place_residual():
    m = frn()
    try:
        m.set_launch_table("5120 4 0 sandwich 0 * p2")
        inp = workloads.make(4, 700, 5120, epilogue="sandwich", sigma=0.5, seed=5101)
        ref = oracle_ref(inp)
        d = to_dev(inp)
        y, x = gpu_fused(d, residual_out=d.residual)
        torch.cuda.synchronize()
        assert x.data_ptr() == d.residual.data_ptr()
        check("pipelined in-place residual", y, x, ref)
    finally:
        m.set_launch_table(None)


@pytest.mark.parametrize("cid", [2, 3])
def test_pipelined_equals_one_row_kernel_at_full_size(cid):
    """The full-size sandwich workloads at T=4096, every row: the built-in
    choice against the one-row kernel forced by a numeric rule, bit for bit
    (H=5120 R=4 takes the row-pipelined kernel, H=8192 R=8 does not)."""
    m = frn()
    w = workloads.WORKLOADS[cid]
    d = workloads.make_workload(cid, 4096, device=DEV)
    pipelined = m.launch_pipelined(w.R, 0, 4096, w.H, m.EPI_SANDWICH)
    log(f"full size w{cid}: built-in takes the row-pipelined kernel: {pipelined}")
    assert pipelined == (cid == 2)
    y0, x0 = gpu_fused(d)
    try:
        m.set_launch_table("* * 0 * 0 * 2")
        assert not m.launch_pipelined(w.R, 0, 4096, w.H, m.EPI_SANDWICH)
        y1, x1 = gpu_fused(d)
    finally:
        m.set_launch_table(None)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    assert torch.equal(x0.view(torch.int16), x1.view(torch.int16))


def test_pipelined_graph_replay():
    """Captured calls of the row-pipelined kernel replayed several times,
    with eager work in between, match the eager results every time."""
    m = frn()
    sets = [to_dev(workloads.make(4, 1600 + 37 * i, 5120, epilogue="sandwich", sigma=0.5,
                                  seed=5200 + i)) for i in range(3)]
    for s in sets:
        assert m.launch_pipelined(4, 0, s.T, 5120, m.EPI_SANDWICH)
    eager = [gpu_fused(s) for s in sets]
    outs = [(torch.empty_like(e[0]), torch.empty_like(e[1])) for e in eager]
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for s, (o, r) in zip(sets, outs):
            gpu_fused(s, out=o, residual_out=r)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s, (o, r) in zip(sets, outs):
            gpu_fused(s, out=o, residual_out=r)
    for rep in range(3):
        for o, r in outs:
            o.zero_()
            r.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (ey, ex), (o, r) in zip(eager, outs):
            assert torch.equal(ey.view(torch.int16), o.view(torch.int16)), f"replay {rep}"
            assert torch.equal(ex.view(torch.int16), r.view(torch.int16)), f"replay {rep}"
        gpu_fused(sets[0])  # eager work between replays
    del g


def test_pipelined_calls_on_two_streams_at_once():
    """Row-pipelined calls queued on two streams together (each launch has its
    own LDS and no state outside its arguments) match the oracle."""
    m = frn()
    try:
        m.set_launch_table("5120 4 0 sandwich 0 * p2\n5120 2 0 rmsnorm 0 * p1")
        cases = [workloads.make(4, 600, 5120, epilogue="sandwich", sigma=0.5, seed=5301),
                 workloads.make(2, 777, 5120, epilogue="rmsnorm", sigma=0.5, seed=5302)]
        devs = [to_dev(c) for c in cases]
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        outs = []
        for d, s in zip(devs, streams):
            with torch.cuda.stream(s):
                for _ in range(3):          # several launches in flight on each stream
                    y, x = gpu_fused(d)
                outs.append((y, x))
        for s in streams:
            torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for c, (y, x) in zip(cases, outs):
            check(f"two streams R{c.R} T{c.T} {c.epilogue}", y, x, oracle_ref(c))
    finally:
        m.set_launch_table(None)
