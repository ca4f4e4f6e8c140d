"""GPU parity: the HIP library, called through its C ABI (via the Python
binding), against the CPU oracle, element by element.

Moderate sizes run the whole batch through the oracle; they span many
workgroups, partially filled waves (ragged H) and odd T.  The full-size
workloads (sandwich H=5120 R=4 and H=8192 R=8 at T=4096; MoE finalize
H=7168 R=2 k=8 at T=16384, fused and split) run on the GPU in the launch
configuration the benchmark times, and the oracle recomputes a sample of
rows (rows are independent, so a row's result does not depend on the
others).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import parity
from tests import pin_battery as B

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def frn():
    import tp_reduction_rmsnorm_amd as m
    return m


def log(msg):
    print(msg, flush=True)


def to_dev(inp: workloads.Inputs) -> workloads.Inputs:
    mv = lambda t: None if t is None else t.to(DEV)
    ml = lambda ts: None if ts is None else [t.to(DEV) for t in ts]
    return workloads.Inputs(R=inp.R, T=inp.T, H=inp.H, epilogue=inp.epilogue,
                            residual=mv(inp.residual), gamma1=mv(inp.gamma1),
                            gamma2=mv(inp.gamma2), eps=inp.eps, partials=ml(inp.partials),
                            expert_rows=ml(inp.expert_rows), shared=ml(inp.shared),
                            topk_w=mv(inp.topk_w), topk_idx=mv(inp.topk_idx), k=inp.k)


def epi_code(inp):
    return oracle.EPI_SANDWICH if inp.epilogue == "sandwich" else oracle.EPI_RMSNORM


def oracle_ref(inp, split=False, epilogue=None):
    kw = dict(residual=workloads.bits(inp.residual), gamma1=workloads.f32(inp.gamma1),
              gamma2=workloads.f32(inp.gamma2) if inp.gamma2 is not None else None,
              eps=inp.eps, epilogue=epi_code(inp) if epilogue is None else epilogue,
              split=split, nthreads=8)
    if inp.k:
        kw.update(topk_w=workloads.f32(inp.topk_w),
                  topk_idx=inp.topk_idx.cpu().numpy().astype(np.int32),
                  shared=[workloads.bits(s) for s in inp.shared] if inp.shared else None)
    return oracle.boundary([workloads.bits(s) for s in inp.sources], **kw)


def gpu_fused(d, **kw):
    m = frn()
    if d.k:
        return m.moe_finalize_reduce_norm(
            d.expert_rows, d.topk_w, d.topk_idx, d.residual, d.gamma1, d.gamma2, d.eps,
            shared=d.shared,
            epilogue=m.EPI_SANDWICH if d.epilogue == "sandwich" else m.EPI_RMSNORM, **kw)
    if d.epilogue == "sandwich":
        return m.reduce_sandwich_norm(d.partials, d.residual, d.gamma1, d.gamma2, d.eps, **kw)
    return m.reduce_residual_rmsnorm(d.partials, d.residual, d.gamma1, d.eps, **kw)


def gpu_split(d):
    m = frn()
    return m.split_reduce_norm(
        d.sources, d.residual, d.gamma1, d.gamma2, d.eps,
        topk_weights=d.topk_w if d.k else None, topk_rows=d.topk_idx if d.k else None,
        shared=d.shared if d.k else None,
        epilogue=m.EPI_SANDWICH if d.epilogue == "sandwich" else m.EPI_RMSNORM)


def check(name, y, x, ref):
    torch.cuda.synchronize()
    parity.compare(f"{name} out", workloads.bits(y), ref.y)
    parity.compare(f"{name} residual_out", workloads.bits(x), ref.xout)


# (R, T, H, epilogue, k, shared): the five workloads at sizes the oracle
# finishes in seconds, plus ragged shapes (H not a multiple of the lanes of
# a row; T odd) and the extremes of the supported range.
MODERATE = [
    (2, 8, 512, "rmsnorm", 0, False),        # tiny workload, full size
    (4, 64, 5120, "sandwich", 0, False),     # sandwich H=5120 R=4
    (4, 37, 5120, "rmsnorm", 0, False),
    (8, 16, 8192, "sandwich", 0, False),     # sandwich H=8192 R=8
    (8, 8, 6144, "rmsnorm", 10, True),       # MoE finalize workload
    (8, 64, 6144, "rmsnorm", 10, True),
    (2, 32, 7168, "rmsnorm", 8, True),       # split workload's shapes, fused
    (2, 9, 7168, "sandwich", 8, True),
    (3, 5, 5128, "sandwich", 0, False),      # ragged: 641 vectors
    (2, 7, 520, "rmsnorm", 0, False),        # ragged: 65 vectors
    (5, 3, 8, "rmsnorm", 0, False),          # minimum H
    (16, 3, 16384, "sandwich", 0, False),    # maximum R and H
    (1, 9, 4096, "rmsnorm", 0, False),       # R = 1
    (3, 4, 2056, "sandwich", 16, True),      # maximum k, ragged
    (4, 6, 1024, "rmsnorm", 1, False),       # k = 1, no shared expert
    (3, 5, 16384, "rmsnorm", 3, True),       # finalize at maximum H (2 vectors/lane)
    (9, 3, 1536, "sandwich", 0, False),      # R not a power of two, > 8
    (3, 1100, 5128, "sandwich", 0, False),   # T > 1024: two vectors per lane, ragged
    (4, 150, 520, "rmsnorm", 2, False),      # finalize, split-row, ragged, no shared
    (2, 300, 520, "sandwich", 2, True),      # finalize above the split-row range
]


def mid_id(c):
    R, T, H, epi, k, sh = c
    return f"R{R}_T{T}_H{H}_{epi}" + (f"_k{k}" if k else "") + ("_shared" if sh else "")


@pytest.mark.parametrize("case", MODERATE, ids=[mid_id(c) for c in MODERATE])
def test_fused_matches_oracle(case):
    R, T, H, epi, k, sh = case
    log(f"fused {mid_id(case)}")
    inp = workloads.make(R, T, H, epilogue=epi, sigma=0.5, k=k, shared=sh,
                         seed=1000 + R * 7 + T * 13 + H)
    y, x = gpu_fused(to_dev(inp))
    check(f"fused {mid_id(case)}", y, x, oracle_ref(inp))


@pytest.mark.parametrize("case", [c for c in MODERATE if c[2] >= 512 and c[1] > 3],
                         ids=[mid_id(c) for c in MODERATE if c[2] >= 512 and c[1] > 3])
def test_split_matches_oracle(case):
    R, T, H, epi, k, sh = case
    log(f"split {mid_id(case)}")
    inp = workloads.make(R, T, H, epilogue=epi, sigma=0.5, k=k, shared=sh,
                         seed=2000 + R * 7 + T * 13 + H)
    d = to_dev(inp)
    y, x = gpu_split(d)
    ref = oracle_ref(inp, split=True)
    check(f"split {mid_id(case)}", y, x, ref)
    # pass 1 alone
    m = frn()
    if k:
        u = m.moe_finalize_reduce_bf16(d.expert_rows, d.topk_w, d.topk_idx, shared=d.shared)
    else:
        u = m.reduce_bf16(d.partials)
    torch.cuda.synchronize()
    u_ref = oracle_ref(inp, epilogue=oracle.EPI_NONE).u
    parity.compare(f"pass1 {mid_id(case)}", workloads.bits(u), u_ref)


def test_boundary_threshold_picks_fused_or_split():
    """frn.boundary: at or below max_fused_tokens the fused result, above it
    the split path's (each against its own oracle path)."""
    m = frn()
    for k in (0, 4):
        inp = workloads.make(2, 40, 1024, epilogue="rmsnorm", k=k, shared=bool(k), seed=70 + k)
        d = to_dev(inp)
        kw = dict(topk_weights=d.topk_w, topk_rows=d.topk_idx, shared=d.shared) if k else {}
        y, x = m.boundary(d.sources, d.residual, d.gamma1, None, d.eps, max_fused_tokens=40, **kw)
        check(f"boundary k={k} fused", y, x, oracle_ref(inp))
        y, x = m.boundary(d.sources, d.residual, d.gamma1, None, d.eps, max_fused_tokens=39, **kw)
        check(f"boundary k={k} split", y, x, oracle_ref(inp, split=True))


# ------------------------------------------------------ full sizes --- #

def sample_rows(T, n=48, seed=0):
    g = np.random.default_rng(seed)
    rows = set(range(min(8, T))) | set(range(max(0, T - 8), T))
    rows |= set(int(r) for r in g.choice(T, size=min(n, T), replace=False))
    return np.array(sorted(rows))


def sub_inputs(d: workloads.Inputs, rows: np.ndarray) -> workloads.Inputs:
    """Host copy of the sampled token rows (with the expert rows they use)."""
    ri = torch.as_tensor(rows, device=DEV)
    cpu = lambda t: t.index_select(0, ri).cpu()
    sub = workloads.Inputs(R=d.R, T=len(rows), H=d.H, epilogue=d.epilogue,
                           residual=cpu(d.residual), gamma1=d.gamma1.cpu(),
                           gamma2=d.gamma2.cpu() if d.gamma2 is not None else None,
                           eps=d.eps, k=d.k)
    if d.k:
        idx = d.topk_idx.index_select(0, ri)                    # [S,k]
        flat = idx.reshape(-1).long()
        sub.expert_rows = [e.index_select(0, flat).cpu() for e in d.expert_rows]
        sub.topk_idx = torch.arange(flat.numel(), dtype=torch.int32).reshape(idx.shape)
        sub.topk_w = cpu(d.topk_w)
        sub.shared = [cpu(s) for s in d.shared] if d.shared else None
    else:
        sub.partials = [cpu(p) for p in d.partials]
    return sub


# the workloads' largest bench sizes, plus T=16384 for both sandwich
# workloads (the measured table's last ranges: the row-pipelined kernel with
# two vectors per lane at H=5120, one vector per lane at H=8192)
FULL = [(2, 4096, False), (3, 4096, False), (5, 16384, False), (5, 16384, True),
        (4, 64, False), (2, 16384, False), (3, 16384, False)]


@pytest.mark.parametrize("cid,T,split", FULL,
                         ids=[f"{workloads.WORKLOADS[c].name}_T{T}{'_split' if s else ''}"
                              for c, T, s in FULL])
def test_full_size_sampled_rows(cid, T, split):
    name = f"{workloads.WORKLOADS[cid].name}_T{T}{'_split' if split else ''}"
    log(f"full size {name}")
    d = workloads.make_workload(cid, T, device=DEV)
    y, x = gpu_split(d) if split else gpu_fused(d)
    torch.cuda.synchronize()
    rows = sample_rows(T, seed=cid)
    ri = torch.as_tensor(rows, device=DEV)
    ref = oracle_ref(sub_inputs(d, rows), split=split)
    parity.compare(f"full {name} out (rows sampled)", workloads.bits(y.index_select(0, ri)), ref.y)
    parity.compare(f"full {name} residual_out (rows sampled)",
                   workloads.bits(x.index_select(0, ri)), ref.xout)
    # properties that hold at any size: finite, and the residual stream is
    # the one the outputs were normalised from (y = 0 exactly where h = 0)
    assert torch.isfinite(y.float()).all() and torch.isfinite(x.float()).all()
    del d, y, x
    torch.cuda.empty_cache()


# ----------------------------------------------------------- structure --- #

def test_fused_finalize_equals_materialized():
    """Fused finalize == the standalone finalize (moe_finalize, R BF16
    tensors) followed by the plain reduction: bit for bit, both epilogues,
    with and without the split-row workspace."""
    m = frn()
    for epi in ("rmsnorm", "sandwich"):
        for T in (24, 300):
            inp = to_dev(workloads.make(4, T, 6144, epilogue=epi, k=10, shared=True, seed=77 + T))
            y, x = gpu_fused(inp)
            mats = m.moe_finalize(inp.expert_rows, inp.topk_w, inp.topk_idx, shared=inp.shared)
            plain = workloads.Inputs(R=4, T=T, H=6144, epilogue=epi, residual=inp.residual,
                                     gamma1=inp.gamma1, gamma2=inp.gamma2, partials=mats)
            y2, x2 = gpu_fused(plain)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), (epi, T)
            assert torch.equal(x.view(torch.int16), x2.view(torch.int16)), (epi, T)


FINALIZE_CASES = [(8, 8, 6144, 10, True), (2, 32, 7168, 8, True), (3, 5, 2056, 16, True),
                  (4, 6, 1024, 1, False), (2, 70, 16384, 3, True)]


@pytest.mark.parametrize("case", FINALIZE_CASES,
                         ids=[f"R{c[0]}_T{c[1]}_H{c[2]}_k{c[3]}{'_shared' if c[4] else ''}"
                              for c in FINALIZE_CASES])
def test_standalone_finalize_matches_oracle(case):
    """moe_finalize writes exactly the oracle's per-rank BF16 partials."""
    R, T, H, k, sh = case
    log(f"standalone finalize {case}")
    inp = workloads.make(R, T, H, k=k, shared=sh, seed=900 + T)
    d = to_dev(inp)
    parts = frn().moe_finalize(d.expert_rows, d.topk_w, d.topk_idx, shared=d.shared)
    torch.cuda.synchronize()
    ref = oracle.boundary([workloads.bits(e) for e in inp.expert_rows],
                          residual=workloads.bits(inp.residual), gamma1=workloads.f32(inp.gamma1),
                          eps=inp.eps, topk_w=workloads.f32(inp.topk_w),
                          topk_idx=inp.topk_idx.numpy(),
                          shared=[workloads.bits(s) for s in inp.shared] if sh else None,
                          debug=True, nthreads=8)
    for r in range(R):
        parity.compare(f"finalize {case} rank {r}", workloads.bits(parts[r]), ref.p[r],
                       min_exact=1.0)


def test_deterministic_across_runs():
    inp = to_dev(workloads.make_workload(3, 64))
    y0, x0 = gpu_fused(inp)
    for _ in range(5):
        y, x = gpu_fused(inp)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y0.view(torch.int16))
        assert torch.equal(x.view(torch.int16), x0.view(torch.int16))


def test_in_place_residual():
    # one, two and four vectors per lane (the last two store residual_out
    # after every load of the row), and the split-row finalize
    for cid, T in ((2, 33), (3, 33), (2, 600), (4, 5)):
        inp = workloads.make_workload(cid, T)
        ref = oracle_ref(inp)
        d = to_dev(inp)
        y, x = gpu_fused(d, residual_out=d.residual)
        torch.cuda.synchronize()
        assert x.data_ptr() == d.residual.data_ptr()
        check(f"in-place residual w{cid} T{T}", y, x, ref)


def test_batch_changes_in_one_process():
    """Different T back to back (the pages' numerics worker changes batch
    sizes between calls)."""
    for T in (1, 300, 7, 64, 2):
        inp = workloads.make_workload(2, T, salt=5)
        y, x = gpu_fused(to_dev(inp))
        check(f"batch change T={T}", y, x, oracle_ref(inp))


def test_side_stream():
    inp = workloads.make_workload(2, 40, salt=9)
    d = to_dev(inp)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        y, x = gpu_fused(d)
    s.synchronize()
    check("side stream", y, x, oracle_ref(inp))


def test_concurrent_streams_with_their_own_workspaces():
    """Finalize calls queued on two streams at once (small T, where each
    takes the split-row finalize through the workspace the binding keeps per
    stream) and a plain call on a third: every result matches the oracle."""
    assert frn().split_rows(8, 10, 48, 6144) and frn().split_rows(8, 10, 40, 6144)
    a = workloads.make_workload(4, 48, salt=3)
    b = workloads.make_workload(4, 40, salt=4)
    c = workloads.make_workload(2, 64, salt=5)
    da, db, dc = to_dev(a), to_dev(b), to_dev(c)
    streams = [torch.cuda.Stream() for _ in range(3)]
    torch.cuda.synchronize()
    outs = []
    for _ in range(3):  # several rounds, so the streams' calls overlap
        with torch.cuda.stream(streams[0]):
            ya, xa = gpu_fused(da)
        with torch.cuda.stream(streams[1]):
            yb, xb = gpu_fused(db)
        with torch.cuda.stream(streams[2]):
            yc, xc = gpu_fused(dc)
        outs.append(((ya, xa), (yb, xb), (yc, xc)))
    torch.cuda.synchronize()
    refs = (oracle_ref(a), oracle_ref(b), oracle_ref(c))
    for rnd, trio in enumerate(outs):
        for name, (y, x), ref in zip("abc", trio, refs):
            check(f"concurrent streams round {rnd} call {name}", y, x, ref)


def test_graph_capture_and_replay_with_new_data():
    """Capture the fused call in a HIP graph; replay it several times with
    new input data copied in between (eager work and synchronisation between
    replays), checking every replay against the oracle."""
    m = frn()
    T, H, R = 48, 5120, 4
    base = to_dev(workloads.make(R, T, H, epilogue="sandwich", sigma=0.5, seed=5))
    out = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    rout = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        m.reduce_sandwich_norm(base.partials, base.residual, base.gamma1, base.gamma2, base.eps,
                               out=out, residual_out=rout)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        m.reduce_sandwich_norm(base.partials, base.residual, base.gamma1, base.gamma2, base.eps,
                               out=out, residual_out=rout)
    for rep in range(4):
        new = workloads.make(R, T, H, epilogue="sandwich", sigma=0.5, seed=100 + rep)
        for dst, src in zip(base.partials, new.partials):
            dst.copy_(src.to(DEV))
        base.residual.copy_(new.residual.to(DEV))
        base.gamma1.copy_(new.gamma1.to(DEV))
        base.gamma2.copy_(new.gamma2.to(DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(f"graph replay {rep}", out, rout, oracle_ref(new))


# ------------------------------------------------------------ edge cases --- #

def test_out_of_range_index_gives_nan_row_without_fault():
    inp = workloads.make(2, 6, 1024, k=3, shared=True, seed=31)
    nr = inp.expert_rows[0].shape[0]
    inp.topk_idx[2, 1] = nr
    inp.topk_idx[4, 0] = -5
    ref = oracle_ref(inp)
    y, x = gpu_fused(to_dev(inp))
    check("out-of-range index", y, x, ref)
    assert torch.isnan(y[2].float()).all() and torch.isnan(y[4].float()).all()


def test_zero_rows_give_zero_outputs():
    m = frn()
    z = torch.zeros(5, 5120, dtype=torch.bfloat16, device=DEV)
    g = torch.ones(5120, device=DEV)
    y, x = m.reduce_sandwich_norm([z, z, z], z, g, g, 1e-6)
    torch.cuda.synchronize()
    assert not torch.any(y.view(torch.int16) & 0x7FFF) and not torch.any(x.view(torch.int16) & 0x7FFF)


def test_non_finite_inputs_follow_ieee_like_the_oracle():
    """Inf and NaN in the inputs propagate as IEEE arithmetic dictates, the
    same way on both sides: NaN positions and every finite value match."""
    for epi in ("rmsnorm", "sandwich"):
        inp = workloads.make(3, 6, 1024, epilogue=epi, sigma=0.5, seed=606)
        inf, nan = torch.tensor(float("inf")), torch.tensor(float("nan"))
        inp.partials[0][1, 7] = inf.to(torch.bfloat16)           # row 1: one +inf
        inp.partials[1][2, 9] = nan.to(torch.bfloat16)           # row 2: one NaN
        inp.partials[0][3, 0] = inf.to(torch.bfloat16)           # row 3: +inf - inf
        inp.partials[2][3, 0] = (-inf).to(torch.bfloat16)
        inp.residual[4, 5] = inf.to(torch.bfloat16)              # row 4: residual inf
        y, x = gpu_fused(to_dev(inp))
        check(f"non-finite {epi}", y, x, oracle_ref(inp))


def test_zero_tokens():
    m = frn()
    p = torch.empty(0, 512, dtype=torch.bfloat16, device=DEV)
    y, x = m.reduce_residual_rmsnorm([p, p], p, torch.ones(512, device=DEV))
    assert y.shape == (0, 512)


def test_rejected_call_leaves_outputs_untouched():
    m = frn()
    buf = torch.zeros(4 * 64 + 8, dtype=torch.bfloat16, device=DEV)
    bad = buf[1:1 + 4 * 64].view(4, 64)  # 2-byte offset: not 16-byte aligned
    good = torch.zeros(4, 64, dtype=torch.bfloat16, device=DEV)
    out = torch.full((4, 64), 7.0, dtype=torch.bfloat16, device=DEV)
    rout = torch.full((4, 64), 9.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(m.FusedReduceNormUnsupported):
        m.reduce_residual_rmsnorm([good, bad], good, torch.ones(64, device=DEV),
                                  out=out, residual_out=rout)
    with pytest.raises(m.FusedReduceNormUnsupported):
        h12 = torch.zeros(4, 12, dtype=torch.bfloat16, device=DEV)
        m.reduce_residual_rmsnorm([h12], h12, torch.ones(12, device=DEV))
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(rout == 9.0)


# ---------------------------------------------------- contraction probes --- #

def test_no_fma_contraction_in_finalize():
    """Slot 1's product is inexact and slot 0 cancels its rounded value:
    uncontracted the finalize is exactly 0, so the pass-1 sum is 0 and the
    zero-residual row normalises to 0; an FMA would leave the rounding error,
    which the norm scales up to +-1."""
    m = frn()
    d = B.contraction_probe_finalize(64)
    rows = torch.from_numpy(d["src"][0].view(np.int16)).view(torch.bfloat16).to(DEV)
    w = torch.from_numpy(d["topk_w"]).to(DEV)
    idx = torch.from_numpy(d["topk_idx"]).to(DEV)
    zero = torch.zeros(1, 64, dtype=torch.bfloat16, device=DEV)
    y, x = m.moe_finalize_reduce_norm([rows], w, idx, zero, torch.ones(64, device=DEV))
    u = m.moe_finalize_reduce_bf16([rows], w, idx)
    torch.cuda.synchronize()
    assert not torch.any(u.view(torch.int16) & 0x7FFF), "finalize was contracted"
    assert not torch.any(y.view(torch.int16) & 0x7FFF)


def test_no_fma_contraction_in_sandwich():
    """gamma1 and the residual are chosen so that (s*r1)*gamma1 is inexact and
    the residual cancels its rounded value: h is exactly 0 unless the
    multiply-add was fused."""
    m = frn()
    H = 64
    p = B._bf16_bits(np.random.default_rng(23).normal(0, 1, H))[None, :]
    first = oracle.boundary([p], residual=np.zeros((1, H), np.uint16),
                            gamma1=np.ones(H, np.float32), gamma2=np.ones(H, np.float32),
                            eps=1e-6, epilogue=oracle.EPI_SANDWICH, debug=True)
    g1, xr = B.contraction_probe_sandwich(first.r1[0], first.s[0], H)
    tp = torch.from_numpy(p.view(np.int16)).view(torch.bfloat16).to(DEV)
    tx = torch.from_numpy(xr.view(np.int16)).view(torch.bfloat16).to(DEV)
    y, x = m.reduce_sandwich_norm([tp], tx, torch.from_numpy(g1).to(DEV),
                                  torch.ones(H, device=DEV), 1e-6)
    torch.cuda.synchronize()
    assert not torch.any(x.view(torch.int16) & 0x7FFF), "sandwich add was contracted"
    assert not torch.any(y.view(torch.int16) & 0x7FFF)


# ------------------------------------------------- split-row finalize --- #

MOE_CASES = [c for c in MODERATE if c[4] > 0]


@pytest.mark.parametrize("case", MOE_CASES, ids=[mid_id(c) for c in MOE_CASES])
def test_finalize_without_workspace_uses_row_kernel(case):
    """The same finalize cases through the one-row-per-workgroup kernel (no
    workspace): identical to the oracle, so identical to the split-row path."""
    R, T, H, epi, k, sh = case
    log(f"finalize row kernel {mid_id(case)}")
    inp = workloads.make(R, T, H, epilogue=epi, sigma=0.5, k=k, shared=sh,
                         seed=1000 + R * 7 + T * 13 + H)
    y, x = gpu_fused(to_dev(inp), workspace=None)
    check(f"row-kernel finalize {mid_id(case)}", y, x, oracle_ref(inp))


def test_split_row_workspace_explicit_and_reused():
    m = frn()
    R, H, k = 8, 6144, 10
    need = m.workspace_bytes(128, H, R, k)
    assert need == 128 * H * 4 + 128 * 12 * 8  # FP32 rows and FP64 slice sums, 128 tokens
    assert m.workspace_bytes(1000, H, R, k) == need  # the largest T that splits here
    assert m.workspace_bytes(64, H, R, 0) == 0
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=DEV)  # no initialisation needed
    for T in (1, 7, 64, 128, 200, 3):  # T=200 takes the one-row kernel, ignoring it
        inp = workloads.make(R, T, H, k=k, shared=True, seed=400 + T)
        y, x = gpu_fused(to_dev(inp), workspace=ws)
        check(f"explicit workspace T={T}", y, x, oracle_ref(inp))


def test_split_row_small_or_misaligned_workspace():
    m = frn()
    assert m.split_rows(4, 3, 8, 2048)
    inp = workloads.make(4, 8, 2048, k=3, shared=True, seed=55)
    ref = oracle_ref(inp)
    d = to_dev(inp)
    out = torch.full((8, 2048), 3.0, dtype=torch.bfloat16, device=DEV)
    rout = torch.full((8, 2048), 5.0, dtype=torch.bfloat16, device=DEV)
    small = torch.zeros(64, dtype=torch.uint8, device=DEV)   # too small: declined
    with pytest.raises(m.FusedReduceNormUnsupported, match="smaller than"):
        gpu_fused(d, workspace=small, out=out, residual_out=rout)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()) and bool((rout == 5.0).all())   # untouched
    y, x = gpu_fused(d, workspace=None)                        # none: the one-row kernel
    check("no workspace", y, x, ref)
    big = torch.zeros(m.workspace_bytes(8, 2048, 4, 3) + 512, dtype=torch.uint8, device=DEV)
    with pytest.raises(m.FusedReduceNormUnsupported):
        gpu_fused(d, workspace=big[16:])                      # 16-byte, not 256-byte aligned


@pytest.mark.parametrize("epi", ["rmsnorm", "sandwich"])
def test_boundary_materializes_a_declined_finalize(epi):
    """A fused finalize call declined for its workspace (too small): with
    on_decline='raise' the layer boundary raises and leaves the outputs
    alone; with 'materialize' it finalizes each rank alone and reduces the
    partials -- bit for bit the fused call's result, and the oracle's."""
    m = frn()
    R, T, H, k = 4, 8, 2048, 3
    assert m.split_rows(R, k, T, H, m.EPI_SANDWICH if epi == "sandwich" else m.EPI_RMSNORM)
    inp = workloads.make(R, T, H, k=k, shared=True, epilogue=epi, seed=58)
    d = to_dev(inp)
    e = m.EPI_SANDWICH if epi == "sandwich" else m.EPI_RMSNORM
    small = torch.zeros(64, dtype=torch.uint8, device=DEV)
    out = torch.full((T, H), 3.0, dtype=torch.bfloat16, device=DEV)
    rout = torch.full((T, H), 5.0, dtype=torch.bfloat16, device=DEV)
    kw = dict(topk_weights=d.topk_w, topk_rows=d.topk_idx, shared=d.shared, epilogue=e,
              workspace=small)
    with pytest.raises(m.FusedReduceNormUnsupported, match="smaller than"):
        m.boundary(d.expert_rows, d.residual, d.gamma1, d.gamma2, d.eps, out=out,
                   residual_out=rout, **kw)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()) and bool((rout == 5.0).all())
    y, x = m.boundary(d.expert_rows, d.residual, d.gamma1, d.gamma2, d.eps,
                      on_decline="materialize", out=out, residual_out=rout, **kw)
    yf, xf = gpu_fused(d)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), yf.view(torch.int16))
    assert torch.equal(x.view(torch.int16), xf.view(torch.int16))
    check(f"boundary materialized after a decline {epi}", y, x, oracle_ref(inp))


def test_split_row_graph_replay():
    """Graph-captured split-row finalize (two kernels through the workspace):
    every replay, with new data, matches the oracle."""
    m = frn()
    R, T, H, k = 8, 4, 6144, 10
    assert m.split_rows(R, k, T, H)
    base = to_dev(workloads.make(R, T, H, k=k, shared=True, seed=600))
    ws = torch.empty(m.workspace_bytes(T, H, R, k), dtype=torch.uint8, device=DEV)
    out = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    rout = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)

    def call():
        m.moe_finalize_reduce_norm(base.expert_rows, base.topk_w, base.topk_idx, base.residual,
                                   base.gamma1, None, base.eps, shared=base.shared,
                                   out=out, residual_out=rout, workspace=ws)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        new = workloads.make(R, T, H, k=k, shared=True, seed=700 + rep)
        for dst, src in zip(base.expert_rows + base.shared, new.expert_rows + new.shared):
            dst.copy_(src.to(DEV))
        base.topk_w.copy_(new.topk_w.to(DEV))
        base.topk_idx.copy_(new.topk_idx.to(DEV))
        base.residual.copy_(new.residual.to(DEV))
        base.gamma1.copy_(new.gamma1.to(DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(f"split-row graph replay {rep}", out, rout, oracle_ref(new))


@pytest.mark.parametrize("side", [0, 1])
def test_finalize_at_the_split_row_edge(side):
    """Either side of the split-row edge the library applies at R=8,
    H=6144, k=10 (read from the library, as a re-tune may move it): the
    automatic workspace's path, the one-row kernel and the oracle agree bit
    for bit."""
    m = frn()
    edge = max(t for t in range(1, 257) if m.split_rows(8, 10, t, 6144))
    T = edge + side
    assert m.split_rows(8, 10, T, 6144) == (side == 0)
    log(f"split-row edge {edge}: T={T}")
    inp = workloads.make(8, T, 6144, k=10, shared=True, seed=640 + T)
    d = to_dev(inp)
    y, x = gpu_fused(d)
    y2, x2 = gpu_fused(d, workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(x.view(torch.int16), x2.view(torch.int16))
    check(f"split-row edge T={T}", y, x, oracle_ref(inp))


def test_auto_workspace_graphs_survive_a_larger_capture():
    """Two graphs captured with the automatic workspace on torch's shared
    capture stream, the second needing a larger buffer: the first graph's
    buffer stays alive, and every replay of both matches the oracle."""
    m = frn()
    R, H, k = 8, 6144, 10
    graphs = []
    for T, seed in ((4, 610), (64, 620)):
        assert m.split_rows(R, k, T, H)
        base = to_dev(workloads.make(R, T, H, k=k, shared=True, seed=seed))
        out = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
        rout = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)

        def call(base=base, out=out, rout=rout):
            m.moe_finalize_reduce_norm(base.expert_rows, base.topk_w, base.topk_idx,
                                       base.residual, base.gamma1, None, base.eps,
                                       shared=base.shared, out=out, residual_out=rout,
                                       workspace="auto")
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            call()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call()
        graphs.append((T, base, out, rout, g))
    assert any(len(kept) >= 2 for kept in m._AUTO_WS.values())   # grown, old one kept
    scratch = [torch.full((1 << 22,), 7, dtype=torch.uint8, device=DEV) for _ in range(8)]
    for rep in range(3):
        for T, base, out, rout, g in graphs:
            new = workloads.make(R, T, H, k=k, shared=True, seed=900 + 10 * T + rep)
            for dst, src in zip(base.expert_rows + base.shared, new.expert_rows + new.shared):
                dst.copy_(src.to(DEV))
            base.topk_w.copy_(new.topk_w.to(DEV))
            base.topk_idx.copy_(new.topk_idx.to(DEV))
            base.residual.copy_(new.residual.to(DEV))
            base.gamma1.copy_(new.gamma1.to(DEV))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            check(f"auto-workspace graph T={T} replay {rep}", out, rout, oracle_ref(new))
    del scratch


# ------------------------------------------------------ launch shapes --- #

SHAPE_CASES = [(4, 300, 5120, "sandwich", 0, False), (3, 7, 5128, "rmsnorm", 0, False),
               (8, 40, 8192, "sandwich", 0, False), (2, 260, 7168, "rmsnorm", 8, True),
               (16, 5, 16384, "rmsnorm", 0, False),
               (4, 40, 4096, "rmsnorm", 4, True)]   # split-row finalize: fixed shapes


@pytest.mark.parametrize("vec", ["1", "2", "4", "p1", "p2"])
def test_results_do_not_depend_on_launch_shape(vec):
    """Force every launch choice through a launch table -- the one-row
    kernel's vectors per lane, and the row-pipelined kernel (p1 / p2), which
    then also runs the k = 0 pass of the split path: fused and split results
    stay equal to the oracle (rules that do not fit a call are skipped, so
    the built-in rule takes over there; the split-row finalize's two kernels
    take fixed shapes)."""
    m = frn()
    try:
        m.set_launch_table(f"* * * * 0 * {vec}")
        for case in SHAPE_CASES:
            R, T, H, epi, k, sh = case
            log(f"launch shape vec={vec} {mid_id(case)} -> {m.launch_shape(R, k, T, H)}, "
                f"pipelined {m.launch_pipelined(R, k, T, H)}")
            inp = workloads.make(R, T, H, epilogue=epi, sigma=0.5, k=k, shared=sh,
                                 seed=3000 + int(vec[-1]) * 11 + T)
            d = to_dev(inp)
            y, x = gpu_fused(d)
            check(f"vec={vec} fused {mid_id(case)}", y, x, oracle_ref(inp))
            y, x = gpu_split(d)
            check(f"vec={vec} split {mid_id(case)}", y, x, oracle_ref(inp, split=True))
    finally:
        m.set_launch_table(None)


def test_tuner_writes_a_loadable_table(tmp_path):
    import importlib.util
    import os
    spec = importlib.util.spec_from_file_location(
        "frn_tune", os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                                 "tp_reduction_rmsnorm_amd", "tune.py"))
    tune = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(tune)
    rows = tune.tune_shape(512, 2, 0, "rmsnorm", [1, 300], 4, DEV, log=log)
    assert [r[0] for r in rows] == [1, 300] and all(r[1] in r[2] for r in rows)
    text = "\n".join(tune.rules_for(512, 2, 0, "rmsnorm", rows))
    m = frn()
    try:
        m.set_launch_table(text)
        best = rows[1][1]  # a rule value: '1', '2', '4', 'p1' or 'p2'
        assert m.launch_shape(2, 0, 300, 512)[1] == int(best[-1])
        assert m.launch_pipelined(2, 0, 300, 512) == best.startswith("p")
    finally:
        m.set_launch_table(None)


def test_tuner_runs_and_its_table_drives_calls(tmp_path):
    """tune.py on one small finalize shape: it times the vec choices and the
    split-row finalize against the one-row kernel, writes a table that
    loads, and calls under that table still match the oracle."""
    import importlib.util
    import os
    m = frn()
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location(
        "frn_tune", os.path.join(root, "tp_reduction_rmsnorm_amd", "tune.py"))
    tune = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(tune)
    H, R, k, epi = 1024, 4, 3, "rmsnorm"
    rows = tune.tune_shape(H, R, k, epi, [8, 300], calls=4, dev=DEV, log=log)
    split = tune.tune_split(H, R, k, epi, [8, 64], calls=4, dev=DEV, log=log)
    lines = tune.rules_for(H, R, k, epi, rows) + tune.rules_for(H, R, k, epi, split, last="256")
    try:
        m.set_launch_table("\n".join(lines))
        for T, best, _ in split:
            assert m.split_rows(R, k, T, H) == (best == "split")
        for T in (8, 64, 300):
            inp = workloads.make(R, T, H, k=k, shared=True, seed=880 + T)
            y, x = gpu_fused(to_dev(inp))
            check(f"tuned table T={T}", y, x, oracle_ref(inp))
    finally:
        m.set_launch_table(None)
