"""GPU parity of the split-row finalize at the edges of its two kernels.

Every finalize call up to 256 tokens is sent to the split-row finalize by a
caller launch table ("* * * * 0 256 split"), then run again without a
workspace (the one-row kernel).  Each result is compared with the oracle,
and the two GPU results with each other bit for bit.  The shapes cover
what the kernels special-case:

* one wave per rank: R = 1 (one wave) up to R = 16 (1024 lanes);
* 64-vector slices: H = 8 (one vector, 63 idle lanes), H = 520 (a partial
  second slice), H = 16384 (32 slices);
* the sandwich's per-token epilogue with one vector per lane and with two
  (H = 8200: 1025 vectors, a ragged second vector);
* the top-k chunk sized to k (k = 1, 2, 4, 5, 10, 16), with and without
  shared-expert rows;
* T = 256, the largest T any rule can split at;
* expert-parallel routing (ranks without a live slot idle in their wave).
"""
import pytest
import torch

import workloads
from tests import parity
from tests import test_gpu_ep as E
from tests.test_gpu_parity import DEV, frn, gpu_fused, log, oracle_ref, to_dev

pytestmark = pytest.mark.gpu

SPLIT_ALL = "* * * * 0 256 split\n"


@pytest.fixture
def split_everywhere():
    m = frn()
    m.set_launch_table(SPLIT_ALL)
    yield m
    m.set_launch_table(None)


def _same(name, a, b):
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name


# (R, T, H, epilogue, k, shared)
TP = [
    (1, 5, 4096, "rmsnorm", 4, True),
    (3, 7, 520, "sandwich", 2, True),
    (3, 7, 520, "rmsnorm", 2, False),
    (16, 3, 16384, "rmsnorm", 16, True),
    (16, 3, 16384, "sandwich", 3, True),
    (4, 9, 8200, "sandwich", 5, True),
    (4, 9, 8200, "rmsnorm", 5, True),
    (2, 256, 2048, "rmsnorm", 8, True),
    (5, 33, 8, "rmsnorm", 1, True),
    (8, 64, 6144, "sandwich", 10, True),
]


@pytest.mark.parametrize("case", TP, ids=[f"R{c[0]}_T{c[1]}_H{c[2]}_{c[3]}_k{c[4]}"
                                          + ("_shared" if c[5] else "") for c in TP])
def test_split_rows_tp(case, split_everywhere):
    m = split_everywhere
    R, T, H, epi, k, shared = case
    e = m.EPI_SANDWICH if epi == "sandwich" else m.EPI_RMSNORM
    assert m.split_rows(R, k, T, H, e)
    log(f"split-row TP R={R} T={T} H={H} {epi} k={k}")
    inp = workloads.make(R, T, H, k=k, shared=shared, epilogue=epi, sigma=0.5,
                         seed=3100 + R * 7 + k)
    d = to_dev(inp)
    y, x = gpu_fused(d, workspace="auto")
    yf, xf = gpu_fused(d, workspace=None)
    ref = oracle_ref(inp)
    torch.cuda.synchronize()
    parity.compare(f"split-row {case} out", workloads.bits(y), ref.y)
    parity.compare(f"split-row {case} residual_out", workloads.bits(x), ref.xout)
    _same("split-row out vs one-row kernel", y, yf)
    _same("split-row residual_out vs one-row kernel", x, xf)


# (R, T, H, epilogue, k, shared rank or None)
EP = [
    (8, 40, 6144, "rmsnorm", 10, 0),
    (16, 5, 16384, "sandwich", 16, 15),
    (3, 7, 520, "rmsnorm", 4, None),
    (2, 256, 1024, "sandwich", 6, 1),
]


@pytest.mark.parametrize("case", EP, ids=[f"R{c[0]}_T{c[1]}_H{c[2]}_{c[3]}_k{c[4]}"
                                          for c in EP])
def test_split_rows_ep(case, split_everywhere):
    m = split_everywhere
    R, T, H, epi, k, shared_rank = case
    e = m.EPI_SANDWICH if epi == "sandwich" else m.EPI_RMSNORM
    assert m.split_rows(R, k, T, H, e, ep=True)
    log(f"split-row EP R={R} T={T} H={H} {epi} k={k}")
    experts = R * (-(-k // R) + 1)
    inp = workloads.make_ep(R, T, H, k=k, experts=experts, epilogue=epi,
                            shared_rank=shared_rank, seed=3300 + R + k)
    d = E.dev(inp)
    y, x = E.gpu_ep(d, workspace="auto")
    yf, xf = E.gpu_ep(d, workspace=None)
    ref = E.oracle_ep(inp)
    torch.cuda.synchronize()
    parity.compare(f"split-row EP {case} out", workloads.bits(y), ref.y)
    parity.compare(f"split-row EP {case} residual_out", workloads.bits(x), ref.xout)
    _same("split-row EP out vs one-row kernel", y, yf)
    _same("split-row EP residual_out vs one-row kernel", x, xf)


@pytest.mark.parametrize("epi", ["rmsnorm", "sandwich"])
def test_split_rows_out_of_range_and_non_finite(epi, split_everywhere):
    """Through the split-row finalize: an index past the expert buffer (or
    negative, under TP routing) reads as a NaN row without a fault, and inf
    or NaN in expert and shared rows propagate as IEEE arithmetic dictates;
    the oracle and the one-row kernel agree element for element (NaN
    positions included)."""
    m = split_everywhere
    R, T, H, k = 3, 6, 1024, 3
    assert m.split_rows(R, k, T, H)
    log(f"split-row non-finite {epi}")
    inp = workloads.make(R, T, H, k=k, shared=True, epilogue=epi, seed=3500)
    nr = inp.expert_rows[0].shape[0]
    inf, nan = torch.tensor(float("inf")), torch.tensor(float("nan"))
    inp.topk_idx[2, 1] = nr                                       # row 2: past the buffer
    inp.topk_idx[4, 0] = -5                                       # row 4: negative
    inp.expert_rows[1][int(inp.topk_idx[1, 2]), 17] = inf.to(torch.bfloat16)  # row 1: inf
    inp.shared[2][3, 40] = nan.to(torch.bfloat16)                 # row 3: NaN shared
    inp.expert_rows[0][int(inp.topk_idx[5, 0]), 3] = inf.to(torch.bfloat16)   # row 5: inf - inf
    inp.expert_rows[1][int(inp.topk_idx[5, 0]), 3] = (-inf).to(torch.bfloat16)
    d = to_dev(inp)
    y, x = gpu_fused(d, workspace="auto")
    yf, xf = gpu_fused(d, workspace=None)
    ref = oracle_ref(inp)
    torch.cuda.synchronize()
    parity.compare(f"split-row non-finite {epi} out", workloads.bits(y), ref.y)
    parity.compare(f"split-row non-finite {epi} residual_out", workloads.bits(x), ref.xout)
    _same("split-row non-finite out vs one-row kernel", y, yf)
    _same("split-row non-finite residual_out vs one-row kernel", x, xf)
    assert torch.isnan(y[2].float()).all() and torch.isnan(y[4].float()).all()
