"""Seeded random shapes across the supported range, each call checked
against the oracle: plain, sandwich, TP and expert-parallel finalize, split
path, with and without the split-row workspace (every other TP finalize
case given one goes through the no-allocation entry point instead, whose
scratch array then holds the partials).  The shapes are drawn from
a fixed seed, so the set is the same on every run: 48 of them by default;
FRN_RANDOM_SHAPES=<n> and FRN_RANDOM_SEED=<s> draw a larger or another
set."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import parity
from tests import test_gpu_ep as E
from tests import test_gpu_parity as P

pytestmark = pytest.mark.gpu


def _cases(n=None, seed=None):
    n = int(os.environ.get("FRN_RANDOM_SHAPES", "48")) if n is None else n
    seed = int(os.environ.get("FRN_RANDOM_SEED", "20261202")) if seed is None else seed
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = ["plain", "tp", "ep", "split"][i % 4]
        H = int(rng.choice([8, 24, 64, 136, 512, 520, 1024, 2056, 3072, 4096, 5128, 6144, 7168,
                            8200, 12288, 16384]))
        T = int(rng.choice([1, 2, 5, 9, 16, 17, 33, 48, 64, 96, 97, 128, 200, 257, 300, 513]))
        R = int(rng.integers(1, 17))
        k = int(rng.integers(1, 17)) if kind in ("tp", "ep") or (kind == "split" and i % 8 == 3) else 0
        # keep each case within a second or two of oracle time
        while T > 1 and T * H * max(1, R * (k + 1)) > 6e8:
            T //= 2
        epi = "sandwich" if rng.random() < 0.5 else "rmsnorm"
        ws = bool(rng.random() < 0.6)
        out.append((i, kind, R, T, H, k, epi, ws))
    return out


CASES = _cases()


def _id(c):
    i, kind, R, T, H, k, epi, ws = c
    return f"{i}_{kind}_R{R}_T{T}_H{H}_k{k}_{epi}" + ("_ws" if ws else "")


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_random_shape_matches_oracle(case):
    i, kind, R, T, H, k, epi, ws = case
    P.log(f"random {_id(case)}")
    m = P.frn()
    if kind == "ep":
        experts = R * int(np.ceil(k / R) + 1)
        inp = workloads.make_ep(R, T, H, k=k, experts=experts, epilogue=epi,
                                shared_rank=(i % R) if i % 3 else None, seed=7000 + i)
        y, x = E.gpu_ep(E.dev(inp), workspace="auto" if ws else None)
        torch.cuda.synchronize()
        ref = E.oracle_ep(inp)
    else:
        inp = workloads.make(R, T, H, epilogue=epi, sigma=0.5, k=k, shared=bool(k and i % 2),
                             seed=7000 + i)
        d = P.to_dev(inp)
        if kind == "split":
            y, x = P.gpu_split(d)
            ref = P.oracle_ref(inp, split=True)
        elif kind == "tp" and ws and (i // 4) % 2 == 1:
            e = m.EPI_SANDWICH if epi == "sandwich" else m.EPI_RMSNORM
            y = torch.empty(T, H, dtype=torch.bfloat16, device=P.DEV)
            x = torch.empty(T, H, dtype=torch.bfloat16, device=P.DEV)
            m.moe_finalize_reduce_norm_noalloc(d.expert_rows, d.topk_w, d.topk_idx, d.residual,
                                               d.gamma1, d.gamma2, d.eps, out=y, residual_out=x,
                                               shared=d.shared, epilogue=e)
            ref = P.oracle_ref(inp)
        else:
            y, x = P.gpu_fused(d, workspace="auto" if (ws and k) else None)
            ref = P.oracle_ref(inp)
        torch.cuda.synchronize()
    parity.compare(f"random {_id(case)} out", workloads.bits(y), ref.y)
    parity.compare(f"random {_id(case)} residual_out", workloads.bits(x), ref.xout)


# The same kind of shapes with a launch table that sends every call two (or
# four) vectors per lane where they fit: the one-row kernel's epilogue with
# several vectors per lane (every gamma load ahead of the first store) and
# its ragged last vectors, at many H.
FORCED = [(v, c) for v in (2, 4) for c in _cases(24, seed=6100 + v)]


@pytest.mark.parametrize("vec,case", FORCED, ids=[f"v{v}_{_id(c)}" for v, c in FORCED])
def test_random_shape_forced_vectors_matches_oracle(vec, case):
    m = P.frn()
    m.set_launch_table(f"* * * * 0 * {vec}\n")
    try:
        test_random_shape_matches_oracle(case)
    finally:
        m.set_launch_table(None)
