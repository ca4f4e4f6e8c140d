"""Seeded random shapes across the supported range, each call checked
against the oracle: plain, sandwich, TP and expert-parallel finalize, split
path, with and without the split-row workspace.  The shapes are drawn once
from a fixed seed, so the set is the same on every run."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import parity
from tests import test_gpu_ep as E
from tests import test_gpu_parity as P

pytestmark = pytest.mark.gpu


def _cases(n=48, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = ["plain", "tp", "ep", "split"][i % 4]
        H = int(rng.choice([8, 16, 64, 136, 512, 520, 1024, 2056, 4096, 5128, 6144, 8200, 16384]))
        T = int(rng.choice([1, 2, 3, 7, 17, 40, 257, 300]))
        if H >= 8192 and T > 40:
            T = 17
        R = int(rng.integers(1, 17))
        k = int(rng.integers(1, 17)) if kind in ("tp", "ep") or (kind == "split" and i % 8 == 3) else 0
        epi = "sandwich" if rng.random() < 0.5 else "rmsnorm"
        ws = bool(rng.random() < 0.5)
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
        else:
            y, x = P.gpu_fused(d, workspace="auto" if (ws and k) else None)
            ref = P.oracle_ref(inp)
        torch.cuda.synchronize()
    parity.compare(f"random {_id(case)} out", workloads.bits(y), ref.y)
    parity.compare(f"random {_id(case)} residual_out", workloads.bits(x), ref.xout)
