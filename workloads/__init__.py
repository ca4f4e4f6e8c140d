"""Seeded synthetic inputs for the fused reduce + norm boundary.

This module serves both sides -- the CPU oracle and the GPU library -- and
therefore holds none of the method's arithmetic: it only draws random
tensors of the right shapes, dtypes and distributions and names the
workloads.  Every draw comes from one ``torch.Generator`` seeded from the
workload id and the token count, in a fixed order (partials r ascending,
residual, gamma1, gamma2, expert rows r ascending, shared rows r ascending,
router logits, row permutation).

The workloads follow the shapes the pages measure (vLLM PR #62366,
kernel microbenchmark table: hidden 5120 and 8192, 1..4096 tokens, TP 4 and
8; SGLang PR #34134: H=6144 MoE finalize + shared expert at decode sizes,
top-k 10; the large-batch split path at prefill sizes).  The
expert-parallel workload (the replicated-token deferral that vLLM PR #62366
names in "Overview") has no measured shape on the pages; it reuses the
H=6144, top-10-of-256 MoE shape over 8 ranks.  No dataset is involved
anywhere.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

EPS = 1e-6


@dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    epilogue: str            # "rmsnorm" or "sandwich"
    R: int                   # partials (TP ranks)
    H: int                   # hidden size
    tokens: Sequence[int]    # T sweep
    sigma: float = 1.0       # std of the BF16 partials
    k: int = 0               # top-k (0: no finalize)
    experts: int = 0         # experts the top-k is taken from (context only)
    shared: bool = False     # shared-expert add inside the finalize
    split: bool = False      # large-batch two-pass path measured too
    ep: bool = False         # expert-parallel routing: each rank owns experts/R experts


WORKLOADS = {
    1: Workload(1, "tiny_rmsnorm_h512_r2", "rmsnorm", R=2, H=512, tokens=(8,), sigma=1.0),
    2: Workload(2, "sandwich_h5120_r4", "sandwich", R=4, H=5120,
                tokens=(1, 8, 64, 256, 1024, 4096), sigma=0.5),
    3: Workload(3, "sandwich_h8192_r8", "sandwich", R=8, H=8192,
                tokens=(1, 8, 64, 256, 1024, 4096), sigma=0.5),
    4: Workload(4, "moe_finalize_h6144_r8_k10", "rmsnorm", R=8, H=6144,
                tokens=(1, 2, 4, 8, 16, 32, 64), k=10, experts=256, shared=True),
    5: Workload(5, "split_h7168_r2_k8", "rmsnorm", R=2, H=7168,
                tokens=(4096, 16384), k=8, experts=256, shared=True, split=True),
    6: Workload(6, "ep_moe_h6144_r8_k10", "rmsnorm", R=8, H=6144,
                tokens=(1, 8, 64, 1024, 4096), k=10, experts=256, shared=True, ep=True),
}


def seed_for(cid: int, T: int, salt: int = 0) -> int:
    return (2026 * 1_000_003 + cid * 10_007 + T * 101 + salt) & 0x7FFF_FFFF


@dataclass
class Inputs:
    """One batch of boundary inputs (torch tensors, all on one device)."""
    R: int
    T: int
    H: int
    epilogue: str
    residual: torch.Tensor                 # [T,H] bf16
    gamma1: torch.Tensor                   # [H] f32
    gamma2: Optional[torch.Tensor]         # [H] f32 (sandwich)
    eps: float = EPS
    partials: Optional[List[torch.Tensor]] = None      # R x [T,H] bf16
    expert_rows: Optional[List[torch.Tensor]] = None   # R x [T*k,H] bf16
    shared: Optional[List[torch.Tensor]] = None        # R x [T,H] bf16
    topk_w: Optional[torch.Tensor] = None              # [T,k] f32
    topk_idx: Optional[torch.Tensor] = None            # [T,k] int32
    ep_rows: Optional[List[torch.Tensor]] = None       # R x [T,k] int32 (expert-parallel)
    k: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def sources(self) -> List[torch.Tensor]:
        return self.expert_rows if self.k > 0 else self.partials


def _normal_bf16(g: torch.Generator, shape, sigma: float, device) -> torch.Tensor:
    """~N(0, sigma) draws rounded to BF16, drawn in chunks to bound memory."""
    rows = shape[0]
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    chunk = max(1, (1 << 26) // max(1, int(np.prod(shape[1:]))))
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        v = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g, device=device,
                        dtype=torch.float32)
        if sigma != 1.0:
            v.mul_(sigma)
        out[r0:r1] = v.to(torch.bfloat16)
    return out


def make(R: int, T: int, H: int, *, epilogue: str = "rmsnorm", sigma: float = 1.0,
         k: int = 0, shared: bool = False, num_rows: Optional[int] = None,
         seed: int = 0, device="cpu", residual_sigma: float = 1.0) -> Inputs:
    """Draw one batch.  k > 0 draws expert rows, top-k weights and indices."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    partials = None
    if k == 0:
        partials = [_normal_bf16(g, (T, H), sigma, device) for _ in range(R)]
    residual = _normal_bf16(g, (T, H), residual_sigma, device)
    gamma1 = torch.rand((H,), generator=g, device=device, dtype=torch.float32) + 0.5
    gamma2 = None
    if epilogue == "sandwich":
        gamma2 = torch.rand((H,), generator=g, device=device, dtype=torch.float32) + 0.5
    inp = Inputs(R=R, T=T, H=H, epilogue=epilogue, residual=residual,
                 gamma1=gamma1, gamma2=gamma2, partials=partials, k=k)
    if k > 0:
        nr = T * k if num_rows is None else num_rows
        inp.expert_rows = [_normal_bf16(g, (nr, H), 1.0, device) for _ in range(R)]
        if shared:
            inp.shared = [_normal_bf16(g, (T, H), 1.0, device) for _ in range(R)]
        logits = torch.randn((T, k), generator=g, device=device, dtype=torch.float32)
        inp.topk_w = torch.softmax(logits, dim=-1).contiguous()
        perm = torch.randperm(T * k, generator=g, device=device)
        if nr != T * k:  # spread the rows over a larger buffer
            perm = (perm * (nr // max(1, T * k))) % nr
        inp.topk_idx = perm.to(torch.int32).reshape(T, k).contiguous()
    return inp


def make_ep(R: int, T: int, H: int, *, k: int, experts: int, epilogue: str = "rmsnorm",
            shared_rank: Optional[int] = 0, seed: int = 0, device="cpu") -> Inputs:
    """Draw one expert-parallel batch: every rank sees all T tokens and the
    same top-k weights, and owns experts [r*E/R, (r+1)*E/R).  Each token picks
    k distinct experts uniformly; rank r's expert-output buffer holds one row
    per slot routed to its experts, grouped by expert (tokens ascending within
    an expert), and ``ep_rows[r][t,j]`` is that row, or -1 when slot j's
    expert lives on another rank.  Only ``shared_rank`` holds a shared-expert
    row (None: no rank does).  Draw order: residual, gamma1, gamma2, expert
    choice keys, router logits, expert rows (r ascending), shared rows."""
    if experts % R or k > experts:
        raise ValueError("experts must split evenly over R ranks and be >= k")
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    residual = _normal_bf16(g, (T, H), 1.0, device)
    gamma1 = torch.rand((H,), generator=g, device=device, dtype=torch.float32) + 0.5
    gamma2 = None
    if epilogue == "sandwich":
        gamma2 = torch.rand((H,), generator=g, device=device, dtype=torch.float32) + 0.5
    keys = torch.rand((T, experts), generator=g, device=device, dtype=torch.float32)
    chosen = keys.topk(k, dim=1).indices                       # [T,k] distinct experts
    logits = torch.randn((T, k), generator=g, device=device, dtype=torch.float32)
    flat = chosen.reshape(-1)
    owner = flat // (experts // R)
    ep_rows, counts = [], []
    for r in range(R):
        slots = (owner == r).nonzero().squeeze(1)             # slot = t*k + j, ascending
        slots = slots[torch.argsort(flat[slots], stable=True)]
        idx = torch.full((T * k,), -1, dtype=torch.int32, device=device)
        idx[slots] = torch.arange(slots.numel(), dtype=torch.int32, device=device)
        ep_rows.append(idx.reshape(T, k).contiguous())
        counts.append(int(slots.numel()))
    inp = Inputs(R=R, T=T, H=H, epilogue=epilogue, residual=residual, gamma1=gamma1,
                 gamma2=gamma2, k=k)
    inp.topk_w = torch.softmax(logits, dim=-1).contiguous()
    inp.ep_rows = ep_rows
    inp.expert_rows = [_normal_bf16(g, (n, H), 1.0, device) for n in counts]
    if shared_rank is not None:
        inp.shared = [_normal_bf16(g, (T, H), 1.0, device) if r == shared_rank else None
                      for r in range(R)]
    return inp


def make_workload(cid: int, T: int, device="cpu", salt: int = 0) -> Inputs:
    w = WORKLOADS[cid]
    if w.ep:
        return make_ep(w.R, T, w.H, k=w.k, experts=w.experts, epilogue=w.epilogue,
                       shared_rank=0 if w.shared else None, seed=seed_for(cid, T, salt),
                       device=device)
    return make(w.R, T, w.H, epilogue=w.epilogue, sigma=w.sigma, k=w.k,
                shared=w.shared, seed=seed_for(cid, T, salt), device=device)


def bits(t: torch.Tensor) -> np.ndarray:
    """BF16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy().astype(np.float32, copy=False)


def algorithmic_bytes(R: int, T: int, H: int, *, epilogue: str, k: int = 0,
                      shared: bool = True, part: str = "fused", ep: bool = False) -> int:
    """Bytes the method must move per call (gamma counted once).

    expert-parallel finalize (ep): T*k*H*2 [each routed row once] + 2TH [one
    rank's shared row] + 4TkR [each rank's index array] + 4Tk [weights] + 6TH
    + gammas
    fused/plain:    T*H*(2R+6) + 4H*(1 or 2 gammas)
    fused/finalize: T*H*2R(k+1) [k expert rows + shared row per rank; k without shared] + 8Tk + 6TH + gammas
    split pass 1:   T*H*2R(k+1) + 8Tk + 2TH  (k=0: T*H*2R + 2TH)
    split pass 2:   8TH + gammas
    """
    ng = 2 if epilogue == "sandwich" else 1
    if ep:
        assert part == "fused" and k > 0
        return (T * k * H * 2 + (2 * T * H if shared else 0) + 4 * T * k * R + 4 * T * k
                + 6 * T * H + 4 * H * ng)
    rows = k + (1 if shared else 0)
    if part == "pass1":
        if k > 0:
            return T * H * 2 * R * rows + 8 * T * k + 2 * T * H
        return T * H * 2 * R + 2 * T * H
    if part == "pass2":
        return 8 * T * H + 4 * H * ng
    if k > 0:
        return T * H * 2 * R * rows + 8 * T * k + 6 * T * H + 4 * H * ng
    return T * H * (2 * R + 6) + 4 * H * ng
