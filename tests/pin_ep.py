"""Pins of the oracle's expert-parallel finalize.

The variant is the replicated-token deferral that vLLM PR #62366 names in
"Overview" and "Details" (TP = 1, EP > 1): every rank holds all T tokens and
the same top-k weights, but only its own experts' output rows.  Rank r's
finalize sums the slots routed to its experts (a negative row index marks a
slot of another rank), adds its shared-expert row if it holds one, and rounds
to BF16; the R partials then take the reduction and epilogue of the TP path.

Each ``pin_*`` returns failure messages (empty: the pin holds):

* ``pin_ep_exact``: exact arithmetic with derived bounds, per rank and step;
* ``pin_ep_closed_forms``: integer-valued rows, where every sum is exact, so
  the result cannot depend on how the slots are split over ranks -- the EP
  result must equal the one-rank TP result over all slots;
* ``pin_ep_invariants``: EP with one rank owning every slot is the TP
  finalize; a rank's partial equals the TP finalize over its own slots; a
  slot that no rank owns is a removed slot; zero weights leave the shared
  row; an index past a rank's own buffer turns the row into NaN; the thread
  count changes nothing;
* ``pin_ep_contraction``: the TP contraction probe routed through EP.
"""
from __future__ import annotations

from typing import List

import numpy as np

import oracle
import workloads
from tests import exact as X
from tests import pin_battery as B

EPS = B.EPS


def make_ep_case(R, T, H, epilogue, k, experts, shared_rank=0, seed=1, row_shifts=None):
    inp = workloads.make_ep(R, T, H, k=k, experts=experts, epilogue=epilogue,
                            shared_rank=shared_rank, seed=seed)
    d = dict(residual=workloads.bits(inp.residual), gamma1=workloads.f32(inp.gamma1),
             gamma2=workloads.f32(inp.gamma2) if inp.gamma2 is not None else None,
             src=[workloads.bits(e) for e in inp.expert_rows],
             topk_w=workloads.f32(inp.topk_w),
             topk_rows=[r.numpy().astype(np.int32) for r in inp.ep_rows],
             shared=(None if inp.shared is None else
                     [None if s is None else workloads.bits(s) for s in inp.shared]))
    # make the weights non-trivial in the sign, so cancellation occurs too
    d["topk_w"][:, 1::2] *= -1.0
    if row_shifts is not None:
        for t, sh in enumerate(row_shifts[:T]):
            if sh == 0:
                continue
            d["residual"] = B._scale_rows(d["residual"], [t], sh)
            for r in range(R):
                own = [int(i) for i in d["topk_rows"][r][t] if i >= 0]
                if own:
                    d["src"][r] = B._scale_rows(d["src"][r], own, sh)
                if d["shared"] is not None and d["shared"][r] is not None:
                    d["shared"][r] = B._scale_rows(d["shared"][r], [t], sh)
    return d


def run_ep(d, epilogue, debug=True, nthreads=1, split=False):
    epi = oracle.EPI_SANDWICH if epilogue == "sandwich" else oracle.EPI_RMSNORM
    return oracle.ep_boundary(d["src"], topk_w=d["topk_w"], topk_rows=d["topk_rows"],
                              residual=d["residual"], gamma1=d["gamma1"],
                              gamma2=d["gamma2"], eps=EPS, epilogue=epi,
                              shared=d["shared"], num_rows=d.get("num_rows"),
                              H=d["residual"].shape[1], debug=debug, nthreads=nthreads,
                              split=split)


# ------------------------------------------------------------- exact --- #

EP_EXACT_CASES = [
    # (R, T, H, epilogue, k, experts, shared_rank)
    (2, 4, 24, "rmsnorm", 3, 8, 0),
    (4, 4, 40, "sandwich", 4, 16, 1),
    (3, 3, 32, "rmsnorm", 2, 6, None),
]


def pin_ep_exact(case, seed=31, min_decided=0.9) -> List[str]:
    R, T, H, epilogue, k, experts, shared_rank = case
    d = make_ep_case(R, T, H, epilogue, k, experts, shared_rank, seed=seed,
                     row_shifts=B.ROW_SHIFTS)
    res = run_ep(d, epilogue)
    tally = X.Tally()
    for t in range(T):
        p_rows = []
        for r in range(R):
            own = [j for j in range(k) if d["topk_rows"][r][t, j] >= 0]
            w = d["topk_w"][t, own]
            idx = d["topk_rows"][r][t, own]
            sh = None
            if d["shared"] is not None and d["shared"][r] is not None:
                sh = d["shared"][r][t]
            for i in range(H):
                ex, bd = X.exact_finalize(d["src"][r], sh, w, idx, i)
                X.check_bf16(tally, f"P[{r},{t},{i}]", int(res.p[r, t, i]), ex, bd)
            p_rows.append(res.p[r, t])
        if not np.all(np.isfinite(oracle.bf16_to_f32(np.stack(p_rows)))):
            tally.fail(f"token {t}: a finalized partial is not finite")
            break
        s_ex, s_bd = [], []
        for i in range(H):
            ex, bd = X.exact_reduce(p_rows, i)
            s_ex.append(ex)
            s_bd.append(bd)
        for i in range(H):
            X.check_fp32(tally, f"s[{t},{i}]", res.s[t, i], s_ex[i], s_bd[i])
        X.check_epilogue(tally, t, s_ex, s_bd, d["residual"][t], d["gamma1"], d["gamma2"],
                         EPS, res, epilogue == "sandwich")
    out = [f"ep exact {case}: {m}" for m in tally.failures]
    total = tally.decided + tally.undecided
    if total and tally.decided < min_decided * total:
        out.append(f"ep exact {case}: only {tally.decided}/{total} outputs decided")
    return out


# -------------------------------------------------------- closed forms --- #

def _one_rank_tp(d, epilogue, shared_rank):
    """The same tokens with every expert on one rank: the ranks' buffers
    concatenated, each slot's row shifted by the rows before its rank."""
    R = len(d["src"])
    T, k = d["topk_w"].shape
    H = d["residual"].shape[1]
    bufs = [e if e is not None else np.zeros((0, H), np.uint16) for e in d["src"]]
    offs = np.cumsum([0] + [b.shape[0] for b in bufs])
    idx = np.full((T, k), -1, np.int32)
    for r in range(R):
        m = d["topk_rows"][r] >= 0
        idx[m] = d["topk_rows"][r][m] + offs[r]
    tp = dict(src=[np.ascontiguousarray(np.concatenate(bufs))], topk_w=d["topk_w"],
              topk_idx=idx, residual=d["residual"], gamma1=d["gamma1"], gamma2=d["gamma2"],
              shared=None if shared_rank is None else [d["shared"][shared_rank]])
    return B._run(tp, epilogue, debug=False)


def pin_ep_closed_forms() -> List[str]:
    """Integer expert rows, weights +-1 and +-2: every finalize sum and the
    rank sum are exact in FP32 and BF16 (|values| < 256), so the split of the
    slots over the ranks cannot show in the result."""
    fails = []
    for epilogue, shared_rank, seed in (("rmsnorm", 0, 3), ("sandwich", 2, 4),
                                        ("rmsnorm", None, 5)):
        d = make_ep_case(4, 6, 48, epilogue, 4, 16, shared_rank, seed=seed)
        rng = np.random.default_rng(seed)
        d["src"] = [B._bf16_bits(rng.integers(-8, 9, e.shape).astype(np.float64))
                    for e in d["src"]]
        if d["shared"] is not None:
            d["shared"] = [None if s is None else
                           B._bf16_bits(rng.integers(-8, 9, s.shape).astype(np.float64))
                           for s in d["shared"]]
        d["topk_w"] = rng.choice(np.array([-2.0, -1.0, 1.0, 2.0], np.float32),
                                 d["topk_w"].shape).astype(np.float32)
        a = run_ep(d, epilogue, debug=False)
        b = _one_rank_tp(d, epilogue, shared_rank)
        if not (np.array_equal(a.y, b.y) and np.array_equal(a.xout, b.xout)):
            fails.append(f"ep closed form ({epilogue}, shared on {shared_rank}): exact "
                         "sums differ from the one-rank result")
    return fails


# ---------------------------------------------------------- invariants --- #

def pin_ep_invariants() -> List[str]:
    fails = []
    # one rank owning every slot: the EP finalize is the TP finalize
    d = B.make_case(1, 5, 64, "sandwich", k=3, shared=True, seed=41)
    tp = B._run(d, "sandwich", debug=False)
    ep = dict(d, topk_rows=[d["topk_idx"]])
    a = run_ep(ep, "sandwich", debug=False)
    if not (np.array_equal(a.y, tp.y) and np.array_equal(a.xout, tp.xout)):
        fails.append("ep with one rank owning every slot differs from the TP finalize")
    # each rank's partial is the TP finalize over that rank's own slots
    d = make_ep_case(4, 5, 40, "rmsnorm", 5, 16, 1, seed=42)
    res = run_ep(d, "rmsnorm", debug=True)
    T, k = d["topk_w"].shape
    for r in range(4):
        sh = d["shared"][r]
        for t in range(T):
            own = [j for j in range(k) if d["topk_rows"][r][t, j] >= 0]
            if not own:
                want = sh[t] if sh is not None else np.zeros(40, np.uint16)
            else:
                one = oracle.boundary([d["src"][r]], topk_w=d["topk_w"][t:t + 1, own],
                                      topk_idx=d["topk_rows"][r][t:t + 1, own],
                                      shared=None if sh is None else [sh[t:t + 1]],
                                      epilogue=oracle.EPI_NONE)
                want = one.u[0]
            if not np.array_equal(res.p[r, t], want):
                fails.append(f"ep partial of rank {r}, token {t} differs from the TP "
                             "finalize over its own slots")
    # the partials reduce like any partials
    plain = dict(src=[np.ascontiguousarray(res.p[r]) for r in range(4)], shared=None,
                 residual=d["residual"], gamma1=d["gamma1"], gamma2=d["gamma2"])
    b = B._run(plain, "rmsnorm", debug=False)
    if not (np.array_equal(res.y, b.y) and np.array_equal(res.xout, b.xout)):
        fails.append("ep: the reduction of the partials differs from the plain reduction")
    # a slot that no rank owns is a removed slot
    d = make_ep_case(3, 4, 32, "sandwich", 4, 12, 0, seed=43)
    d1 = dict(d, topk_rows=[r.copy() for r in d["topk_rows"]])
    for r in d1["topk_rows"]:
        r[:, 2] = -1
    keep = [0, 1, 3]
    d2 = dict(d, topk_w=np.ascontiguousarray(d["topk_w"][:, keep]),
              topk_rows=[np.ascontiguousarray(r[:, keep]) for r in d1["topk_rows"]])
    a, b = run_ep(d1, "sandwich", debug=False), run_ep(d2, "sandwich", debug=False)
    if not (np.array_equal(a.y, b.y) and np.array_equal(a.xout, b.xout)):
        fails.append("ep: a slot owned by no rank is not the same as a removed slot")
    # zero weights: rank 0's partial is its shared row, the others +0
    d = make_ep_case(3, 4, 32, "rmsnorm", 3, 9, 0, seed=44)
    d["topk_w"] = np.zeros_like(d["topk_w"])
    a = run_ep(d, "rmsnorm", debug=False)
    b = B._run(dict(src=[d["shared"][0]], shared=None, residual=d["residual"],
                    gamma1=d["gamma1"], gamma2=None), "rmsnorm", debug=False)
    if not (np.array_equal(a.y, b.y) and np.array_equal(a.xout, b.xout)):
        fails.append("ep: zero weights do not leave the shared row alone")
    # an index past the rank's own buffer turns that token's row into NaN
    d = make_ep_case(3, 6, 32, "rmsnorm", 4, 12, 0, seed=45)
    nr = [e.shape[0] for e in d["src"]]
    r_small = int(np.argmin(nr))
    bad = [r.copy() for r in d["topk_rows"]]
    t_bad = 4
    j = int(np.flatnonzero(d["topk_rows"][r_small][t_bad] < 0)[0])
    for r in range(3):  # hand slot j of token t_bad to the smallest rank
        bad[r][t_bad, j] = -1
    bad[r_small][t_bad, j] = nr[r_small]
    a = run_ep(dict(d, topk_rows=bad), "rmsnorm", debug=False)
    ok = run_ep(d, "rmsnorm", debug=False)
    rows = [t for t in range(6) if t != t_bad]
    if not (np.all(np.isnan(oracle.bf16_to_f32(a.y[t_bad])))
            and np.array_equal(a.y[rows], ok.y[rows])):
        fails.append("ep: an index past the rank's buffer did not give a NaN row alone")
    # the thread count changes nothing
    d = make_ep_case(4, 23, 64, "sandwich", 6, 32, 3, seed=46)
    a = run_ep(d, "sandwich", debug=False, nthreads=1)
    b = run_ep(d, "sandwich", debug=False, nthreads=4)
    if not (np.array_equal(a.y, b.y) and np.array_equal(a.xout, b.xout)):
        fails.append("ep: results depend on the thread count")
    return fails


def pin_ep_contraction() -> List[str]:
    """The TP finalize probe with its two slots on one rank of two (the other
    rank owns nothing): uncontracted, every output is exactly 0."""
    d = B.contraction_probe_finalize(64)
    idx = d["topk_idx"]
    ep = dict(src=[d["src"][0], None], topk_w=d["topk_w"],
              topk_rows=[idx, np.full_like(idx, -1)], shared=None,
              residual=d["residual"], gamma1=d["gamma1"], gamma2=None, num_rows=[2, 0])
    res = run_ep(ep, "rmsnorm", debug=True)
    if np.any(res.p != 0) or np.any(res.y != 0):
        return ["ep finalize probe: nonzero result, the weighted sum was contracted"]
    return []


def all_ep_pins(quick: bool = False) -> List[str]:
    fails = []
    for c in (EP_EXACT_CASES[:1] if quick else EP_EXACT_CASES):
        fails += pin_ep_exact(c)
    fails += pin_ep_closed_forms()
    fails += pin_ep_invariants()
    fails += pin_ep_contraction()
    return fails
