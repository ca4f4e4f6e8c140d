"""The pins that hold the CPU oracle to the method's definition.

Each ``pin_*`` function runs the oracle (through the ``oracle`` package, so a
test can swap in a deliberately broken build of its source) and returns a
list of failure messages; an empty list means the pin holds.  The pins are
chosen so that a plausible mistake anywhere in the oracle -- a dropped term,
a wrong sign or index, a swapped operand, a missing rounding, an FMA
contraction -- fails at least one of them:

* ``pin_exact``: exact real arithmetic (tests/exact.py) with derived error
  bounds, at tiny sizes, for every variant (plain, sandwich, finalize with
  and without shared expert, split).
* ``pin_bf16``: BF16 widening (exhaustive) and narrowing against torch's CPU
  conversion (a library routine).
* ``pin_library_rmsnorm``: R=1 without finalize is plain residual + RMSNorm;
  compared with ``torch.nn.functional.rms_norm`` in float64.
* ``pin_closed_forms``: rows whose result is known exactly.
* ``pin_invariants``: permutation, zero partial, zero-weight slot, unit
  weight, zero weights with shared expert, split structure, thread count,
  out-of-range index.
* ``pin_contraction``: inputs on which an FMA-contracted finalize or sandwich
  gives a visibly different answer than the uncontracted one the pages ask
  for (vLLM PR #62366 "Details").
"""
from __future__ import annotations

from typing import List

import numpy as np
import torch

import oracle
import workloads
from tests import exact as X

EPS = 1e-6


def _np_inputs(inp: workloads.Inputs):
    d = dict(residual=workloads.bits(inp.residual), gamma1=workloads.f32(inp.gamma1),
             gamma2=workloads.f32(inp.gamma2) if inp.gamma2 is not None else None)
    if inp.k > 0:
        d["src"] = [workloads.bits(e) for e in inp.expert_rows]
        d["shared"] = [workloads.bits(s) for s in inp.shared] if inp.shared else None
        d["topk_w"] = workloads.f32(inp.topk_w)
        d["topk_idx"] = inp.topk_idx.cpu().numpy().astype(np.int32)
    else:
        d["src"] = [workloads.bits(p) for p in inp.partials]
        d["shared"] = None
    return d


def _scale_rows(bits: np.ndarray, rows, shift: int) -> np.ndarray:
    """Scale the given rows of a BF16 array by 2**shift (exact)."""
    out = bits.copy()
    v = torch.from_numpy(out.view(np.int16)).view(torch.bfloat16)
    v[rows] = (v[rows].float() * (2.0 ** shift)).to(torch.bfloat16)
    return out


def make_case(R, T, H, epilogue, k=0, shared=False, seed=1, row_shifts=None):
    """Tiny seeded case; row t of every input is scaled by 2**row_shifts[t]
    so that eps matters in some rows and not in others."""
    inp = workloads.make(R, T, H, epilogue=epilogue, k=k, shared=shared,
                         num_rows=(T * k + 3) if k else None, seed=seed, sigma=0.5)
    d = _np_inputs(inp)
    if row_shifts is not None:
        for t, sh in enumerate(row_shifts[:T]):
            if sh == 0:
                continue
            d["residual"] = _scale_rows(d["residual"], [t], sh)
            if k > 0:
                rows = [int(i) for i in d["topk_idx"][t]]
                d["src"] = [_scale_rows(e, rows, sh) for e in d["src"]]
                if d["shared"] is not None:
                    d["shared"] = [_scale_rows(s, [t], sh) for s in d["shared"]]
            else:
                d["src"] = [_scale_rows(p, [t], sh) for p in d["src"]]
    return d


def _run(d, epilogue, split=False, debug=True, **kw):
    epi = oracle.EPI_SANDWICH if epilogue == "sandwich" else oracle.EPI_RMSNORM
    return oracle.boundary(d["src"], residual=d["residual"], gamma1=d["gamma1"],
                           gamma2=d["gamma2"], eps=kw.get("eps", EPS), epilogue=epi,
                           split=split, topk_w=d.get("topk_w"), topk_idx=d.get("topk_idx"),
                           shared=d.get("shared"), debug=debug,
                           nthreads=kw.get("nthreads", 1))


# ------------------------------------------------------------- exact --- #

EXACT_CASES = [
    # (R, T, H, epilogue, k, shared, split)
    (1, 3, 16, "rmsnorm", 0, False, False),
    (2, 4, 40, "rmsnorm", 0, False, False),
    (3, 4, 64, "rmsnorm", 0, False, False),
    (1, 3, 16, "sandwich", 0, False, False),
    (2, 4, 40, "sandwich", 0, False, False),
    (3, 4, 64, "sandwich", 0, False, False),
    (2, 3, 24, "rmsnorm", 1, False, False),
    (3, 3, 32, "rmsnorm", 3, True, False),
    (2, 3, 24, "sandwich", 2, True, False),
    (2, 4, 40, "rmsnorm", 0, False, True),
    (2, 3, 24, "sandwich", 0, False, True),
    (2, 3, 24, "rmsnorm", 2, True, True),
]
ROW_SHIFTS = [0, -10, 3, -7]


def pin_exact(case, seed=11, min_decided=0.9) -> List[str]:
    R, T, H, epilogue, k, shared, split = case
    d = make_case(R, T, H, epilogue, k=k, shared=shared, seed=seed, row_shifts=ROW_SHIFTS)
    res = _run(d, epilogue, split=split)
    tally = X.Tally()
    for t in range(T):
        if k > 0:
            p_rows = []
            for r in range(R):
                for i in range(H):
                    ex, bd = X.exact_finalize(d["src"][r], d["shared"][r][t] if shared else None,
                                              d["topk_w"][t], d["topk_idx"][t], i)
                    X.check_bf16(tally, f"P[{r},{t},{i}]", int(res.p[r, t, i]), ex, bd)
                p_rows.append(res.p[r, t])
            if not np.all(np.isfinite(oracle.bf16_to_f32(np.stack(p_rows)))):
                tally.fail(f"token {t}: a finalized partial is not finite")
                break
        else:
            p_rows = [p[t] for p in d["src"]]
        s_ex, s_bd = [], []
        for i in range(H):
            ex, bd = X.exact_reduce(p_rows, i)
            s_ex.append(ex)
            s_bd.append(bd)
        if split:
            for i in range(H):
                X.check_bf16(tally, f"U[{t},{i}]", int(res.u[t, i]), s_ex[i], s_bd[i])
            s_ex = [X.bf16_val(b) for b in res.u[t]]
            s_bd = [0.0] * H
        for i in range(H):
            X.check_fp32(tally, f"s[{t},{i}]", res.s[t, i], s_ex[i], s_bd[i])
        X.check_epilogue(tally, t, s_ex, s_bd, d["residual"][t], d["gamma1"], d["gamma2"],
                         EPS, res, epilogue == "sandwich")
    out = list(tally.failures)
    total = tally.decided + tally.undecided
    if total and tally.decided < min_decided * total:
        out.append(f"only {tally.decided}/{total} outputs decided: bounds too loose to pin")
    return out


def pin_exact_rows(partials, residual, g1, g2, epilogue, label) -> List[str]:
    """Exact-arithmetic check of hand-built rows (no finalize)."""
    d = dict(src=partials, residual=residual, gamma1=g1, gamma2=g2, shared=None)
    res = _run(d, epilogue)
    tally = X.Tally()
    T, H = residual.shape
    for t in range(T):
        p_rows = [p[t] for p in partials]
        s_ex, s_bd = zip(*[X.exact_reduce(p_rows, i) for i in range(H)])
        X.check_epilogue(tally, t, list(s_ex), list(s_bd), residual[t], g1, g2, EPS, res,
                         epilogue == "sandwich")
    return [f"{label}: {m}" for m in tally.failures]


def pin_hard_rows() -> List[str]:
    """Rows where a sloppy sum of squares shows: one large element and many
    small ones whose squares an FP32 accumulator would absorb (1 + 2^-26 is
    1 in FP32), and a row spanning a wide dynamic range."""
    fails = []
    H = 512
    big_small = np.full((1, H), 2.0 ** -13, np.float32)
    big_small[0, 0] = 1.0
    wide = np.array([[2.0 ** (e % 40 - 20) * (1 if e % 3 else -1) for e in range(H)]], np.float32)
    ones = np.ones(H, np.float32)
    g = np.random.default_rng(29).uniform(0.5, 1.5, H).astype(np.float32)
    zero = np.zeros((1, H), np.uint16)
    for name, row in (("absorbed squares", big_small), ("wide range", wide)):
        p = _bf16_bits(row)
        fails += pin_exact_rows([p], zero, ones, None, "rmsnorm", f"{name}/rmsnorm")
        fails += pin_exact_rows([p], zero, g, ones, "sandwich", f"{name}/sandwich")
    return fails


# -------------------------------------------------------------- BF16 --- #

def pin_bf16() -> List[str]:
    fails = []
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_f32(allbits)
    ref = torch.from_numpy(allbits.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan_o, nan_r = np.isnan(ours), np.isnan(ref)
    if not np.array_equal(nan_o, nan_r):
        fails.append("widening: NaN set differs from torch")
    ok = ~nan_r
    if not np.array_equal(ours[ok].view(np.uint32), ref[ok].view(np.uint32)):
        fails.append("widening differs from torch on finite/inf patterns")
    # narrowing: random patterns, ties of both parities, specials
    rng = np.random.default_rng(5)
    pats = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    hi = rng.integers(0, 2 ** 16, size=1 << 16, dtype=np.uint64).astype(np.uint32)
    ties = (hi << 16) | 0x8000
    near = np.concatenate([(hi << 16) | 0x7FFF, (hi << 16) | 0x8001])
    special = np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x7F7FFFFF, 0xFF7FFFFF,
                        0x7F7F8000, 0x7F7F7FFF, 0x00000001, 0x80000001, 0x00008000,
                        0x00018000, 0x007FFFFF, 0x00800000, 0x3F808000, 0x3F818000],
                       dtype=np.uint32)
    allp = np.concatenate([pats, ties, near, special])
    vals = allp.view(np.float32)
    got = oracle.f32_to_bf16(vals)
    want = torch.from_numpy(vals.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    isnan = np.isnan(vals)
    if not np.array_equal(got[~isnan], want[~isnan]):
        bad = np.nonzero(got[~isnan] != want[~isnan])[0][:5]
        fails.append(f"narrowing differs from torch at {allp[~isnan][bad]}")
    g = got[isnan].astype(np.uint32)
    if not np.all(((g & 0x7F80) == 0x7F80) & ((g & 0x0040) != 0)):
        fails.append("narrowing: NaN is not a quiet BF16 NaN")
    if not np.array_equal(g >> 15, allp[isnan] >> 31):
        fails.append("narrowing: NaN lost its sign")
    # narrowing against the exact definition on a sample
    for b in list(allp[:2000]) + list(special):
        f = np.uint32(b).view(np.float32)
        if np.isnan(f) or np.isinf(f):
            continue
        want_v = X.bf16_round(X.to_frac(f))
        got_v = X.bf16_val(int(oracle.f32_to_bf16(np.array([f], np.float32))[0]))
        if want_v != got_v and not (want_v in (X.INF, -X.INF)):
            fails.append(f"narrowing of {float(f)!r}: {float(got_v)} vs exact {float(want_v)}")
            break
    return fails


# -------------------------------------------------- library special case --- #

def pin_library_rmsnorm() -> List[str]:
    """R=1, no finalize: residual + RMSNorm.  Also the sandwich as two
    library RMSNorms around the residual add."""
    fails = []
    for epilogue in ("rmsnorm", "sandwich"):
        d = make_case(1, 16, 512, epilogue, seed=3, row_shifts=[0, -9, 2, -11] * 4)
        res = _run(d, epilogue, debug=False)
        p = torch.from_numpy(d["src"][0].view(np.int16)).view(torch.bfloat16).double()
        x = torch.from_numpy(d["residual"].view(np.int16)).view(torch.bfloat16).double()
        g1 = torch.from_numpy(d["gamma1"]).double()
        eps32 = float(np.float32(EPS))
        if epilogue == "rmsnorm":
            h = p + x
            y = torch.nn.functional.rms_norm(h, (h.shape[-1],), weight=g1, eps=eps32)
            mask = torch.ones_like(h, dtype=torch.bool)
        else:
            g2 = torch.from_numpy(d["gamma2"]).double()
            a = torch.nn.functional.rms_norm(p, (p.shape[-1],), weight=g1, eps=eps32)
            h = a + x
            y = torch.nn.functional.rms_norm(h, (h.shape[-1],), weight=g2, eps=eps32)
            # outside heavy cancellation in a + x the FP32 path stays < 1 ulp
            mask = h.abs() > 2.0 ** -6 * a.abs()
        want_y = y.float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        want_h = h.float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        m = mask.numpy()
        for name, got, want in (("y", res.y, want_y), ("xout", res.xout, want_h)):
            dist = X.ulp_dist(got, want)[m]
            if dist.max() > 1:
                fails.append(f"{epilogue} {name}: {int(dist.max())} ulp from torch rms_norm")
            if (dist == 0).mean() < 0.99:
                fails.append(f"{epilogue} {name}: only {(dist == 0).mean():.4f} bit-equal")
    return fails


# ------------------------------------------------------ closed forms --- #

def _bf16_bits(vals) -> np.ndarray:
    return torch.tensor(np.asarray(vals, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def pin_closed_forms() -> List[str]:
    fails = []
    rng = np.random.default_rng(7)
    for H in (8, 100, 512):
        g1 = rng.uniform(0.5, 1.5, H).astype(np.float32)
        g2 = rng.uniform(0.5, 1.5, H).astype(np.float32)
        for c in (8.0, -8.0, 64.0, 2.0 ** 20):
            p = _bf16_bits(np.full((1, H), c))
            x0 = np.zeros((1, H), np.uint16)
            # residual + RMSNorm of a constant row 2^m (m >= 3): y = gamma exactly
            res = oracle.boundary([p], residual=x0, gamma1=g1, eps=EPS,
                                  epilogue=oracle.EPI_RMSNORM)
            want = _bf16_bits(np.sign(c) * g1)[None, :]
            if not np.array_equal(res.y, want):
                fails.append(f"rmsnorm constant row {c}, H={H}: y != bf16(gamma)")
            if not np.array_equal(res.xout, p):
                fails.append(f"rmsnorm constant row {c}, H={H}: xout != row")
            # sandwich: first norm of a constant row is gamma1 exactly
            res = oracle.boundary([p], residual=x0, gamma1=g1, gamma2=g2, eps=EPS,
                                  epilogue=oracle.EPI_SANDWICH, debug=True)
            if not np.array_equal(res.xout, _bf16_bits(np.sign(c) * g1)[None, :]):
                fails.append(f"sandwich constant row {c}, H={H}: xout != bf16(gamma1)")
            if not np.array_equal(res.a[0].view(np.uint32), (np.sign(c) * g1).astype(np.float32).view(np.uint32)):
                fails.append(f"sandwich constant row {c}, H={H}: a != gamma1")
        # split of two partials summing to a constant row: U is that constant
        p1 = _bf16_bits(np.full((1, H), 6.0))
        p2 = _bf16_bits(np.full((1, H), 2.0))
        res = oracle.boundary([p1, p2], residual=np.zeros((1, H), np.uint16), gamma1=g1,
                              eps=EPS, epilogue=oracle.EPI_RMSNORM, split=True, debug=True)
        if not np.array_equal(res.u, _bf16_bits(np.full((1, H), 8.0))):
            fails.append(f"split constant: U != 8, H={H}")
        if not np.array_equal(res.y, _bf16_bits(g1)[None, :]):
            fails.append(f"split constant: y != bf16(gamma), H={H}")
        # all-zero row: no NaN, y = 0, r = 1/sqrt(eps)
        z = np.zeros((1, H), np.uint16)
        res = oracle.boundary([z, z], residual=z, gamma1=g1, gamma2=g2, eps=EPS,
                              epilogue=oracle.EPI_SANDWICH, debug=True)
        if np.any(res.y != 0) or np.any(res.xout != 0):
            fails.append(f"zero row: outputs not zero, H={H}")
        r_eps = np.float32(1.0) / np.sqrt(np.float32(EPS))
        if not (res.r1[0] == r_eps and res.r2[0] == r_eps):
            fails.append(f"zero row: r != 1/sqrt(eps), H={H}")
        # eps = 0: scaling by 2^m leaves y bit-identical.  RMSNorm: scale the
        # partials and the residual (xout scales exactly).  Sandwich: scale
        # the partials only (the first norm removes the scale before the add).
        for epi in ("rmsnorm", "sandwich"):
            d = make_case(3, 4, H, epi, seed=H)
            base = _run(d, epi, debug=False, eps=0.0)
            for sh in (-5, 6):
                d2 = dict(d)
                d2["src"] = [_scale_rows(p, slice(None), sh) for p in d["src"]]
                if epi == "rmsnorm":
                    d2["residual"] = _scale_rows(d["residual"], slice(None), sh)
                res = _run(d2, epi, debug=False, eps=0.0)
                if not np.array_equal(res.y, base.y):
                    fails.append(f"{epi} eps=0 scale 2^{sh}: y changed, H={H}")
                want_x = _scale_rows(base.xout, slice(None), sh) if epi == "rmsnorm" else base.xout
                if not np.array_equal(res.xout, want_x):
                    fails.append(f"{epi} eps=0 scale 2^{sh}: xout not scaled exactly, H={H}")
    # a worked example whose every step is exact or hand-roundable:
    # h = [3, 1 x7, 0 x8] -> mean square 1; v = 1 + 8*2^-23 (eps rounds to 8
    # ulps of 1), d = 1 + 2^-21, rinv = 1 - 2^-21, y = h*rinv -> BF16 = h.
    H = 16
    hrow = np.array([3.0] + [1.0] * 7 + [0.0] * 8, np.float32)
    p0 = _bf16_bits(hrow - 0.5)[None, :]
    xr = np.full((1, H), 0.5, np.float32)
    xr[0, 8:] = 0.0
    p0[0, 8:] = _bf16_bits(np.zeros(8))
    ones = np.ones(H, np.float32)
    res = oracle.boundary([p0], residual=_bf16_bits(xr), gamma1=ones, eps=EPS,
                          epilogue=oracle.EPI_RMSNORM, debug=True)
    if res.r1[0] != np.float32(1.0 - 2.0 ** -21):
        fails.append(f"worked example: rinv {res.r1[0]!r} != 1 - 2^-21")
    if not np.array_equal(res.y[0], _bf16_bits(hrow)):
        fails.append("worked example: y != h")
    if res.y32[0, 0] != np.float32(3.0 - 6 * 2.0 ** -22):
        fails.append("worked example: y32[0] != 3 - 6*2^-22")
    return fails


# -------------------------------------------------------- invariants --- #

def pin_invariants() -> List[str]:
    fails = []
    # permuting the partials moves s by at most 2*gamma_{R-1}*sum|P|, and the
    # outputs by at most 1 ulp (usually not at all)
    d = make_case(4, 8, 320, "sandwich", seed=21)
    base = _run(d, "sandwich")
    perm = dict(d)
    perm["src"] = [d["src"][i] for i in (2, 0, 3, 1)]
    res = _run(perm, "sandwich")
    absP = sum(np.abs(oracle.bf16_to_f32(p)) for p in d["src"])
    if np.any(np.abs(res.s - base.s) > 2 * 3 * X.U * absP * 1.01):
        fails.append("permutation: s moved beyond the summation bound")
    for name in ("y", "xout"):
        dist = X.ulp_dist(getattr(res, name), getattr(base, name))
        if dist.max() > 1 or (dist == 0).mean() < 0.98:
            fails.append(f"permutation: {name} max {dist.max()} ulp, "
                         f"{(dist == 0).mean():.4f} equal")
    # a zero partial adds nothing
    z = np.zeros_like(d["src"][0])
    more = dict(d)
    more["src"] = d["src"] + [z]
    res = _run(more, "sandwich")
    for name in ("y", "xout"):
        if X.ulp_dist(getattr(res, name), getattr(base, name)).max() != 0:
            fails.append(f"zero partial changed {name}")
    # R=1 with no finalize equals the same row given as two halves? no: it
    # equals plain residual+RMSNorm on f(P0) -- checked by the library pin.
    # thread count does not change any bit
    for epi in ("rmsnorm", "sandwich"):
        d = make_case(3, 37, 128, epi, seed=5)
        a = _run(d, epi, debug=False, nthreads=1)
        b = _run(d, epi, debug=False, nthreads=5)
        if not (np.array_equal(a.y, b.y) and np.array_equal(a.xout, b.xout)):
            fails.append(f"{epi}: results depend on the thread count")
    # finalize: zero-weight slot contributes nothing, whatever its row holds
    d = make_case(2, 6, 64, "rmsnorm", k=3, shared=True, seed=8)
    w = d["topk_w"].copy()
    w[:, 1] = 0.0
    d1 = dict(d)
    d1["topk_w"] = w
    d1["src"] = [e.copy() for e in d["src"]]
    for e in d1["src"]:
        e[d["topk_idx"][:, 1]] = _bf16_bits(np.full(64, 1.5e38))
    d2 = dict(d)
    d2["topk_w"] = np.ascontiguousarray(w[:, [0, 2]])
    d2["topk_idx"] = np.ascontiguousarray(d["topk_idx"][:, [0, 2]])
    a, b = _run(d1, "rmsnorm", debug=False), _run(d2, "rmsnorm", debug=False)
    for name in ("y", "xout"):
        if X.ulp_dist(getattr(a, name), getattr(b, name)).max() != 0:
            fails.append(f"zero-weight slot changed {name}")
    # k=1, weight 1, no shared: finalize is a gather, the rest a plain reduce
    d = make_case(3, 5, 96, "sandwich", k=1, shared=False, seed=9)
    d["topk_w"] = np.ones_like(d["topk_w"])
    a = _run(d, "sandwich", debug=False)
    plain = dict(d)
    plain["src"] = [np.ascontiguousarray(e[d["topk_idx"][:, 0]]) for e in d["src"]]
    plain.pop("topk_w")
    plain.pop("topk_idx")
    b = _run(plain, "sandwich", debug=False)
    if not (np.array_equal(a.y, b.y) and np.array_equal(a.xout, b.xout)):
        fails.append("k=1, w=1: finalize is not the plain gather")
    # zero weights with a shared expert: the partials are the shared rows
    d = make_case(2, 5, 96, "rmsnorm", k=4, shared=True, seed=10)
    d["topk_w"] = np.zeros_like(d["topk_w"])
    a = _run(d, "rmsnorm", debug=False)
    plain = dict(d)
    plain["src"] = d["shared"]
    plain.pop("topk_w")
    plain.pop("topk_idx")
    plain["shared"] = None
    b = _run(plain, "rmsnorm", debug=False)
    if X.ulp_dist(a.y, b.y).max() != 0 or X.ulp_dist(a.xout, b.xout).max() != 0:
        fails.append("w=0 with shared: partials are not the shared rows")
    # fused finalize equals finalize materialized to BF16, then plain reduce
    d = make_case(3, 6, 64, "sandwich", k=3, shared=True, seed=12)
    a = _run(d, "sandwich", debug=True)
    plain = dict(d)
    plain["src"] = [np.ascontiguousarray(a.p[r]) for r in range(3)]
    plain.pop("topk_w")
    plain.pop("topk_idx")
    plain["shared"] = None
    b = _run(plain, "sandwich", debug=False)
    if not (np.array_equal(a.y, b.y) and np.array_equal(a.xout, b.xout)):
        fails.append("fused finalize differs from the materialized one")
    # split: pass 2 is the R=1 boundary on U
    for epi in ("rmsnorm", "sandwich"):
        d = make_case(3, 6, 64, epi, seed=13)
        a = _run(d, epi, split=True, debug=True)
        one = dict(d)
        one["src"] = [a.u]
        b = _run(one, epi, debug=False)
        if not (np.array_equal(a.y, b.y) and np.array_equal(a.xout, b.xout)):
            fails.append(f"split {epi}: pass 2 differs from the R=1 boundary on U")
        u_only = oracle.boundary(d["src"], epilogue=oracle.EPI_NONE)
        if not np.array_equal(u_only.u, a.u):
            fails.append(f"split {epi}: pass 1 alone differs")
    # an index outside the expert buffer turns that token's row into NaN
    d = make_case(2, 4, 64, "rmsnorm", k=2, shared=True, seed=14)
    nr = d["src"][0].shape[0]
    bad = d["topk_idx"].copy()
    bad[2, 1] = nr
    bad[3, 0] = -1
    d1 = dict(d)
    d1["topk_idx"] = bad
    a = _run(d1, "rmsnorm", debug=False)
    b = _run(d, "rmsnorm", debug=False)
    ya = oracle.bf16_to_f32(a.y)
    if not (np.all(np.isnan(ya[2:])) and np.array_equal(a.y[:2], b.y[:2])):
        fails.append("out-of-range index: row not NaN, or other rows touched")
    return fails


# ------------------------------------------------- contraction probes --- #

def contraction_probe_finalize(H=64):
    """Inputs where slot 1's product is inexact and slot 0 cancels its
    rounded value: uncontracted, the finalize is exactly 0 (so with a zero
    residual the whole row normalises to 0); contracted into an FMA it is
    the product's rounding error, which RMSNorm blows up to +-gamma."""
    rng = np.random.default_rng(17)
    w1 = np.float32(rng.uniform(0.3, 0.7))
    while float(w1) * 1.8125 == float(np.float32(w1 * np.float32(1.8125))):
        w1 = np.nextafter(w1, np.float32(1))
    e1 = 1.8125  # BF16-exact, product with w1 is inexact in FP32
    q = np.float32(w1 * np.float32(e1))
    rows = np.zeros((2, H), np.uint16)
    rows[0] = _bf16_bits(np.full(H, -1.0))
    rows[1] = _bf16_bits(np.full(H, e1))
    w = np.array([[q, w1]], np.float32)
    idx = np.array([[0, 1]], np.int32)
    return dict(src=[rows], topk_w=w, topk_idx=idx, shared=None,
                residual=np.zeros((1, H), np.uint16),
                gamma1=np.ones(H, np.float32), gamma2=None)


def contraction_probe_sandwich(r1: float, s_row: np.ndarray, H: int):
    """Given the FP32 s row and its r1, choose gamma1 and the residual so that
    q*gamma1 is inexact and the residual cancels its rounded value:
    uncontracted h = 0 exactly; contracted, h is the rounding error."""
    rng = np.random.default_rng(19)
    q = (s_row.astype(np.float32) * np.float32(r1)).astype(np.float32)
    g1 = np.empty(H, np.float32)
    xr = np.empty(H, np.float32)
    for i in range(H):
        if q[i] == 0:  # nothing to probe: h = 0 + 0
            g1[i], xr[i] = 1.0, 0.0
            continue
        found = None
        for _attempt in range(32):  # target b: a BF16 value of the sign of q
            b = float(torch.tensor(float(rng.uniform(0.5, 1.5)) * np.sign(q[i])).to(torch.bfloat16))
            g0 = np.float32(b / float(q[i]))
            for g in (g0, np.nextafter(g0, np.float32(np.inf)), np.nextafter(g0, np.float32(-np.inf))):
                prod = float(q[i]) * float(g)  # exact in binary64
                if np.float32(prod) == np.float32(b) and prod != b:
                    found = g
                    break
            if found is not None:
                break
        if found is None:
            # q is a power of two: every product is exact; keep h = 0 exactly
            assert float(q[i]) * float(g0) == b, "probe construction failed"
            found = g0
        g1[i] = found
        xr[i] = -b
    return g1, _bf16_bits(xr)[None, :]


def pin_contraction() -> List[str]:
    fails = []
    H = 64
    d = contraction_probe_finalize(H)
    res = _run(d, "rmsnorm", debug=True)
    if np.any(res.p != 0):
        fails.append("finalize probe: P != 0, the weighted sum was contracted")
    if np.any(res.y != 0):
        fails.append("finalize probe: y != 0")
    # sandwich probe
    p = _bf16_bits(np.random.default_rng(23).normal(0, 1, H))[None, :]
    g2 = np.ones(H, np.float32)
    first = oracle.boundary([p], residual=np.zeros((1, H), np.uint16),
                            gamma1=np.ones(H, np.float32), gamma2=g2, eps=EPS,
                            epilogue=oracle.EPI_SANDWICH, debug=True)
    g1, xr = contraction_probe_sandwich(first.r1[0], first.s[0], H)
    res = oracle.boundary([p], residual=xr, gamma1=g1, gamma2=g2, eps=EPS,
                          epilogue=oracle.EPI_SANDWICH, debug=True)
    if np.any(res.h != 0) or np.any(res.xout != 0) or np.any(res.y != 0):
        fails.append("sandwich probe: h != 0, (s*r1)*gamma1 + x was contracted")
    return fails


def all_pins(quick: bool = False) -> List[str]:
    fails = []
    cases = EXACT_CASES[::3] if quick else EXACT_CASES
    for c in cases:
        fails += [f"exact {c}: {m}" for m in pin_exact(c)]
    fails += pin_hard_rows()
    fails += pin_bf16()
    fails += pin_library_rmsnorm()
    fails += pin_closed_forms()
    fails += pin_invariants()
    fails += pin_contraction()
    from tests import pin_ep  # the expert-parallel finalize's pins
    fails += pin_ep.all_ep_pins(quick=quick)
    return fails
