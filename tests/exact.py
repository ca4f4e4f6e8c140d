"""Exact real-number model of the boundary, used to pin the CPU oracle.

Nothing here shares code with the oracle's C source.  Sums and products are
exact rationals (``fractions.Fraction``); the square root and everything
after it run in ``mpmath`` at 256 bits; rounding to bfloat16 is written from
the IEEE 754 definition (nearest, ties to even) on exact rationals.

The model follows the definition of the method, not the oracle's operation
order: the finalize is the exact weighted sum plus the shared expert, rounded
once to BF16 (the BF16 rounding on each rank is part of the method, vLLM PR
#62366 "Claims"); the reduction is the exact sum of the partials; RMSNorm is
x / sqrt(mean(x^2) + eps) * gamma with exact arithmetic.

The oracle computes in FP32 with one rounding per operation, so its results
differ from the exact ones by rounding error.  For every intermediate this
module derives a first-order absolute error bound (standard error analysis,
unit roundoff u = 2^-24, inflated by 25% and by a few u to cover
second-order terms) and checks:

* the oracle's FP32 debug value lies within the bound of the exact value;
* where the whole bound interval rounds to one BF16 value, the oracle's BF16
  output IS that value, bit for bit; elsewhere it is within one BF16 ulp.

To avoid one legitimate 1-ulp flip cascading, each stage is fed with the
oracle's own output of the previous stage (step-wise checking): the reduction
starts from the oracle's finalized partials, the split pass 2 from its BF16
pass-1 tensor.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from fractions import Fraction
from typing import List, Optional

import mpmath
import numpy as np

mpmath.mp.prec = 256
U = 2.0 ** -24          # binary32 unit roundoff
U64 = 2.0 ** -53        # binary64 unit roundoff
INF = float("inf")


# ------------------------------------------------------------ rounding --- #

def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_binary(q: Fraction, p: int, emin: int = -126, emax: int = 127):
    """Round an exact rational to a binary format with p significand bits
    (nearest, ties to even; gradual underflow; overflow to +-inf)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = max(_floor_log2(a), emin)
    ulp = Fraction(2) ** (e - p + 1)
    m = a / ulp
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    res = n * ulp
    if res > (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax:
        return sign * INF
    return sign * res


def bf16_round(q: Fraction):
    return round_binary(q, 8)


def bf16_bits_of(v) -> int:
    """Bit pattern of a value that is exactly representable in BF16."""
    f = np.float32(float(v))
    b = int(f.view(np.uint32))
    assert b & 0xFFFF == 0, "value is not a BF16 number"
    return b >> 16


def bf16_ord(bits) -> np.ndarray:
    """Monotone integer image of BF16 bit patterns, +0 and -0 both 0."""
    b = np.asarray(bits, dtype=np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def ulp_dist(a_bits, b_bits) -> np.ndarray:
    return np.abs(bf16_ord(a_bits) - bf16_ord(b_bits))


def to_frac(x) -> Fraction:
    return Fraction(float(x))


def mp_to_frac(x) -> Fraction:
    """Exact rational value of an mpf (sign, mantissa, exponent)."""
    sign, man, exp, _ = mpmath.mpf(x)._mpf_
    man = -int(man) if sign else int(man)
    exp = int(exp)
    return Fraction(man) * Fraction(2) ** exp if exp >= 0 else Fraction(man, 2 ** (-exp))


def bf16_val(bits: int):
    """Exact value of a BF16 bit pattern (a Fraction; +-inf and NaN as a float)."""
    f = np.uint32(int(bits) << 16).view(np.float32)
    if not np.isfinite(f):
        return float(f)
    return to_frac(f)


# ------------------------------------------------------------- checking --- #

@dataclass
class Tally:
    """Counts of checked BF16 outputs."""
    decided: int = 0        # bound interval inside one rounding cell: bit-exact
    undecided: int = 0      # interval straddles a rounding boundary: <= 1 ulp
    failures: List[str] = field(default_factory=list)

    def fail(self, msg: str):
        if len(self.failures) < 20:
            self.failures.append(msg)
        else:
            self.failures.append("...")

    def ok(self) -> bool:
        return not self.failures


def check_fp32(tally: Tally, label: str, got, exact, bound: float):
    ex = mpf_of(exact)
    err = abs(float(mpmath.mpf(float(got)) - ex))
    if not err <= bound:
        tally.fail(f"{label}: FP32 {float(got)!r} vs exact {float(ex)!r}: "
                   f"|err| {err:.3e} > bound {bound:.3e}")


def check_bf16(tally: Tally, label: str, got_bits: int, exact, bound: float):
    """exact: Fraction or mpf; bound: absolute bound on the oracle's FP32
    value before rounding."""
    if np.isnan(np.uint32(int(got_bits) << 16).view(np.float32)):
        tally.fail(f"{label}: BF16 NaN where a finite value is defined")
        return
    ex = mp_to_frac(exact) if not isinstance(exact, Fraction) else exact
    bnd = Fraction(bound)
    if bnd == 0:  # the FP32 value is exact: its rounding is fully decided
        lo = hi = bf16_round(ex)
    else:
        lo = bf16_round(ex - bnd)
        hi = bf16_round(ex + bnd)
    got = bf16_val(got_bits)
    if lo == hi:
        tally.decided += 1
        if got != lo:
            tally.fail(f"{label}: BF16 {float(got)!r} but every value within the "
                       f"bound of exact {float(ex)!r} rounds to {float(lo)!r}")
    else:
        tally.undecided += 1
        want = bf16_round(ex)
        d = abs(int(bf16_ord(bf16_bits_of(got))) - int(bf16_ord(bf16_bits_of(want))))
        if d > 1:
            tally.fail(f"{label}: BF16 {float(got)!r} is {d} ulp from exact "
                       f"{float(ex)!r}")


# ------------------------------------------------------ stage models --- #

def inv_rms_model(x_exact: List, x_bound: List[float], eps32: float):
    """Exact inverse RMS of a row with known per-element bounds on the
    values the oracle actually squares.  Returns (r_exact (mpf), rel_bound)."""
    H = len(x_exact)
    xs = [mpmath.mpf(v) if not isinstance(v, Fraction) else
          mpmath.mpf(v.numerator) / v.denominator for v in x_exact]
    sq = mpmath.fsum(v * v for v in xs)
    ms = sq / H
    v = ms + mpmath.mpf(to_frac(np.float32(eps32)).numerator) / to_frac(np.float32(eps32)).denominator
    r = 1 / mpmath.sqrt(v)
    # relative error of the oracle's sum of squares (its x carry errors)
    if sq == 0:
        rho_ms = 0.0
    else:
        cross = sum(2 * abs(float(a)) * b + b * b for a, b in zip(xs, x_bound))
        rho_ms = cross / float(sq) + H * U64 + U
    rho_v = float(ms) * rho_ms / float(v) + U
    rho_r = 1.25 * (rho_v / 2 + 2 * U) + 1e-3 * U
    return r, rho_r


def mpf_of(q) -> mpmath.mpf:
    if isinstance(q, Fraction):
        return mpmath.mpf(q.numerator) / q.denominator
    return mpmath.mpf(q)


def check_epilogue(tally: Tally, t: int, s_exact: List, s_bound: List[float],
                   x_bits: np.ndarray, g1: np.ndarray, g2: Optional[np.ndarray],
                   eps: float, res, sandwich: bool):
    """Check one row of the oracle's epilogue against the exact model.

    s_exact/s_bound: exact reduced sum fed in and the bound on the oracle's
    FP32 s.  res: oracle Result with debug arrays.
    """
    H = len(s_exact)
    x = [bf16_val(b) for b in x_bits]
    if sandwich:
        r1, rho1 = inv_rms_model(s_exact, s_bound, eps)
        check_fp32(tally, f"r1[{t}]", res.r1[t], r1, rho1 * float(r1))
        a_ex, a_bd = [], []
        for i in range(H):
            s_i = mpf_of(s_exact[i])
            a_i = s_i * r1 * mpf_of(to_frac(g1[i]))
            bd = 1.25 * (abs(float(g1[i])) * float(r1) * (s_bound[i] + abs(float(s_i)) * rho1)
                         + 2 * U * abs(float(a_i))) + 1e-45
            check_fp32(tally, f"a[{t},{i}]", res.a[t, i], a_i, bd)
            a_ex.append(a_i)
            a_bd.append(bd)
        h_ex = [a_ex[i] + mpf_of(x[i]) for i in range(H)]
        h_bd = [a_bd[i] + 1.25 * U * (abs(float(h_ex[i])) + a_bd[i]) for i in range(H)]
        gam = g2
    else:
        h_ex = [mpf_of(s_exact[i]) + mpf_of(x[i]) for i in range(H)]
        h_bd = []
        for i in range(H):
            if s_bound[i] == 0:
                # s is exact, so h is one IEEE addition of known operands
                hq = s_exact[i] + x[i]
                h_bd.append(float(abs(round_binary(hq, 24) - hq)))
            else:
                h_bd.append(s_bound[i] + 1.25 * U * (abs(float(h_ex[i])) + s_bound[i]))
        gam = g1
    for i in range(H):
        check_fp32(tally, f"h[{t},{i}]", res.h[t, i], h_ex[i], h_bd[i])
        check_bf16(tally, f"xout[{t},{i}]", int(res.xout[t, i]), h_ex[i], h_bd[i])
    r2, rho2 = inv_rms_model(h_ex, h_bd, eps)
    rr = res.r2[t] if sandwich else res.r1[t]
    check_fp32(tally, f"r_out[{t}]", rr, r2, rho2 * float(r2))
    for i in range(H):
        y_i = h_ex[i] * r2 * mpf_of(to_frac(gam[i]))
        bd = 1.25 * (abs(float(gam[i])) * float(r2) * (h_bd[i] + abs(float(h_ex[i])) * rho2)
                     + 2 * U * abs(float(y_i))) + 1e-45
        check_fp32(tally, f"y32[{t},{i}]", res.y32[t, i], y_i, bd)
        check_bf16(tally, f"y[{t},{i}]", int(res.y[t, i]), y_i, bd)


def exact_reduce(p_rows: List[np.ndarray], i: int):
    """Exact sum of the partials' element i and the bound on the oracle's
    recursive FP32 sum (gamma_{R-1} * sum |P_r|)."""
    vals = [bf16_val(p[i]) for p in p_rows]
    R = len(vals)
    ex = sum(vals, Fraction(0))
    if R == 2:
        # one IEEE addition: its error is exactly |RN32(exact) - exact|
        bd = float(abs(round_binary(ex, 24) - ex))
    else:
        bd = 1.25 * (R - 1) * U * float(sum(abs(v) for v in vals))
    return ex, bd


def exact_finalize(rows: np.ndarray, shared_row: Optional[np.ndarray], w: np.ndarray,
                   idx: np.ndarray, i: int):
    """Exact finalize value of element i and the bound on the oracle's FP32
    accumulator (gamma_{k+1} * sum |terms|)."""
    terms = [to_frac(w[j]) * bf16_val(rows[int(idx[j]), i]) for j in range(len(w))]
    if shared_row is not None:
        terms.append(bf16_val(shared_row[i]))
    ex = sum(terms, Fraction(0))
    n = len(terms)
    bd = 1.25 * (n + 1) * U * float(sum(abs(t) for t in terms))
    return ex, bd
