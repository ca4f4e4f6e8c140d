"""The CPU oracle against what the pages and the mathematics fix.

No page prints a worked numeric example for this path, so the oracle is
pinned by exact arithmetic with error bounds, a library special case, closed
forms, invariants and contraction probes (see tests/pin_battery.py).
"""
import pytest

from tests import pin_battery as B


@pytest.mark.parametrize("case", B.EXACT_CASES, ids=lambda c: "R{}_T{}_H{}_{}_k{}{}{}".format(
    c[0], c[1], c[2], c[3], c[4], "_shared" if c[5] else "", "_split" if c[6] else ""))
def test_exact_arithmetic(case):
    fails = B.pin_exact(case)
    assert not fails, "\n".join(fails)


def test_exact_arithmetic_hard_rows():
    fails = B.pin_hard_rows()
    assert not fails, "\n".join(fails)


def test_bf16_conversions_match_torch():
    fails = B.pin_bf16()
    assert not fails, "\n".join(fails)


def test_library_rmsnorm_special_case():
    fails = B.pin_library_rmsnorm()
    assert not fails, "\n".join(fails)


def test_closed_forms():
    fails = B.pin_closed_forms()
    assert not fails, "\n".join(fails)


def test_invariants():
    fails = B.pin_invariants()
    assert not fails, "\n".join(fails)


def test_no_fma_contraction():
    fails = B.pin_contraction()
    assert not fails, "\n".join(fails)


@pytest.mark.parametrize("case", __import__("tests.pin_ep", fromlist=["x"]).EP_EXACT_CASES,
                         ids=lambda c: "ep_R{}_T{}_H{}_{}_k{}_of{}_shared{}".format(*c))
def test_ep_exact_arithmetic(case):
    from tests import pin_ep as E
    fails = E.pin_ep_exact(case)
    assert not fails, "\n".join(fails)


def test_ep_closed_forms():
    from tests import pin_ep as E
    fails = E.pin_ep_closed_forms()
    assert not fails, "\n".join(fails)


def test_ep_invariants():
    from tests import pin_ep as E
    fails = E.pin_ep_invariants()
    assert not fails, "\n".join(fails)


def test_ep_no_fma_contraction():
    from tests import pin_ep as E
    fails = E.pin_ep_contraction()
    assert not fails, "\n".join(fails)
