"""Pins of the oracle's flow-shifted noise schedule (CPU only).

The shift map of "Cosmos 3 方法原理全解" §6.3 is pinned by what fixes it
without retyping it: its end points, its reduction to the linear schedule at
s = 1, the direction the page gives it (towards high noise), its odds form
(a pure scaling by s, so two shifts compose by multiplying), and the exact
landing of the Euler sampler on the rectified-flow path (§6.3, §7.2).  The
cases are the step counts and shifts of the page's §12.1 table.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import euler, schedule

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "recommended_sampler_settings.json")
SETTINGS = json.load(open(GOLDEN, encoding="utf-8"))["settings"]
CASES = sorted({(s["steps"], float(s["shift"])) for s in SETTINGS}
               | {(1, 5.0), (3, 2.5), (10, 1.0), (7, 0.25), (16, 7.5)})


def _ids(c):
    return "n%d_s%g" % c


def test_golden_table_holds_the_policy_row():
    rows = [s for s in SETTINGS if s["steps"] == 4]
    assert rows and rows[0]["shift"] == 5 and rows[0]["guidance"] == [3]
    assert {s["shift"] for s in SETTINGS} == {3, 5, 10}


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_end_points_and_strict_decrease(case):
    n, s = case
    sig = schedule.shifted_schedule(n, s)
    assert len(sig) == n + 1
    assert sig[0] == pytest.approx(1.0, abs=1e-15) and sig[-1] == 0.0
    assert all(a > b for a, b in zip(sig[:-1], sig[1:]))


@pytest.mark.parametrize("n", [1, 4, 10, 50])
def test_unit_shift_is_the_linear_schedule(n):
    sig = schedule.shifted_schedule(n, 1.0)
    for k, x in enumerate(sig):
        assert Fraction(x) == Fraction(n - k, n) or abs(Fraction(x) - Fraction(n - k, n)) < Fraction(1, 2**52)
    np.testing.assert_allclose(sig, euler.linear_schedule(n), rtol=0, atol=1e-15)


@pytest.mark.parametrize("case", [c for c in CASES if c[1] != 1.0], ids=_ids)
def test_shift_moves_interior_points_the_way_the_page_says(case):
    # §6.3: the shift biases sampling towards high noise for s > 1, and the
    # other way for s < 1; the ends stay where they are.
    n, s = case
    sig = schedule.shifted_schedule(n, s)
    for k in range(1, n):
        lin = 1.0 - k / n
        assert (sig[k] > lin) if s > 1 else (sig[k] < lin)


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_odds_form_is_a_scaling_by_the_shift(case):
    # σ/(1-σ) = s·t̄/(1-t̄): from the exact odds, σ = odds/(1+odds) exactly.
    n, s = case
    sig = schedule.shifted_schedule(n, s)
    for k in range(1, n):
        odds = Fraction(s) * Fraction(n - k, k)
        exact = odds / (1 + odds)
        assert abs(Fraction(sig[k]) - exact) <= 4 * Fraction(2.0 ** -53)


def test_two_shifts_compose_by_multiplying():
    for s1, s2 in [(2.0, 5.0), (10.0, 0.5), (3.0, 3.0)]:
        for tb in (0.1, 0.25, 0.5, 0.9):
            once = schedule.shift_sigma(tb, s1 * s2)
            twice = schedule.shift_sigma(schedule.shift_sigma(tb, s2), s1)
            assert once == pytest.approx(twice, rel=1e-14)


@pytest.mark.parametrize("s", [3.0, 5.0, 10.0])
def test_midpoint_closed_form(s):
    # t̄ = 1/2: σ = s / (s + 1); 4 steps, shift 5 gives 1, 15/16, 5/6, 5/8, 0.
    assert schedule.shifted_schedule(2, s)[1] == pytest.approx(s / (s + 1), rel=1e-15)
    assert schedule.shifted_schedule(4, 5.0) == pytest.approx([1.0, 15 / 16, 5 / 6, 5 / 8, 0.0],
                                                              rel=1e-15, abs=0)


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_euler_on_the_flow_path_lands_on_the_data(case):
    # §6.3 / §7.2: with the true velocity, any schedule from 1 to 0 ends on x0.
    n, s = case
    rng = np.random.default_rng(n)
    eps, x0 = rng.standard_normal(32), rng.standard_normal(32)
    sig = schedule.shifted_schedule(n, s)
    x = euler.flow_path(eps, x0, sig[0])
    for a, b in zip(sig[:-1], sig[1:]):
        x = np.asarray(x, np.float64) + (b - a) * euler.true_velocity(eps, x0)
    np.testing.assert_allclose(x, x0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("bad", [(0, 5.0), (4, 0.0), (4, -1.0), (4, float("inf")), (4, float("nan"))])
def test_bad_arguments_raise(bad):
    with pytest.raises(ValueError):
        schedule.shifted_schedule(*bad)
