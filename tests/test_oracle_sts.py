"""The STS / ECE oracle against what fixes it independently (CPU only):
hand-worked ECE values, closed-form temperatures (a constant logit whose
sigmoid hits the label rate exactly, position by position, so the second
position's temperature only comes out right if the first position's
calibrated value is used), the all-accepted and none-accepted limits,
causality (later positions never move earlier temperatures), rank
preservation, and recovery of a planted overconfidence factor."""
import math

import numpy as np

import workloads
from oracle import sts


def test_hand_worked_ece():
    a = np.array([0.1, 0.4, 0.6, 0.9])
    y = np.array([0.0, 1.0, 1.0, 1.0])
    # two bins: [0.1, 0.4] -> |0.1 + (0.4 - 1)| = 0.5; [0.6, 0.9] -> |-0.4 - 0.1| = 0.5
    assert math.isclose(sts.ece(a, y, 2), (0.5 + 0.5) / 4, abs_tol=1e-15)
    # one bin: |(0.1 + 0.4 + 0.6 + 0.9) - 3| / 4
    assert math.isclose(sts.ece(a, y, 1), 0.25, abs_tol=1e-15)
    # ten bins, every value alone: (0.1 + 0.6 + 0.4 + 0.1) / 4
    assert math.isclose(sts.ece(a, y, 10), 1.2 / 4, abs_tol=1e-15)
    # a value of exactly 1 lands in the last bin: bins 9 -> |1 + (0.95 - 1)|,
    # 0 -> |0.05|
    assert math.isclose(sts.ece(np.array([1.0, 0.95, 0.05]), np.array([0.0, 1.0, 0.0]), 10),
                        1.0 / 3, abs_tol=1e-15)


def _blocks(rates, N=8):
    """Accepted lengths so that the fraction of blocks with A >= k is rates[k-1]."""
    A = np.zeros(N, np.int32)
    for k, r in enumerate(rates, start=1):
        A[: int(round(r * N))] = k
    return A


def test_closed_form_temperatures_are_sequential():
    # position 1: z = 2 ln 3, 3/4 of the blocks pass: sigmoid(z / 2) = 3/4 exactly
    # position 2: z = 2 ln 2, 1/2 pass: with a_1 = 3/4, sigmoid(z / 2) = 2/3
    # gives a_2 = 1/2; from the raw a_1 = sigmoid(2 ln 3) = 0.9 it would take
    # t = 2 ln 2 / ln(5/4) ~ 6.2 instead
    N = 8
    z = np.zeros((N, 2), np.float32)
    z[:, 0] = 2.0 * math.log(3.0)
    z[:, 1] = 2.0 * math.log(2.0)
    A = _blocks([0.75, 0.5], N)
    grid = np.array([0.5, 1.0, 2.0, 4.0, 6.0, 8.0])
    out = sts.sts_calibrate(z, A, grid, bins=1)
    assert list(out["temperatures"]) == [2.0, 2.0]
    assert out["ece"][0] < 1e-7 and out["ece"][1] < 1e-7


def test_all_accepted_prefers_the_smallest_temperature():
    # every block passes every position: ECE = 1 - mean(a), so the sharpest
    # scores win for positive logits
    g = np.random.default_rng(0)
    z = g.uniform(0.5, 3.0, size=(50, 3)).astype(np.float32)
    A = np.full(50, 3, np.int32)
    grid = np.array([0.3, 0.6, 1.0, 2.0])
    out = sts.sts_calibrate(z, A, grid, bins=15)
    assert np.all(out["temperatures"] == 0.3)
    a = np.ones(50)
    for k in range(3):
        a = a * (1.0 / (1.0 + np.exp(-z[:, k].astype(np.float64) / 0.3)))
        assert math.isclose(out["ece"][k], 1.0 - a.mean(), rel_tol=1e-12)


def test_none_accepted_prefers_the_largest_temperature():
    # no block passes: ECE = mean(a); positive logits are flattest at the largest t
    z = np.full((20, 2), 1.5, np.float32)
    A = np.zeros(20, np.int32)
    grid = np.array([0.5, 1.0, 4.0])
    out = sts.sts_calibrate(z, A, grid, bins=7)
    assert np.all(out["temperatures"] == 4.0)
    s = 1.0 / (1.0 + math.exp(-1.5 / 4.0))
    assert math.isclose(out["ece"][0], s, rel_tol=1e-12)
    assert math.isclose(out["ece"][1], s * s, rel_tol=1e-12)


def test_ties_take_the_first_grid_point():
    z = np.zeros((4, 1), np.float32)           # sigmoid(0 / t) = 1/2 for every t
    A = np.array([1, 1, 0, 0], np.int32)
    out = sts.sts_calibrate(z, A, np.array([3.0, 1.0, 2.0]), bins=4)
    assert out["temperatures"][0] == 3.0 and out["ece"][0] == 0.0


def test_later_positions_do_not_move_earlier_temperatures():
    c = workloads.sts_case(seed=3, N=600, gamma=4, G=24)
    base = sts.sts_calibrate(c.z, c.accepted, c.grid)
    z2 = c.z.copy()
    z2[:, 2:] = -z2[:, 2:] * 3.0
    A2 = np.where(c.accepted >= 2, 4, c.accepted).astype(np.int32)  # same [A >= 1], [A >= 2]
    other = sts.sts_calibrate(z2, A2, c.grid)
    np.testing.assert_array_equal(base["temperatures"][:2], other["temperatures"][:2])
    np.testing.assert_array_equal(base["ece"][:2], other["ece"][:2])


def test_temperature_keeps_the_ranking():
    g = np.random.default_rng(1)
    z = g.normal(0, 2, size=200)
    for t in (0.3, 1.0, 5.0):
        np.testing.assert_array_equal(np.argsort(z, kind="stable"),
                                      np.argsort(sts.sigmoid(z / t), kind="stable"))


def test_recovers_a_planted_overconfidence():
    # one position, raw logit = 2 * true logit, labels drawn from the truth:
    # the calibrated temperature lands near 2 and beats the raw scores
    g = np.random.default_rng(5)
    N = 40000
    lg = g.normal(0.5, 1.5, size=N)
    y = g.random(N) < 1.0 / (1.0 + np.exp(-lg))
    z = (2.0 * lg).astype(np.float32)[:, None]
    grid = np.exp(np.linspace(np.log(0.25), np.log(8.0), 61))
    out = sts.sts_calibrate(z, y.astype(np.int32), grid, bins=15)
    assert 1.7 < out["temperatures"][0] < 2.35
    raw = sts.ece(sts.sigmoid(z[:, 0].astype(np.float64)), y.astype(np.float64), 15)
    assert out["ece"][0] < 0.4 * raw


def test_workload_is_overconfident_and_calibration_helps():
    c = workloads.sts_case(seed=10, N=4096, gamma=7, G=64)
    assert c.accepted.min() >= 0 and c.accepted.max() <= 7
    raw = sts.sts_calibrate(c.z, c.accepted, np.array([1.0]))
    cal = sts.sts_calibrate(c.z, c.accepted, c.grid)
    assert raw["ece"].mean() > 0.03           # several percent before
    assert cal["ece"].mean() < 0.5 * raw["ece"].mean()
    assert np.all(cal["temperatures"] > 1.0)  # overconfident head: t > 1
