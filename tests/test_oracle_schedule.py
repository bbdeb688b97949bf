"""The scheduler oracle against what the DSpark "scheduler" section fixes
(CPU only): the greedy optimum against brute force over every length vector,
the top-K variant against the best sum of K survival probabilities, the
early stop at the first drop of Theta (also when the cost curve has a later,
higher peak), prefix-closed lengths, and the degenerate tables."""
import math

import numpy as np
import pytest

from oracle import schedule as sch


def smooth_sps(bmax, scale=40.0):
    """A step-rate curve that falls smoothly with the batch size."""
    B = np.arange(bmax + 1, dtype=np.float64)
    return (1000.0 / (1.0 + B / scale)).astype(np.float32)


def test_survival_is_left_to_right_fp32_product():
    c = np.array([[0.5, 0.5, 0.25], [1.0, 0.1, 0.9]], np.float32)
    a = sch.survival(c)
    assert a.dtype == np.float32
    assert a.tolist() == [[0.5, 0.25, 0.0625], [1.0, np.float32(0.1), np.float32(np.float32(0.1) * np.float32(0.9))]]


def test_hand_case():
    # two requests; a = [[.9, .45], [.6, .06]]; pool order .9 (0,1), .6 (1,1), .45 (0,2), .06 (1,2)
    c = np.array([[0.9, 0.5], [0.6, 0.1]], np.float32)
    sps = np.array([0, 0, 100, 90, 60, 55, 50], np.float32)
    # B=2 tau=2 -> 200; +.9: B3 tau2.9 -> 261; +.6: B4 tau3.5 -> 210 (drop) -> stop
    res = sch.schedule(c, sps)
    assert res["len"].tolist() == [1, 0]
    assert res["admitted"] == 1
    assert math.isclose(res["theta"], (2.0 + float(np.float32(0.9))) * 90.0, rel_tol=1e-15)
    top = sch.schedule(c, sps, topk=3)
    assert top["len"].tolist() == [2, 1]


@pytest.mark.parametrize("seed", range(12))
def test_greedy_equals_brute_force_on_unimodal_curves(seed):
    rng = np.random.default_rng(seed)
    R, G = 3, 3
    c = rng.uniform(0.05, 1.0, size=(R, G)).astype(np.float32)
    sps = smooth_sps(R * (G + 1) + 2, scale=float(rng.uniform(2.0, 30.0)))
    res = sch.schedule(c, sps)
    best, arg = sch.brute_force_best(c, sps)
    assert math.isclose(res["theta"], best, rel_tol=1e-12), (res, best, arg)


@pytest.mark.parametrize("seed", range(6))
def test_topk_maximises_tau_for_its_batch(seed):
    rng = np.random.default_rng(100 + seed)
    R, G = 3, 3
    c = rng.uniform(0.0, 1.0, size=(R, G)).astype(np.float32)
    a = sch.survival(c)
    flat = sorted(a.ravel().tolist(), reverse=True)
    sps = np.ones(R * (G + 1) + 1, np.float32)
    for K in range(R * G + 1):
        res = sch.schedule(c, sps, topk=K)
        assert res["admitted"] == K
        assert int(res["len"].sum()) == K
        tau = float(R) + sum(float(a[r, j]) for r in range(R) for j in range(res["len"][r]))
        assert math.isclose(tau, float(R) + sum(flat[:K]), rel_tol=1e-12)


def test_stops_at_first_drop_even_with_a_later_peak():
    # a cliff in the step-rate table: Theta drops at B = R + 2, then a later
    # batch is much faster; the early stop must not look past the drop
    R, G = 2, 3
    c = np.full((R, G), 0.99, np.float32)
    sps = np.array([0, 0, 100, 100, 40, 1000, 1000, 1000, 1000], np.float32)
    res = sch.schedule(c, sps)
    assert res["admitted"] == 1
    best, _ = sch.brute_force_best(c, sps)
    assert best > res["theta"]


def test_lengths_are_prefixes_and_ties_follow_request_order():
    c = np.ones((4, 5), np.float32)  # every a is 1: the order is (r, j) ascending
    sps = np.ones(4 * 6 + 1, np.float32)
    top = sch.schedule(c, sps, topk=7)
    assert top["len"].tolist() == [5, 2, 0, 0]
    full = sch.schedule(c, sps)  # constant rate, a = 1: every admission raises Theta
    assert full["len"].tolist() == [5, 5, 5, 5]


def test_zero_confidence_admits_nothing_on_a_falling_curve():
    c = np.zeros((3, 4), np.float32)
    res = sch.schedule(c, smooth_sps(20))
    assert res["len"].tolist() == [0, 0, 0]


def test_table_end_stops_the_walk():
    c = np.ones((2, 4), np.float32)
    sps = np.ones(5, np.float32)  # B <= 4: at most 2 admissions
    res = sch.schedule(c, sps)
    assert res["admitted"] == 2 and res["len"].tolist() == [2, 0]


def test_invalid_inputs():
    c = np.array([[0.5, 1.5]], np.float32)
    res = sch.schedule(c, np.ones(4, np.float32))
    assert not res["valid"] and res["len"].tolist() == [-1]
    c = np.array([[0.5, np.nan]], np.float32)
    assert not sch.schedule(c, np.ones(4, np.float32))["valid"]
    assert not sch.schedule(np.full((1, 2), 0.5, np.float32), np.array([1, np.inf, 1, 1], np.float32))["valid"]


def test_no_gain_no_admission():
    # zero confidence on a flat curve: every admission leaves Theta equal,
    # which does not raise it, so nothing is admitted
    c = np.zeros((2, 3), np.float32)
    res = sch.schedule(c, np.ones(9, np.float32))
    assert res["admitted"] == 0 and res["tie_margin"] == 0.0
