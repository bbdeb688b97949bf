"""Plain CPU oracle of sequential temperature scaling (STS) and the expected
calibration error (ECE) of cumulative survival probabilities.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may call this; the product library never does.  It shares
no code with the HIP library.

Method (DSpark paper guide, personal-site-bgy.pages.dev, the confidence-head
section, "STS"): the confidence head's per-position scores are calibrated
after training on a held-out set.  Positions are taken left to right; for
each a one-dimensional grid search picks the temperature scalar that
minimises the ECE of the cumulative (multiplied) probabilities, with the
positions already calibrated kept at their chosen temperatures.  Temperature
scaling keeps the ranking of the scores.

Readings where the pages leave a step open (listed in the design notes):
  * the score of position k is c = sigmoid(z / t) for the head's raw logit z
    and temperature t > 0; the cumulative probability is
    a_k = c_1(t_1) ... c_k(t_k);
  * the label of a_k is the event that positions 1..k were all accepted,
    y_k = [A >= k] for the block's accepted prefix length A;
  * ECE uses `bins` equal-width bins over [0, 1] (a value of 1 falls in the
    last bin): ECE = sum over bins of |sum_{n in bin} (a_n - y_n)| / N, i.e.
    the bin-weighted gap between mean confidence and accuracy;
  * the grid is a caller-given list of temperatures; ties go to the first
    grid point that reaches the minimum;
  * arithmetic is fp64 throughout.
"""
from __future__ import annotations

import numpy as np

# Reported near ties: ECE gap between the best and the runner-up grid point,
# and the distance of a value a * bins to a bin edge.
ECE_TIE = 1e-12
EDGE_TIE = 1e-9


def sigmoid(x: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def bin_index(a: np.ndarray, bins: int) -> np.ndarray:
    """Equal-width bin of each value in [0, 1]; 1 goes to the last bin."""
    return np.minimum(np.floor(a * bins).astype(np.int64), bins - 1)


def ece(a: np.ndarray, y: np.ndarray, bins: int) -> float:
    """sum_m |sum_{n in bin m} (a_n - y_n)| / N."""
    a = np.asarray(a, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    gap = np.zeros(bins)
    np.add.at(gap, bin_index(a, bins), a - y)
    return float(np.abs(gap).sum() / len(a))


def edge_margin(a: np.ndarray, bins: int) -> float:
    """Smallest distance of a * bins to an interior bin edge."""
    s = np.asarray(a, dtype=np.float64) * bins
    inner = (s > 0.5) & (s < bins - 0.5)
    if not inner.any():
        return np.inf
    return float(np.abs(s[inner] - np.round(s[inner])).min())


def sts_calibrate(z, accepted, grid, bins: int = 15) -> dict:
    """temperatures [gamma], ece [gamma] (after calibration), curves
    [gamma][G] (ECE at every grid point), tie_gap [gamma] (best vs runner-up
    ECE), edge [gamma] (edge_margin over every grid point's values)."""
    z = np.asarray(z, dtype=np.float64)
    A = np.asarray(accepted)
    grid = np.asarray(grid, dtype=np.float64)
    N, gamma = z.shape
    G = len(grid)
    a_prev = np.ones(N)
    temps = np.zeros(gamma)
    eces = np.zeros(gamma)
    curves = np.zeros((gamma, G))
    gaps = np.full(gamma, np.inf)
    edges = np.full(gamma, np.inf)
    for k in range(gamma):
        y = (A >= k + 1).astype(np.float64)
        for g in range(G):
            a = a_prev * sigmoid(z[:, k] / grid[g])
            curves[k, g] = ece(a, y, bins)
            edges[k] = min(edges[k], edge_margin(a, bins))
        best = int(np.argmin(curves[k]))           # first minimum
        temps[k] = grid[best]
        eces[k] = curves[k, best]
        if G > 1:
            others = np.delete(curves[k], best)
            gaps[k] = float(others.min() - eces[k])
        a_prev = a_prev * sigmoid(z[:, k] / temps[k])
    return dict(temperatures=temps, ece=eces, curves=curves, tie_gap=gaps, edge=edges)
