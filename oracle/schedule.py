"""Plain CPU oracle of the confidence-scheduled verify length.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may call this; the product library never does.  It shares
no code with the HIP library.

Method (DSpark paper guide, personal-site-bgy.pages.dev, "scheduler"):
each request r has per-position conditional acceptance confidences
c[r][k] (k = 1..gamma); the survival probability of position j is the
running product a[r][j] = prod_{i <= j} c[r][i], non-increasing in j.  One
verify step sends B = sum_r (1 + l_r) rows to the target and expects
tau = sum_r (1 + sum_{j <= l_r} a[r][j]) accepted tokens; the step rate of
the engine at batch B comes from a profiled table SPS(B), and the system
throughput is Theta = tau * SPS(B).  All candidate extensions (r, j) go into
one pool sorted by a descending; they are admitted from the top, B and tau
updated with each, and the walk stops at the first admission that does not
raise Theta, returning the verify lengths before it.  The production
variant admits the top K of the same order with no early stop.

Readings where the pages leave a step open (listed in the design notes):
  * a[r][j] is the fp32 product taken left to right, a[r][0] = 1;
  * the walk starts from l_r = 0 for every request: B = R, tau = R;
  * ties in a are ordered by request, then position (ascending), which keeps
    every request's admitted positions a prefix;
  * tau and Theta are fp64; SPS is a table indexed by B (entries 0..bmax);
    an admission whose B is past the table ends the walk;
  * inputs outside c in [0, 1] or SPS finite and >= 0 make the schedule
    invalid (every length -1).
"""
from __future__ import annotations

import math

import numpy as np

# Relative gap under which a stopping decision is reported as a near tie.
TIE_REL = 1e-12


def survival(conf: np.ndarray) -> np.ndarray:
    """a[r][j-1] = c[r][1] * ... * c[r][j] in fp32, multiplied left to right."""
    c = np.asarray(conf, dtype=np.float32)
    R, G = c.shape
    a = np.empty((R, G), dtype=np.float32)
    for r in range(R):
        run = np.float32(1.0)
        for j in range(G):
            run = np.float32(run * c[r, j])
            a[r, j] = run
    return a


def pool_order(a: np.ndarray) -> list:
    """The candidate extensions (r, j) (j = 1..gamma) in admission order."""
    R, G = a.shape
    return sorted(((r, j + 1) for r in range(R) for j in range(G)),
                  key=lambda rj: (-float(a[rj[0], rj[1] - 1]), rj[0], rj[1]))


def schedule(conf, sps, topk: int = -1) -> dict:
    """Verify lengths l[R] (int32), the number admitted, Theta of the
    result, and tie_margin: the smallest relative gap |Theta_k -
    Theta_{k-1}| / Theta_{k-1} among the stopping comparisons the walk made
    (inf when it made none; only the greedy walk compares)."""
    c = np.asarray(conf, dtype=np.float32)
    table = np.asarray(sps, dtype=np.float32)
    R, G = c.shape
    bmax = len(table) - 1
    ok = bool(np.all((c >= 0.0) & (c <= 1.0))) and bool(np.all(np.isfinite(table) & (table >= 0.0)))
    if not ok:
        return dict(len=np.full(R, -1, np.int32), admitted=0, theta=float("nan"),
                    tie_margin=math.inf, valid=False)
    a = survival(c)
    order = pool_order(a)
    lens = np.zeros(R, dtype=np.int32)
    B = R
    tau = float(R)
    theta = tau * float(table[B]) if B <= bmax else 0.0
    margin = math.inf
    admitted = 0
    for (r, j) in order:
        if topk >= 0 and admitted >= topk:
            break
        if B + 1 > bmax:
            break
        t_new = tau + float(a[r, j - 1])
        th_new = t_new * float(table[B + 1])
        if topk < 0:
            if theta > 0.0:
                margin = min(margin, abs(th_new - theta) / theta)
            elif th_new == theta:
                margin = 0.0
            if th_new <= theta:
                break
        B += 1
        tau = t_new
        theta = th_new
        lens[r] = j
        admitted += 1
    return dict(len=lens, admitted=admitted, theta=theta, tie_margin=margin, valid=True)


def brute_force_best(conf, sps) -> tuple:
    """max over every length vector l in {0..gamma}^R of tau(l) * SPS(B(l))
    (tiny R and gamma only), and one maximiser."""
    c = np.asarray(conf, dtype=np.float32)
    table = np.asarray(sps, dtype=np.float32)
    R, G = c.shape
    a = survival(c)
    best, arg = -math.inf, None
    for code in range((G + 1) ** R):
        lens, rest = [], code
        for _ in range(R):
            lens.append(rest % (G + 1))
            rest //= G + 1
        B = R + sum(lens)
        if B > len(table) - 1:
            continue
        tau = float(R) + sum(float(a[r, j]) for r in range(R) for j in range(lens[r]))
        th = tau * float(table[B])
        if th > best:
            best, arg = th, np.array(lens, dtype=np.int32)
    return best, arg
