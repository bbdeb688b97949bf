"""Pins for the fp64 oracle: each check ties the oracle to something other
than itself -- exact enumeration over uniform grids, closed forms, library
routines (scipy softmax, numpy argmax / searchsorted / matmul), Monte-Carlo
estimates of the pages' eq. (2), and hand-derived golden cases.

Every pin takes the loaded oracle library as `lib`, so the same pins run
against the real oracle (test_oracle_pins.py) and against copies with planted
mistakes (test_oracle_mutants.py), where at least one pin must fail.

Sources: DART reading note (zhongzhuzhou.org) sec. 2.2 eq. (2), sec. 2.3
eq. (3)-(4) and its T = 0 remark; DSpark paper guide, "basics", "Markov head",
"confidence head"; speculative-decoding survey (zhifeiding.github.io) sec. 1.3.
"""
from __future__ import annotations

import glob
import json
import os
from fractions import Fraction

import numpy as np
from scipy.special import log_softmax, softmax

import oracle
import workloads

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _logits_from_probs(probs) -> np.ndarray:
    """fp32 logits whose softmax at T = 1 is `probs` (zeros -> -inf)."""
    p = np.asarray(probs, dtype=np.float64)
    with np.errstate(divide="ignore"):
        return np.log(p).astype(np.float32)


# ---------------------------------------------------------------------------
# library-routine pins for c*, Res and log q
# ---------------------------------------------------------------------------

def pin_tv_library(lib):
    """c* = 1 - 1/2 ||p - q||_1 and Res = sum [q - p]_+ = 1/2 ||p - q||_1 for
    softmaxes computed by scipy in fp64 (DSpark confidence label; DART eq. (3)).
    Also the T = 0 one-hot limit against numpy.argmax."""
    gen = np.random.default_rng(11)
    N, V = 24, 333
    zt = (gen.standard_normal((N, V)) * 2.5).astype(np.float32)
    zd = (zt + gen.standard_normal((N, V)) * np.linspace(0.1, 3.0, N)[:, None]).astype(np.float32)
    # includes a small temperature: z / T reaches ~5000, so the max must be
    # taken of z / T (not z) before exponentiating
    T = np.array([1.0, 0.7, 1.9, 0.002] * (N // 4), dtype=np.float32)
    cs, rs = oracle.tv_accept_rate(zd, zt, T, lib=lib)
    for n in range(N):
        q = softmax(zt[n].astype(np.float64) / float(T[n]))
        p = softmax(zd[n].astype(np.float64) / float(T[n]))
        tv = 0.5 * np.abs(p - q).sum()
        assert abs(cs[n] - (1.0 - tv)) < 1e-12, (n, cs[n], 1.0 - tv)
        assert np.isfinite(cs[n])
        assert abs(rs[n] - tv) < 1e-12, (n, rs[n], tv)
    # bf16 rows
    tb = workloads.f32_to_bf16_bits(zt)
    db = workloads.f32_to_bf16_bits(zd)
    cs2, _ = oracle.tv_accept_rate(db, tb, T, lib=lib)
    for n in range(N):
        q = softmax(workloads.bf16_bits_to_f32(tb[n]).astype(np.float64) / float(T[n]))
        p = softmax(workloads.bf16_bits_to_f32(db[n]).astype(np.float64) / float(T[n]))
        assert abs(cs2[n] - (1.0 - 0.5 * np.abs(p - q).sum())) < 1e-12
    # T = 0: indicator of equal argmaxes
    T0 = np.zeros(N, np.float32)
    zd0 = zd.copy()
    zd0[::3] = zt[::3]  # some rows share the argmax
    cs0, rs0 = oracle.tv_accept_rate(zd0, zt, T0, lib=lib)
    for n in range(N):
        same = float(np.argmax(zd0[n]) == np.argmax(zt[n]))
        assert cs0[n] == same and rs0[n] == 1.0 - same


def pin_verify_floats_library(lib):
    """Per-position c*, Res and the log q of committed tokens from the batched
    call against scipy's fp64 softmax / log_softmax."""
    case = workloads.make_verify_case(6, 5, 257, "bf16", seed=21, target_std=2.0,
                                      noise_std=np.linspace(0.3, 2.0, 5),
                                      verify_len=[0, 1, 5, 3, 5, 2],
                                      temperature=[1.0, 0.8, 1.3, 1.0, 0.5, 2.0])
    out = oracle.verify_case(case, lib=lib)
    zt = workloads.as_f32(case.target).astype(np.float64)
    zd = workloads.as_f32(case.draft).astype(np.float64)
    for r in range(case.R):
        T = float(case.temperature[r])
        l = int(case.verify_len[r])
        A = int(out["num_accepted"][r])
        assert 0 <= A <= l
        for i in range(case.gamma):
            if i < l:
                q = softmax(zt[r, i] / T)
                p = softmax(zd[r, i] / T)
                assert abs(out["cstar"][r, i] - (1 - 0.5 * np.abs(p - q).sum())) < 1e-12
                assert abs(out["resid"][r, i] - 0.5 * np.abs(p - q).sum()) < 1e-12
            else:
                assert np.isnan(out["cstar"][r, i]) and np.isnan(out["resid"][r, i])
        for j in range(case.gamma + 1):
            t = int(out["tokens"][r, j])
            if j <= A:
                assert 0 <= t < case.V
                lq = log_softmax(zt[r, j] / T)[t]
                assert abs(out["logq"][r, j] - lq) < 1e-10, (r, j, out["logq"][r, j], lq)
            else:
                assert t == -1 and np.isnan(out["logq"][r, j])
        # committed prefix is the draft prefix
        assert np.array_equal(out["tokens"][r, :A], case.draft_tokens[r, :A])


# ---------------------------------------------------------------------------
# exact enumeration: the committed token's law equals q (DART eq. (3)-(4))
# ---------------------------------------------------------------------------

EXACT_CASES = [
    # (denominator, p0, q0, q1) as integer numerators; row 0 is verified, row 1
    # is the bonus row.  Every decision threshold is k/m with m dividing the
    # grid size (840 = lcm(1..8) for eighths, 24 for quarters).
    (8, [4, 1, 2, 1], [2, 3, 1, 2], [1, 1, 4, 2]),
    (8, [1, 1, 1, 5], [5, 1, 1, 1], [2, 2, 2, 2]),
    (4, [1, 1, 1, 1], [2, 0, 1, 1], [1, 1, 1, 1]),   # q(1) = 0: x = 1 never passes
    (4, [1, 1, 1, 1], [1, 1, 1, 1], [4, 0, 0, 0]),   # p == q: always accept
    (4, [2, 2, 0, 0], [0, 0, 1, 3], [0, 1, 0, 3]),   # disjoint supports: always reject
    (4, [3, 0, 1, 0], [1, 1, 1, 1], [1, 0, 1, 2]),   # zero-probability ids (-inf logits)
]
GRID_FOR_DEN = {8: 840, 4: 24}


def _exact_grid_case(lib, den, p0, q0, q1):
    V = 4
    n_grid = GRID_FOR_DEN[den]
    p0f = [Fraction(a, den) for a in p0]
    q0f = [Fraction(a, den) for a in q0]
    q1f = [Fraction(a, den) for a in q1]
    xs = [x for x in range(V) if p0[x] > 0]          # drafts are drawn from p0
    g = (np.arange(n_grid, dtype=np.float64) + 0.5) / n_grid
    ua_grid, us_grid = np.meshgrid(g, g, indexing="ij")
    n = ua_grid.size
    R = n * len(xs)
    target = np.empty((R, 2, V), np.float32)
    target[:, 0, :] = _logits_from_probs(np.array(q0) / den)
    target[:, 1, :] = _logits_from_probs(np.array(q1) / den)
    draft = np.empty((R, 1, V), np.float32)
    draft[:, 0, :] = _logits_from_probs(np.array(p0) / den)
    tokens = np.repeat(np.array(xs, np.int32), n)[:, None]
    ua = np.tile(ua_grid.ravel(), len(xs)).astype(np.float32)[:, None]
    us = np.tile(us_grid.ravel(), len(xs)).astype(np.float32)
    us = np.stack([us, us], axis=1)
    out = oracle.verify_batch(target, draft, tokens, np.ones(R, np.int32), np.ones(R, np.float32),
                              ua, us, lib=lib)
    assert out["invalid"] == 0
    tok0 = out["tokens"][:, 0].reshape(len(xs), n)
    tok1 = out["tokens"][:, 1].reshape(len(xs), n)
    A = out["num_accepted"].reshape(len(xs), n)
    law0 = [Fraction(0)] * V
    pA = Fraction(0)
    law1 = [Fraction(0)] * V
    for k, x in enumerate(xs):
        w = p0f[x] / n
        for v in range(V):
            law0[v] += w * int((tok0[k] == v).sum())
            law1[v] += w * int(((tok1[k] == v) & (A[k] == 1)).sum())
        pA += w * int((A[k] == 1).sum())
    cstar = sum(min(a, b) for a, b in zip(p0f, q0f))
    assert law0 == q0f, ("first committed token law", law0, q0f)       # eq. (4)
    assert pA == cstar, ("P(accept)", pA, cstar)                          # eq. (3)
    if cstar > 0:
        assert [x / pA for x in law1] == q1f, ("bonus law", law1, q1f)
    # logits are fp32 roundings of log-probabilities, so the floats are ~1e-7 off
    assert np.allclose(out["cstar"][:, 0], float(cstar), atol=1e-6, rtol=0)
    assert np.allclose(out["resid"][:, 0], float(1 - cstar), atol=1e-6, rtol=0)


def pin_exact_grid(lib):
    """Runs the oracle over every draft token and a midpoint grid of both
    uniforms; with probabilities in eighths (quarters) and a grid of 840 (24)
    points per uniform the integral is exact, so the law of the first committed token must equal q0 exactly,
    P(accept) must equal sum min(p0, q0), and the bonus law must equal q1."""
    for den, p0, q0, q1 in EXACT_CASES:
        _exact_grid_case(lib, den, p0, q0, q1)


# ---------------------------------------------------------------------------
# Monte Carlo: prefix survival and eq. (2)
# ---------------------------------------------------------------------------

def pin_monte_carlo_prefix(lib):
    """gamma = 3 fixed rows, drafts drawn from p_i, random uniforms.  Checks
    P(A >= k) = prod_{j<k} c*_j, E[A] = sum_i prod_{j<=i} c*_j (DART eq. (2)
    with a_j = c*_j), and that the committed token at position k, given
    survival to k, follows q_k (chi-square)."""
    gen = np.random.default_rng(5)
    R, gamma, V, T = 200_000, 3, 5, 0.8
    zt = (gen.standard_normal((gamma + 1, V)) * 1.2).astype(np.float32)
    zd = (zt[:gamma] + gen.standard_normal((gamma, V)) * 0.8).astype(np.float32)
    q = softmax(zt.astype(np.float64) / T, axis=1)
    p = softmax(zd.astype(np.float64) / T, axis=1)
    c = 1.0 - 0.5 * np.abs(p - q[:gamma]).sum(axis=1)
    tokens = np.stack([gen.choice(V, size=R, p=p[i]) for i in range(gamma)], axis=1).astype(np.int32)
    target = np.broadcast_to(zt, (R, gamma + 1, V))
    draft = np.broadcast_to(zd, (R, gamma, V))
    ua = gen.random((R, gamma), dtype=np.float32)
    us = gen.random((R, gamma + 1), dtype=np.float32)
    out = oracle.verify_batch(target, draft, tokens, np.full(R, gamma, np.int32),
                              np.full(R, T, np.float32), ua, us, lib=lib)
    A = out["num_accepted"]
    surv = np.concatenate([[1.0], np.cumprod(c)])
    for k in range(gamma + 1):
        est = (A >= k).mean()
        se = np.sqrt(surv[k] * (1 - surv[k]) / R) + 1e-9
        assert abs(est - surv[k]) < 5 * se + 1e-12, ("P(A>=k)", k, est, surv[k])
    ea = surv[1:].sum()
    assert abs(A.mean() - ea) < 5 * A.std() / np.sqrt(R), (A.mean(), ea)
    for k in range(gamma + 1):
        sel = A >= k
        m = int(sel.sum())
        counts = np.bincount(out["tokens"][sel, k], minlength=V)
        expct = m * q[k]
        chi2 = ((counts - expct) ** 2 / expct).sum()
        assert chi2 < 30.0, ("committed token law at position", k, chi2)   # 4 dof


# ---------------------------------------------------------------------------
# greedy path, inverse CDF, degenerate cases, validation
# ---------------------------------------------------------------------------

def pin_greedy_argmax(lib):
    """T = 0: accept iff x == numpy.argmax(target row) (first index on ties),
    the committed next token is that argmax, log q = 0 (survey sec. 1.3; DART
    note sec. 2.3)."""
    gen = np.random.default_rng(7)
    R, gamma, V = 64, 4, 40
    zt = np.round(gen.standard_normal((R, gamma + 1, V)) * 2).astype(np.float32)  # many ties
    zd = np.round(zt[:, :gamma] + gen.standard_normal((R, gamma, V))).astype(np.float32)
    g = np.argmax(zt, axis=2)
    tokens = np.where(gen.random((R, gamma)) < 0.7, g[:, :gamma],
                      gen.integers(0, V, (R, gamma))).astype(np.int32)
    vl = gen.integers(0, gamma + 1, R).astype(np.int32)
    out = oracle.verify_batch(zt, zd, tokens, vl, np.zeros(R, np.float32),
                              np.full((R, gamma), 0.5, np.float32),
                              np.full((R, gamma + 1), 0.5, np.float32), lib=lib)
    for r in range(R):
        l = vl[r]
        A = 0
        while A < l and tokens[r, A] == g[r, A]:
            A += 1
        assert out["num_accepted"][r] == A
        assert list(out["tokens"][r, :A]) == list(tokens[r, :A])
        assert out["tokens"][r, A] == g[r, A]
        assert (out["tokens"][r, A + 1:] == -1).all()
        assert (out["logq"][r, :A + 1] == 0).all()
        for i in range(gamma):
            if i < l:
                assert out["cstar"][r, i] == float(np.argmax(zd[r, i]) == g[r, i])
            else:
                assert np.isnan(out["cstar"][r, i])


def pin_inverse_cdf_searchsorted(lib):
    """The inverse-CDF draw equals numpy.searchsorted(cumsum(w), u W,
    side='right'): the smallest id whose running sum exceeds u W; zero-weight
    ids are never chosen."""
    gen = np.random.default_rng(9)
    for trial in range(200):
        V = int(gen.integers(1, 50))
        w = gen.random(V) * (gen.random(V) < 0.6)
        if w.sum() == 0:
            w[gen.integers(0, V)] = 1.0
        for u in [0.0, float(gen.random()), float(np.float32(1 - 2**-24)), 0.5]:
            t, _ = oracle.inverse_cdf(w, u, lib=lib)
            cs = np.cumsum(w)
            ref = int(np.searchsorted(cs, u * cs[-1], side="right"))
            if ref == V:  # u W rounded up to the total: last positive id
                ref = int(np.nonzero(w > 0)[0][-1])
            assert t == ref, (trial, V, u, t, ref)
            assert w[t] > 0


def pin_degenerate(lib):
    """p == q: every draft accepted, c* = 1, Res = 0, bonus from q_l.
    l = 0: one token from target row 0 (a plain autoregressive step).
    Disjoint supports: c* = 0 and the committed token lies in q's support."""
    gen = np.random.default_rng(13)
    R, gamma, V = 32, 5, 64
    zt = (gen.standard_normal((R, gamma + 1, V)) * 2).astype(np.float32)
    zd = zt[:, :gamma].copy()
    tokens = gen.integers(0, V, (R, gamma)).astype(np.int32)
    ua = gen.random((R, gamma), dtype=np.float32)
    us = gen.random((R, gamma + 1), dtype=np.float32)
    out = oracle.verify_batch(zt, zd, tokens, np.full(R, gamma, np.int32),
                              np.ones(R, np.float32), ua, us, lib=lib)
    assert (out["num_accepted"] == gamma).all()
    assert np.allclose(out["cstar"], 1.0, atol=1e-12) and np.allclose(out["resid"], 0, atol=1e-15)
    # l = 0: the committed token is an inverse-CDF draw from target row 0
    out0 = oracle.verify_batch(zt, zd, tokens, np.zeros(R, np.int32), np.ones(R, np.float32),
                               ua, us, lib=lib)
    assert (out0["num_accepted"] == 0).all()
    for r in range(R):
        q = softmax(zt[r, 0].astype(np.float64))
        cs = np.cumsum(q)
        assert out0["tokens"][r, 0] == int(np.searchsorted(cs, float(us[r, 0]) * cs[-1], side="right"))
    # disjoint supports: draft mass on even ids, target mass on odd ids
    zt2 = zt.copy()
    zd2 = zd.copy()
    zt2[:, :, 0::2] = -np.inf
    zd2[:, :, 1::2] = -np.inf
    tok2 = (2 * gen.integers(0, V // 2, (R, gamma))).astype(np.int32)
    out2 = oracle.verify_batch(zt2, zd2, tok2, np.full(R, gamma, np.int32), np.ones(R, np.float32),
                               ua, us, lib=lib)
    assert (out2["num_accepted"] == 0).all()
    assert (out2["tokens"][:, 0] % 2 == 1).all()
    assert np.allclose(out2["cstar"], 0.0) and np.allclose(out2["resid"], 1.0)


def pin_validation(lib):
    """Invalid requests are flagged: l outside [0, gamma], draft token outside
    [0, V), NaN / +inf logits, a row of only -inf, negative or NaN T, uniforms
    outside [0, 1).  A valid neighbour request is unaffected."""
    case = workloads.make_verify_case(2, 3, 16, "f32", seed=3, verify_len=3, temperature=1.0)
    base = oracle.verify_case(case, lib=lib)
    assert base["invalid"] == 0

    def run(mut):
        c = workloads.VerifyCase(case.name, case.target.copy(), case.draft.copy(),
                                 case.draft_tokens.copy(), case.verify_len.copy(),
                                 case.temperature.copy(), case.u_accept.copy(),
                                 case.u_sample.copy())
        mut(c)
        return oracle.verify_case(c, lib=lib)

    muts = [
        lambda c: c.verify_len.__setitem__(0, 4),
        lambda c: c.verify_len.__setitem__(0, -1),
        lambda c: c.draft_tokens.__setitem__((0, 1), 16),
        lambda c: c.draft_tokens.__setitem__((0, 2), -3),
        lambda c: c.target.__setitem__((0, 3, 5), np.nan),
        lambda c: c.draft.__setitem__((0, 0, 5), np.inf),
        lambda c: c.target.__setitem__((0, 2), -np.inf),
        lambda c: c.temperature.__setitem__(0, -1.0),
        lambda c: c.temperature.__setitem__(0, np.nan),
        lambda c: c.u_accept.__setitem__((0, 0), 1.0),
        lambda c: c.u_sample.__setitem__((0, 3), np.nan),
    ]
    for k, m in enumerate(muts):
        out = run(m)
        assert out["invalid"] == 1, k
        assert out["num_accepted"][0] == -1 and (out["tokens"][0] == -1).all(), k
        assert np.isnan(out["cstar"][0]).all(), k
        assert out["num_accepted"][1] == base["num_accepted"][1], k
        assert np.array_equal(out["tokens"][1], base["tokens"][1]), k
    # -inf logits that are not a whole row are valid (masked ids)
    out = run(lambda c: c.target.__setitem__((0, 1, 3), -np.inf))
    assert out["invalid"] == 0


# ---------------------------------------------------------------------------
# Markov head (DSpark guide, "Markov head")
# ---------------------------------------------------------------------------

def pin_markov_matmul(lib):
    """Stored draft logits equal float32(U + W1[x_{k-1}] @ W2) with numpy's
    fp64 matmul, the previous token feeding each step (x_0 = anchor); tokens
    are the oracle's own inverse-CDF draws from softmax(l / T)."""
    gen = np.random.default_rng(17)
    R, gamma, V, rank = 3, 4, 300, 16
    U = workloads.f32_to_bf16_bits(gen.standard_normal((R, gamma, V)).astype(np.float32) * 2)
    W1 = workloads.f32_to_bf16_bits(gen.standard_normal((V, rank)).astype(np.float32) * 0.5)
    W2 = workloads.f32_to_bf16_bits(gen.standard_normal((rank, V)).astype(np.float32) * 0.5)
    anchor = gen.integers(0, V, R).astype(np.int32)
    T = np.array([1.0, 0.6, 1.5], np.float32)
    ud = gen.random((R, gamma), dtype=np.float32)
    out = oracle.markov_draft(U, W1, W2, anchor, T, ud, lib=lib)
    assert out["invalid"] == 0
    Uf = workloads.bf16_bits_to_f32(U).astype(np.float64)
    W1f = workloads.bf16_bits_to_f32(W1).astype(np.float64)
    W2f = workloads.bf16_bits_to_f32(W2).astype(np.float64)
    for r in range(R):
        x = int(anchor[r])
        for k in range(gamma):
            l = (Uf[r, k] + W1f[x] @ W2f).astype(np.float32)
            got = out["logits"][r, k]
            ulp = np.spacing(np.abs(l))
            assert (np.abs(got - l) <= ulp).all()
            p = softmax(got.astype(np.float64) / float(T[r]))
            cs = np.cumsum(p)
            ref = int(np.searchsorted(cs, float(ud[r, k]) * cs[-1], side="right"))
            assert out["tokens"][r, k] == ref
            x = ref


def pin_markov_collision(lib):
    """The pages' collision example: with ids {of, course, no, problem} the base
    logits at position 2 favour 'course' and 'problem' equally; the Markov
    bias of 'of' lifts 'course' and lowers 'problem'.  Over a uniform grid the
    oracle's second draft token follows softmax(U_2 + W1[of] W2) exactly (to
    the grid resolution), and x_1 feeds the second step."""
    OF, COURSE, NO, PROBLEM = 0, 1, 2, 3
    V, rank, n = 4, 2, 4096
    U = np.zeros((n, 2, V), np.float32)
    U[:, 0] = [3.0, -9.0, 3.0, -9.0]       # position 1: "of" or "no"
    U[:, 1] = [-9.0, 2.0, -9.0, 2.0]       # position 2: "course" or "problem"
    W1 = np.zeros((V, rank), np.float32)
    W2 = np.zeros((rank, V), np.float32)
    W1[OF] = [1.0, 0.0]
    W1[NO] = [0.0, 1.0]
    W2[0, COURSE], W2[0, PROBLEM] = 2.0, -2.0   # after "of": course up, problem down
    W2[1, COURSE], W2[1, PROBLEM] = -2.0, 2.0   # after "no": the reverse
    g = ((np.arange(n) + 0.5) / n).astype(np.float32)
    ud = np.stack([np.full(n, 0.25, np.float32), g], axis=1)   # u=0.25 draws "of" first
    out = oracle.markov_draft(U, W1, W2, np.full(n, NO, np.int32), np.ones(n, np.float32), ud,
                              lib=lib)
    assert (out["tokens"][:, 0] == OF).all()
    law = np.bincount(out["tokens"][:, 1], minlength=V) / n
    expect = softmax(np.array([-9.0, 4.0, -9.0, 0.0]))
    assert np.abs(law - expect).max() < 2.0 / n, (law, expect)
    assert law[COURSE] > 0.95


# ---------------------------------------------------------------------------
# hand-derived golden cases
# ---------------------------------------------------------------------------

def pin_golden(lib):
    """Small cases derived by hand from eq. (3)-(4) and the greedy rule; each
    JSON file carries its derivation and citation."""
    files = sorted(glob.glob(os.path.join(GOLDEN_DIR, "*.json")))
    assert files, "no golden fixtures"
    for f in files:
        with open(f) as fh:
            g = json.load(fh)
        for c in g["cases"]:
            zt = np.array(c["target_probs"], np.float64)
            zd = np.array(c["draft_probs"], np.float64)
            if g.get("logits_are_probs", True):
                zt = _logits_from_probs(zt)
                zd = _logits_from_probs(zd)
            else:
                zt = zt.astype(np.float32)
                zd = zd.astype(np.float32)
            out = oracle.verify_batch(zt[None], zd[None], np.array([c["draft_tokens"]], np.int32),
                                      np.array([c["verify_len"]], np.int32),
                                      np.array([c["temperature"]], np.float32),
                                      np.array([c["u_accept"]], np.float32),
                                      np.array([c["u_sample"]], np.float32), lib=lib)
            assert out["num_accepted"][0] == c["expect_num_accepted"], (f, c["name"])
            assert list(out["tokens"][0]) == c["expect_tokens"], (f, c["name"], out["tokens"][0])
            for i, v in enumerate(c.get("expect_cstar", [])):
                if v is None:
                    assert np.isnan(out["cstar"][0, i])
                else:
                    # logits are fp32 roundings of log-probabilities: ~1e-7 off
                    assert abs(out["cstar"][0, i] - v) < 1e-6, (f, c["name"], i)


# cheapest first: the mutant test stops at the first pin that fails
ALL_PINS = [
    pin_golden,
    pin_inverse_cdf_searchsorted,
    pin_tv_library,
    pin_greedy_argmax,
    pin_verify_floats_library,
    pin_degenerate,
    pin_validation,
    pin_markov_matmul,
    pin_markov_collision,
    pin_monte_carlo_prefix,
    pin_exact_grid,
]
