"""Plants plausible mistakes in copies of the oracle (on the CPU) and checks
that at least one pin rejects each copy: evidence that the pins constrain
every part of the oracle (accept rule, residual, bonus, prefix survival,
temperature, inverse CDF, argmax tie-break, uniform indexing, Markov head)."""
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
import oracle_pins

# (name, text in oracle.c, replacement, expected occurrence count)
MUTANTS = [
    ("accept_ratio_inverted", "const double ratio = q[x] / p[x];",
     "const double ratio = p[x] / q[x];", 1),
    ("accept_uses_first_uniform", "const double u = (double)u_accept[(size_t)r * gamma + i];",
     "const double u = (double)u_accept[(size_t)r * gamma];", 1),
    ("residual_sign_flipped", "w[v] = (q[v] > p[v]) ? (q[v] - p[v]) : 0.0;",
     "w[v] = (p[v] > q[v]) ? (p[v] - q[v]) : 0.0;", 1),
    ("residual_without_draft", "w[v] = (q[v] > p[v]) ? (q[v] - p[v]) : 0.0;",
     "w[v] = q[v];", 1),
    ("final_draw_wrong_target_row",
     "softmax_row(zt, t_dtype, trow0 + (size_t)A * V, V, T, q, &mq, &lSq);",
     "softmax_row(zt, t_dtype, trow0 + (size_t)(A > 0 ? A - 1 : A) * V, V, T, q, &mq, &lSq);", 1),
    ("final_draw_first_uniform", "const double us = (double)u_sample[(size_t)r * (gamma + 1) + A];",
     "const double us = (double)u_sample[(size_t)r * (gamma + 1)];", 1),
    ("no_prefix_stop", "            alive = 0;\n            continue;", "            continue;", 1),
    ("cstar_uses_max", "smin += (p[v] < q[v]) ? p[v] : q[v];", "smin += (p[v] > q[v]) ? p[v] : q[v];", 1),
    ("tv_cstar_uses_max", "c += (p[v] < q[v]) ? p[v] : q[v];", "c += (p[v] > q[v]) ? p[v] : q[v];", 1),
    ("resid_uses_abs", "sres += (q[v] > p[v]) ? (q[v] - p[v]) : 0.0;", "sres += fabs(q[v] - p[v]);", 1),
    ("temperature_ignored_in_max", "double a = z / T;", "double a = z;", 1),
    ("temperature_ignored_in_exp", "double a = logit_at(base, dtype, row_off, v) / T;",
     "double a = logit_at(base, dtype, row_off, v);", 1),
    ("cdf_non_strict", "if (C > t) {", "if (C >= t) {", 1),
    ("argmax_last_on_ties", "if (z > bv) {", "if (z >= bv) {", 1),
    ("greedy_compares_draft_argmax", "if (draft_tokens[(size_t)r * gamma + i] == g) {",
     "if (draft_tokens[(size_t)r * gamma + i] == gd) {", 1),
    ("logq_missing_normaliser",
     "if (lq) lq[A] = logit_at(zt, t_dtype, trow0 + (size_t)i * V, x) / T - mq - lSq;",
     "if (lq) lq[A] = logit_at(zt, t_dtype, trow0 + (size_t)i * V, x) / T - mq;", 1),
    ("markov_bias_from_anchor_only", "            x_prev = x;\n", "            (void)x_prev;\n", 1),
    ("markov_w1_transposed", "logit_at(W1, w_dtype, (size_t)x_prev * rank, j)",
     "logit_at(W1, w_dtype, (size_t)j * V, x_prev)", 1),
    ("markov_bias_dropped", "l32[v] = (float)(uv + b[v]);", "l32[v] = (float)uv;", 1),
]


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def _build_mutant(workdir, name, old, new, count):
    with open(oracle.SRC) as f:
        src = f.read()
    assert src.count(old) == count, f"mutation site for {name} not found exactly {count}x"
    src = src.replace(old, new)
    c = os.path.join(workdir, name + ".c")
    so = os.path.join(workdir, name + ".so")
    with open(c, "w") as f:
        f.write(src)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", so, c, "-lm"])
    return oracle.load(so)


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m[0])
def test_mutant_is_caught(workdir, mutant):
    name, old, new, count = mutant
    lib = _build_mutant(workdir, name, old, new, count)
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            return  # caught
        except (ValueError, IndexError, TypeError):
            return  # the mutant produced unusable output: caught as well
    pytest.fail(f"no pin caught the planted mistake {name}")
