"""Plants plausible mistakes in copies of the Python oracles (the RNN head,
the verify-length scheduler, the STS calibration and greedy tree
verification) and checks that at least one of their pins
rejects each copy.  The copy is executed as a module of the oracle package
and swapped in for the pin module's reference while its tests run (CPU)."""
import importlib
import pathlib
import types

import pytest

import oracle

ROOT = pathlib.Path(__file__).resolve().parent.parent

# (oracle module, pin module, name, text, replacement)
MUTANTS = [
    ("rnn", "test_oracle_rnn", "gate_mix_swapped", "s = (1.0 - z) * s + z * n",
     "s = z * s + (1.0 - z) * n"),
    ("rnn", "test_oracle_rnn", "hidden_of_first_step", "c = np.concatenate([s, w1[x], h[r, k - 1]])",
     "c = np.concatenate([s, w1[x], h[r, 0]])"),
    ("rnn", "test_oracle_rnn", "state_slot_dropped", "c = np.concatenate([s, w1[x], h[r, k - 1]])",
     "c = np.concatenate([0.0 * s, w1[x], h[r, k - 1]])"),
    ("rnn", "test_oracle_rnn", "candidate_from_gate_columns", "n = np.tanh(g[rank:])",
     "n = np.tanh(g[:rank])"),
    ("rnn", "test_oracle_rnn", "sigmoid_sign", "z = 1.0 / (1.0 + np.exp(-g[:rank]))",
     "z = 1.0 / (1.0 + np.exp(g[:rank]))"),
    ("rnn", "test_oracle_rnn", "bias_dropped", "l32 = (U64[r, k - 1] + s @ w2).astype(np.float32)",
     "l32 = U64[r, k - 1].astype(np.float32)"),
    ("rnn", "test_oracle_rnn", "token_not_fed_back", "x, mg = inverse_cdf(p, u, lib)",
     "_, mg = inverse_cdf(p, u, lib)"),
    ("rnn", "test_oracle_rnn", "bias_missing", "g = c @ wg + b", "g = c @ wg"),
    ("schedule", "test_oracle_schedule", "survival_not_a_product",
     "run = np.float32(run * c[r, j])", "run = np.float32(c[r, j])"),
    ("schedule", "test_oracle_schedule", "pool_ascending",
     "key=lambda rj: (-float(a[rj[0], rj[1] - 1]), rj[0], rj[1])",
     "key=lambda rj: (float(a[rj[0], rj[1] - 1]), rj[0], rj[1])"),
    ("schedule", "test_oracle_schedule", "ties_by_request_descending",
     "key=lambda rj: (-float(a[rj[0], rj[1] - 1]), rj[0], rj[1])",
     "key=lambda rj: (-float(a[rj[0], rj[1] - 1]), -rj[0], rj[1])"),
    ("schedule", "test_oracle_schedule", "stop_only_on_strict_drop",
     "if th_new <= theta:", "if th_new < theta:"),
    ("schedule", "test_oracle_schedule", "walk_starts_empty", "    B = R\n", "    B = 0\n"),
    ("schedule", "test_oracle_schedule", "tau_without_bonus", "    tau = float(R)\n", "    tau = 0.0\n"),
    ("schedule", "test_oracle_schedule", "table_at_old_batch",
     "th_new = t_new * float(table[B + 1])", "th_new = t_new * float(table[B])"),
    ("schedule", "test_oracle_schedule", "table_end_off_by_one",
     "if B + 1 > bmax:", "if B + 2 > bmax:"),
    ("schedule", "test_oracle_schedule", "topk_one_extra",
     "if topk >= 0 and admitted >= topk:", "if topk >= 0 and admitted > topk:"),
    ("sts", "test_oracle_sts", "temperature_multiplies",
     "a = a_prev * sigmoid(z[:, k] / grid[g])", "a = a_prev * sigmoid(z[:, k] * grid[g])"),
    ("sts", "test_oracle_sts", "earlier_positions_raw",
     "a_prev = a_prev * sigmoid(z[:, k] / temps[k])", "a_prev = a_prev * sigmoid(z[:, k])"),
    ("sts", "test_oracle_sts", "top_bin_unclamped",
     "return np.minimum(np.floor(a * bins).astype(np.int64), bins - 1)",
     "return np.floor(a * bins).astype(np.int64) % bins"),
    ("sts", "test_oracle_sts", "signed_bin_gaps",
     "return float(np.abs(gap).sum() / len(a))", "return float(abs(gap.sum()) / len(a))"),
    ("sts", "test_oracle_sts", "ties_to_last",
     "best = int(np.argmin(curves[k]))", "best = int(len(grid) - 1 - np.argmin(curves[k][::-1]))"),
    ("sts", "test_oracle_sts", "label_off_by_one",
     "y = (A >= k + 1).astype(np.float64)", "y = (A > k + 1).astype(np.float64)"),
    ("tree", "test_oracle_tree", "always_root_row", "g = _row_argmax(L[r, cur])",
     "g = _row_argmax(L[r, 0])"),
    ("tree", "test_oracle_tree", "any_node_not_children", "if P[r, v] == cur and X[r, v] == g:",
     "if X[r, v] == g:"),
    ("tree", "test_oracle_tree", "bonus_dropped", "                toks.append(g)\n",
     "                toks.append(-1)\n"),
    ("tree", "test_oracle_tree", "argmax_ties_last", "return int(np.argmax(r))",
     "return int(len(r) - 1 - np.argmax(r[::-1]))"),
    ("tree", "test_oracle_tree", "last_equal_sibling",
     "                    nxt = v\n                    break\n", "                    nxt = v\n"),
    ("tree", "test_oracle_tree", "parent_may_be_self", "ok = ok and 0 <= P[r, v] < v and",
     "ok = ok and 0 <= P[r, v] <= v and"),
]


def _mutant_module(name, old, new):
    src = (ROOT / "oracle" / f"{name}.py").read_text()
    assert src.count(old) == 1, f"mutation site not unique in oracle/{name}.py: {old!r}"
    mod = types.ModuleType(f"oracle._mutant_{name}")
    mod.__package__ = "oracle"
    mod.__file__ = str(ROOT / "oracle" / f"{name}.py")
    exec(compile(src.replace(old, new), mod.__file__, "exec"), mod.__dict__)
    return mod


def _calls(fn, lib):
    """Every (args) a pin function runs with: its parametrize values, and the
    lib fixture where it asks for one."""
    params = [{}]
    for mark in getattr(fn, "pytestmark", []):
        if mark.name == "parametrize":
            names = [n.strip() for n in mark.args[0].split(",")]
            vals = list(mark.args[1])
            params = [dict(p, **dict(zip(names, v if len(names) > 1 else (v,))))
                      for p in params for v in vals]
    need_lib = "lib" in fn.__code__.co_varnames[:fn.__code__.co_argcount]
    for p in params:
        yield dict(p, lib=lib) if need_lib else p


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: f"{m[0]}-{m[2]}")
def test_python_oracle_mutant_is_caught(mutant, monkeypatch):
    mod_name, pins_name, _, old, new = mutant
    pins = importlib.import_module(pins_name)
    ref_attr = {"rnn": "rnn", "schedule": "sch", "sts": "sts", "tree": "otree"}[mod_name]
    assert getattr(pins, ref_attr) is importlib.import_module(f"oracle.{mod_name}")
    monkeypatch.setattr(pins, ref_attr, _mutant_module(mod_name, old, new))
    oracle.build(force=False)
    lib = oracle.load()
    failed = []
    for fname in dir(pins):
        fn = getattr(pins, fname)
        if not fname.startswith("test_") or not callable(fn):
            continue
        for kw in _calls(fn, lib):
            try:
                fn(**kw)
            except Exception:  # an assertion, or the mutant breaking outright
                failed.append(fname)
                break
    assert failed, f"no pin rejects the mutant {mutant[2]}"
