"""The greedy tree-verification oracle against what fixes it independently
(CPU only): on chain trees it is the C oracle's greedy chain verification;
on random trees its path is the set of nodes whose every edge matches the
parent row's argmax (checked node by node, not by walking); a hand-worked
tree; the lowest-index child among equal siblings; invalid trees."""
import numpy as np
import pytest

import oracle
import workloads
from oracle import tree as otree


def test_chain_trees_are_greedy_chain_verification():
    R, G, V = 6, 5, 700
    case = workloads.make_verify_case(R, G, V, "f32", seed=21, noise_std=0.3,
                                      verify_len=[5, 3, 0, 5, 4, 2], temperature=[0.0] * R)
    ref = oracle.verify_case(case)
    M = G + 1
    parent = np.full((R, M), -1, np.int32)
    tokens = np.full((R, M), -1, np.int32)
    n = case.verify_len.astype(np.int32) + 1
    for r in range(R):
        for v in range(1, n[r]):
            parent[r, v] = v - 1
            tokens[r, v] = case.draft_tokens[r, v - 1]
    out = otree.tree_verify(case.target, parent, tokens, n)
    np.testing.assert_array_equal(out["accepted"], ref["num_accepted"])
    for r in range(R):
        A = ref["num_accepted"][r]
        np.testing.assert_array_equal(out["committed"][r, :A + 1], ref["tokens"][r, :A + 1])
        np.testing.assert_array_equal(out["path"][r, :A], np.arange(1, A + 1))


def test_hand_worked_tree():
    # root -> {1: tok 2, 2: tok 4}; 1 -> {3: tok 0}; 2 -> {4: tok 5, 5: tok 1}
    V = 6
    L = np.zeros((1, 6, V), np.float32)
    L[0, 0, 4] = 1.0          # root row: argmax 4 -> node 2
    L[0, 2, 1] = 2.0          # node 2 row: argmax 1 -> node 5
    L[0, 5, 3] = 1.0          # node 5 row: argmax 3 -> no child, bonus 3
    L[0, 1, 0] = 9.0          # node 1's row would accept node 3, but node 1 is rejected
    parent = np.array([[-1, 0, 0, 1, 2, 2]], np.int32)
    tokens = np.array([[-1, 2, 4, 0, 5, 1]], np.int32)
    out = otree.tree_verify(L, parent, tokens, np.array([6]))
    assert out["accepted"][0] == 2
    assert list(out["path"][0, :3]) == [2, 5, -1]
    assert list(out["committed"][0, :4]) == [4, 1, 3, -1]


def test_path_is_the_set_of_fully_matching_nodes():
    c = workloads.tree_case(seed=3, R=24, M=20, V=300, dtype="f32")
    out = otree.tree_verify(c.logits, c.parent, c.tokens, c.n_nodes)
    for r in range(c.R):
        n = c.n_nodes[r]
        am = [int(np.argmax(c.logits[r, u])) for u in range(n)]
        good = []
        for v in range(1, n):
            u, ok = v, True
            while u != 0:                      # every edge on root .. v
                ok = ok and c.tokens[r, u] == am[c.parent[r, u]]
                u = c.parent[r, u]
            if ok:
                good.append(v)
        A = out["accepted"][r]
        assert sorted(out["path"][r, :A].tolist()) == sorted(good)
        last = out["path"][r, A - 1] if A > 0 else 0
        assert out["committed"][r, A] == am[last]
    assert out["accepted"].max() >= 2


def test_equal_siblings_take_the_lowest_index():
    V = 5
    L = np.zeros((1, 4, V), np.float32)
    L[0, 0, 3] = 1.0
    L[0, 2, 0] = 1.0
    L[0, 3, 1] = 1.0
    parent = np.array([[-1, 0, 0, 0]], np.int32)
    tokens = np.array([[-1, 1, 3, 3]], np.int32)
    out = otree.tree_verify(L, parent, tokens, np.array([4]))
    assert out["accepted"][0] == 1 and out["path"][0, 0] == 2 and out["committed"][0, 1] == 0


def test_argmax_ties_take_the_lowest_id():
    L = np.zeros((1, 2, 4), np.float32)
    L[0, 0, [1, 3]] = 2.0
    out = otree.tree_verify(L, np.array([[-1, 0]]), np.array([[-1, 3]]), np.array([2]))
    assert out["accepted"][0] == 0 and out["committed"][0, 0] == 1


@pytest.mark.parametrize("fault", ["parent_forward", "parent_root_missing", "token_high", "n_zero",
                                   "nan_row", "inf_row"])
def test_invalid_trees(fault):
    c = workloads.tree_case(seed=4, R=3, M=8, V=50, dtype="f32")
    L, P, X, n = c.logits.copy(), c.parent.copy(), c.tokens.copy(), c.n_nodes.copy()
    if fault == "parent_forward":
        P[1, 3] = 3
    elif fault == "parent_root_missing":
        P[1, 2] = -1
    elif fault == "token_high":
        X[1, 5] = 50
    elif fault == "n_zero":
        n[1] = 0
    elif fault == "nan_row":
        L[1, 0, 7] = np.nan
    else:
        L[1, 0, 7] = np.inf
    out = otree.tree_verify(L, P, X, n)
    assert out["accepted"][1] == -1 and np.all(out["committed"][1] == -1)
    assert out["accepted"][0] >= 0 and out["accepted"][2] >= 0


def test_only_children_are_candidates():
    # root -> {1: tok 7, 2: tok 9}; 1 -> {3: tok 4}.  The root row accepts
    # node 2, whose row's argmax 4 is carried by node 3 -- a child of node 1,
    # not of node 2 -- so the walk stops at node 2 with bonus 4
    V = 10
    L = np.zeros((1, 4, V), np.float32)
    L[0, 0, 9] = 1.0
    L[0, 2, 4] = 1.0
    parent = np.array([[-1, 0, 0, 1]], np.int32)
    tokens = np.array([[-1, 7, 9, 4]], np.int32)
    out = otree.tree_verify(L, parent, tokens, np.array([4]))
    assert out["accepted"][0] == 1 and out["path"][0, 0] == 2
    assert list(out["committed"][0, :2]) == [9, 4]
