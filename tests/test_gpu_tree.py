"""GPU parity of spec_tree_verify against the greedy tree oracle: accepted
counts, paths and committed tokens bit-exact (argmax of the same values, no
floating-point arithmetic in between), for bf16 and fp32 rows, vector and
scalar loads (odd V), ragged slices, chain trees, single-node trees, deep
and wide trees, equal siblings, argmax ties across slices, invalid trees and
rows, repeated calls."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import to_device
from oracle import tree as otree

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    import lossless_verification_sampling_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


@pytest.fixture(scope="module")
def dev(sv):
    return torch.device("cuda:0")


def run(sv, dev, L, P, X, n, max_depth, ws=None):
    acc, path, tok = sv.spec_tree_verify(to_device(L, dev), to_device(P, dev), to_device(X, dev),
                                         to_device(np.asarray(n, np.int32), dev), max_depth,
                                         workspace=ws)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), path.cpu().numpy(), tok.cpu().numpy()


def check(out, ref):
    acc, path, tok = out
    np.testing.assert_array_equal(acc, ref["accepted"])
    np.testing.assert_array_equal(path, ref["path"])
    np.testing.assert_array_equal(tok, ref["committed"])


@pytest.mark.parametrize("R,M,V,dtype", [
    (5, 12, 3000, "bf16"),       # one slice
    (6, 20, 20000, "f32"),       # three slices, the last ragged
    (4, 16, 8193, "bf16"),       # odd V: the scalar path, a one-logit slice
    (3, 24, 70001, "f32"),       # odd V, fp32
    (8, 32, 151936, "bf16"),     # the benchmark's vocabulary
])
def test_tree_matches_oracle(sv, dev, R, M, V, dtype):
    print(f"[tree] R={R} M={M} V={V} {dtype}", flush=True)
    c = workloads.tree_case(seed=R * 7 + M, R=R, M=M, V=V, dtype=dtype)
    ref = otree.tree_verify(c.logits, c.parent, c.tokens, c.n_nodes)
    check(run(sv, dev, c.logits, c.parent, c.tokens, c.n_nodes, c.max_depth), ref)
    assert ref["accepted"].max() >= 1


def test_tree_benchmark_workload(sv, dev):
    # the benchmark's trees: 64 of 48 nodes, widths 3 / 2 / 2 / 1, V = 151936 bf16
    print("[tree] R=64 M=48 V=151936 bf16 (benchmark)", flush=True)
    c = workloads.tree_case(seed=12, R=64, M=48, V=151936, dtype="bf16",
                            widths=(3, 2, 2, 1, 1, 1, 1, 1))
    ref = otree.tree_verify(c.logits, c.parent, c.tokens, c.n_nodes)
    check(run(sv, dev, c.logits, c.parent, c.tokens, c.n_nodes, c.max_depth), ref)
    assert ref["accepted"].max() >= 4


def test_chain_deep_and_single_node_trees(sv, dev):
    V, M = 5000, 40
    c = workloads.tree_case(seed=2, R=4, M=M, V=V, dtype="bf16", widths=(1,) * 39, p_hit=0.95)
    c.n_nodes[3] = 1                                       # a root alone: bonus only
    ref = otree.tree_verify(c.logits, c.parent, c.tokens, c.n_nodes)
    check(run(sv, dev, c.logits, c.parent, c.tokens, c.n_nodes, M - 1), ref)
    assert ref["accepted"][3] == 0 and ref["accepted"].max() >= 5


def test_largest_tree_walked_to_the_bottom(sv, dev):
    # 1024 nodes in one chain, every edge planted: the walk accepts 1023
    # nodes over 1025 launches (max_depth = M - 1)
    M, V = 1024, 3000
    print(f"[tree] chain M={M} V={V}", flush=True)
    c = workloads.tree_case(seed=31, R=2, M=M, V=V, dtype="f32", widths=(1,) * (M - 1),
                            p_hit=1.0)
    ref = otree.tree_verify(c.logits, c.parent, c.tokens, c.n_nodes)
    assert ref["accepted"][0] == M - 1
    check(run(sv, dev, c.logits, c.parent, c.tokens, c.n_nodes, M - 1), ref)


def test_equal_siblings_and_ties_across_slices(sv, dev):
    V, M = 20000, 6
    L = np.zeros((1, M, V), np.float32)
    L[0, 0, [9000, 17000]] = 3.0                           # tie across slices: id 9000
    L[0, 2, [100, 16500]] = 2.0
    parent = np.array([[-1, 0, 0, 0, 2, 2]], np.int32)
    tokens = np.array([[-1, 17000, 9000, 9000, 16500, 100]], np.int32)
    ref = otree.tree_verify(L, parent, tokens, np.array([M]))
    assert ref["accepted"][0] == 2 and list(ref["path"][0, :2]) == [2, 5]
    check(run(sv, dev, L, parent, tokens, [M], 2), ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_signed_zero_maximum_across_slices(sv, dev, dtype):
    """A row whose maximum is zero, -0.0 at a lower id (one slice) and +0.0 at
    a higher one (another slice): the two are equal, so the lower id is the
    argmax, as for any tie."""
    V, M = 20000, 3
    L = np.full((1, M, V), -1.0, np.float32)
    L[0, 0, 9000] = -0.0
    L[0, 0, 17000] = 0.0
    L[0, 1, 17000] = -0.0                                  # same again one level down,
    L[0, 1, 9000] = 0.0                                    # with the signs swapped
    assert np.signbit(L[0, 0, 9000]) and not np.signbit(L[0, 0, 17000])
    parent = np.array([[-1, 0, 1]], np.int32)
    tokens = np.array([[-1, 9000, 9000]], np.int32)
    ref = otree.tree_verify(L, parent, tokens, np.array([M]))
    assert ref["accepted"][0] == 2 and ref["committed"][0, 2] == int(np.argmax(L[0, 2]))
    Ls = workloads.f32_to_bf16_bits(L) if dtype == "bf16" else L
    check(run(sv, dev, Ls, parent, tokens, [M], 2), ref)


@pytest.mark.parametrize("fault", ["parent_forward", "token_high", "n_zero", "too_deep",
                                   "nan_on_path", "inf_on_path"])
def test_invalid_trees(sv, dev, fault):
    c = workloads.tree_case(seed=5, R=3, M=10, V=4000, dtype="f32", p_hit=1.0)
    L, P, X, n = c.logits.copy(), c.parent.copy(), c.tokens.copy(), c.n_nodes.copy()
    depth = c.max_depth
    if fault == "parent_forward":
        P[1, 4] = 6
    elif fault == "token_high":
        X[1, 3] = 4000
    elif fault == "n_zero":
        n[1] = 0
    elif fault == "too_deep":
        depth = c.max_depth - 1                            # every tree is too deep
    elif fault == "nan_on_path":
        L[1, 0, 11] = np.nan
    else:
        L[1, 0, 3999] = -np.inf
    ws = sv.Workspace(dev, sv.spec_tree_workspace_bytes(3, 10, 4000))
    acc, path, tok = run(sv, dev, L, P, X, n, depth, ws)
    assert acc[1] == -1 and np.all(path[1] == -1) and np.all(tok[1] == -1)
    assert sv.spec_get_device_status(ws, clear=True) & sv.SPEC_DEV_BAD_REQUEST
    if fault != "too_deep":
        ref = otree.tree_verify(L, P, X, n)
        np.testing.assert_array_equal(acc, ref["accepted"])
        np.testing.assert_array_equal(tok, ref["committed"])
    good = run(sv, dev, c.logits, c.parent, c.tokens, c.n_nodes, c.max_depth, ws)
    check(good, otree.tree_verify(c.logits, c.parent, c.tokens, c.n_nodes))


def test_repeated_calls_share_a_workspace(sv, dev):
    c = workloads.tree_case(seed=8, R=16, M=24, V=30000, dtype="bf16")
    ref = otree.tree_verify(c.logits, c.parent, c.tokens, c.n_nodes)
    ws = sv.Workspace(dev, sv.spec_tree_workspace_bytes(16, 24, 30000))
    for _ in range(3):
        check(run(sv, dev, c.logits, c.parent, c.tokens, c.n_nodes, c.max_depth, ws), ref)
