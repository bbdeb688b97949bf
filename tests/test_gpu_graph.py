"""HIP graph capture of the entry points that allow it (Markov draft, tree
verification, STS, verify-length scheduler): every replay, with new inputs
copied into the captured buffers and eager calls and synchronisations in
between, must equal an eager call on the same inputs.  The verification entry
points must refuse capture with SPEC_EUNSUPPORTED."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    import lossless_verification_sampling_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


@pytest.fixture(scope="module")
def dev(sv):
    return torch.device("cuda:0")


def capture(fn):
    """Captures fn() on a side stream (after one warm-up call there) and
    returns (graph, captured outputs)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    torch.cuda.synchronize()
    return g, out


def replay_and_compare(g, out, fill, eager, rounds=3):
    for k in range(rounds):
        fill(k)                       # new inputs into the captured buffers
        torch.cuda.synchronize()
        ref = [t.clone() for t in eager()]
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(out, ref):
            if a is None:
                continue
            assert torch.equal(a, b), f"replay {k} differs from the eager call"


def test_markov_draft_graph(sv, dev):
    mks = [workloads.dspark_markov(seed=s, R=8, gamma=4, V=5000) for s in (1, 2, 3)]
    U, W1, W2 = (to_device(x, dev) for x in (mks[0].U, mks[0].W1, mks[0].W2))
    anc, T, ud = (to_device(x, dev) for x in (mks[0].anchor, mks[0].temperature, mks[0].u_draft))
    ws = sv.Workspace(dev, sv.spec_markov_workspace_bytes(8, 4, 5000, 256))
    fn = lambda: sv.spec_markov_draft_sample(U, W1, W2, anc, T, ud, workspace=ws)
    g, out = capture(fn)

    def fill(k):
        U.copy_(to_device(mks[k].U, dev))
        anc.copy_(to_device(mks[k].anchor, dev))
        ud.copy_(to_device(mks[k].u_draft, dev))

    ws2 = sv.Workspace(dev, sv.spec_markov_workspace_bytes(8, 4, 5000, 256))
    eager = lambda: sv.spec_markov_draft_sample(U, W1, W2, anc, T, ud, workspace=ws2)
    replay_and_compare(g, out, fill, eager)


def test_tree_verify_graph(sv, dev):
    cs = [workloads.tree_case(seed=s, R=6, M=16, V=9000, dtype="bf16") for s in (4, 5, 6)]
    depth = max(c.max_depth for c in cs)
    L, P, X, n = (to_device(x, dev) for x in (cs[0].logits, cs[0].parent, cs[0].tokens,
                                             cs[0].n_nodes))
    ws = sv.Workspace(dev, sv.spec_tree_workspace_bytes(6, 16, 9000))
    g, out = capture(lambda: sv.spec_tree_verify(L, P, X, n, depth, workspace=ws))

    def fill(k):
        for dst, src in ((L, cs[k].logits), (P, cs[k].parent), (X, cs[k].tokens),
                         (n, cs[k].n_nodes)):
            dst.copy_(to_device(src, dev))

    ws2 = sv.Workspace(dev, sv.spec_tree_workspace_bytes(6, 16, 9000))
    replay_and_compare(g, out, fill, lambda: sv.spec_tree_verify(L, P, X, n, depth, workspace=ws2))


def test_sts_graph(sv, dev):
    cs = [workloads.sts_case(seed=s, N=2000, gamma=4, G=32) for s in (7, 8, 9)]
    z, A, grid = (to_device(x, dev) for x in (cs[0].z, cs[0].accepted, cs[0].grid))
    ws = sv.Workspace(dev, sv.spec_sts_workspace_bytes(2000, 4, 32, 15))
    g, out = capture(lambda: sv.spec_sts_calibrate(z, A, grid, want_curve=True, workspace=ws))

    def fill(k):
        z.copy_(to_device(cs[k].z, dev))
        A.copy_(to_device(cs[k].accepted, dev))

    ws2 = sv.Workspace(dev, sv.spec_sts_workspace_bytes(2000, 4, 32, 15))
    replay_and_compare(g, out, fill,
                       lambda: sv.spec_sts_calibrate(z, A, grid, want_curve=True, workspace=ws2))


def test_schedule_graph(sv, dev):
    cs = [workloads.schedule_case(seed=s, R=64, gamma=7) for s in (10, 11, 12)]
    conf, sps = to_device(cs[0].conf, dev), to_device(cs[0].sps, dev)
    ws = sv.Workspace(dev, sv.spec_schedule_workspace_bytes())
    g, out = capture(lambda: sv.spec_schedule_verify_len(conf, sps, workspace=ws))

    def fill(k):
        conf.copy_(to_device(cs[k].conf, dev))

    ws2 = sv.Workspace(dev, sv.spec_schedule_workspace_bytes())
    replay_and_compare(g, out, fill, lambda: sv.spec_schedule_verify_len(conf, sps, workspace=ws2))


def test_verify_refuses_capture(sv, dev):
    case = workloads.make_verify_case(2, 3, 1000, "bf16", seed=3)
    args = [to_device(x, dev) for x in (case.target, case.draft, case.draft_tokens,
                                        case.verify_len, case.temperature, case.u_accept,
                                        case.u_sample)]
    ws = sv.Workspace(dev, sv.spec_verify_workspace_bytes(2, 3, 1000))
    sv.spec_verify_batch(*args, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(Exception, match="SPEC_EUNSUPPORTED"):
        with torch.cuda.graph(g):
            sv.spec_verify_batch(*args, workspace=ws)
    torch.cuda.synchronize()
    out = sv.spec_verify_batch(*args, workspace=ws)   # still usable afterwards
    torch.cuda.synchronize()
    assert out["num_accepted"].min().item() >= 0
