"""HIP graph capture of the entry points (batched verification, the
acceptance rate, Markov draft, tree verification, STS, verify-length
scheduler): every replay, with new inputs copied into the captured buffers
and eager calls and synchronisations in between, must equal an eager call on
the same inputs."""
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
            if a.is_floating_point():   # bit patterns: NaN outputs compare equal
                it = torch.int32 if a.element_size() == 4 else torch.int64
                a, b = a.view(it), b.view(it)
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


def test_verify_batch_graph(sv, dev):
    cases = [workloads.make_verify_case(6, 5, 3000, "bf16", seed=s, noise_std=1.0,
                                        temperature=[1.0, 0.0, 0.7, 1.0, 1.0, 0.0])
             for s in (13, 14, 15)]
    names = ("target", "draft", "draft_tokens", "verify_len", "temperature", "u_accept",
             "u_sample")
    args = [to_device(getattr(cases[0], nm), dev) for nm in names]
    ws = sv.Workspace(dev, sv.spec_verify_workspace_bytes(6, 5, 3000))

    def outs(d):
        return [d["tokens"], d["num_accepted"], d["cstar"], d["resid_mass"], d["logq"]]

    g, out = capture(lambda: outs(sv.spec_verify_batch(*args, workspace=ws)))

    def fill(k):
        for t, nm in zip(args, names):
            t.copy_(to_device(getattr(cases[k], nm), dev))

    ws2 = sv.Workspace(dev, sv.spec_verify_workspace_bytes(6, 5, 3000))
    # replays and eager calls share the captured workspace too: the device
    # tag keeps their words apart
    replay_and_compare(g, out, fill, lambda: outs(sv.spec_verify_batch(*args, workspace=ws2)))
    replay_and_compare(g, out, fill, lambda: outs(sv.spec_verify_batch(*args, workspace=ws)))


def test_tv_accept_rate_graph(sv, dev):
    g0 = np.random.default_rng(3)
    rows = [(g0.standard_normal((16, 2000)).astype(np.float32),
             g0.standard_normal((16, 2000)).astype(np.float32)) for _ in range(3)]
    d, t = to_device(rows[0][0], dev), to_device(rows[0][1], dev)
    T = to_device(np.ones(16, np.float32), dev)
    ws = sv.Workspace(dev, sv.spec_tv_workspace_bytes(16, 2000))
    g, out = capture(lambda: list(sv.spec_tv_accept_rate(d, t, T, workspace=ws)))

    def fill(k):
        d.copy_(to_device(rows[k][0], dev))
        t.copy_(to_device(rows[k][1], dev))

    ws2 = sv.Workspace(dev, sv.spec_tv_workspace_bytes(16, 2000))
    replay_and_compare(g, out, fill, lambda: list(sv.spec_tv_accept_rate(d, t, T, workspace=ws2)))


def test_verify_graph_shared_workspace(sv, dev):
    """One workspace serves a captured verification, eager Markov drafts and an
    eager verification with fewer requests between the replays: every replay
    must still equal an eager call (no state of an earlier call is trusted)."""
    cases = [workloads.make_verify_case(6, 5, 3000, "bf16", seed=s, noise_std=1.0,
                                        temperature=[1.0, 0.0, 0.7, 1.0, 1.0, 0.0])
             for s in (21, 22, 23)]
    names = ("target", "draft", "draft_tokens", "verify_len", "temperature", "u_accept",
             "u_sample")
    args = [to_device(getattr(cases[0], nm), dev) for nm in names]
    mk = workloads.dspark_markov(seed=24, R=8, gamma=4, V=3000)
    small = workloads.make_verify_case(2, 3, 3000, "bf16", seed=25, noise_std=0.8)
    nbytes = max(sv.spec_verify_workspace_bytes(6, 5, 3000),
                 sv.spec_markov_workspace_bytes(8, 4, 3000, 256))
    ws = sv.Workspace(dev, nbytes)

    def outs(d):
        return [d["tokens"], d["num_accepted"], d["cstar"], d["resid_mass"], d["logq"]]

    g, out = capture(lambda: outs(sv.spec_verify_batch(*args, workspace=ws)))
    mk_args = [to_device(x, dev) for x in (mk.U, mk.W1, mk.W2, mk.anchor, mk.temperature,
                                          mk.u_draft)]
    small_args = [to_device(getattr(small, nm), dev) for nm in names]
    ws2 = sv.Workspace(dev, nbytes)
    for k in range(3):
        for t, nm in zip(args, names):
            t.copy_(to_device(getattr(cases[k], nm), dev))
        # other calls write the same workspace between the replays
        sv.spec_markov_draft_sample(*mk_args, workspace=ws)
        sv.spec_verify_batch(*small_args, workspace=ws)
        torch.cuda.synchronize()
        ref = [t.clone() for t in outs(sv.spec_verify_batch(*args, workspace=ws2))]
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(out, ref):
            if a.is_floating_point():
                a, b = a.view(torch.int32), b.view(torch.int32)
            assert torch.equal(a, b), f"replay {k} differs from the eager call"
    assert sv.spec_get_device_status(ws, clear=True) == 0
