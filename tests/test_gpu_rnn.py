"""GPU parity of spec_rnn_draft_sample against the RNN-head oracle: states
and logits to the fp32 state update's rounding, tokens exact up to the
oracle's first near tie."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import to_device
from oracle import rnn as ornn

pytestmark = pytest.mark.gpu

# fp32 gate sums of 2 rank + hidden terms (|c Wg| ~ 1) carried through up to
# seven steps: measured |ds| <= 1.1e-6 and |dl| <= 1e-6 (one ulp of logits of
# size 4..8); the bounds leave a factor of four.  Near ties as for the Markov
# head: a draw within 1e-6 of a CDF boundary is not graded.
STATE_TOL = 5e-6
LOGIT_TOL = 4e-6
TIE_EPS = 1e-6


@pytest.fixture(scope="module")
def sv():
    import lossless_verification_sampling_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


@pytest.fixture(scope="module")
def dev(sv):
    return torch.device("cuda:0")


def run(sv, dev, c, anchor=None, T=None):
    mk = c.mk
    tok, lg, st = sv.spec_rnn_draft_sample(
        to_device(mk.U, dev), to_device(mk.W1, dev), to_device(mk.W2, dev), to_device(c.H, dev),
        to_device(c.Wg, dev), to_device(c.bg, dev),
        to_device(mk.anchor if anchor is None else anchor, dev),
        to_device(mk.temperature if T is None else T, dev), to_device(mk.u_draft, dev),
        want_state=True)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), lg.cpu().numpy(), st.cpu().numpy()


@pytest.mark.parametrize("R,gamma,V,hidden,T", [
    (3, 4, 1000, 64, 1.0),
    (2, 3, 1001, 32, 0.7),       # ragged V: the guarded logits kernel
    (70, 2, 2048, 128, 1.0),     # two MFMA request blocks, a partial gate block
    (4, 3, 4096, 256, 0.0),      # greedy
    (2, 7, 129280, 1024, 1.0),   # the DSpark vocabulary
    (3, 2, 2000, 3072, 1.0),     # the largest hidden size
])
def test_rnn_matches_oracle(sv, dev, R, gamma, V, hidden, T):
    print(f"[rnn] R={R} gamma={gamma} V={V} hidden={hidden} T={T}", flush=True)
    c = workloads.rnn_head(seed=R + V + hidden, R=R, gamma=gamma, V=V, hidden=hidden,
                           temperature=T)
    tok, lg, st = run(sv, dev, c)
    mk = c.mk
    ref = ornn.rnn_draft(mk.U, mk.W1, mk.W2, c.H, c.Wg, c.bg, mk.anchor, mk.temperature,
                         mk.u_draft, tie_eps=TIE_EPS)
    ties = 0
    worst_s = worst_l = 0.0
    for r in range(R):
        ft = int(ref["first_tie"][r])
        upto = gamma if ft < 0 else ft
        ties += ft >= 0
        assert np.array_equal(tok[r, :upto], ref["tokens"][r, :upto]), (r, tok[r], ref["tokens"][r])
        steps = upto + 1 if ft >= 0 else gamma
        serr = np.abs(st[r, :steps].astype(np.float64) - ref["states"][r, :steps]).max()
        assert serr <= STATE_TOL, (r, serr)
        worst_s = max(worst_s, serr)
        lerr = np.abs(lg[r, :steps].astype(np.float64) - ref["logits"][r, :steps]).max()
        assert lerr <= LOGIT_TOL, (r, lerr)
        worst_l = max(worst_l, lerr)
    print(f"[rnn] near ties: {ties}  max |ds| {worst_s:.2e}  max |dl| {worst_l:.2e}", flush=True)


def test_rnn_full_size(sv, dev):
    """The benchmark's workload (R = 64, gamma = 7, V = 129280, hidden 1024,
    the gate product over 16 request blocks): all 64 requests on the GPU and
    on the oracle."""
    print("[rnn] R=64 gamma=7 V=129280 hidden=1024", flush=True)
    c = workloads.rnn_head(seed=6, hidden=1024)
    tok, lg, st = run(sv, dev, c)
    mk = c.mk
    ref = ornn.rnn_draft(mk.U, mk.W1, mk.W2, c.H, c.Wg, c.bg, mk.anchor, mk.temperature,
                         mk.u_draft, tie_eps=TIE_EPS)
    assert (tok >= 0).all() and (tok < mk.V).all()
    ties = 0
    for r in range(mk.R):
        ft = int(ref["first_tie"][r])
        upto = mk.gamma if ft < 0 else ft
        ties += ft >= 0
        assert np.array_equal(tok[r, :upto], ref["tokens"][r, :upto]), (r, tok[r], ref["tokens"][r])
        steps = upto + 1 if ft >= 0 else mk.gamma
        assert np.abs(st[r, :steps].astype(np.float64) - ref["states"][r, :steps]).max() <= STATE_TOL
        assert np.abs(lg[r, :steps].astype(np.float64) - ref["logits"][r, :steps]).max() <= LOGIT_TOL
    print(f"[rnn] full size: near ties {ties} of {mk.R}", flush=True)


def test_rnn_invalid_requests(sv, dev):
    c = workloads.rnn_head(seed=5, R=4, gamma=3, V=777, hidden=16)
    mk = c.mk
    anchor = mk.anchor.copy()
    anchor[1] = 777
    T = mk.temperature.copy()
    T[2] = -1.0
    tok, _, _ = run(sv, dev, c, anchor=anchor, T=T)
    ref = ornn.rnn_draft(mk.U, mk.W1, mk.W2, c.H, c.Wg, c.bg, anchor, T, mk.u_draft,
                         tie_eps=TIE_EPS)
    assert (tok[1] == -1).all() and (tok[2] == -1).all()
    for r in (0, 3):
        ft = int(ref["first_tie"][r])
        upto = mk.gamma if ft < 0 else ft
        assert np.array_equal(tok[r, :upto], ref["tokens"][r, :upto])
