"""The RNN-head oracle against what fixes it independently (CPU only):
with the update gate shut it is sampling from U alone (the C Markov oracle
with a zero embedding), with the gate open and the candidate reading only the
embedding it is a Markov head with embedding tanh(W1) (the C Markov oracle on
fp32 tables), and its state stays inside (-1, 1).  Gate weights made of
identity blocks reduce the update to scalar recurrences per state unit that
are written out here: the candidate reading the hidden state alone, the
previous state plus the hidden state, and the gate held at one half."""
import numpy as np
import pytest

import oracle
import workloads
from oracle import rnn


@pytest.fixture(scope="module")
def lib():
    oracle.build(force=False)
    return oracle.load()


def small(seed, R=3, gamma=4, V=300, hidden=16, T=1.0):
    return workloads.rnn_head(seed=seed, R=R, gamma=gamma, V=V, hidden=hidden, temperature=T)


def test_shut_gate_is_sampling_from_u(lib):
    c = small(1)
    mk = c.mk
    bg = c.bg.copy()
    bg[:mk.rank] = -1e4                      # z = 0: the state stays 0
    out = rnn.rnn_draft(mk.U, mk.W1, mk.W2, c.H, c.Wg, bg, mk.anchor, mk.temperature,
                        mk.u_draft, lib=lib)
    zero_w1 = np.zeros_like(mk.W1)
    ref = oracle.markov_draft(mk.U, zero_w1, mk.W2, mk.anchor, mk.temperature, mk.u_draft, lib=lib)
    assert np.all(out["states"] == 0.0)
    np.testing.assert_array_equal(out["logits"], ref["logits"])
    np.testing.assert_array_equal(out["tokens"], ref["tokens"])


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_open_gate_on_the_embedding_is_a_markov_head(lib, T):
    c = small(2, T=T)
    mk = c.mk
    r = mk.rank
    hidden = c.H.shape[2]
    wg = np.zeros((2 * r + hidden, 2 * r), np.float32)
    wg[r:2 * r, r:2 * r] = np.eye(r, dtype=np.float32)   # candidate = the embedding slot
    bg = np.zeros(2 * r, np.float32)
    bg[:r] = 1e4                                         # z = 1: s_k = tanh(W1[x_{k-1}])
    out = rnn.rnn_draft(mk.U, mk.W1, mk.W2, c.H, wg, bg, mk.anchor, mk.temperature,
                        mk.u_draft, lib=lib)
    w1t = np.tanh(workloads.bf16_bits_to_f32(mk.W1).astype(np.float64)).astype(np.float32)
    w2 = workloads.bf16_bits_to_f32(mk.W2)
    ref = oracle.markov_draft(mk.U, w1t, w2, mk.anchor, mk.temperature, mk.u_draft, lib=lib)
    for i in range(mk.R):
        ft = int(ref["first_tie"][i])
        upto = mk.gamma if ft < 0 else ft
        np.testing.assert_array_equal(out["tokens"][i, :upto], ref["tokens"][i, :upto])
        steps = upto + 1 if ft >= 0 else mk.gamma
        np.testing.assert_allclose(out["logits"][i, :steps], ref["logits"][i, :steps],
                                   rtol=0, atol=2e-6)


def test_state_stays_in_the_open_unit_interval(lib):
    c = small(3, R=4, gamma=6)
    mk = c.mk
    out = rnn.rnn_draft(mk.U, mk.W1, mk.W2, c.H, c.Wg, c.bg, mk.anchor, mk.temperature,
                        mk.u_draft, lib=lib)
    assert np.all(np.abs(out["states"]) < 1.0)
    assert np.all(out["tokens"] >= 0)
    # the state carries history: with the same anchor and hidden, different
    # earlier tokens give different states after the first step
    assert not np.allclose(out["states"][:, 1], out["states"][:, 1].mean(axis=0))


def test_invalid_requests(lib):
    c = small(4)
    mk = c.mk
    anchor = mk.anchor.copy()
    anchor[1] = mk.V
    T = mk.temperature.copy()
    T[2] = -1.0
    out = rnn.rnn_draft(mk.U, mk.W1, mk.W2, c.H, c.Wg, c.bg, anchor, T, mk.u_draft, lib=lib)
    assert (out["tokens"][1] == -1).all() and (out["tokens"][2] == -1).all()
    assert (out["tokens"][0] >= 0).all()


def _identity_gate(rank, hidden, cand_from_state, cand_from_hidden, z_bias):
    """Wg with Wz = 0 (z = sigmoid(z_bias)) and the candidate's pre-activation
    the chosen sum of the state slot and the first rank hidden values."""
    wg = np.zeros((2 * rank + hidden, 2 * rank), np.float32)
    eye = np.eye(rank, dtype=np.float32)
    if cand_from_state:
        wg[0:rank, rank:2 * rank] = eye
    if cand_from_hidden:
        wg[2 * rank:3 * rank, rank:2 * rank] = eye
    bg = np.zeros(2 * rank, np.float32)
    bg[:rank] = z_bias
    return wg, bg


def _check_recurrence(c, wg, bg, step, lib):
    """States against s_k = step(s_{k-1}, h_k[:rank]) with s_0 = 0, and the
    logits against U_k + s_k W2, while the tokens follow the oracle's draws."""
    mk = c.mk
    r = mk.rank
    out = rnn.rnn_draft(mk.U, mk.W1, mk.W2, c.H, wg, bg, mk.anchor, mk.temperature,
                        mk.u_draft, lib=lib)
    w2 = workloads.bf16_bits_to_f32(mk.W2).astype(np.float64)
    u = workloads.bf16_bits_to_f32(mk.U).astype(np.float64) if mk.U.dtype == np.uint16 \
        else mk.U.astype(np.float64)
    for i in range(mk.R):
        s = np.zeros(r)
        for k in range(mk.gamma):
            s = step(s, c.H[i, k, :r].astype(np.float64))
            np.testing.assert_allclose(out["states"][i, k], s, rtol=0, atol=1e-12)
            want = (u[i, k] + s @ w2).astype(np.float32)
            np.testing.assert_allclose(out["logits"][i, k], want, rtol=0, atol=2e-6)
    assert np.all(out["tokens"] >= 0)
    return out


def test_candidate_reads_the_hidden_state(lib):
    # z = 1, n = tanh(h_k): s_k = tanh(h_k), no dependence on the tokens
    c = small(5, R=3, gamma=4, V=300, hidden=300)
    wg, bg = _identity_gate(c.mk.rank, 300, False, True, 1e4)
    _check_recurrence(c, wg, bg, lambda s, h: np.tanh(h), lib)


def test_candidate_reads_state_and_hidden(lib):
    # z = 1, n = tanh(s_{k-1} + h_k): s_k = tanh(s_{k-1} + h_k)
    c = small(6, R=2, gamma=5, V=300, hidden=256)
    wg, bg = _identity_gate(c.mk.rank, 256, True, True, 1e4)
    _check_recurrence(c, wg, bg, lambda s, h: np.tanh(s + h), lib)


def test_half_open_gate_averages(lib):
    # z = sigmoid(0) = 1/2: s_k = (s_{k-1} + tanh(h_k)) / 2
    c = small(7, R=2, gamma=6, V=300, hidden=256, T=0.0)
    wg, bg = _identity_gate(c.mk.rank, 256, False, True, 0.0)
    _check_recurrence(c, wg, bg, lambda s, h: 0.5 * s + 0.5 * np.tanh(h), lib)
