"""Plain CPU oracle of the RNN serial head (fp64).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may call this; the product library never does.  It shares
no code with the HIP library; the inverse-CDF draw is the C oracle's.

Method (DSpark paper guide, personal-site-bgy.pages.dev, the serial-head
section: "Markov head" and the RNN variant after it): the RNN head keeps a
state s_k that accumulates the block's prefix.  Each step concatenates the
previous state s_{k-1}, the previous token's embedding W1[x_{k-1}] and the
backbone hidden h_k, makes one gated update, and projects the state to the
transition bias added to the base logits U_k; s_0 = 0 and x_0 is the anchor.
Sampling is as for the Markov head: softmax of (U_k + bias) / T, inverse CDF
in ascending token id (argmax, lowest id, at T = 0).

Readings where the pages leave a step open (listed in the design notes):
  * the gated update has one update gate on the concatenation
    c = [s_{k-1}; W1[x_{k-1}]; h_k]:
        z = sigmoid(c Wz + bz),  n = tanh(c Wn + bn),
        s_k = (1 - z) * s_{k-1} + z * n,
    with Wg = [Wz | Wn] of shape (2 r + hidden) x 2 r and bg = [bz | bn];
  * the state has the rank r of W1 and W2, and the bias is s_k W2 (W2 is the
    Markov head's logit projection);
  * the stored logits are the fp32 rounding of U_k + s_k W2 taken in fp64.
"""
from __future__ import annotations

import numpy as np

from . import TIE_EPS, inverse_cdf, load


def _f64(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:  # bf16 bit patterns
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def _temperature_ok(t: float) -> bool:
    if not np.isfinite(t) or t < 0.0:
        return False
    return t == 0.0 or 1e-30 <= t <= 1e30


def rnn_draft(U, W1, W2, H, Wg, bg, anchor, temperature, u_draft,
              tie_eps: float = TIE_EPS, lib=None) -> dict:
    """tokens [R, gamma] int32 (-1 for an invalid request), logits
    [R, gamma, V] fp32, states [R, gamma, r] fp64, margin_min [R],
    first_tie [R] (step index k-1 of the first draw within tie_eps)."""
    lib = lib or load()
    U64 = _f64(U)
    R, G, V = U64.shape
    w1, w2 = _f64(W1), _f64(W2)
    rank = w1.shape[1]
    h = _f64(H)
    wg, b = _f64(Wg), np.asarray(bg, dtype=np.float64)
    tokens = np.full((R, G), -1, np.int32)
    logits = np.zeros((R, G, V), np.float32)
    states = np.zeros((R, G, rank), np.float64)
    margin_min = np.full(R, np.inf)
    first_tie = np.full(R, -1, np.int32)
    for r in range(R):
        T = float(temperature[r])
        x = int(anchor[r])
        ok = _temperature_ok(T) and 0 <= x < V
        s = np.zeros(rank)
        mm, ft = np.inf, -1
        for k in range(1, G + 1):
            if not ok:
                break
            c = np.concatenate([s, w1[x], h[r, k - 1]])
            g = c @ wg + b
            with np.errstate(over="ignore"):  # exp(+large) = inf gives z = 0 exactly
                z = 1.0 / (1.0 + np.exp(-g[:rank]))
            n = np.tanh(g[rank:])
            s = (1.0 - z) * s + z * n
            states[r, k - 1] = s
            l32 = (U64[r, k - 1] + s @ w2).astype(np.float32)
            if np.any(np.isnan(l32)) or np.any(l32 == np.inf):
                ok = False
                break
            logits[r, k - 1] = l32
            if T == 0.0:
                x = int(np.argmax(l32))
            else:
                u = float(u_draft[r, k - 1])
                if not (0.0 <= u < 1.0):
                    ok = False
                    break
                a = l32.astype(np.float64) / T
                e = np.exp(a - a.max())
                p = e / e.sum()
                x, mg = inverse_cdf(p, u, lib)
                mm = min(mm, mg)
                if ft < 0 and mg < tie_eps:
                    ft = k - 1
            if x < 0:
                ok = False
                break
            tokens[r, k - 1] = x
        if not ok:
            tokens[r] = -1
            mm, ft = np.inf, -1
        margin_min[r], first_tie[r] = mm, ft
    return dict(tokens=tokens, logits=logits, states=states, margin_min=margin_min,
                first_tie=first_tie)
