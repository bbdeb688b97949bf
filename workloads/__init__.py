"""Seeded synthetic workloads for the verification and Markov-draft paths.

This module only draws random inputs.  It holds none of the method's
arithmetic (no softmax, no accept test, no inverse-CDF draw): the oracle and
the HIP library both consume what it produces, and neither imports the other.

Random numbers come from numpy's Philox counter-based generator
(``numpy.random.Philox``), one independent key per (seed, stream id):

  stream 0  draft tokens (Gumbel-max draws from the draft logits)
  stream 1  u_accept   [R, gamma]       uniforms for the accept tests
  stream 2  u_sample   [R, gamma + 1]   uniforms for the residual / bonus draw
  stream 3  u_draft    [R, gamma]       uniforms for the Markov-head draft
  stream 4  target logits
  stream 5  draft-logit noise
  stream 6  per-request parameters (verify lengths, noise scales, anchors)
  stream 7  Markov tables W1, W2 and base logits U
  stream 8  scheduler confidences and step-rate tables
  stream 9  RNN-head backbone hidden states and gate weights

Uniforms are fp32 values (w >> 8) * 2**-24 of 32-bit Philox words: exact in
fp32 and always in [0, 1).

bf16 tensors are carried as ``numpy.uint16`` bit patterns (round to nearest
even from fp32); fp32 tensors as ``numpy.float32``.

The five named workloads follow the shapes, value distributions and
structure of the pages' settings (gamma = 7 for DSpark's block, gamma = 8 for
DART's default draft length, Qwen3- and DeepSeek-scale vocabularies, batch 1
to 256, suffix decay of acceptance across positions).  The pages evaluate on
public benchmark suites that are not used here: these synthetic inputs stand
in for them.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

STREAM_DRAFT_TOKENS = 0
STREAM_U_ACCEPT = 1
STREAM_U_SAMPLE = 2
STREAM_U_DRAFT = 3
STREAM_TARGET = 4
STREAM_NOISE = 5
STREAM_PARAMS = 6
STREAM_MARKOV = 7
STREAM_SCHEDULE = 8
STREAM_RNN = 9
STREAM_STS = 10
STREAM_TREE = 11


def rng(seed: int, stream: int) -> np.random.Generator:
    """Philox generator keyed by (seed, stream)."""
    return np.random.Generator(np.random.Philox(key=[int(seed), int(stream)]))


def uniforms(gen: np.random.Generator, shape) -> np.ndarray:
    """fp32 uniforms in [0, 1): top 24 bits of a 32-bit word times 2**-24."""
    w = gen.integers(0, 2**32, size=shape, dtype=np.uint32)
    return ((w >> np.uint32(8)).astype(np.float32) * np.float32(2.0**-24)).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = b >> np.uint32(16)
    out &= np.uint32(1)
    out += np.uint32(0x7FFF)
    out += b
    out >>= np.uint32(16)
    return out.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f32(x: np.ndarray) -> np.ndarray:
    """fp32 values of a logit array (uint16 = bf16 bits, float32 as is)."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x)
    return np.asarray(x, dtype=np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dtype)


def gumbel_max_tokens(zd: np.ndarray, temperature: np.ndarray, seed: int) -> np.ndarray:
    """Draft tokens x_{i+1} drawn from softmax(zd[r, i] / T_r) by the Gumbel-max
    construction (argmax of z/T + Gumbel noise); argmax of zd at T = 0.  This is
    how a draft model hands its samples to verification; it is not the
    verifier's own inverse-CDF rule."""
    R, G, V = zd.shape
    gen = rng(seed, STREAM_DRAFT_TOKENS)
    out = np.empty((R, G), dtype=np.int32)
    for r in range(R):
        z = as_f32(zd[r]).astype(np.float64)
        T = float(temperature[r])
        if T == 0.0:
            out[r] = np.argmax(z, axis=1)
            continue
        w = gen.integers(1, 2**32, size=(G, V), dtype=np.uint64).astype(np.float64) * 2.0**-32
        out[r] = np.argmax(z / T - np.log(-np.log(w)), axis=1)
    return out


@dataclasses.dataclass
class VerifyCase:
    """Inputs of one batched verification call (shapes follow the C ABI)."""

    name: str
    target: np.ndarray          # [R, gamma+1, V] uint16 (bf16) or float32
    draft: np.ndarray           # [R, gamma, V]   uint16 (bf16) or float32
    draft_tokens: np.ndarray    # [R, gamma] int32
    verify_len: np.ndarray      # [R] int32
    temperature: np.ndarray     # [R] float32
    u_accept: np.ndarray        # [R, gamma] float32
    u_sample: np.ndarray        # [R, gamma+1] float32
    seed: int = 0

    @property
    def R(self) -> int:
        return int(self.target.shape[0])

    @property
    def gamma(self) -> int:
        return int(self.draft.shape[1])

    @property
    def V(self) -> int:
        return int(self.target.shape[2])

    def subset(self, rows) -> "VerifyCase":
        rows = np.asarray(rows)
        return VerifyCase(self.name + "[sub]", self.target[rows], self.draft[rows],
                          self.draft_tokens[rows], self.verify_len[rows],
                          self.temperature[rows], self.u_accept[rows], self.u_sample[rows],
                          self.seed)


@dataclasses.dataclass
class MarkovCase:
    """Inputs of one Markov-head draft call plus the target for verification."""

    name: str
    U: np.ndarray               # [R, gamma, V] base draft logits
    W1: np.ndarray              # [V, rank]
    W2: np.ndarray              # [rank, V]
    anchor: np.ndarray          # [R] int32
    temperature: np.ndarray     # [R] float32
    u_draft: np.ndarray         # [R, gamma] float32
    target: np.ndarray          # [R, gamma+1, V]
    verify_len: np.ndarray      # [R] int32
    u_accept: np.ndarray        # [R, gamma]
    u_sample: np.ndarray        # [R, gamma+1]
    seed: int = 0

    @property
    def R(self) -> int:
        return int(self.U.shape[0])

    @property
    def gamma(self) -> int:
        return int(self.U.shape[1])

    @property
    def V(self) -> int:
        return int(self.U.shape[2])

    @property
    def rank(self) -> int:
        return int(self.W1.shape[1])


def _uniform_streams(seed: int, R: int, gamma: int):
    return (uniforms(rng(seed, STREAM_U_ACCEPT), (R, gamma)),
            uniforms(rng(seed, STREAM_U_SAMPLE), (R, gamma + 1)))


def make_verify_case(R: int, gamma: int, V: int, dtype: str = "bf16", seed: int = 0,
                     target_std: float = 3.0, noise_std=1.0,
                     verify_len=None, temperature=1.0, draft_dtype: Optional[str] = None,
                     planted_boost: float = 0.0, name: str = "custom") -> VerifyCase:
    """Generic case: target ~ N(0, target_std^2) (optionally one planted id per
    target row raised by `planted_boost`), draft = target + N(0, sigma^2) with
    sigma per position (array of length gamma), per request (array of length R)
    or scalar; verify lengths and temperatures scalar or per request."""
    draft_dtype = draft_dtype or dtype
    gt = rng(seed, STREAM_TARGET)
    z = gt.standard_normal((R, gamma + 1, V), dtype=np.float32)
    z *= np.float32(target_std)
    if planted_boost:
        ids = rng(seed, STREAM_PARAMS).integers(0, V, size=(R, gamma + 1))
        rr, ii = np.meshgrid(np.arange(R), np.arange(gamma + 1), indexing="ij")
        z[rr, ii, ids] += np.float32(planted_boost)
    target = _store(z, dtype)
    del z
    zt = as_f32(target)[:, :gamma, :]
    sig = np.asarray(noise_std, dtype=np.float32)
    if sig.ndim == 0:
        sig = np.full((R, gamma), float(sig), dtype=np.float32)
    elif sig.shape == (gamma,):
        sig = np.broadcast_to(sig[None, :], (R, gamma))
    elif sig.shape == (R,):
        sig = np.broadcast_to(sig[:, None], (R, gamma))
    gn = rng(seed, STREAM_NOISE)
    noise = gn.standard_normal((R, gamma, V), dtype=np.float32)
    noise *= sig[:, :, None].astype(np.float32)
    noise += zt
    draft = _store(noise, draft_dtype)
    del noise, zt
    if verify_len is None:
        verify_len = gamma
    vl = np.asarray(verify_len, dtype=np.int32)
    if vl.ndim == 0:
        vl = np.full((R,), int(vl), dtype=np.int32)
    T = np.asarray(temperature, dtype=np.float32)
    if T.ndim == 0:
        T = np.full((R,), float(T), dtype=np.float32)
    tokens = gumbel_max_tokens(draft, T, seed)
    ua, us = _uniform_streams(seed, R, gamma)
    return VerifyCase(name, target, draft, tokens, vl.astype(np.int32), T.astype(np.float32),
                      ua, us, seed)


# ---------------------------------------------------------------------------
# the five named workloads
# ---------------------------------------------------------------------------

def tiny_chain(temperature: float = 1.0, seed: int = 1) -> VerifyCase:
    """R=1, gamma=4 (+1 bonus row), V=32, fp32 target ~ N(0, 2^2), draft =
    target + N(0, 1), l = 4; run at T = 1 and T = 0."""
    return make_verify_case(1, 4, 32, "f32", seed, target_std=2.0, noise_std=1.0,
                            verify_len=4, temperature=temperature,
                            name=f"tiny_chain_T{temperature:g}")


def single_user(seed: int = 2) -> VerifyCase:
    """R=1, gamma=8, V=151936, fp32 target ~ N(0, 3^2) with one planted
    dominant id per row (+8), draft = target + N(0, 1.5^2), l = 8, T = 1."""
    return make_verify_case(1, 8, 151936, "f32", seed, target_std=3.0, noise_std=1.5,
                            verify_len=8, temperature=1.0, planted_boost=8.0,
                            name="single_user")


def batched(seed: int = 3, R: int = 64, gamma: int = 7, V: int = 151936) -> VerifyCase:
    """R=64, gamma=7, V=151936, bf16 target ~ N(0, 3^2); draft noise sigma
    rising linearly 0.5 -> 2.5 across positions (suffix decay); l_r uniform on
    0..7; T = 1."""
    sig = (0.5 + 2.0 * np.arange(gamma) / max(gamma - 1, 1)).astype(np.float32)
    vl = rng(seed, STREAM_PARAMS).integers(0, gamma + 1, size=R).astype(np.int32)
    return make_verify_case(R, gamma, V, "bf16", seed, target_std=3.0, noise_std=sig,
                            verify_len=vl, temperature=1.0, name="batched")


def truncated_geometric(gen: np.random.Generator, p: float, kmax: int, size: int) -> np.ndarray:
    """Draws on 0..kmax with P(k) proportional to p (1-p)^k."""
    k = np.arange(kmax + 1)
    w = p * (1.0 - p) ** k
    return gen.choice(k, size=size, p=w / w.sum()).astype(np.int32)


def high_load_mixed(seed: int = 5, R: int = 256, gamma: int = 7, V: int = 129280) -> VerifyCase:
    """R=256, gamma=7, V=129280, bf16 target ~ N(0, 3^2); per-request noise
    sigma ~ U[0.5, 3]; l_r truncated geometric(0.3) on 0..7; even requests at
    T = 0 (greedy), odd requests at T = 1."""
    gp = rng(seed, STREAM_PARAMS)
    vl = truncated_geometric(gp, 0.3, gamma, R)
    sig = gp.uniform(0.5, 3.0, size=R).astype(np.float32)
    T = np.where(np.arange(R) % 2 == 0, 0.0, 1.0).astype(np.float32)
    return make_verify_case(R, gamma, V, "bf16", seed, target_std=3.0, noise_std=sig,
                            verify_len=vl, temperature=T, name="high_load_mixed")


def dspark_markov(seed: int = 4, R: int = 64, gamma: int = 7, V: int = 129280,
                  rank: int = 256, temperature: float = 1.0) -> MarkovCase:
    """R=64, gamma=7, V=129280: bf16 base draft logits U_k ~ N(0, 2^2); W1
    [V, 256] and W2 [256, V] bf16 ~ N(0, 0.02^2); anchor uniform over V; target
    rows 0..gamma-1 = U_k + N(0, 1), target row gamma a fresh N(0, 2^2) +
    N(0, 1); l = gamma; T = 1."""
    gm = rng(seed, STREAM_MARKOV)
    U32 = gm.standard_normal((R, gamma, V), dtype=np.float32) * np.float32(2.0)
    W1 = f32_to_bf16_bits(gm.standard_normal((V, rank), dtype=np.float32) * np.float32(0.02))
    W2 = f32_to_bf16_bits(gm.standard_normal((rank, V), dtype=np.float32) * np.float32(0.02))
    U = f32_to_bf16_bits(U32)
    del U32
    gp = rng(seed, STREAM_PARAMS)
    anchor = gp.integers(0, V, size=R).astype(np.int32)
    gt = rng(seed, STREAM_TARGET)
    extra = gt.standard_normal((R, 1, V), dtype=np.float32) * np.float32(2.0)
    base = np.concatenate([bf16_bits_to_f32(U), extra], axis=1)
    del extra
    base += rng(seed, STREAM_NOISE).standard_normal((R, gamma + 1, V), dtype=np.float32)
    target = f32_to_bf16_bits(base)
    del base
    T = np.full((R,), float(temperature), dtype=np.float32)
    ud = uniforms(rng(seed, STREAM_U_DRAFT), (R, gamma))
    ua, us = _uniform_streams(seed, R, gamma)
    return MarkovCase("dspark_markov", U, W1, W2, anchor, T, ud, target,
                      np.full((R,), gamma, dtype=np.int32), ua, us, seed)


# name -> (builder, description) for the parity tests and the benchmark
WORKLOADS = {
    "tiny_chain": tiny_chain,
    "single_user": single_user,
    "batched": batched,
    "dspark_markov": dspark_markov,
    "high_load_mixed": high_load_mixed,
}


@dataclasses.dataclass
class RnnCase:
    """Inputs of one RNN-head draft call: the Markov head's U, W1, W2,
    anchors, temperatures and uniforms, plus the backbone hidden states and
    the gate weights."""
    mk: MarkovCase
    H: np.ndarray    # [R, gamma, hidden] fp32 backbone hidden states h_k
    Wg: np.ndarray   # [2 rank + hidden, 2 rank] bf16 bits: update-gate and candidate weights
    bg: np.ndarray   # [2 rank] fp32 biases


def rnn_head(seed: int = 6, R: int = 64, gamma: int = 7, V: int = 129280, hidden: int = 1024,
             temperature: float = 1.0) -> RnnCase:
    """The Markov workload's U, W1, W2 (same recipe), hidden states
    h_k ~ N(0, 1), gate weights ~ N(0, 1 / (2 rank + hidden)) in bf16 and
    biases ~ N(0, 0.1^2)."""
    mk = dspark_markov(seed=seed, R=R, gamma=gamma, V=V, temperature=temperature)
    g = rng(seed, STREAM_RNN)
    rank = mk.rank
    din = 2 * rank + hidden
    H = g.standard_normal((R, gamma, hidden), dtype=np.float32)
    Wg = f32_to_bf16_bits(g.standard_normal((din, 2 * rank), dtype=np.float32)
                          * np.float32(1.0 / np.sqrt(din)))
    bg = (g.standard_normal(2 * rank, dtype=np.float32) * np.float32(0.1)).astype(np.float32)
    return RnnCase(mk=mk, H=H, Wg=Wg, bg=bg)


@dataclasses.dataclass
class ScheduleCase:
    """Inputs of the confidence-scheduled verify length: per-position
    confidences (the confidence head's outputs) and a step-rate table."""
    conf: np.ndarray  # [R, gamma] fp32 in [0, 1]
    sps: np.ndarray   # [bmax + 1] fp32, steps per second at batch size B
    R: int
    gamma: int


def schedule_case(seed: int = 8, R: int = 64, gamma: int = 7, curve: str = "smooth",
                  bmax: Optional[int] = None) -> ScheduleCase:
    """Confidences with a per-request level and a decay along the block (the
    suffix decay of acceptance), and one of three step-rate curves over batch
    sizes 0..bmax: "smooth" (falls as 1 / (1 + B / (2 R))), "cliff" (the same
    curve taken at B rounded up to a multiple of 128 rows: flat inside a tile,
    a step down past each boundary, the saw-tooth of a padded engine) or
    "flat"."""
    gen = rng(seed, STREAM_SCHEDULE)
    level = gen.uniform(0.55, 0.98, size=(R, 1))
    decay = gen.uniform(0.0, 0.06, size=(R, 1))
    noise = gen.normal(0.0, 0.05, size=(R, gamma))
    conf = np.clip(level - decay * np.arange(gamma)[None, :] + noise, 0.01, 0.999)
    conf = conf.astype(np.float32)
    bmax = R * (gamma + 1) if bmax is None else bmax
    B = np.arange(bmax + 1, dtype=np.float64)
    if curve == "flat":
        sps = np.full(bmax + 1, 50.0)
    elif curve == "smooth":
        sps = 1000.0 / (1.0 + B / (2.0 * max(R, 1)))
    elif curve == "cliff":
        sps = 1000.0 / (1.0 + np.ceil(B / 128.0) * 128.0 / (2.0 * max(R, 1)))
    else:
        raise ValueError(curve)
    return ScheduleCase(conf=conf, sps=sps.astype(np.float32), R=R, gamma=gamma)


def algorithmic_bytes(verify_len: np.ndarray, V: int, t_elt: int, d_elt: int) -> int:
    """Bytes the method must move for one verification call: every verified
    draft row and target row, read once, plus the bonus target row."""
    vl = np.asarray(verify_len, dtype=np.int64)
    vl = vl[(vl >= 0)]
    return int(((vl * (t_elt + d_elt)).sum() + vl.size * t_elt) * V)


@dataclasses.dataclass
class StsCase:
    """A held-out set for confidence calibration: the confidence head's raw
    logits per draft position and each block's accepted prefix length."""
    z: np.ndarray       # [N, gamma] fp32 raw confidence logits
    accepted: np.ndarray  # [N] int32 leading accepted positions, 0..gamma
    grid: np.ndarray    # [G] fp64 candidate temperatures, ascending
    N: int
    gamma: int


def sts_case(seed: int = 10, N: int = 4096, gamma: int = 7, G: int = 64,
             kappa: float = 1.2) -> StsCase:
    """Per block a difficulty u ~ N(1, 1) and per position a suffix decay of
    0.15; the true conditional acceptance is pi = sigmoid(u - 0.15 (k - 1) +
    N(0, 0.5^2)), acceptance of each position is drawn from pi and the block
    keeps its leading accepts.  The head is overconfident: its raw logit is
    (kappa + 0.1 k) logit(pi) + N(0, 0.3^2).  Candidate temperatures: G values
    spaced evenly in log between 0.25 and 8."""
    g = rng(seed, STREAM_STS)
    u = g.normal(1.0, 1.0, size=(N, 1))
    k = np.arange(1, gamma + 1)[None, :]
    lg = u - 0.15 * (k - 1) + g.normal(0.0, 0.5, size=(N, gamma))
    pi = 1.0 / (1.0 + np.exp(-lg))
    acc = g.random(size=(N, gamma)) < pi
    rej = ~acc
    first_rej = np.where(rej.any(axis=1), rej.argmax(axis=1), gamma)
    z = ((kappa + 0.1 * k) * lg + g.normal(0.0, 0.3, size=(N, gamma))).astype(np.float32)
    grid = np.exp(np.linspace(np.log(0.25), np.log(8.0), G))
    return StsCase(z=z, accepted=first_rej.astype(np.int32), grid=grid, N=N, gamma=gamma)


@dataclasses.dataclass
class TreeCase:
    """A draft tree per request (topological order, node 0 the root) and the
    target's logits at every node."""
    logits: np.ndarray   # [R, M, V] bf16 bits (uint16) or fp32
    parent: np.ndarray   # [R, M] int32, -1 for the root and unused slots
    tokens: np.ndarray   # [R, M] int32 draft token of each node (root: -1)
    n_nodes: np.ndarray  # [R] int32
    R: int
    M: int
    V: int
    max_depth: int


def tree_case(seed: int = 12, R: int = 64, M: int = 32, V: int = 151936, dtype: str = "bf16",
              widths=(4, 3, 2, 2, 1, 1, 1, 1), p_hit: float = 0.7,
              n_nodes: Optional[np.ndarray] = None) -> TreeCase:
    """Trees grown breadth first with at most widths[d] children per node at
    depth d (distinct sibling tokens) until M nodes; target rows ~ N(0, 3^2)
    with, for each node, probability p_hit that one of its children's tokens
    is planted as the row's argmax (+24, eight standard deviations: above the
    largest of 151936 draws), so accepted paths run a few levels deep."""
    g = rng(seed, STREAM_TREE)
    parent = np.full((R, M), -1, np.int32)
    tokens = np.full((R, M), -1, np.int32)
    nn = np.full(R, M, np.int32) if n_nodes is None else np.asarray(n_nodes, np.int32)
    depth_max = 0
    for r in range(R):
        depth = [0]
        n = 1
        frontier = [0]
        while frontier and n < nn[r]:
            nxt = []
            for u in frontier:
                w = widths[depth[u]] if depth[u] < len(widths) else 0
                ids = g.choice(V, size=w, replace=False) if w else []
                for t in ids:
                    if n >= nn[r]:
                        break
                    parent[r, n] = u
                    tokens[r, n] = int(t)
                    depth.append(depth[u] + 1)
                    nxt.append(n)
                    n += 1
            frontier = nxt
        nn[r] = n
        depth_max = max(depth_max, max(depth))
    z = (g.standard_normal((R, M, V), dtype=np.float32) * np.float32(3.0))
    for r in range(R):
        for u in range(nn[r]):
            kids = [v for v in range(u + 1, nn[r]) if parent[r, v] == u]
            if kids and g.random() < p_hit:
                z[r, u, tokens[r, g.choice(kids)]] += np.float32(24.0)
    logits = f32_to_bf16_bits(z) if dtype == "bf16" else z
    return TreeCase(logits=logits, parent=parent, tokens=tokens, n_nodes=nn, R=R, M=M, V=V,
                    max_depth=depth_max)
