"""GPU parity of spec_verify_batch and spec_tv_accept_rate against the oracle
(called through the C ABI via the binding).  The named workloads run at their
full sizes; small cases span several chunks and a ragged tail; edge cases cover
empty, degenerate and invalid inputs."""
import numpy as np
import pytest
import torch

import oracle
import oracle_pins
import workloads
from gpu_util import compare_verify, run_verify, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    import lossless_verification_sampling_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


@pytest.fixture(scope="module")
def dev(sv):
    return torch.device("cuda:0")


def _report(name, stats):
    print(f"[{name}] exact={stats['exact']} near_ties={stats['near_ties']} "
          f"(matched anyway {stats['near_ties_matched']}) invalid={stats['invalid']} "
          f"max_rel c*={stats['max_rel_cstar']:.2e} res={stats['max_rel_resid']:.2e} "
          f"(abs {stats['max_abs_resid']:.1e}) logq={stats['max_rel_logq']:.2e}", flush=True)


def _check(sv, dev, case, name, workspace=None, rtol=None):
    print(f"[{name}] R={case.R} gamma={case.gamma} V={case.V} "
          f"dtypes={case.target.dtype},{case.draft.dtype}", flush=True)
    gpu = run_verify(sv, case, dev, workspace)
    ref = oracle.verify_case(case)
    stats = compare_verify(case, gpu, ref, rtol)
    _report(name, stats)
    return gpu, ref, stats


# ---------------------------------------------------------------------------
# the named workloads at full size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1.0, 0.0])
def test_tiny_chain(sv, dev, T):
    _check(sv, dev, workloads.tiny_chain(temperature=T), f"tiny_chain_T{T}")


def test_single_user_full(sv, dev):
    gpu, ref, st = _check(sv, dev, workloads.single_user(), "single_user")
    assert st["exact"] + st["near_ties"] == 1


def test_batched_full(sv, dev):
    case = workloads.batched()
    gpu, ref, st = _check(sv, dev, case, "batched")
    assert st["exact"] + st["near_ties"] == case.R


def test_high_load_mixed_full(sv, dev):
    case = workloads.high_load_mixed()
    gpu, ref, st = _check(sv, dev, case, "high_load_mixed")
    assert st["exact"] + st["near_ties"] == case.R
    # greedy requests are exact by construction
    greedy = case.temperature == 0
    assert (ref["first_tie"][greedy] < 0).all()


# ---------------------------------------------------------------------------
# small cases: several chunks, ragged tails, dtypes, temperatures
# ---------------------------------------------------------------------------

SMALL = [
    # R, gamma, V, t_dtype, d_dtype
    (5, 4, 1000, "bf16", "bf16"),
    (3, 7, 70001, "bf16", "bf16"),     # odd V: scalar-load path, ragged chunk
    (4, 3, 65536, "f32", "f32"),
    (6, 5, 9000, "bf16", "f32"),       # mixed dtypes (Markov-draft verify layout)
    (6, 5, 9000, "f32", "bf16"),
    (2, 8, 151936, "bf16", "bf16"),
    (9, 2, 17, "f32", "f32"),          # V smaller than one vector group
    (1, 1, 1, "f32", "f32"),           # single-token vocabulary
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "R%d_g%d_V%d_%s_%s" % s)
def test_small_shapes(sv, dev, shape):
    R, gamma, V, tdt, ddt = shape
    gen = np.random.default_rng(R * 1000 + V)
    vl = gen.integers(0, gamma + 1, R).astype(np.int32)
    vl[0] = gamma
    T = np.array([1.0, 0.0, 0.6, 1.7, 1.0, 0.05][:R] * (R // 6 + 1), np.float32)[:R]
    case = workloads.make_verify_case(R, gamma, V, tdt, seed=V + R, draft_dtype=ddt,
                                      target_std=2.5, noise_std=1.0, verify_len=vl,
                                      temperature=T)
    _check(sv, dev, case, f"small_{R}_{gamma}_{V}_{tdt}_{ddt}")


def test_gamma_zero(sv, dev):
    """gamma = 0: each request commits one token drawn from target row 0."""
    case = workloads.make_verify_case(7, 0, 5000, "bf16", seed=4, verify_len=0,
                                      temperature=[1.0, 0.0, 1.0, 0.5, 2.0, 0.0, 1.0])
    _check(sv, dev, case, "gamma0")


def test_verify_len_extremes(sv, dev):
    for l in (0, 6):
        case = workloads.make_verify_case(8, 6, 20000, "bf16", seed=10 + l, verify_len=l,
                                          temperature=1.0)
        _check(sv, dev, case, f"all_l{l}")


def test_max_gamma(sv, dev):
    case = workloads.make_verify_case(2, 64, 3000, "bf16", seed=64, noise_std=0.05,
                                      verify_len=[64, 40], temperature=1.0)
    _check(sv, dev, case, "gamma64")


def test_large_batch_walks_all_candidates(sv, dev):
    # R = 160, gamma = 48: the unit table (4 (3 R + R (gamma + 1)) = 33.3 KB)
    # exceeds the 32 KB the streaming kernels list in LDS, so they walk every
    # candidate item instead; greedy and sampled requests mixed
    R, G = 160, 48
    g = np.random.default_rng(160)
    case = workloads.make_verify_case(R, G, 1500, "bf16", seed=160, noise_std=0.3,
                                      verify_len=g.integers(0, G + 1, size=R).tolist(),
                                      temperature=[0.0 if r % 3 == 0 else 0.9 for r in range(R)])
    gpu, ref, st = _check(sv, dev, case, "large_batch")
    assert st["exact"] + st["near_ties"] == R


@pytest.mark.parametrize("V,dtype", [(262144, "bf16"), (262143, "f32")])
def test_largest_vocabulary(sv, dev, V, dtype):
    # V = 262144: 256 chunks per row, every chunk block of the unit combines
    # in use; V - 1 (odd) takes the scalar loads
    case = workloads.make_verify_case(3, 3, V, dtype, seed=V % 1000, noise_std=1.0,
                                      verify_len=[3, 2, 3], temperature=[1.0, 0.0, 0.8])
    gpu, ref, st = _check(sv, dev, case, f"V{V}")
    assert st["exact"] + st["near_ties"] == case.R


def test_identical_and_disjoint_rows(sv, dev):
    case = workloads.make_verify_case(6, 4, 4096, "f32", seed=8, verify_len=4, temperature=1.0)
    case.draft[:3] = case.target[:3, :4]                 # p == q: every draft accepted
    case.draft[3:, :, 1::2] = -np.inf                    # disjoint supports: draft on
    case.target[3:, :, 0::2] = -np.inf                   # even ids, target on odd ids
    case.draft_tokens[3:] = 2 * (case.draft_tokens[3:] // 2)
    gpu, ref, _ = _check(sv, dev, case, "identical_disjoint")
    assert (gpu["num_accepted"][:3] == 4).all()
    assert np.allclose(gpu["cstar"][:3], 1.0, atol=1e-6)
    assert np.allclose(gpu["resid_mass"][:3], 0.0, atol=1e-6)
    assert (gpu["num_accepted"][3:] == 0).all() and (gpu["tokens"][3:, 0] % 2 == 1).all()
    assert np.allclose(gpu["cstar"][3:], 0.0, atol=1e-6)


def test_small_and_large_temperature(sv, dev):
    case = workloads.make_verify_case(4, 3, 8192, "bf16", seed=12, verify_len=3,
                                      temperature=[0.01, 0.2, 5.0, 50.0])
    _check(sv, dev, case, "temperatures")


def test_invalid_requests(sv, dev):
    """Invalid inputs flag only their own request (num_accepted -1, tokens -1,
    NaN floats) and raise the device status bit."""
    from lossless_verification_sampling_amd import (SPEC_DEV_BAD_REQUEST, Workspace,
                                                    spec_get_device_status)
    R = 10
    case = workloads.make_verify_case(R, 3, 2048, "f32", seed=5, verify_len=3, temperature=1.0)
    case.verify_len[1] = 4              # l > gamma
    case.draft_tokens[2, 1] = 2048      # token out of range
    case.target[3, 2, 7] = np.nan       # NaN logit
    case.draft[4, 0, 9] = np.inf        # +inf logit
    case.temperature[5] = -1.0          # negative temperature
    case.u_accept[6, 0] = 1.0           # uniform out of range
    case.target[7, 1] = -np.inf         # a row of only -inf
    case.temperature[8] = 0.0
    case.target[8, 0, 3] = np.nan       # NaN at T = 0
    ws = Workspace(dev)
    gpu, ref, st = _check(sv, dev, case, "invalid", workspace=ws)
    assert st["invalid"] == 8 and gpu["num_accepted"][0] >= 0 and gpu["num_accepted"][9] >= 0
    bits = spec_get_device_status(ws, clear=True)
    assert bits & SPEC_DEV_BAD_REQUEST
    assert spec_get_device_status(ws, clear=True) == 0


def test_masked_ids_are_valid(sv, dev):
    case = workloads.make_verify_case(4, 3, 5000, "bf16", seed=6, verify_len=3, temperature=1.0)
    ninf = workloads.f32_to_bf16_bits(np.array([-np.inf], np.float32))[0]
    case.target[:, :, 4000:] = ninf     # padded vocabulary tail
    case.draft[:, :, 4000:] = ninf
    case.draft_tokens[:] = np.minimum(case.draft_tokens, 3999)
    gpu, _, st = _check(sv, dev, case, "masked")
    assert st["invalid"] == 0 and (gpu["tokens"] < 4000).all()


# ---------------------------------------------------------------------------
# exact law on the GPU: the committed token follows q exactly
# ---------------------------------------------------------------------------

def test_exact_grid_law_on_gpu(sv, dev):
    """The oracle's exact-enumeration pin, replayed through the GPU: over every
    draft token and an 840-point grid of both uniforms the law of the first
    committed token equals q0 exactly (DART note eq. (3)-(4))."""
    from fractions import Fraction
    den, p0, q0, q1 = oracle_pins.EXACT_CASES[0]
    V, n_grid = 4, oracle_pins.GRID_FOR_DEN[den]
    g = (np.arange(n_grid, dtype=np.float64) + 0.5) / n_grid
    ua, us = np.meshgrid(g, g, indexing="ij")
    xs = [x for x in range(V) if p0[x] > 0]
    n = ua.size
    R = n * len(xs)
    target = np.empty((R, 2, V), np.float32)
    target[:, 0] = oracle_pins._logits_from_probs(np.array(q0) / den)
    target[:, 1] = oracle_pins._logits_from_probs(np.array(q1) / den)
    draft = np.empty((R, 1, V), np.float32)
    draft[:, 0] = oracle_pins._logits_from_probs(np.array(p0) / den)
    case = workloads.VerifyCase("grid", target, draft,
                                np.repeat(np.array(xs, np.int32), n)[:, None],
                                np.ones(R, np.int32), np.ones(R, np.float32),
                                np.tile(ua.ravel(), len(xs)).astype(np.float32)[:, None],
                                np.stack([np.tile(us.ravel(), len(xs))] * 2, 1).astype(np.float32))
    gpu = run_verify(sv, case, dev)
    tok0 = gpu["tokens"][:, 0].reshape(len(xs), n)
    law = [Fraction(0)] * V
    for k, x in enumerate(xs):
        for v in range(V):
            law[v] += Fraction(p0[x], den) / n * int((tok0[k] == v).sum())
    assert law == [Fraction(a, den) for a in q0], law


# ---------------------------------------------------------------------------
# determinism, workspace reuse, and the standalone c* entry point
# ---------------------------------------------------------------------------

def test_run_twice_bit_identical(sv, dev):
    case = workloads.make_verify_case(16, 7, 151936, "bf16", seed=77,
                                      noise_std=np.linspace(0.5, 2.5, 7),
                                      verify_len=np.arange(16) % 8, temperature=1.0)
    a = run_verify(sv, case, dev)
    b = run_verify(sv, case, dev)
    for k in a:
        if a[k] is not None:
            assert np.array_equal(a[k], b[k], equal_nan=True), k


def test_workspace_reuse_across_shapes(sv, dev):
    from lossless_verification_sampling_amd import Workspace
    ws = Workspace(dev)
    shapes = [(3, 2, 50000), (40, 7, 4096), (1, 8, 151936), (40, 7, 4096), (2, 1, 33)]
    for i, (R, gamma, V) in enumerate(shapes):
        case = workloads.make_verify_case(R, gamma, V, "bf16", seed=200 + i,
                                          verify_len=np.arange(R) % (gamma + 1),
                                          temperature=1.0)
        _check(sv, dev, case, f"reuse_{i}", workspace=ws)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tv_accept_rate(sv, dev, dtype):
    N, V = 37, 30011
    gen = np.random.default_rng(3)
    zt = (gen.standard_normal((N, V)) * 3).astype(np.float32)
    zd = (zt + gen.standard_normal((N, V)) * np.linspace(0.05, 3, N)[:, None]).astype(np.float32)
    zd[0] = zt[0]
    T = np.array([1.0, 0.0, 0.7, 2.0] * 10, np.float32)[:N]
    if dtype == "bf16":
        zt, zd = workloads.f32_to_bf16_bits(zt), workloads.f32_to_bf16_bits(zd)
    cs, rs = sv.spec_tv_accept_rate(to_device(zd, dev), to_device(zt, dev), to_device(T, dev))
    torch.cuda.synchronize()
    ref_c, ref_r = oracle.tv_accept_rate(zd, zt, T)
    tol = 1e-5 if dtype == "f32" else 2e-3
    assert np.allclose(cs.cpu().numpy(), ref_c, rtol=tol, atol=1e-6)
    assert np.allclose(rs.cpu().numpy(), ref_r, rtol=tol, atol=1e-6)
    assert abs(cs[0].item() - 1.0) < 1e-6


def _same_bits(a, b, what):
    for k, x in a.items():
        y = b[k]
        if x is None or y is None:
            assert x is None and y is None, (what, k)
            continue
        assert x.shape == y.shape and np.array_equal(x.view(np.uint8), y.view(np.uint8)), \
            (what, k)


def test_verify_path_choice(sv, dev, monkeypatch):
    """The batched workload's shape takes the held path on this GPU, the
    high-load batch (R = 256) and fp32 rows the split path, and the
    environment switch forces the split path."""
    bf = torch.bfloat16
    assert sv.spec_verify_path(64, 7, 151936, bf, bf) == sv.SPEC_PATH_HELD
    assert sv.spec_verify_path(256, 7, 129280, bf, bf) == sv.SPEC_PATH_SPLIT
    assert sv.spec_verify_path(1, 8, 151936, torch.float32, torch.float32) == sv.SPEC_PATH_SPLIT
    assert sv.spec_verify_path(64, 7, 65536, bf, bf) == sv.SPEC_PATH_SPLIT  # 64 chunks
    monkeypatch.setenv("SPECVERIFY_SPLIT", "1")
    assert sv.spec_verify_path(64, 7, 151936, bf, bf) == sv.SPEC_PATH_SPLIT


@pytest.mark.parametrize("seed", [51, 52])
def test_held_and_split_paths_identical(sv, dev, seed, monkeypatch):
    """bf16 rows of more than 64 chunks take the held-pair launch (one
    workgroup keeps each row pair on chip between the two passes); the split
    launches (SPECVERIFY_SPLIT=1) must give the same bits, and both the
    oracle's, on a batch mixing T > 0 and T = 0 requests, every verify length
    and an invalid request."""
    R, g, V = 24, 7, 151936
    T = np.array([1.0, 0.0, 0.7, 1.3] * 6, np.float32)
    lens = (np.arange(R) % (g + 1)).astype(np.int32)
    case = workloads.make_verify_case(R, g, V, "bf16", seed=seed,
                                      noise_std=np.linspace(0.5, 2.5, g), verify_len=lens,
                                      temperature=T)
    case.verify_len[5] = g + 3   # invalid
    held = run_verify(sv, case, dev)
    monkeypatch.setenv("SPECVERIFY_SPLIT", "1")
    split = run_verify(sv, case, dev)
    monkeypatch.delenv("SPECVERIFY_SPLIT")
    _same_bits(held, split, "verify")
    st = compare_verify(case, held, oracle.verify_case(case))
    assert st["invalid"] == 1 and st["exact"] + st["near_ties"] == R - 1, st


@pytest.mark.parametrize("R,V,lmode", [(16, 65 * 1024 - 8, "mixed"),   # 65 chunks: one slot
                                         (40, 129280, "mixed"),
                                         (64, 151936, "full"),          # 448 pairs: two rounds
                                         (72, 131072, "full")],         # 504 pairs, whole chunks
                         ids=["V66552", "V129280", "two_rounds", "V131072_two_rounds"])
def test_held_path_edges(sv, dev, R, V, lmode, monkeypatch):
    """The held path at its edges: the smallest vocabulary it takes (65
    chunks, one shared-memory slot, a ragged last chunk), V = 129280, and
    batches with more pairs than compute units (a workgroup holds two pairs
    in turn): the same bits as the split path and the oracle's tokens."""
    g = 7
    assert sv.spec_verify_path(R, g, V, torch.bfloat16, torch.bfloat16) == sv.SPEC_PATH_HELD
    lens = np.full(R, g, np.int32) if lmode == "full" else (np.arange(R) % (g + 1)).astype(np.int32)
    T = np.array([1.0, 0.7, 0.0, 1.5], np.float32)[np.arange(R) % 4]
    case = workloads.make_verify_case(R, g, V, "bf16", seed=61 + R,
                                      noise_std=np.linspace(0.5, 2.5, g), verify_len=lens,
                                      temperature=T)
    held = run_verify(sv, case, dev)
    monkeypatch.setenv("SPECVERIFY_SPLIT", "1")
    split = run_verify(sv, case, dev)
    monkeypatch.delenv("SPECVERIFY_SPLIT")
    _same_bits(held, split, "verify")
    st = compare_verify(case, held, oracle.verify_case(case))
    assert st["exact"] + st["near_ties"] == R, st


def test_held_and_split_accept_rate_identical(sv, dev, monkeypatch):
    """Row-pair mode on bf16 rows of V = 151936, with more pairs than compute
    units (two rounds per workgroup): held and split launches give the same
    bits, within the bf16 tolerance of the oracle."""
    N, V = 300, 151936
    gen = np.random.default_rng(5)
    zt = (gen.standard_normal((N, V)) * 3).astype(np.float32)
    zd = (zt + gen.standard_normal((N, V)) * np.linspace(0.05, 3, N)[:, None]).astype(np.float32)
    T = np.array([1.0, 0.0, 0.7, 2.0] * 75, np.float32)[:N]
    zt, zd = workloads.f32_to_bf16_bits(zt), workloads.f32_to_bf16_bits(zd)
    args = (to_device(zd, dev), to_device(zt, dev), to_device(T, dev))
    held = [t.cpu().numpy() for t in sv.spec_tv_accept_rate(*args)]
    monkeypatch.setenv("SPECVERIFY_SPLIT", "1")
    split = [t.cpu().numpy() for t in sv.spec_tv_accept_rate(*args)]
    monkeypatch.delenv("SPECVERIFY_SPLIT")
    torch.cuda.synchronize()
    _same_bits({"c": held[0], "r": held[1]}, {"c": split[0], "r": split[1]}, "accept rate")
    ref_c, ref_r = oracle.tv_accept_rate(zd, zt, T)
    assert np.allclose(held[0], ref_c, rtol=2e-3, atol=1e-6)
    assert np.allclose(held[1], ref_r, rtol=2e-3, atol=1e-6)


def test_concurrent_calls_on_two_streams(sv, dev):
    """Two verification calls with distinct workspaces run concurrently on two
    streams: both must match the oracle, with no device status bit (no wait
    gave up)."""
    cases = [workloads.make_verify_case(48, 7, 151936, "bf16", seed=s,
                                        noise_std=[0.5, 0.8, 1.1, 1.4, 1.7, 2.0, 2.5],
                                        verify_len=7) for s in (41, 42)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [sv.Workspace(dev, sv.spec_verify_workspace_bytes(48, 7, 151936)) for _ in range(2)]
    names = ("target", "draft", "draft_tokens", "verify_len", "temperature", "u_accept",
             "u_sample")
    args = [[to_device(getattr(c, nm), dev) for nm in names] for c in cases]
    torch.cuda.synchronize()
    outs = [None, None]
    for rep in range(3):
        for k in range(2):
            with torch.cuda.stream(streams[k]):
                outs[k] = sv.spec_verify_batch(*args[k], workspace=wss[k])
        torch.cuda.synchronize()
    for k in range(2):
        assert sv.spec_get_device_status(wss[k], clear=True) == 0
        gpu = {n: (v.cpu().numpy() if v is not None else None) for n, v in outs[k].items()}
        ref = oracle.verify_case(cases[k])
        st = compare_verify(cases[k], gpu, ref)
        assert st["exact"] + st["near_ties"] == cases[k].R


def test_stats_launch_timing_hook(sv, dev):
    """spec_time_stats_launch brackets the statistics launch of the next calls
    with the caller's events: each pair spans a positive time shorter than the
    whole call, the outputs are those of an untimed call, and calls past the
    n requested (or after n = 0) record nothing."""
    import bench
    case = workloads.make_verify_case(8, 7, 151936, "bf16", seed=91,
                                      noise_std=np.linspace(0.5, 2.5, 7),
                                      verify_len=np.arange(8) % 8, temperature=1.0)
    plain = run_verify(sv, case, dev)
    hev = bench.HipEvents(4)
    try:
        sv.spec_time_stats_launch(hev.events[:2], hev.events[2:])
        s0 = torch.cuda.Event(enable_timing=True)
        s1 = torch.cuda.Event(enable_timing=True)
        s0.record()
        timed = [run_verify(sv, case, dev) for _ in range(2)]
        s1.record()
        extra = run_verify(sv, case, dev)   # past the two requested: untimed
        torch.cuda.synchronize()
        spans = [hev.elapsed_ms(k, 2 + k) for k in range(2)]
        whole = s0.elapsed_time(s1)
        print(f"[timing hook] statistics launches {spans} ms, two calls {whole:.4f} ms",
              flush=True)
        assert all(0.0 < t < whole for t in spans), (spans, whole)
        for out in timed + [extra]:
            for k in plain:
                if plain[k] is not None:
                    assert np.array_equal(plain[k], out[k], equal_nan=True), k
    finally:
        sv.spec_time_stats_launch([], [])
        hev.close()
