"""GPU parity of spec_schedule_verify_len against the scheduler oracle
(DSpark guide, "scheduler"): verify lengths exact, Theta to fp64 rounding,
except where the oracle reports a stopping comparison within 1e-12 of a tie
(the GPU sums tau in a different order), where the GPU's answer must still be
a valid prefix schedule one admission from the oracle's."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import to_device
from oracle import schedule as osch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    import lossless_verification_sampling_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


@pytest.fixture(scope="module")
def dev(sv):
    return torch.device("cuda:0")


def run(sv, dev, conf, sps, topk=-1, ws=None):
    ln, th = sv.spec_schedule_verify_len(to_device(conf, dev), to_device(sps, dev), topk=topk,
                                         workspace=ws)
    torch.cuda.synchronize()
    return ln.cpu().numpy(), float(th.cpu().numpy()[0])


def walk_lengths(conf, k):
    """The verify lengths after admitting the first k candidates of the
    oracle's pool order."""
    a = osch.survival(conf)
    lens = np.zeros(conf.shape[0], np.int32)
    for (r, j) in osch.pool_order(a)[:k]:
        lens[r] = j
    return lens


def compare(conf, sps, topk, ln, th):
    ref = osch.schedule(conf, sps, topk)
    print(f"[schedule] admitted={ref['admitted']} sum_len={int(ln.sum())} "
          f"tie_margin={ref['tie_margin']:.3g}", flush=True)
    assert ln.shape == ref["len"].shape
    if ref["tie_margin"] < osch.TIE_REL:
        # the stopping comparison is within rounding of a tie: the GPU may stop
        # one admission earlier or later, but always on the oracle's walk
        npool = conf.shape[0] * conf.shape[1]
        cands = [walk_lengths(conf, k) for k in (ref["admitted"] - 1, ref["admitted"],
                                                  ref["admitted"] + 1) if 0 <= k <= npool]
        assert any(np.array_equal(ln, c) for c in cands), (ln, ref["len"])
        return ref
    np.testing.assert_array_equal(ln, ref["len"])
    assert th == pytest.approx(ref["theta"], rel=1e-12, abs=0.0)
    return ref


@pytest.mark.parametrize("R,gamma,curve,topk", [
    (64, 7, "smooth", -1),
    (64, 7, "cliff", -1),
    (64, 7, "flat", -1),
    (256, 7, "smooth", -1),
    (256, 7, "cliff", -1),
    (1, 7, "smooth", -1),
    (64, 7, "smooth", 100),
    (256, 7, "cliff", 1000),
    (100, 5, "smooth", 17),        # pool of 500: not a power of two
    (1024, 8, "smooth", -1),       # the largest pool, 8192 candidates
    (1024, 8, "cliff", 5000),
])
def test_schedule_matches_oracle(sv, dev, R, gamma, curve, topk):
    case = workloads.schedule_case(seed=R + gamma, R=R, gamma=gamma, curve=curve)
    ln, th = run(sv, dev, case.conf, case.sps, topk)
    compare(case.conf, case.sps, topk, ln, th)


def test_schedule_ties_and_table_end(sv, dev):
    # every survival probability equal: the order is (request, position)
    conf = np.ones((8, 4), np.float32)
    sps = np.ones(8 * 5 + 1, np.float32)
    for topk in (0, 1, 5, 13, 32, 40):
        ln, th = run(sv, dev, conf, sps, topk)
        compare(conf, sps, topk, ln, th)
    ln, th = run(sv, dev, conf, sps, -1)          # flat curve: everything admitted
    compare(conf, sps, -1, ln, th)
    short = np.ones(8 + 3, np.float32)            # B up to 10: room for two admissions
    ln, th = run(sv, dev, conf, short, -1)
    compare(conf, short, -1, ln, th)
    tiny = np.ones(5, np.float32)                 # B = R is already past the table
    ln, th = run(sv, dev, conf, tiny, -1)
    assert ln.tolist() == [0] * 8 and th == 0.0


def test_schedule_zero_confidence_and_empty_draft(sv, dev):
    conf = np.zeros((16, 6), np.float32)
    sps = workloads.schedule_case(R=16, gamma=6).sps
    ln, th = run(sv, dev, conf, sps, -1)
    compare(conf, sps, -1, ln, th)
    empty = np.zeros((16, 0), np.float32)
    ln, th = run(sv, dev, empty, sps, -1)
    assert ln.tolist() == [0] * 16 and th == pytest.approx(16.0 * float(sps[16]), rel=1e-15)


def test_schedule_invalid_inputs_flagged(sv, dev):
    ws = sv.Workspace(dev, 1 << 16)
    conf = np.full((4, 3), 0.5, np.float32)
    conf[2, 1] = 1.5
    sps = np.ones(20, np.float32)
    ln, th = run(sv, dev, conf, sps, -1, ws)
    assert ln.tolist() == [-1] * 4 and np.isnan(th)
    assert sv.spec_get_device_status(ws, clear=True) & sv.SPEC_DEV_BAD_REQUEST
    bad_table = sps.copy()
    bad_table[7] = -1.0
    ln, _ = run(sv, dev, np.full((4, 3), 0.5, np.float32), bad_table, -1, ws)
    assert ln.tolist() == [-1] * 4
    assert sv.spec_get_device_status(ws, clear=True) & sv.SPEC_DEV_BAD_REQUEST
    ln, _ = run(sv, dev, np.full((4, 3), 0.5, np.float32), sps, -1, ws)   # a valid call after
    assert np.all(ln >= 0)
    assert sv.spec_get_device_status(ws, clear=True) == 0
