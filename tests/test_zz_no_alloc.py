"""The no-allocation verification entry point (spec_verify_batch_noalloc)
against spec_verify_batch on the same inputs: two calls in a row on the
library's fixed scratch, the second smaller than the first, then the first
again; outputs bit-identical to the workspace entry point's (the same kernels
on the same inputs) and, through the same comparison rule as every verify
test, to the oracle.  A call too large for the scratch is refused on the
host."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import compare_verify, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    import lossless_verification_sampling_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


@pytest.fixture(scope="module")
def dev(sv):
    return torch.device("cuda:0")


def _inputs(case, dev):
    g = case.gamma > 0
    return (to_device(case.target, dev), to_device(case.draft, dev) if g else None,
            to_device(case.draft_tokens, dev) if g else None, to_device(case.verify_len, dev),
            to_device(case.temperature, dev), to_device(case.u_accept, dev) if g else None,
            to_device(case.u_sample, dev))


def _outputs(case, dev):
    R, G = case.R, case.gamma
    return dict(tokens=torch.full((R, G + 1), -7, dtype=torch.int32, device=dev),
                num_accepted=torch.full((R,), -7, dtype=torch.int32, device=dev),
                cstar=torch.full((R, G), 7.0, dtype=torch.float32, device=dev),
                resid_mass=torch.full((R, G), 7.0, dtype=torch.float32, device=dev),
                logq=torch.full((R, G + 1), 7.0, dtype=torch.float32, device=dev))


def _host(o):
    return {k: v.cpu().numpy() for k, v in o.items()}


def _same(a, b):
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k


CASES = [
    # 48 requests at the largest vocabulary of the batched workloads, bf16,
    # mixed temperatures (greedy included) and every verify length
    lambda: workloads.make_verify_case(48, 7, 151936, "bf16", seed=81,
                                       noise_std=[0.5, 0.8, 1.1, 1.4, 1.7, 2.0, 2.5],
                                       verify_len=np.arange(48) % 8,
                                       temperature=np.where(np.arange(48) % 3 == 0, 0.0,
                                                            np.where(np.arange(48) % 3 == 1,
                                                                     1.0, 0.7))),
    # a smaller second call: 5 requests, fp32, a ragged vocabulary
    lambda: workloads.make_verify_case(5, 3, 4099, "f32", seed=82, noise_std=[0.5, 1.0, 2.0],
                                       verify_len=[3, 0, 2, 3, 1],
                                       temperature=[1.0, 1.0, 0.0, 0.7, 1.3]),
]


def test_noalloc_matches_workspace_entry_point(sv, dev):
    cases = [CASES[0](), CASES[1]()]
    refs = [oracle.verify_case(c) for c in cases]
    # two calls in a row on the fixed scratch, the second smaller, then the
    # first again (the scratch keeps the smaller call's words in between)
    for k in (0, 1, 0):
        case = cases[k]
        ins = _inputs(case, dev)
        ws = sv.Workspace(dev, sv.spec_verify_workspace_bytes(case.R, case.gamma, case.V))
        o_ws = sv.spec_verify_batch(*ins, out=_outputs(case, dev), workspace=ws)
        o_na = sv.spec_verify_batch_noalloc(*ins, out=_outputs(case, dev))
        torch.cuda.synchronize()
        a, b = _host(o_ws), _host(o_na)
        print(f"[noalloc] case {k}: R={case.R} gamma={case.gamma} V={case.V} "
              f"accepted {b['num_accepted'].tolist()[:12]}", flush=True)
        _same(a, b)
        assert sv.spec_get_device_status(ws, clear=True) == 0
        stats = compare_verify(case, b, refs[k])
        assert stats["exact"] + stats["near_ties"] == case.R, stats


def test_noalloc_refuses_oversized_calls(sv, dev):
    need = sv.spec_verify_workspace_bytes(512, 7, 151936)
    assert need > sv.SPEC_NOALLOC_SCRATCH_BYTES
    # shapes only: the library refuses before touching any buffer
    t = torch.empty((512, 8, 151936), dtype=torch.bfloat16, device=dev)
    d = torch.empty((512, 7, 151936), dtype=torch.bfloat16, device=dev)
    i32 = lambda *s: torch.zeros(s, dtype=torch.int32, device=dev)  # noqa: E731
    f32 = lambda *s: torch.zeros(s, dtype=torch.float32, device=dev)  # noqa: E731
    out = dict(tokens=i32(512, 8), num_accepted=i32(512), cstar=None, resid_mass=None,
               logq=None)
    with pytest.raises(sv.SpecError) as e:
        sv.spec_verify_batch_noalloc(t, d, i32(512, 7), i32(512), f32(512), f32(512, 7),
                                     f32(512, 8), out=out)
    assert e.value.status == sv.SPEC_ETOOLARGE
    del t, d
