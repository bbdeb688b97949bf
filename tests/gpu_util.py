"""Helpers for the GPU parity tests: host <-> device marshalling of the seeded
cases and the comparison rule against the oracle.

Comparison rule (per request):
  * validity must agree (num_accepted == -1 on both sides or on neither);
  * if the oracle saw no near tie (every decision margin >= 1e-6), tokens and
    num_accepted are bit-exact;
  * if its first near tie is the accept test at row j, the GPU must have
    accepted rows 0..j-1 too, with the same tokens; later outputs of that
    request are not graded;
  * if its first near tie is the final draw, num_accepted and the accepted
    tokens are bit-exact and only the drawn token is not graded;
  * c*, Res and log q agree within a relative tolerance (1e-5 for fp32
    inputs, 2e-3 for bf16 inputs) plus an absolute floor of 1e-6 for values
    near zero.
"""
from __future__ import annotations

import numpy as np
import torch

NEAR_TIE_EPS = 1e-6
ATOL = 1e-6


def to_device(x: np.ndarray, dev) -> torch.Tensor:
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:  # bf16 bit patterns
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(x).to(dev)


def run_verify(sv, case, dev, workspace=None) -> dict:
    out = sv.spec_verify_batch(to_device(case.target, dev),
                               to_device(case.draft, dev) if case.gamma > 0 else None,
                               to_device(case.draft_tokens, dev) if case.gamma > 0 else None,
                               to_device(case.verify_len, dev), to_device(case.temperature, dev),
                               to_device(case.u_accept, dev) if case.gamma > 0 else None,
                               to_device(case.u_sample, dev), workspace=workspace)
    torch.cuda.synchronize()
    return {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}


def float_tol(case) -> float:
    both_f32 = case.target.dtype == np.float32 and case.draft.dtype == np.float32
    return 1e-5 if both_f32 else 2e-3


def compare_verify(case, gpu: dict, ref: dict, rtol: float = None) -> dict:
    """Asserts parity; returns counts and the largest float errors seen."""
    rtol = float_tol(case) if rtol is None else rtol
    R, gamma = case.R, case.gamma
    stats = dict(near_ties=0, near_ties_matched=0, exact=0, max_rel_cstar=0.0, max_rel_resid=0.0,
                 max_rel_logq=0.0, max_abs_resid=0.0, invalid=0)
    for r in range(R):
        n_ref = int(ref["num_accepted"][r])
        n_gpu = int(gpu["num_accepted"][r])
        tag = f"request {r} (l={case.verify_len[r]}, T={case.temperature[r]})"
        if n_ref < 0 or n_gpu < 0:
            assert n_ref == n_gpu, f"{tag}: validity differs (gpu {n_gpu}, oracle {n_ref})"
            assert (gpu["tokens"][r] == -1).all(), tag
            stats["invalid"] += 1
            continue
        ft = int(ref["first_tie"][r])
        if ft < 0:
            assert n_gpu == n_ref, f"{tag}: num_accepted gpu {n_gpu} vs oracle {n_ref}"
            assert np.array_equal(gpu["tokens"][r], ref["tokens"][r]), \
                f"{tag}: tokens gpu {gpu['tokens'][r]} vs oracle {ref['tokens'][r]}"
            stats["exact"] += 1
            upto = n_ref + 1
        elif ft == gamma + 1:
            stats["near_ties"] += 1
            stats["near_ties_matched"] += int(n_gpu == n_ref and
                                              np.array_equal(gpu["tokens"][r], ref["tokens"][r]))
            assert n_gpu == n_ref, f"{tag}: num_accepted gpu {n_gpu} vs oracle {n_ref}"
            assert np.array_equal(gpu["tokens"][r, :n_ref], ref["tokens"][r, :n_ref]), tag
            upto = n_ref
        else:
            stats["near_ties"] += 1
            stats["near_ties_matched"] += int(n_gpu == n_ref and
                                              np.array_equal(gpu["tokens"][r], ref["tokens"][r]))
            assert n_gpu >= ft, f"{tag}: gpu stopped at {n_gpu} before the near tie at row {ft}"
            assert np.array_equal(gpu["tokens"][r, :ft], ref["tokens"][r, :ft]), tag
            upto = ft
        # floats: c*, Res for verified positions; NaN beyond
        l = int(case.verify_len[r])
        for key, sk in (("cstar", "max_rel_cstar"), ("resid", "max_rel_resid")):
            gk = "cstar" if key == "cstar" else "resid_mass"
            if gpu.get(gk) is None:
                continue
            g = gpu[gk][r].astype(np.float64)
            o = ref[key][r]
            assert np.isnan(g[l:]).all(), f"{tag}: {key} beyond l must be NaN"
            err = np.abs(g[:l] - o[:l])
            lim = rtol * np.abs(o[:l]) + ATOL
            assert (err <= lim).all(), f"{tag}: {key} gpu {g[:l]} vs oracle {o[:l]}"
            if l:
                big = np.abs(o[:l]) > 1e-3   # relative error where it is meaningful
                if big.any():
                    stats[sk] = max(stats[sk], float((err[big] / np.abs(o[:l][big])).max()))
                if key == "resid":
                    stats["max_abs_resid"] = max(stats["max_abs_resid"], float(err.max()))
        if gpu.get("logq") is not None:
            g = gpu["logq"][r, :upto].astype(np.float64)
            o = ref["logq"][r, :upto]
            err = np.abs(g - o)
            assert (err <= rtol * np.abs(o) + ATOL).all(), f"{tag}: logq gpu {g} vs oracle {o}"
            big = np.abs(o) > 1e-3
            if big.any():
                stats["max_rel_logq"] = max(stats["max_rel_logq"], float((err[big] / np.abs(o[big])).max()))
            if ft < 0:
                assert np.isnan(gpu["logq"][r, n_ref + 1:]).all(), tag
    return stats


def markov_oracle_all(mk, workers: int = 16) -> dict:
    """oracle.markov_draft over every request of a Markov case, the requests
    split over host threads (the C oracle keeps no shared state, and ctypes
    releases the interpreter lock during the call)."""
    import concurrent.futures
    import os
    import oracle
    R = mk.R
    n = max(1, min(workers, os.cpu_count() or 1, R))
    parts = [list(range(k, R, n)) for k in range(n)]

    def one(rows):
        return rows, oracle.markov_draft(mk.U[rows], mk.W1, mk.W2, mk.anchor[rows],
                                         mk.temperature[rows], mk.u_draft[rows])

    out = dict(tokens=np.empty((R, mk.gamma), np.int32),
               logits=np.empty((R, mk.gamma, mk.V), np.float32),
               margin_min=np.empty((R,), np.float64), first_tie=np.empty((R,), np.int32))
    with concurrent.futures.ThreadPoolExecutor(n) as ex:
        for rows, ref in ex.map(one, parts):
            for k in ("tokens", "logits", "margin_min", "first_tie"):
                out[k][rows] = ref[k]
    return out
