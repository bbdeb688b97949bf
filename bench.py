"""Benchmark of batched speculative-sampling verification on one MI355X.

A step is one spec_verify_batch call over the batched workload (R = 64
requests, gamma = 7, V = 151936, bf16 logits, verify lengths uniform on 0..7,
T = 1): every row of the hot path (softmax statistics, c*, accept tests,
prefix survival, residual / bonus draw, commit) runs in that one call.  For
bf16 rows of more than 64 chunks (this workload) the call launches two
kernels on the current stream: the held-pair kernel (one workgroup per row
pair keeps most of the pair on its compute unit between the statistics pass
and the total-variation pass, so the pair is read from memory about once) and
the per-request combine with the draw and the commit.  Other shapes take the
split path's four launches (chunk statistics, normaliser folds, the
total-variation pass, the combine); spec_verify_path says which.

Inputs are generated once (seeded), uploaded, and replicated into enough
device copies that consecutive steps never find their logits in the 256 MB
Infinity Cache: each step reads a copy untouched for at least 512 MB of other
traffic, so the timed region streams from HBM.

Prints one JSON line:
  value      verified draft positions per second (sum of l_r per call / time)
  roofline   the dominant kernel, the call's first launch (the held-pair
             kernel, or on the split path the statistics launch; either reads
             every needed row): algorithmic bytes (every verified draft row
             and target row plus the bonus row, read once) / its average
             HIP-event time inside the timed calls, against 8 TB/s;
             call_roofline the same bytes over the whole call
  cpu_baseline  the fp64 oracle on the host over the same batch: all usable
             cores (up to a one-GPU share of 16, requests split over
             threads), with the one-thread figure beside it

The other verify workloads (--workload single_user, dspark_verify,
high_load, tiny) give the same line for the other batch shapes; --workload
dspark measures the Markov-head draft (R = 64, gamma = 7, V = 129280, rank
256); --workload schedule the confidence-scheduled verify lengths of the same
batch size (448 candidates); --workload rnn the RNN serial head at the Markov
workload's size; --workload sts the confidence head's sequential temperature
scaling on a held-out set; --workload tree greedy verification of draft
trees.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("verified draft positions/sec and achieved HBM GB/s (% of peak), "
          "R=64 γ=7 V=151936")
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


# The sources each counter entry's kernels are built from.
TRAFFIC_SOURCES = {
    "verify_batched": ("common.h", "verify.hip"),
    "verify_single_user": ("common.h", "verify.hip"),
    "verify_dspark_verify": ("common.h", "verify.hip"),
    "verify_high_load": ("common.h", "verify.hip"),
    "verify_tiny": ("common.h", "verify.hip"),
    "markov_dspark": ("common.h", "markov.hip"),
    "rnn_head": ("common.h", "markov.hip"),
    "tree_greedy": ("common.h", "tree.hip"),
}


def source_hash(key: str) -> str:
    """Hash of the code of entry `key`'s kernel sources with comments and blank
    space removed, so that counter figures stay tied to the code they were
    measured on."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "lossless_verification_sampling_amd", "csrc")
    for f in TRAFFIC_SOURCES[key]:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            code = fh.read()
        code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        code = " ".join(code.split())
        h.update(f.encode() + b"\0" + code.encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key: str, kernel: str = None):
    """HBM bytes per call (all of the library's kernels), or per launch of the
    kernel whose name contains `kernel`, from the committed rocprofv3 counter
    summary, if it was taken on the current kernel sources; None otherwise."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(kernel_key)
    if not e or e.get("source_hash") != source_hash(kernel_key):
        return None
    if kernel is None:
        return e.get("bytes_per_launch")
    tot = [v for k, v in e.get("per_dispatch_fetch", {}).items() if kernel in k]
    tot += [v for k, v in e.get("per_dispatch_write", {}).items() if kernel in k]
    return sum(tot) if tot else None


def timed_steps(call, steps: int, stream):
    """(wall seconds, per-call GPU ms) of `steps` calls call(k).  The wall
    time is that of the calls issued back to back with a synchronisation on
    both sides and nothing between them; the per-call GPU times come from a
    second pass of the same calls (k = steps .. 2 steps - 1), each bracketed
    by HIP events (an event between two calls adds a gap of its own, hence
    the separate pass)."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        call(k)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for k in range(steps):
        ev[k][0].record(stream)
        call(steps + k)
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    return wall, np.array([a.elapsed_time(b) for a, b in ev])


class HipEvents:
    """hipEvent_t handles made through the HIP runtime torch has loaded, for
    timing a launch inside a library call (torch.cuda.Event cannot be handed
    to the library)."""

    def __init__(self, n: int):
        import ctypes
        try:
            self.hip = ctypes.CDLL("libamdhip64.so")
        except OSError:
            self.hip = ctypes.CDLL("/opt/rocm/lib/libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.events.append(e.value)

    def elapsed_ms(self, a: int, b: int) -> float:
        import ctypes
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.events[a], self.events[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        for e in self.events:
            self.hip.hipEventDestroy(e)
        self.events = []


def to_device(x, dev):
    import torch
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(x).to(dev)


def host_cpu():
    """The host's CPU model and the cores this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return model, int(usable or 1), int(os.cpu_count() or 1)


# Host threads for the all-cores oracle run: a one-GPU share of the host is
# 16 cores, whatever the machine reports.
CPU_SHARE = 16


def cpu_baseline(case, min_seconds: float):
    """The C oracle (fp64, unchanged) over the workload's whole batch, timed on
    one host thread and then on all usable cores with the requests split over
    threads (the oracle keeps no shared state and ctypes releases the
    interpreter lock during the call).  Each leg repeats full passes until
    min_seconds / 2 have passed."""
    import concurrent.futures
    import oracle
    model, usable, logical = host_cpu()
    R = case.R
    positions = int(np.clip(case.verify_len, 0, None).sum())

    last = {}

    def run_rows(r0, r1):
        last[r0] = oracle.verify_batch(case.target[r0:r1], case.draft[r0:r1],
                                       case.draft_tokens[r0:r1], case.verify_len[r0:r1],
                                       case.temperature[r0:r1], case.u_accept[r0:r1],
                                       case.u_sample[r0:r1])

    def timed(fn):
        passes, t0 = 0, time.perf_counter()
        while True:
            fn()
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds / 2:
                return passes, dt

    p1, d1 = timed(lambda: run_rows(0, R))
    n = max(1, min(usable, CPU_SHARE, R))
    cuts = np.linspace(0, R, n + 1).astype(int)
    with concurrent.futures.ThreadPoolExecutor(n) as ex:
        def all_cores():
            list(ex.map(lambda k: run_rows(cuts[k], cuts[k + 1]), range(n)))
        pn, dn = timed(all_cores)
    ref = {k: np.concatenate([last[c][k] for c in cuts[:-1]])
           for k in ("tokens", "num_accepted", "first_tie", "cstar", "resid", "logq")}
    return ref, {"value": positions * pn / dn, "unit": "positions/s", "cores": n, "kind": "oracle",
            "single_thread_value": positions * p1 / d1,
            "host": {"cpu_model": model, "usable_cores": usable, "logical_cpus": logical},
            "sample": f"the full {R}-request batch: {pn} pass(es) in {dn:.1f} s on {n} threads "
                      f"(requests split), {p1} pass(es) in {d1:.1f} s on one thread; "
                      "fp64 C oracle"}


# The kernels of one spec_verify_batch call, in launch order.
VERIFY_KERNELS = {0: "stats_kernel + fold_kernel + tv_kernel + combine_kernel",
                  1: "hold_kernel + combine_kernel"}

# Verify workloads: name -> description.
VERIFY_WORKLOADS = {
    "batched": "R=64 gamma=7 V=151936 bf16, l_r uniform on 0..7, T=1",
    "single_user": "R=1 gamma=8 V=151936 fp32, one planted dominant id per row, l=8, T=1",
    "dspark_verify": "R=64 gamma=7 V=129280: bf16 target, fp32 draft logits from the "
                     "Markov-head draft (made on the GPU before timing), l=7, T=1",
    "high_load": "R=256 gamma=7 V=129280 bf16, l_r truncated geometric(0.3), half T=0",
    "tiny": "R=1 gamma=4 V=32 fp32, l=4, T=1",
}


def verify_inputs(args, dev):
    """(case, device target, device draft) of a verify workload.  The case's
    host arrays are the oracle's inputs; for dspark_verify its draft arrays
    are filled from the GPU draft."""
    import torch
    import workloads
    import lossless_verification_sampling_amd as sv
    w = args.workload
    seed = args.seed
    if w == "batched":
        case = workloads.batched(seed=3 if seed is None else seed)
    elif w == "single_user":
        case = workloads.single_user(seed=2 if seed is None else seed)
    elif w == "high_load":
        case = workloads.high_load_mixed(seed=5 if seed is None else seed)
    elif w == "tiny":
        case = workloads.tiny_chain(seed=1 if seed is None else seed)
    else:
        mk = workloads.dspark_markov(seed=4 if seed is None else seed)
        R, gamma, V = mk.R, mk.gamma, mk.V
        tok = torch.empty((R, gamma), dtype=torch.int32, device=dev)
        lg = torch.empty((R, gamma, V), dtype=torch.float32, device=dev)
        ws = sv.Workspace(dev, sv.spec_markov_workspace_bytes(R, gamma, V, mk.rank))
        sv.spec_markov_draft_sample(to_device(mk.U, dev), to_device(mk.W1, dev),
                                    to_device(mk.W2, dev), to_device(mk.anchor, dev),
                                    to_device(mk.temperature, dev), to_device(mk.u_draft, dev),
                                    out_tokens=tok, out_logits=lg, workspace=ws)
        torch.cuda.synchronize()
        case = workloads.VerifyCase(name="dspark_verify", target=mk.target,
                                    draft=lg.cpu().numpy(), draft_tokens=tok.cpu().numpy(),
                                    verify_len=mk.verify_len, temperature=mk.temperature,
                                    u_accept=mk.u_accept, u_sample=mk.u_sample, seed=mk.seed)
        return case, to_device(case.target, dev), lg
    return case, to_device(case.target, dev), to_device(case.draft, dev)


def bench_verify(args):
    import torch
    import lossless_verification_sampling_amd as sv
    import workloads

    dev = torch.device("cuda:0")
    case, tgt0, drf0 = verify_inputs(args, dev)
    R, G1, V = case.target.shape
    gamma = G1 - 1
    sum_l = int(case.verify_len.sum())
    te = 2 if case.target.dtype == np.uint16 else 4
    de = 2 if case.draft.dtype == np.uint16 else 4
    alg_bytes = workloads.algorithmic_bytes(case.verify_len, V, te, de)
    ncopy = args.copies or max(2, int(np.ceil(2 * MALL_BYTES / alg_bytes)) + 1)
    tgts = [tgt0] + [tgt0.clone() for _ in range(ncopy - 1)]
    drfs = [drf0] + [drf0.clone() for _ in range(ncopy - 1)]
    tok = to_device(case.draft_tokens, dev)
    vl = to_device(case.verify_len, dev)
    T = to_device(case.temperature, dev)
    ua = to_device(case.u_accept, dev)
    us = to_device(case.u_sample, dev)
    ws = sv.Workspace(dev, sv.spec_verify_workspace_bytes(R, gamma, V))
    out = dict(tokens=torch.empty((R, G1), dtype=torch.int32, device=dev),
               num_accepted=torch.empty((R,), dtype=torch.int32, device=dev),
               cstar=torch.empty((R, gamma), dtype=torch.float32, device=dev),
               resid_mass=torch.empty((R, gamma), dtype=torch.float32, device=dev),
               logq=torch.empty((R, G1), dtype=torch.float32, device=dev))

    def step(k):
        sv.spec_verify_batch(tgts[k % ncopy], drfs[k % ncopy], tok, vl, T, ua, us, out=out,
                             workspace=ws)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    if sv.spec_get_device_status(ws, clear=True):
        raise RuntimeError("device status bits set during warm-up")
    wall, kern_ms = timed_steps(lambda k: step(args.warmup + k), args.steps,
                                torch.cuda.current_stream(dev))
    # third pass of the same steps: the first launch of every call bracketed
    # by HIP events that the library records on the call's stream (events
    # inside a call add launch gaps, hence a pass of its own)
    hev = HipEvents(2 * args.steps)
    sv.spec_time_stats_launch(hev.events[:args.steps], hev.events[args.steps:])
    for k in range(args.steps):
        step(args.warmup + 2 * args.steps + k)
    torch.cuda.synchronize()
    sv.spec_time_stats_launch([], [])
    stats_ms = np.array([hev.elapsed_ms(k, args.steps + k) for k in range(args.steps)])
    hev.close()
    bits = sv.spec_get_device_status(ws, clear=True)
    if bits:
        raise RuntimeError(f"device status bits {bits:#x} during the timed steps")
    avg_kernel_s = float(kern_ms.mean()) / 1e3
    avg_stats_s = float(stats_ms.mean()) / 1e3
    ms_per_step = wall / args.steps * 1e3
    achieved = alg_bytes / avg_stats_s / 1e9
    call_achieved = alg_bytes / avg_kernel_s / 1e9
    key = "verify_" + args.workload
    tname = "bf16" if te == 2 else "f32"
    dname = "bf16" if de == 2 else "f32"
    path = sv.spec_verify_path(R, gamma, V, sv.SPEC_BF16 if te == 2 else sv.SPEC_F32,
                               sv.SPEC_BF16 if de == 2 else sv.SPEC_F32)
    first = "hold_kernel" if path == sv.SPEC_PATH_HELD else "stats_kernel"
    traffic = measured_traffic(key, first)
    Ts = sorted(set(float(t) for t in np.asarray(case.temperature).ravel()))
    result = {
        "metric": METRIC if args.workload == "batched" else
        f"verified draft positions/sec and achieved HBM GB/s (% of peak), {args.workload}: "
        + VERIFY_WORKLOADS[args.workload],
        "value": sum_l / (ms_per_step / 1e3),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "R": R, "gamma": gamma, "V": V,
                   "logits": tname if tname == dname else f"target {tname}, draft {dname}",
                   "sum_verify_len": sum_l, "temperature": Ts, "seed": case.seed,
                   "input_copies": ncopy, "parallelism": "none (one GPU)"},
        # the dominant kernel, the first launch: it reads every needed row,
        # so its algorithmic bytes are the call's
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": alg_bytes,
                     "kernel_ms_mean": float(stats_ms.mean()),
                     "kernel_ms_p10": float(np.percentile(stats_ms, 10)),
                     "kernel_ms_p90": float(np.percentile(stats_ms, 90)),
                     "kernel": f"{first}<{tname}, {dname}> (HIP events around the launch "
                               "inside each call of a third pass)"},
        # the whole call against the same bytes
        "call_roofline": {"achieved": call_achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": call_achieved / HBM_PEAK_GBS,
                          "traffic": measured_traffic(key),
                          "call_ms_mean": float(kern_ms.mean()),
                          "call_ms_p10": float(np.percentile(kern_ms, 10)),
                          "call_ms_p90": float(np.percentile(kern_ms, 90)),
                          "kernels": f"spec_verify_batch: {VERIFY_KERNELS[path]} "
                                     f"({tname}, {dname})"},
        "kernel_positions_per_s": sum_l / avg_kernel_s,
    }
    if not args.no_cpu_baseline:
        ref, result["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
        result["parity"] = parity_summary(case, {k: v.cpu().numpy() for k, v in out.items()}, ref)
    return result


def parity_summary(case, gpu: dict, ref: dict) -> dict:
    """How the last timed call's outputs compare with the oracle's from the
    baseline leg: requests graded exactly (no decision within 1e-6 of its
    boundary), near ties, exact mismatches among the graded, and the largest
    relative errors of c*, Res and log q (where the oracle's value exceeds
    1e-3)."""
    R = case.R
    graded = mism = ties = 0
    err = {"cstar": 0.0, "resid": 0.0, "logq": 0.0}
    for r in range(R):
        n = int(ref["num_accepted"][r])
        if n < 0:
            mism += int(gpu["num_accepted"][r] != -1)
            continue
        if int(ref["first_tie"][r]) >= 0:
            ties += 1
            continue
        graded += 1
        mism += int(gpu["num_accepted"][r] != n or
                    not np.array_equal(gpu["tokens"][r], ref["tokens"][r]))
        l = int(case.verify_len[r])
        for k, gk, m in (("cstar", "cstar", l), ("resid", "resid_mass", l), ("logq", "logq", n + 1)):
            o = ref[k][r, :m]
            g = gpu[gk][r, :m].astype(np.float64)
            big = np.abs(o) > 1e-3
            if big.any():
                err[k] = max(err[k], float((np.abs(g - o)[big] / np.abs(o[big])).max()))
    return {"requests": R, "graded_exact": graded, "near_ties": ties,
            "mismatches_among_graded": mism, "max_rel_err": err,
            "tolerance": 1e-5 if case.target.dtype == case.draft.dtype == np.float32 else 2e-3}


def bench_dspark(args):
    import torch
    import lossless_verification_sampling_amd as sv
    import workloads

    dev = torch.device("cuda:0")
    mk = workloads.dspark_markov(seed=args.seed + 1)
    R, gamma, V, rank = mk.R, mk.gamma, mk.V, mk.rank
    U = to_device(mk.U, dev)
    W1 = to_device(mk.W1, dev)
    W2 = to_device(mk.W2, dev)
    anc = to_device(mk.anchor, dev)
    T = to_device(mk.temperature, dev)
    ud = to_device(mk.u_draft, dev)
    tok = torch.empty((R, gamma), dtype=torch.int32, device=dev)
    lg = torch.empty((R, gamma, V), dtype=torch.float32, device=dev)
    ws = sv.Workspace(dev, sv.spec_markov_workspace_bytes(R, gamma, V, rank))
    for _ in range(args.warmup):
        sv.spec_markov_draft_sample(U, W1, W2, anc, T, ud, out_tokens=tok, out_logits=lg,
                                    workspace=ws)
    torch.cuda.synchronize()

    def call(k):
        sv.spec_markov_draft_sample(U, W1, W2, anc, T, ud, out_tokens=tok, out_logits=lg,
                                    workspace=ws)

    wall, ms = timed_steps(call, args.steps, torch.cuda.current_stream(dev))
    flops = 2.0 * R * rank * V * gamma
    per_step_bytes = (R * V * 2 + rank * V * 2 + R * V * 4) * gamma
    res = {
        "metric": "Markov-head draft: drafted tokens/sec",
        "value": R * gamma / (wall / args.steps),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16-mfma/f32", "data": "synthetic",
        "config": {"workload": "dspark_markov", "R": R, "gamma": gamma, "V": V, "rank": rank},
        "roofline": {"bound": "hbm", "achieved": per_step_bytes / (ms.mean() / 1e3) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": per_step_bytes / (ms.mean() / 1e3) / 1e9 / HBM_PEAK_GBS,
                     "traffic": measured_traffic("markov_dspark"),
                     "algorithmic_bytes_per_call": per_step_bytes,
                     "mfma_tflops": flops / (ms.mean() / 1e3) / 1e12},
    }
    if not args.no_cpu_baseline:
        import oracle
        n_cpu = 4
        t1 = time.perf_counter()
        oracle.markov_draft(mk.U[:n_cpu], mk.W1, mk.W2, mk.anchor[:n_cpu],
                            mk.temperature[:n_cpu], mk.u_draft[:n_cpu])
        el = time.perf_counter() - t1
        res["cpu_baseline"] = {"value": n_cpu * gamma / el, "unit": "tokens/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"the first {n_cpu} of the {R} requests, all {gamma} "
                                         "steps, the C oracle (fp64)"}
    return res


def bench_rnn(args):
    """RNN serial head at the Markov workload's size (R = 64, gamma = 7,
    V = 129280, rank 256) with backbone hidden states of 1024."""
    import torch
    import lossless_verification_sampling_amd as sv
    import workloads

    dev = torch.device("cuda:0")
    c = workloads.rnn_head(seed=args.seed + 3, hidden=1024)
    mk = c.mk
    R, gamma, V, rank, hidden = mk.R, mk.gamma, mk.V, mk.rank, c.H.shape[2]
    ins = [to_device(x, dev) for x in (mk.U, mk.W1, mk.W2, c.H, c.Wg, c.bg, mk.anchor,
                                       mk.temperature, mk.u_draft)]
    tok = torch.empty((R, gamma), dtype=torch.int32, device=dev)
    lg = torch.empty((R, gamma, V), dtype=torch.float32, device=dev)
    ws = sv.Workspace(dev, sv.spec_rnn_workspace_bytes(R, gamma, V, rank, hidden))
    for _ in range(args.warmup):
        sv.spec_rnn_draft_sample(*ins, out_tokens=tok, out_logits=lg, workspace=ws)
    torch.cuda.synchronize()

    def call(k):
        sv.spec_rnn_draft_sample(*ins, out_tokens=tok, out_logits=lg, workspace=ws)

    wall, ms = timed_steps(call, args.steps, torch.cuda.current_stream(dev))
    din = 2 * rank + hidden
    per_call = (R * V * 2 + rank * V * 2 + R * V * 4 + din * 2 * rank * 2 + R * hidden * 4) * gamma
    flops = (3 * 2.0 * R * rank * V + 2.0 * R * din * 2 * rank) * gamma
    res = {
        "metric": "RNN-head draft: drafted tokens/sec",
        "value": R * gamma / (wall / args.steps),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16-mfma (state in three bf16 parts)/f32", "data": "synthetic",
        "config": {"workload": "rnn_head", "R": R, "gamma": gamma, "V": V, "rank": rank,
                   "hidden": hidden},
        "roofline": {"bound": "hbm", "achieved": per_call / (ms.mean() / 1e3) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": per_call / (ms.mean() / 1e3) / 1e9 / HBM_PEAK_GBS,
                     "traffic": measured_traffic("rnn_head"),
                     "algorithmic_bytes_per_call": per_call,
                     "mfma_tflops": flops / (ms.mean() / 1e3) / 1e12},
    }
    if not args.no_cpu_baseline:
        from oracle import rnn as ornn
        n_cpu = 4
        t1 = time.perf_counter()
        ornn.rnn_draft(mk.U[:n_cpu], mk.W1, mk.W2, c.H[:n_cpu], c.Wg, c.bg, mk.anchor[:n_cpu],
                       mk.temperature[:n_cpu], mk.u_draft[:n_cpu])
        el = time.perf_counter() - t1
        res["cpu_baseline"] = {"value": n_cpu * gamma / el, "unit": "tokens/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"the first {n_cpu} of the {R} requests, all {gamma} "
                                         "steps, numpy fp64"}
    return res


def bench_schedule(args):
    """Confidence-scheduled verify lengths for the headline batch (R = 64,
    gamma = 7) on the smooth step-rate curve: one workgroup sorts the 448
    candidates and finds the early stop.  The oracle (plain Python) is timed
    beside it."""
    import torch
    import lossless_verification_sampling_amd as sv
    import workloads

    dev = torch.device("cuda:0")
    R, gamma = 64, 7
    case = workloads.schedule_case(seed=args.seed + 5, R=R, gamma=gamma, curve="smooth")
    conf = to_device(case.conf, dev)
    sps = to_device(case.sps, dev)
    ln = torch.empty((R,), dtype=torch.int32, device=dev)
    th = torch.empty((1,), dtype=torch.float64, device=dev)
    ws = sv.Workspace(dev, sv.spec_schedule_workspace_bytes())
    for _ in range(args.warmup):
        sv.spec_schedule_verify_len(conf, sps, out_len=ln, out_theta=th, workspace=ws)
    torch.cuda.synchronize()

    def call(k):
        sv.spec_schedule_verify_len(conf, sps, out_len=ln, out_theta=th, workspace=ws)

    wall, ms = timed_steps(call, args.steps, torch.cuda.current_stream(dev))
    res = {
        "metric": "confidence-scheduled verify lengths: schedules/sec",
        "value": args.steps / wall,
        "unit": "schedules/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 products, f64 sums", "data": "synthetic",
        "config": {"workload": "schedule", "R": R, "gamma": gamma, "candidates": R * gamma,
                   "curve": "smooth", "admitted": int(ln.sum().item())},
        "roofline": None,
        "kernel_us_mean": float(ms.mean()) * 1e3,
        "note": "one workgroup, latency-bound (a bitonic sort of 512 keys in LDS, a block "
                "scan and a block minimum); no HBM or MFMA roofline applies",
    }
    if not args.no_cpu_baseline:
        from oracle import schedule as osch
        n, t1 = 0, time.perf_counter()
        while time.perf_counter() - t1 < min(args.cpu_seconds, 5.0):
            osch.schedule(case.conf, case.sps)
            n += 1
        el = time.perf_counter() - t1
        res["cpu_baseline"] = {"value": n / el, "unit": "schedules/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n} schedules of the same 64 x 7 pool, plain Python"}
    return res


# fp64 VALU instructions the histogram loop issues per (block, temperature)
# score (the sigmoid's exp polynomial, a reciprocal with two Newton steps, the
# bin index, the running product), counted in the kernel's gfx950 assembly;
# the peak is 256 CUs x 64 fp64 lanes per clock x 2.4 GHz.
STS_OPS_PER_SCORE = 35
STS_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12


def bench_sts(args):
    """Sequential temperature scaling of the confidence head on a held-out set
    of 262144 draft blocks (gamma = 7), 64 candidate temperatures, 15 bins:
    every (block, temperature, position) score is evaluated once in fp64.
    The oracle (numpy, fp64) is timed beside it on the first 16384 blocks."""
    import torch
    import lossless_verification_sampling_amd as sv
    import workloads

    dev = torch.device("cuda:0")
    N, gamma, G, bins = 262144, 7, 64, 15
    c = workloads.sts_case(seed=args.seed + 7, N=N, gamma=gamma, G=G)
    z, A, grid = to_device(c.z, dev), to_device(c.accepted, dev), to_device(c.grid, dev)
    ws = sv.Workspace(dev, sv.spec_sts_workspace_bytes(N, gamma, G, bins))
    for _ in range(args.warmup):
        sv.spec_sts_calibrate(z, A, grid, bins=bins, workspace=ws)
    torch.cuda.synchronize()
    last = {}

    def call(k):
        last["r"] = sv.spec_sts_calibrate(z, A, grid, bins=bins, workspace=ws)

    wall, ms = timed_steps(call, args.steps, torch.cuda.current_stream(dev))
    t, e, _ = last["r"]
    evals = N * G * gamma
    achieved = STS_OPS_PER_SCORE * evals / (ms.mean() / 1e3) / 1e12
    res = {
        "metric": "STS calibration: scored (block, temperature, position) triples/sec",
        "value": evals / (wall / args.steps),
        "unit": "scores/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f64", "data": "synthetic",
        "config": {"workload": "sts", "N": N, "gamma": gamma, "grid": G, "bins": bins,
                   "temperatures": [round(float(x), 4) for x in t.cpu().numpy()],
                   "ece": [round(float(x), 5) for x in e.cpu().numpy()]},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": STS_PEAK_TOPS,
                     "unit": "T fp64 lane-instructions/s", "frac": achieved / STS_PEAK_TOPS,
                     "traffic": None,
                     "ops_per_score": STS_OPS_PER_SCORE,
                     "kernel": "spec_sts_calibrate call (sts_hist_kernel dominates)"},
        "kernel_ms_mean": float(ms.mean()),
    }
    if not args.no_cpu_baseline:
        from oracle import sts as osts
        n_cpu = 16384
        t1 = time.perf_counter()
        osts.sts_calibrate(c.z[:n_cpu], c.accepted[:n_cpu], c.grid, bins=bins)
        el = time.perf_counter() - t1
        res["cpu_baseline"] = {"value": n_cpu * G * gamma / el, "unit": "scores/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"the first {n_cpu} blocks, all {G} temperatures and "
                                         f"{gamma} positions, numpy fp64"}
    return res


def bench_tree(args):
    """Greedy (T = 0) tree verification of 64 draft trees of 48 nodes (up to
    3 / 2 / 2 / 1 children per node by depth) over V = 151936 bf16 rows: one
    level launch per depth, each reading the current node's row of every
    unfinished request.  The oracle is timed beside it."""
    import torch
    import lossless_verification_sampling_amd as sv
    import workloads

    dev = torch.device("cuda:0")
    R, M, V = 64, 48, 151936
    c = workloads.tree_case(seed=args.seed + 9, R=R, M=M, V=V, dtype="bf16",
                            widths=(3, 2, 2, 1, 1, 1, 1, 1))
    L = to_device(c.logits, dev)
    P, X = to_device(c.parent, dev), to_device(c.tokens, dev)
    n = to_device(c.n_nodes, dev)
    ws = sv.Workspace(dev, sv.spec_tree_workspace_bytes(R, M, V))
    for _ in range(args.warmup):
        sv.spec_tree_verify(L, P, X, n, c.max_depth, workspace=ws)
    torch.cuda.synchronize()
    last = {}

    def call(k):
        last["r"] = sv.spec_tree_verify(L, P, X, n, c.max_depth, workspace=ws)

    wall, ms = timed_steps(call, args.steps, torch.cuda.current_stream(dev))
    acc, _, _ = last["r"]
    a = acc.cpu().numpy()
    committed = int((a + 1).sum())
    per_call = committed * V * 2          # the rows the walk reads
    res = {
        "metric": "greedy tree verification: committed tokens/sec",
        "value": committed / (wall / args.steps),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 logits, f32 compare", "data": "synthetic",
        "config": {"workload": "tree", "R": R, "nodes": M, "V": V, "max_depth": c.max_depth,
                   "accepted_mean": float(a.mean()), "levels": c.max_depth + 1},
        "roofline": {"bound": "hbm", "achieved": per_call / (ms.mean() / 1e3) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": per_call / (ms.mean() / 1e3) / 1e9 / HBM_PEAK_GBS,
                     "traffic": measured_traffic("tree_greedy"),
                     "algorithmic_bytes_per_call": per_call,
                     "kernel": "spec_tree_verify call (tree_level_kernel per level)"},
        "kernel_ms_mean": float(ms.mean()),
    }
    if not args.no_cpu_baseline:
        from oracle import tree as otree
        nrep, t1 = 0, time.perf_counter()
        while time.perf_counter() - t1 < min(args.cpu_seconds, 5.0):
            otree.tree_verify(c.logits, c.parent, c.tokens, c.n_nodes)
            nrep += 1
        el = time.perf_counter() - t1
        res["cpu_baseline"] = {"value": committed * nrep / el, "unit": "tokens/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{nrep} full calls (64 trees), numpy"}
    return res


def calibrate_copy(args):
    """One device-to-device copy of a known size, repeated: the reference that
    scales rocprofv3's FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    dev = torch.device("cuda:0")
    nbytes = 256 << 20
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(args.warmup + args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"calibration": "device copy", "bytes_read_per_copy": nbytes,
            "bytes_written_per_copy": nbytes, "copies": args.warmup + args.steps}


def counter_rows(d, counter):
    """(kernel name, value) of every dispatch in a rocprofv3 --pmc csv output."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") == counter:
                    rows.append((row.get("Kernel_Name", ""), float(row["Counter_Value"])))
    return rows


def write_traffic(args):
    """Per-call HBM bytes of this library's kernels from two rocprofv3 --pmc
    runs of a workload (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled
    by what the same counter reads for the 256 MiB device copy of
    --calibrate-copy.  Kernels dispatched fewer times than there were calls
    (one-time workspace set-up) are left out.  Writes the entry under --key
    in the traffic file, stamped with the current source hash."""
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = args.traffic_from
    # calls of the counted run: the warm-up, then two passes of the steps
    # (three for the verify workloads, whose last pass times the first launch)
    passes = 3 if args.key.startswith("verify_") else 2
    calls = args.calls or (args.warmup + passes * args.steps)
    copy_bytes = 256 << 20

    def scale(d, counter):
        # the copy kernel is the one dispatched once per copy (the source fill
        # of the calibration run is a different kernel, dispatched once)
        groups = {}
        for name, v in counter_rows(d, counter):
            groups.setdefault(name, []).append(v)
        vals = [v for vs in groups.values() if len(vs) == args.copies_counted for v in vs]
        if not vals:
            raise SystemExit(f"no kernel with {args.copies_counted} {counter} dispatches under {d}")
        return copy_bytes / (sum(vals) / len(vals) * 1024.0)

    def per_call(d, counter, sc):
        per_kernel = {}
        for name, v in counter_rows(d, counter):
            if "sv::" not in name:
                continue
            key = name.split("(")[0].replace("void ", "")
            n, tot = per_kernel.get(key, (0, 0.0))
            per_kernel[key] = (n + 1, tot + v)
        out = {k: tot * 1024.0 * sc / calls for k, (n, tot) in per_kernel.items() if n >= calls}
        per_dispatch = {k: tot * 1024.0 * sc / n for k, (n, tot) in per_kernel.items()
                        if n >= calls}
        return out, per_dispatch

    fs, ws = scale(cfetch_dir, "FETCH_SIZE"), scale(cwrite_dir, "WRITE_SIZE")
    (fk, fkd), (wk, wkd) = per_call(fetch_dir, "FETCH_SIZE", fs), per_call(write_dir, "WRITE_SIZE", ws)
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        t = {}
    t[args.key] = {
        "source_hash": source_hash(args.key),
        "bytes_per_launch": sum(fk.values()) + sum(wk.values()),
        "fetch_bytes": sum(fk.values()), "write_bytes": sum(wk.values()),
        "fetch_scale": fs, "write_scale": ws,
        "per_kernel_fetch": fk, "per_kernel_write": wk,
        "per_dispatch_fetch": fkd, "per_dispatch_write": wkd,
        "note": "per call, summed over the library's kernels; FETCH_SIZE then WRITE_SIZE in "
                "separate rocprofv3 --pmc runs, scaled by a 256 MiB device copy",
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(t, f, indent=1, sort_keys=True)
        f.write("\n")
    return t[args.key]


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--seed", type=int, default=None,
                    help="workload seed (default: the workload's own)")
    ap.add_argument("--copies", type=int, default=0, help="input copies rotated (0 = auto)")
    ap.add_argument("--workload", choices=list(VERIFY_WORKLOADS) +
                    ["dspark", "rnn", "schedule", "sts", "tree"], default="batched")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only copy a 256 MiB buffer (reference for the HBM byte counters)")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="rocprofv3 --pmc output folders: write the traffic entry --key from them "
                         "(--steps/--warmup as in the counted run)")
    ap.add_argument("--key", default="verify_batched")
    ap.add_argument("--calls", type=int, default=0,
                    help="library calls in the counted run (default --warmup + 2 --steps; "
                         "the verify workloads make three passes: --warmup + 3 --steps)")
    ap.add_argument("--copies-counted", type=int, default=6,
                    help="copies in the counted --calibrate-copy run")
    args = ap.parse_args()
    if args.seed is None and args.workload not in VERIFY_WORKLOADS:
        args.seed = 3
    if args.traffic_from:
        print(json.dumps(write_traffic(args)))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(requests shard across GPUs with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        res = calibrate_copy(args)
    else:
        other = {"dspark": bench_dspark, "rnn": bench_rnn, "schedule": bench_schedule,
                 "sts": bench_sts, "tree": bench_tree}
        res = other.get(args.workload, bench_verify)(args)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
