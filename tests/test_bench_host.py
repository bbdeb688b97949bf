"""Host logic of bench.py, on the CPU: the one-GPU guard, the reading and
scaling of rocprofv3 counter summaries into the traffic file, and the source
hash that ties counter figures to the kernel code they were taken on."""
import json
import os
import shutil
import subprocess
import sys
import types

import pytest

import bench


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert p.returncode == 2, p.stderr
    assert "one GPU" in p.stderr
    assert p.stdout == ""


def _counter_csv(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, (name, v) in enumerate(rows):
            f.write(f'{i},"{name}",{counter},{v}\n')


def test_traffic_from_scales_by_the_copy_and_checks_the_hash(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    copy_kib = (256 << 20) / 1024.0
    # the calibration: a one-off source fill, then six copies; FETCH_SIZE
    # reads half the copied bytes, WRITE_SIZE all of them
    _counter_csv(tmp_path / "cf", "FETCH_SIZE",
                 [("fill_kernel", 7.0)] + [("copy_kernel", copy_kib / 2)] * 6)
    _counter_csv(tmp_path / "cw", "WRITE_SIZE",
                 [("fill_kernel", 7.0)] + [("copy_kernel", copy_kib)] * 6)
    # a verify run of 1 warm-up call and two steps: 1 + 3 * 2 = 7 calls; a
    # one-time set-up launch and a kernel outside the library are left out
    work = [("void sv::hold_kernel<16, 8>(sv::VerifyArgs, int)", 100.0),
            ("void sv::combine_kernel<bf16>(sv::VerifyArgs)", 3.0)] * 7
    other = [("sv::zero_fill_kernel(unsigned int*, unsigned long)", 500.0),
             ("__amd_rocclr_copyBuffer", 900.0)]
    _counter_csv(tmp_path / "pf", "FETCH_SIZE", other + work)
    _counter_csv(tmp_path / "pw", "WRITE_SIZE",
                 other + [(n, v / 10.0) for n, v in work])
    args = types.SimpleNamespace(
        traffic_from=[str(tmp_path / d) for d in ("pf", "pw", "cf", "cw")],
        key="verify_batched", calls=0, warmup=1, steps=2, copies_counted=6)
    e = bench.write_traffic(args)
    assert e["fetch_scale"] == pytest.approx(2.0)
    assert e["write_scale"] == pytest.approx(1.0)
    hold = "sv::hold_kernel<16, 8>"
    assert set(e["per_kernel_fetch"]) == {hold, "sv::combine_kernel<bf16>"}
    assert e["per_dispatch_fetch"][hold] == pytest.approx(100.0 * 1024 * 2.0)
    assert e["per_dispatch_write"][hold] == pytest.approx(10.0 * 1024)
    per_call = (100.0 + 3.0) * 1024 * 2.0 + (10.0 + 0.3) * 1024
    assert e["bytes_per_launch"] == pytest.approx(per_call)
    assert e["source_hash"] == bench.source_hash("verify_batched")
    # read back while the hash matches: per call, or per launch of one kernel
    assert bench.measured_traffic("verify_batched") == pytest.approx(per_call)
    assert bench.measured_traffic("verify_batched", "hold_kernel") == \
        pytest.approx(100.0 * 1024 * 2.0 + 10.0 * 1024)
    assert bench.measured_traffic("verify_batched", "no_such_kernel") is None
    assert bench.measured_traffic("markov_dspark") is None
    # counters taken on other code are not used
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    t["verify_batched"]["source_hash"] = "0" * 16
    with open(bench.TRAFFIC_FILE, "w") as f:
        json.dump(t, f)
    assert bench.measured_traffic("verify_batched") is None


def test_traffic_from_needs_the_copy_kernel(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    for d, c in (("cf", "FETCH_SIZE"), ("cw", "WRITE_SIZE"), ("pf", "FETCH_SIZE"),
                 ("pw", "WRITE_SIZE")):
        _counter_csv(tmp_path / d, c, [("copy_kernel", 1.0)] * 5)
    args = types.SimpleNamespace(
        traffic_from=[str(tmp_path / d) for d in ("pf", "pw", "cf", "cw")],
        key="verify_batched", calls=0, warmup=1, steps=2, copies_counted=6)
    with pytest.raises(SystemExit):
        bench.write_traffic(args)
    assert not os.path.exists(bench.TRAFFIC_FILE)


def test_source_hash_follows_code_not_comments(tmp_path, monkeypatch):
    src = os.path.join(bench.ROOT, "lossless_verification_sampling_amd", "csrc")
    dst = tmp_path / "lossless_verification_sampling_amd" / "csrc"
    dst.mkdir(parents=True)
    for f in ("common.h", "verify.hip", "markov.hip"):
        shutil.copy(os.path.join(src, f), dst / f)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.source_hash("verify_batched")
    assert h0 == bench.source_hash("verify_single_user")  # same sources
    m0 = bench.source_hash("markov_dspark")
    with open(dst / "verify.hip", "a") as f:
        f.write("\n// a comment\n/* and\n another */\n\n")
    assert bench.source_hash("verify_batched") == h0
    with open(dst / "verify.hip", "a") as f:
        f.write("static int unused_marker = 1;\n")
    assert bench.source_hash("verify_batched") != h0
    assert bench.source_hash("markov_dspark") == m0
    with open(dst / "common.h", "a") as f:
        f.write("static int another_marker = 2;\n")
    assert bench.source_hash("markov_dspark") != m0
