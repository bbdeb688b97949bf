"""Builds libspecverify.so in-tree from csrc/*.hip with hipcc for gfx950."""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libspecverify.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)


def build(verbose: bool = False) -> str:
    """Compiles every HIP source (in parallel) and links one shared library
    (always rebuilds)."""
    cc = hipcc()
    srcs = sources()
    with tempfile.TemporaryDirectory(prefix="specverify_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(f) + ".o") for f in srcs]
        cmds = [[cc, *HIPCC_FLAGS, "-I" + INCLUDE, "-I" + CSRC, "-c", f, "-o", o]
                for f, o in zip(srcs, objs)]
        workers = max(1, min(len(cmds), os.cpu_count() or 1, 8))
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(_run, cmds))
        tmp = LIB + f".tmp{os.getpid()}"
        link = [cc, "--offload-arch=gfx950", "-fPIC", "-shared", *objs, "-o", tmp]
        _run(link)
        if verbose:
            for c in cmds + [link]:
                print(" ".join(c))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
