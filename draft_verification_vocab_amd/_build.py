"""Compile libspecverify.so (all HIP sources under csrc/) for gfx950, in tree,
and libsvceiling.so (the HIP sources under ceiling/: plain comparison kernels
that bench.py times beside the library -- the streaming-read ceiling, the
drafter's bytes without its arithmetic, and the build as two kernels)."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libspecverify.so")
CEILING_LIB = os.path.join(HERE, "libsvceiling.so")
CEILING_DIR = os.path.join(HERE, "ceiling")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-fvisibility=hidden",
    # no packed-fp32 instructions in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def ceiling_sources():
    return sorted(glob.glob(os.path.join(CEILING_DIR, "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def _compile(srcs, out, verbose):
    """One object per source, compiled in parallel (every source is a
    self-contained translation unit: no device code crosses files), then one
    shared library."""
    tmpdir = tempfile.mkdtemp(prefix="svbuild-")
    try:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in srcs]
        jobs = max(1, min(len(srcs), os.cpu_count() or 1, 8))
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            list(ex.map(lambda so: _run([HIPCC, *FLAGS, "-c", so[0], "-o", so[1]], verbose),
                        zip(srcs, objs)))
        tmp = out + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, out)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)


def build(verbose: bool = False) -> str:
    """Always recompile both libraries; returns the path of the verify library."""
    _compile(sources(), LIB, verbose)
    _compile(ceiling_sources(), CEILING_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
