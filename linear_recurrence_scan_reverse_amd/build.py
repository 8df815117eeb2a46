"""Build librlscan.so in-tree for gfx950 with hipcc.

    python -m linear_recurrence_scan_reverse_amd.build

Each estimator's kernels compile in their own translation unit (in parallel),
then everything links into ``linear_recurrence_scan_reverse_amd/librlscan.so``.
Packed-fp32 instruction selection is switched off for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "librlscan.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# the bench's streaming-ceiling probe: a library of its own, not part of librlscan
PROBE_SRC = os.path.join(CSRC, "probe", "stream_probe.hip")
PROBE_PATH = os.path.join(PKG, "libstreamprobe.so")
OBJ_DIR = os.path.join(PKG, "_build")
ARCH = os.environ.get("RLSCAN_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE,
    "-I" + CSRC,
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: ROCm is required to build librlscan")
    return path


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, res.stdout, res.stderr))
    return obj


def build(jobs: int | None = None, verbose: bool = True) -> str:
    """Compile every HIP source and link librlscan.so; returns its path."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (res.stdout, res.stderr))
    os.replace(tmp, LIB_PATH)
    build_probe()
    if verbose:
        print("built %s from %d sources (and %s)" % (LIB_PATH, len(srcs), os.path.basename(PROBE_PATH)),
              file=sys.stderr)
    return LIB_PATH


def build_probe() -> str:
    """Compile the bench's streaming-ceiling probe into its own shared library."""
    tmp = PROBE_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-shared", PROBE_SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (PROBE_SRC, res.stdout, res.stderr))
    os.replace(tmp, PROBE_PATH)
    return PROBE_PATH


if __name__ == "__main__":
    build()
