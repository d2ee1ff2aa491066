"""Build the gfx950 HIP libraries in-tree with hipcc.

libssm_amd.so: the scan library (the C ABI of include/ssm.h).
libssm_probe.so: measurement kernels (instruction rates, clock, a plain
copy) that bench.py uses to calibrate the bounds; built with the same flags
so that its rates are the ones the scan kernels see.

Every translation unit under csrc/ is compiled for gfx950 only, with packed
fp32 instructions disabled.  Objects go to _build/ (not tracked).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libssm_amd.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

SOURCES = ["abi.cpp", "conv1d.hip", "scan_fwd.hip", "scan_bwd.hip", "step.hip", "model.hip", "scratch.hip"]
PROBE_SOURCES = ["probe.hip"]
PROBE_LIB = os.path.join(HERE, "libssm_probe.so")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    # operations run as written; every fused multiply-add is an explicit fmaf
    "-ffp-contract=off",
    "--offload-arch=" + ARCH,
    # packed fp32 (v_pk_*_f32) stays off: plain fp32 VALU only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    return "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc()] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr[-6000:]))
    return obj


def _link(objs, lib) -> str:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr[-4000:]))
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile and link both libraries; returns the path of libssm_amd.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    jobs = min(len(srcs), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
