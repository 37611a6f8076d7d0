"""Build libtv.so (the HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m tree_speculative_decoding_amd.build

Every call recompiles.  Objects go to ``_build/`` next to this file, the shared
library to ``libtv.so`` in this package directory.  The measurement aid under
``measure/`` (a plain HBM read-stream kernel the benchmark reports the ceiling of)
becomes ``libtv_measure.so``; libtv.so does not contain or need it.
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
OUT = os.path.join(PKG, "libtv.so")
MEASURE_OUT = os.path.join(PKG, "libtv_measure.so")
ARCH = "gfx950"

COMMON_FLAGS = [
    "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-fvisibility=hidden", "-I", INCLUDE, "-I", CSRC,
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtv)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name: harmless, drop it
    log = "\n".join(line for line in r.stdout.splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{log}")
    return log


def build(verbose: bool = False, jobs: int = 8) -> str:
    cc = hipcc()
    bdir = os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "tv_host.cpp")]
    objs = []
    cmds = []
    for s in srcs:
        o = os.path.join(bdir, os.path.basename(s) + ".o")
        objs.append(o)
        cmds.append([cc, *COMMON_FLAGS, "-c", s, "-o", o])
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        for log in ex.map(_run, cmds):
            if verbose and log.strip():
                print(log)
    tmp = OUT + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, OUT)
    msrc = sorted(glob.glob(os.path.join(PKG, "measure", "*.hip")))
    if msrc:
        tmp = MEASURE_OUT + ".tmp"
        _run([cc, *COMMON_FLAGS, "-shared", "-o", tmp, *msrc])
        os.replace(tmp, MEASURE_OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
