"""Builds libkda.so (HIP kernels for gfx950 + the C ABI) and libkda_calib.so (a counter
calibration kernel) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libkda.so")
SOURCES = ["kda_api.hip", "kda_chain.hip", "kda_decode.hip", "kda_fast.hip", "kda_pipe.hip", "kda_plan.hip", "kda_scan.hip"]
HEADERS = ["kda_common.h", "kda_fast_common.h", "kda_launch.h"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 (v_pk_*_f32) instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# a kernel of known MFMA count that scales the profiler's MFMA-busy counter (not KDA)
CALIB_LIB = os.path.join(HERE, "libkda_calib.so")
CALIB_SOURCES = ["calib/kda_calib.hip"]


def _hipcc(out: str, sources, verbose: bool) -> None:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = [os.path.join(HERE, "csrc", s) for s in sources]
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc] + HIPCC_FLAGS + ["-I", os.path.join(ROOT, "include"), "-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building " + os.path.basename(out))
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    _hipcc(LIB, SOURCES, verbose)
    _hipcc(CALIB_LIB, CALIB_SOURCES, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
