"""Build libmsa.so (the HIP kernels + C ABI) and libmsa_calib.so (the benchmark's
measured-ceiling kernels) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmsa.so")
CALIB_SRC = os.path.join(HERE, "calib", "ceilings.hip")
CALIB_LIB = os.path.join(HERE, "libmsa_calib.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc(srcs, out, verbose):
    tmp = out + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-I", os.path.join(HERE, "..", "include")] + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed to build {os.path.basename(out)}")
    # hipcc's host pass does not know the packed-fp32 feature: drop that warning only
    noise = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"
    rest = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if rest.strip() and verbose:
        print(rest)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "msa_api.cpp")]
    _hipcc(srcs, LIB, verbose)
    _hipcc([CALIB_SRC], CALIB_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
