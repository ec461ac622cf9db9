"""Build libsgb.so (gfx950 HIP kernels + C ABI) in-tree with hipcc.

    python sparse_gradient_backward_amd/build.py

(run as a script: importing the package itself needs the built library)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsgb.so")
SOURCES = [os.path.join(CSRC, "kernels.hip"), os.path.join(CSRC, "api.cpp")]
# the atomic scatter-add backward, a comparison baseline kept in its own library
ATOMIC_LIB = os.path.join(HERE, "libsgb_atomic.so")
ATOMIC_SOURCES = [os.path.join(CSRC, "atomic_scatter.hip")]
ARCH = os.environ.get("SGB_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU ops are kept out of the generated code on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, out: str = LIB, defines: tuple = (), sources=None) -> str:
    """Compile every source into libsgb.so (always recompiles).  `defines`
    (e.g. ("SGB_SHORT_UNR=2",)) override the tuning knobs of internal.h."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *FLAGS, *[f"-D{d}" for d in defines], *(sources or SOURCES), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


def build_atomic(verbose: bool = False) -> str:
    """Compile the atomic scatter-add baseline into libsgb_atomic.so."""
    return build(verbose=verbose, out=ATOMIC_LIB, sources=ATOMIC_SOURCES)


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("-o", "--out", default=LIB)
    ap.add_argument("-D", dest="defines", action="append", default=[])
    a = ap.parse_args()
    print(build(verbose=True, out=a.out, defines=tuple(a.defines)))
    if a.out == LIB:
        print(build_atomic(verbose=True))
