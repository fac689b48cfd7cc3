"""Builds libglu.so (the C-ABI library with the gfx950 kernels) in-tree,
and libglu_ref.so (the data-movement reference kernels the benchmark
measures the library against, include/glu_ref.h).

    python -m mlp_gated_activation_amd.build [--out PATH] [-DNAME=VALUE ...]

Extra -D options override the launch-shape macros (GLU_BLOCK, GLU_UNROLL)
for sweeps; the default build uses the values in csrc/glu_internal.h.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libglu.so")
REF_LIB = os.path.join(PKG, "libglu_ref.so")
REF_SOURCES = [os.path.join(CSRC, "stream_ref.hip")]
SOURCES = [os.path.join(CSRC, "glu_kernels.hip"), os.path.join(CSRC, "rmsnorm_kernels.hip"),
           os.path.join(CSRC, "gemm_kernels.hip"), os.path.join(CSRC, "glu_api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function", "-fvisibility=hidden",
    # keep fp32 denormals (subnormal sigmoid tails) and scalar fp32 arithmetic
    "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=on",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(out: str = LIB, defines=(), verbose: bool = False) -> str:
    """Builds libglu.so at `out`, and libglu_ref.so beside the default one."""
    if out == LIB:
        _compile(REF_SOURCES, REF_LIB, defines, verbose)
    return _compile(SOURCES, out, defines, verbose)


def _compile(sources, out, defines, verbose):
    cmd = [HIPCC, *FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", *[f"-D{d}" for d in defines],
           *sources, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is expected
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(out + ".tmp", out)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=LIB)
    ap.add_argument("-D", dest="defines", action="append", default=[])
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.out, a.defines, a.verbose))


if __name__ == "__main__":
    main()
