"""Build libmoe_ep.so (HIP for gfx950) in-tree with hipcc."""
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmoe_ep.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden",
    # keep every binary32 operation as written (combine is specified with
    # separately rounded multiply and add; the kernels also say so explicitly)
    "-ffp-contract=off",
    # no packed-fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["/opt/rocm/bin/hipcc", *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(PKG, "csrc"), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
