"""Build tests/c_abi_check (a plain C++ consumer of libmoe_ep.so, no Python)
with hipcc; run by __graft_entry__.build() after the library is built."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_abi_check.cpp")
BIN = os.path.join(HERE, "c_abi_check")


def build(verbose=False):
    pkg = os.path.join(ROOT, "combine_moe_dispatch_layout_amd")
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O2", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), SRC, "-L", pkg, "-lmoe_ep",
           "-Wl,-rpath,$ORIGIN/../combine_moe_dispatch_layout_amd", "-o", BIN + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
