"""Build the CPU oracle (test infrastructure) into oracle/libmoe_oracle.so.

The oracle is plain scalar C compiled with gcc.  -ffp-contract=off keeps each
binary32 multiply and add separately rounded, as the combine definition needs.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "libmoe_oracle.so")


def build(verbose: bool = False, src: str = SRC, lib: str = LIB) -> str:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c99",
           "-D_DEFAULT_SOURCE", "-Wall", "-Wextra", "-fPIC", "-shared",
           "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
