"""Compile the CPU oracle (oracle.c) into oracle/liboracle.so with gcc.

Test infrastructure: the product library never links or loads it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
OUT = os.path.join(HERE, "liboracle.so")

# IEEE semantics are part of the oracle's contract: no fast-math, no FMA
# contraction (fl32(acc * sX) * sW must be two rounded products).
CFLAGS = ["-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
