"""Build the CPU oracle (oracle/libiqo.so) with gcc.

Test infrastructure: the oracle is the checker, never part of the product
path.  Strict binary32 semantics: no FMA contraction, no fast-math, SSE math.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libiqo.so")
FLAGS = ["-std=c11", "-O3", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
         "-fno-fast-math", "-frounding-math", "-mfpmath=sse", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *FLAGS, os.path.join(HERE, "iqo.c"), "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
