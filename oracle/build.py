"""Compile the CPU oracle (qk_oracle.cpp, g++) into oracle/liboracle.so.

Test infrastructure: the oracle is the correctness reference for the GPU
library and is never linked into it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qk_oracle.cpp")
LIB = os.path.join(HERE, "liboracle.so")

# -ffp-contract=off: g++ contracts a*b+c into an FMA by default on hosts that
# have one; the oracle rounds every multiply and add on its own.
CFLAGS = ["-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(verbose=False):
    cmd = ["g++", *CFLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
