"""Build the CPU oracle (test infrastructure) into oracle/libep_oracle.so.

Plain host C, ISO C11, -O2: the FP32 sums are IEEE binary32 in SSE registers,
with no contraction and no reassociation.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libep_oracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "ep_oracle.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
