"""Compile the CPU oracle (test infrastructure) into oracle/liboracle.so with gcc.

Flags keep IEEE fp32 semantics for the quantizer: no FMA contraction, no fast
math, SSE arithmetic (x86-64 default, no excess precision)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "kvq_oracle.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
           "-fno-fast-math", "-fexcess-precision=standard", "-fopenmp", "-fPIC",
           "-shared", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
