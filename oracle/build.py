"""Compile the CPU oracle (test infrastructure) into oracle/liboracle.so with gcc.

Flags keep IEEE fp32 semantics for the quantizer: no FMA contraction, no fast
math, SSE arithmetic (x86-64 default, no excess precision).

`python oracle/build.py --sanitize` builds oracle/liboracle_san.so with
AddressSanitizer and UndefinedBehaviorSanitizer (errors abort), for the CPU tests:

    ORACLE_LIBRARY=oracle/liboracle_san.so ASAN_OPTIONS=detect_leaks=0 \
    LD_PRELOAD="$(gcc -print-file-name=libasan.so) $(gcc -print-file-name=libubsan.so)" \
    python -m pytest -q -m "not gpu" tests/test_oracle_*.py"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
LIB_SAN = os.path.join(HERE, "liboracle_san.so")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    src = os.path.join(HERE, "kvq_oracle.c")
    out = LIB_SAN if sanitize else LIB
    tmp = out + ".tmp"
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           "-g"] if sanitize else []
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
           "-fno-fast-math", "-fexcess-precision=standard", "-fopenmp", "-fPIC", *san,
           "-shared", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv[1:])
    sys.exit(0)
