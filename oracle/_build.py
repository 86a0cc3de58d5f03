"""Build the CPU oracle shared library (oracle/liblbm_oracle.so) with gcc.

Test infrastructure: the oracle is compiled so the tests, the smoke check and
the benchmark's CPU-baseline leg can call it.  Plain -O2 with floating-point
contraction switched off, single-threaded, no vectorisation pragmas.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lbm_oracle.c")
LIB = os.path.join(HERE, "liblbm_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fno-semantic-interposition", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
