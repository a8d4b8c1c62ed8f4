"""Build the CPU oracle (plain C, OpenMP) into oracle/liboracle.so.

Test infrastructure: compiled by the build step so that the checker exists
before any test runs; only the test suite, the smoke check and the
benchmark's CPU-baseline leg load it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dfssm_oracle.c")
OUT = os.path.join(HERE, "liboracle.so")
# -O3 vectorises the integer dot products; floating point keeps IEEE
# semantics in source order (no fast-math, no contraction, no reassociation).
CFLAGS = ["-O3", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wno-unknown-pragmas"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, "-o", OUT + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
