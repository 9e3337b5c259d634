"""Builds the oracle's C part (``zr_oracle.c`` -> ``liboracle.so``) with gcc.

TEST INFRASTRUCTURE ONLY: the oracle is loaded by the tests, the smoke check
and the benchmark's CPU-baseline leg, never by the product library.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "zr_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

# No fast-math and no contraction: each C operation is one IEEE operation.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SOURCE, "-o", LIBRARY + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIBRARY + ".tmp", LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
