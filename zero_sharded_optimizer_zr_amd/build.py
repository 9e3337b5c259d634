"""Builds libzr.so in-tree with hipcc for gfx950 (MI355X).

Every HIP source is compiled with FP contraction off (each fp32 operation in
the kernels is one IEEE operation, as written) and with packed-fp32 code
generation disabled.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libzr.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-fvisibility=hidden",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.cpp")) + glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, extra=(), output: str = LIBRARY) -> str:
    cmd = ["hipcc", *FLAGS, *extra, f"-I{INCLUDE}", f"-I{CSRC}", *sources(), "-o", output + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(output + ".tmp", output)
    return output


if __name__ == "__main__":
    print(build(verbose=True, extra=sys.argv[1:]))
