"""Builds libzr.so in-tree with hipcc for gfx950 (MI355X).

Every source is compiled with FP contraction off (each fp32 operation is one
IEEE operation, as written) and with packed-fp32 code generation disabled;
the .hip files carry the gfx950 kernels, the .cpp files are host-only.
"""
import glob
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libzr.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-fvisibility=hidden",
]


def device_sources():
    """Translation units with GPU kernels (compiled for gfx950 and the host)."""
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def host_sources():
    """Host-only translation units (layout, the host optimizer): no device pass,
    so they may use host-only builtins."""
    return sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


def sources():
    return device_sources() + host_sources()


def build(verbose: bool = False, extra=(), output: str = LIBRARY) -> str:
    """Compiles every translation unit to an object (in parallel), then links
    libzr.so; the library is replaced only when everything succeeded."""
    include = [f"-I{INCLUDE}", f"-I{CSRC}"]
    with tempfile.TemporaryDirectory(prefix="zr_build_") as tmp:
        jobs = []
        for src in sources():
            obj = os.path.join(tmp, os.path.basename(src).replace(".", "_") + ".o")
            host_only = ["--offload-host-only"] if src.endswith(".cpp") else []
            jobs.append((["hipcc", *FLAGS, *host_only, *extra, *include, "-c", src, "-o", obj], obj))
        if verbose:
            for cmd, _ in jobs:
                print(" ".join(cmd), flush=True)
        workers = max(1, min(len(jobs), os.cpu_count() or 1, 16))
        with ThreadPoolExecutor(workers) as pool:
            results = list(pool.map(lambda j: subprocess.run(j[0], capture_output=True, text=True), jobs))
        failed = [(cmd, r) for (cmd, _), r in zip(jobs, results) if r.returncode != 0]
        if verbose:
            for r in results:
                if r.stderr:
                    print(r.stderr, end="", file=sys.stderr)
        if failed:
            cmd, r = failed[0]
            print(r.stdout + r.stderr, file=sys.stderr)
            raise subprocess.CalledProcessError(r.returncode, cmd)
        link = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for _, o in jobs], "-o", output + ".tmp"]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
    os.replace(output + ".tmp", output)
    return output


MEASURE_SOURCE = os.path.join(HERE, "measure", "stream_pattern.hip")
MEASURE_LIBRARY = os.path.join(HERE, "libzr_measure.so")


def build_measure(verbose: bool = False) -> str:
    """The bench's measurement kernel (the AdamW kernel's access pattern
    without its arithmetic), a library of its own beside libzr.so."""
    cmd = ["hipcc", *FLAGS, "-shared", f"-I{CSRC}", MEASURE_SOURCE, "-o", MEASURE_LIBRARY + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if verbose and r.stderr:
        print(r.stderr, end="", file=sys.stderr)
    if r.returncode != 0:
        print(r.stdout + r.stderr, file=sys.stderr)
        raise subprocess.CalledProcessError(r.returncode, cmd)
    os.replace(MEASURE_LIBRARY + ".tmp", MEASURE_LIBRARY)
    return MEASURE_LIBRARY


if __name__ == "__main__":
    print(build(verbose=True, extra=sys.argv[1:]))
