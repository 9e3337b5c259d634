"""Builds tests/c_abi_step, a C program that drives one rank's step through
libzr's C ABI alone (test infrastructure, run by tests/test_gpu_c_abi.py).
Plain C with gcc against the HIP runtime and the in-tree libzr.so, found at
run time through an rpath relative to the program."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SOURCE = os.path.join(HERE, "c_abi_step.c")
PROGRAM = os.path.join(HERE, "c_abi_step")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROCM, 'include')}", f"-I{os.path.join(ROOT, 'include')}", SOURCE,
           "-o", PROGRAM + ".tmp",
           f"-L{os.path.join(ROOT, 'zero_sharded_optimizer_zr_amd')}", "-l:libzr.so",
           "-Wl,-rpath,$ORIGIN/../zero_sharded_optimizer_zr_amd",
           f"-L{os.path.join(ROCM, 'lib')}", "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(PROGRAM + ".tmp", PROGRAM)
    return PROGRAM


if __name__ == "__main__":
    print(build(verbose=True))
