"""The GPU kernels take the fp32 square root of AdamW's second moment as the
hardware square root (within 1 ulp) refined by one exact FMA residual test on
each neighbour, so that it is correctly rounded like IEEE sqrtf and the host
AdamW of the offload path gives the same bits.  This CPU test applies the
refinement to each start value within 1 ulp of the true root, for every
denormal, every input around the 2^-96 scaling edge, two whole binades (both
exponent parities) and the largest binades, and compares with the C library's
correctly rounded sqrtf.  (Run with the argument "all", the same program checks
every finite input: 6.4e9 cases.)"""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = tmp_path_factory.mktemp("sqrt") / "sqrt_refine_check"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                    os.path.join(HERE, "sqrt_refine_check.c"), "-o", str(exe), "-lm"], check=True)
    return exe


def test_refined_hardware_sqrt_is_correctly_rounded(checker):
    out = subprocess.run([str(checker)], capture_output=True, text=True, timeout=600, check=True).stdout
    n, bad = map(int, out.split())
    assert n > 2e8
    assert bad == 0
