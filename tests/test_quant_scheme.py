"""The int8 and int4 block quantizers take x / s as one Markstein correction step on
the reciprocal (two FMAs) instead of a division.  For bf16 inputs the whole
input space is small enough to enumerate: this CPU test checks, for every
bf16 absmax whose scale is at least 2^-100 and every bf16 x of its block, that
the codes equal those of the correctly rounded quotient (and the quotient
itself wherever it is at least 1/4), and that the uncorrected product alone
would not."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = tmp_path_factory.mktemp("scheme") / "quant_scheme_check"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                    os.path.join(HERE, "quant_scheme_check.c"), "-o", str(exe), "-lm"], check=True)
    return exe


@pytest.mark.parametrize("q", [127, 7])  # int8, int4
def test_corrected_reciprocal_quotient_gives_exact_codes_for_all_bf16(checker, q):
    out = subprocess.run([str(checker), str(q)], capture_output=True, text=True, timeout=600, check=True).stdout
    pairs, bad_code, bad_quot, bad_plain = map(int, out.split())
    assert pairs > 5e8                 # the whole fast domain: about 5.2e8 (x, amax) pairs with x >= 0
    assert bad_code == 0
    assert bad_quot == 0
    assert bad_plain > 100             # the product alone misrounds near half steps
