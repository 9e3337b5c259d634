"""Pins the oracle's memory ledger to the numbers the pages print."""
from fractions import Fraction

import oracle
from oracle import Layout, ledger_closed_form

GB = 10**9


def test_7b_on_4_gpus(golden):
    g = golden("ledger_7b_4gpu.txt")
    psi, n_d = g["psi"], g["n_d"]
    assert g["params_gb"] + g["grads_gb"] + g["optimizer_states_gb"] == g["stage0_gb"]
    for stage in range(4):
        assert ledger_closed_form(psi, n_d, stage) == Fraction(g[f"stage{stage}_gb"]).limit_denominator() * GB
    assert n_d * ledger_closed_form(psi, n_d, 0) == g["cluster_total_stage0_gb"] * GB
    # the same model as one flat tensor, every rank's layout-exact ledger equals the closed form
    lay = Layout([psi], n_d)
    for stage in range(4):
        assert lay.ledger_bytes(stage) == ledger_closed_form(psi, n_d, stage)


def test_7p5b_on_64_gpus(golden):
    g = golden("ledger_7p5b_64gpu.txt")
    psi, n_d = g["psi"], g["n_d"]
    assert ledger_closed_form(psi, n_d, 0) == g["stage0_gb"] * GB
    s3 = ledger_closed_form(psi, n_d, 3)
    assert round(float(s3) / GB, 1) == g["stage3_gb_1dp"]
    assert s3 == Fraction(1875, 1000) * GB  # exact value behind the printed 1.9


def test_fractions_at_nd64(golden):
    g = golden("ledger_fractions_nd64.txt")
    n_d = g["n_d"]
    psi = 10**9
    base = ledger_closed_form(psi, n_d, 0)
    assert base / base * 100 == g["stage0_pct"]
    for stage in (1, 2, 3):
        pct = ledger_closed_form(psi, n_d, stage) / base * 100
        assert round(float(pct), 1) == g[f"stage{stage}_pct_1dp"]


def test_16_bytes_per_param(golden):
    g = golden("ledger_16B_examples.txt")
    per = g["bytes_param"] + g["bytes_grad"] + g["bytes_m"] + g["bytes_v"] + g["bytes_master"]
    assert per == 16
    assert g["bytes_m"] + g["bytes_v"] + g["bytes_master"] == g["k_adam"]
    assert ledger_closed_form(g["psi_175b"], 8, 0) == g["stage0_gb_175b"] * GB
    assert ledger_closed_form(g["psi_7b"], 8, 0) == g["stage0_gb_7b"] * GB
    assert ledger_closed_form(g["psi_7b"], 8, 0) > g["a100_gb"] * GB
    # stage 3 is (2 + 2 + K) psi / N_d for every N_d
    for n_d in (1, 3, 64, 512):
        assert ledger_closed_form(1234567, n_d, 3) == Fraction((2 + 2 + g["k_adam"]) * 1234567, n_d)


def test_savings_limits(golden):
    g = golden("savings_factors.txt")
    psi = 10**12
    base = ledger_closed_form(psi, 1, 0)
    huge = 10**15  # stands in for N_d -> infinity
    assert round(float(base / ledger_closed_form(psi, huge, 1)), 6) == g["stage1_factor"]
    assert round(float(base / ledger_closed_form(psi, huge, 2)), 6) == g["stage2_factor"]
    for n_d in (2, 8, 64):
        assert base / ledger_closed_form(psi, n_d, 3) == n_d


def test_stage_one_equals_data_parallel_at_one_rank():
    for stage in range(4):
        assert ledger_closed_form(999, 1, stage) == 16 * 999


def test_layout_exact_bounds_the_closed_form():
    # with padding and persistent tensors the layout-exact stage-3 bytes sit
    # between the partitioned closed form and one extra element of state
    lists = ([5, 7, 3], [100, 1, 1, 250], [1, 2, 3, 4, 5, 6, 7], [0, 9])
    for numels in lists:
        for n_d in range(1, 9):
            for thr in (0, 4, 10**9):
                lay = Layout(numels, n_d, thr)
                exact = lay.ledger_bytes(3) - 16 * lay.psi_persist
                lo = ledger_closed_form(lay.psi_part, n_d, 3)
                assert lo <= exact < lo + 16


def test_workload_ledgers_match_hand_arithmetic():
    from zr_workloads import FLAT_1T, FLAT_7B, TINY_MLP
    lay = Layout(TINY_MLP.numels, TINY_MLP.n_d)
    # 2 biases (512 + 1024 elements) are persistent; 4 ranks of 262144
    assert lay.ledger_bytes(3) == 16 * 262144 + 16 * 1536
    assert Layout(FLAT_7B.numels, 4).ledger_bytes(3) == 28 * GB
    assert Layout(FLAT_1T.numels, 512).ledger_bytes(3) == 31_250_000_000
    assert oracle.DEFAULT_PERSIST_THRESHOLD == 100_000
