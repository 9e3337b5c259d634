"""The C ABI on its own: tests/c_abi_step (plain C, built by build() against
libzr.so and the HIP runtime, no Python or torch in the process) runs one
rank's step -- layout, pack of the rank's own gradient, mean of the
contributions, AdamW with the bf16 copy, unpack into tensor views -- and one
rejected call.  Its outputs must equal the oracle bit for bit: the mean, the
fp32 state (checked first against the 1e-6 relative + 1e-9 absolute bar, then
bits) and the unpacked bf16 parameters (1 ulp first, then bits) inside the
rank's range, which stay untouched outside it."""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_bf16_exact, assert_bits_equal, assert_fp32_exact, device, say
from zr_workloads import TINY_MLP, synth

pytestmark = pytest.mark.gpu

PROGRAM = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_step")
HP = TINY_MLP.hparams


def _bits(t):
    return t.view(torch.int16).numpy().view(np.uint16).copy()


@pytest.mark.parametrize("numels,n_d,rank,n_contrib", [
    (TINY_MLP.numels, 4, 0, 4),
    (TINY_MLP.numels, 3, 2, 3),                                  # the last rank, padding in its range
    ([5_000, 123_457, 99_999, 250_001, 100_000], 7, 3, 8),       # ragged list, persistent and straddling tensors
])
def test_c_program_step_matches_the_oracle(tmp_path, numels, n_d, rank, n_contrib):
    device()
    assert os.path.exists(PROGRAM), "tests/c_abi_step is missing: build() compiles it"
    ref = oracle.Layout(numels, n_d, 100_000)
    b, e = ref.rank_range(rank)
    S = e - b
    say("C ABI step", numels, "n_d", n_d, "rank", rank)
    step = 7
    d = str(tmp_path)
    with open(os.path.join(d, "config.bin"), "wb") as f:
        np.array([len(numels), *numels, n_d, rank, ref.threshold, n_contrib, step], np.int64).tofile(f)
        np.array([HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"]], np.float64).tofile(f)
    grads = {}
    for t, x in enumerate(numels):
        if not ref.persistent[t]:
            grads[t] = _bits(synth.normal_bf16(x, 1e-3, 300 + t))
            grads[t].tofile(os.path.join(d, f"grad_{t}.bin"))
    peers = [_bits(synth.normal_bf16(S, 1e-3, 400 + k)) for k in range(1, n_contrib)]
    for k, p in enumerate(peers, start=1):
        p.tofile(os.path.join(d, f"contrib_{k}.bin"))
    master = synth.normal_f32(S, 0.02, 500).numpy()
    m = synth.normal_f32(S, 1e-4, 501).numpy()
    v = synth.uniform_f32(S, 1e-6, 502).numpy()
    np.concatenate([master, m, v]).astype(np.float32).tofile(os.path.join(d, "state.bin"))

    r = subprocess.run([PROGRAM, d], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr

    # the oracle: pack, mean, AdamW, unpack
    views = [(grads[t], 0) if t in grads else None for t in range(len(numels))]
    want_mean = oracle.reduce([oracle.pack(ref, views, b, e)] + peers)
    st = [master.copy(), m.copy(), v.copy()]
    flat = np.zeros(S, np.uint16)
    oracle.adamw(want_mean, *st, flat, step=step, **HP)
    assert_bits_equal(np.fromfile(os.path.join(d, "reduced.bin"), np.uint16), want_mean, "C ABI mean")
    got = np.fromfile(os.path.join(d, "state_out.bin"), np.float32).reshape(3, S)
    for name, a, want in zip(("master", "exp_avg", "exp_avg_sq"), got, st):
        assert_fp32_exact(a, want, f"C ABI {name}")
    for t, x in enumerate(numels):
        if ref.persistent[t]:
            continue
        got_p = np.fromfile(os.path.join(d, f"param_{t}.bin"), np.uint16)
        lo, hi = max(b, ref.offset[t]), min(e, ref.offset[t] + x)
        inside = np.zeros(x, bool)
        if lo < hi:
            inside[lo - ref.offset[t]:hi - ref.offset[t]] = True
            assert_bf16_exact(got_p[inside], flat[lo - b:hi - b], f"C ABI param tensor {t}")
        assert not got_p[~inside].any(), f"C ABI unpack wrote tensor {t} outside the rank's range"
