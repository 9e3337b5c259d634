"""CPU tests of the host AdamW used by the ZeRO-Offload step (zr_host_adamw_step):
bit-identity with the oracle (the same double computation), across its
AVX-512 / AVX2 / scalar variants,
ragged sizes and misaligned buffers, thread counts, concurrent callers, and
the validation of both offload entry points (no GPU is touched)."""
import ctypes
import json
import os
import subprocess
import sys
import threading

import numpy as np
import pytest
import torch

import oracle
import zero_sharded_optimizer_zr_amd as zr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HP = dict(lr=5e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def state(n, seed):
    rng = np.random.default_rng(seed)
    g = oracle.bf16_from_f32(rng.normal(0, 1e-3, n).astype(np.float32))
    th = rng.normal(0, 0.02, n).astype(np.float32)
    m = rng.normal(0, 1e-4, n).astype(np.float32)
    v = rng.uniform(0, 1e-6, n).astype(np.float32)
    return g, th, m, v


def host_step(g, th, m, v, offset=0, threads=0, with_param=True, **kw):
    """Runs zr_host_adamw_step on copies placed `offset` elements into larger
    buffers (so the SIMD loops start misaligned); returns (th, m, v, param)."""
    n = g.size

    def place(x, dtype):
        big = torch.zeros(n + offset + 3, dtype=dtype)
        big[offset:offset + n] = torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x.copy())
        return big, big[offset:offset + n]

    _, gt = place(g, torch.int16)
    outs = [place(x, torch.float32) for x in (th, m, v)]
    pb, pt = place(np.zeros(n, np.uint16), torch.int16)
    zr.zr_host_adamw_step(gt, outs[0][1], outs[1][1], outs[2][1], pt if with_param else None,
                          threads=threads, **{**HP, **kw})
    for big, _ in outs:
        assert not big[:offset].any() and not big[offset + n:].any()
    return (*[o[1].numpy().copy() for o in outs], pt.numpy().view(np.uint16).copy())


def assert_bits(got, ref, what):
    g = got.view(np.uint32) if got.dtype == np.float32 else got
    r = ref.view(np.uint32) if ref.dtype == np.float32 else ref
    bad = g != r
    assert not bad.any(), f"{what}: {int(bad.sum())} of {got.size} differ from the oracle"


@pytest.mark.parametrize("n", [0, 1, 7, 15, 16, 17, 31, 100_003])
@pytest.mark.parametrize("offset", [0, 1, 5])
def test_host_adamw_matches_oracle(n, offset):
    """The host AdamW computes the update in double, in the oracle's order of
    operations, and rounds each state once: every bit equals the oracle's."""
    g, th, m, v = state(n, n + offset)
    ref = [th.copy(), m.copy(), v.copy()]
    rp = np.zeros(n, np.uint16)
    if n:
        oracle.adamw(g, *ref, rp, step=10, **HP)
    got = host_step(g, th, m, v, offset=offset, step=10)
    for name, a, b in zip(("master", "m", "v", "param"), got, ref + [rp]):
        assert_bits(a, b, f"{name} n={n}")


@pytest.mark.parametrize("step,kw", [(1, {}), (10, {}), (1000, dict(lr=1e-4, weight_decay=0.1)),
                                     (3, dict(grad_scale=0.25)), (7, dict(beta1=0.0, beta2=0.0))])
def test_host_adamw_hyperparameters(step, kw):
    n = 70_001
    g, th, m, v = state(n, step)
    ref = [th.copy(), m.copy(), v.copy()]
    rp = np.zeros(n, np.uint16)
    oracle.adamw(g, *ref, rp, step=step, **{**HP, **kw})
    got = host_step(g, th, m, v, offset=3, step=step, **kw)
    for name, a, b in zip(("master", "m", "v", "param"), got, ref + [rp]):
        assert_bits(a, b, f"{name} step {step}")


def test_host_adamw_near_total_cancellation():
    """Elements whose update nearly cancels the decayed master (theta' within a
    few 1e-10 of zero at step 1, where the step is lr * g / (|g| + eps)): the
    double computation keeps them exact, so the bf16 copy equals the oracle's
    too (an fp32 evaluation can miss it by several bf16 ulps there)."""
    n = 4096
    rng = np.random.default_rng(5)
    g = oracle.bf16_from_f32(rng.choice([-1.0, 1.0], n).astype(np.float32) * np.float32(1e-3))
    gf = oracle.f32_from_bf16(g).astype(np.float64)
    # theta * (1 - lr wd) equals lr * g / (|g| + eps) up to a tiny offset
    target = 5e-5 * gf / (np.abs(gf) + 1e-8) / (1.0 - 5e-5 * 0.01)
    th = (target + rng.normal(0, 1e-12, n)).astype(np.float32)
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    ref = [th.copy(), m.copy(), v.copy()]
    rp = np.zeros(n, np.uint16)
    oracle.adamw(g, *ref, rp, step=1, **HP)
    assert np.median(np.abs(ref[0])) < 1e-9     # the cancellation is there
    got = host_step(g, th, m, v, step=1)
    for name, a, b in zip(("master", "m", "v", "param"), got, ref + [rp]):
        assert_bits(a, b, f"{name} near cancellation")


SIMD_SCRIPT = r"""
import sys, json
import numpy as np, torch
sys.path.insert(0, sys.argv[1])
import zero_sharded_optimizer_zr_amd as zr
d = np.load(sys.argv[2])
g, th, m, v = (torch.from_numpy(d[k].copy()) for k in ("g", "th", "m", "v"))
p = torch.zeros(g.numel(), dtype=torch.int16)
zr.zr_host_adamw_step(g, th, m, v, p, lr=5e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=10)
np.savez(sys.argv[3], th=th.numpy(), m=m.numpy(), v=v.numpy(), p=p.numpy())
print(zr.zr_host_simd())
"""


def test_simd_variants_agree_bit_for_bit(tmp_path):
    n = 100_003
    g, th, m, v = state(n, 5)
    g = g.copy()
    g[:6] = [0x7F80, 0xFF80, 0x7FC1, 0x0001, 0x8000, 0x0000]   # inf, -inf, NaN, subnormal, -0, 0
    np.savez(tmp_path / "in.npz", g=g.view(np.int16), th=th, m=m, v=v)
    outs = {}
    for isa in ("scalar", "avx2", "avx512"):
        env = {**os.environ, "ZR_HOST_SIMD": isa}
        r = subprocess.run([sys.executable, "-c", SIMD_SCRIPT, ROOT, str(tmp_path / "in.npz"),
                            str(tmp_path / f"{isa}.npz")], env=env, capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stderr
        used = r.stdout.strip().splitlines()[-1]
        outs[used] = np.load(tmp_path / f"{isa}.npz")
    assert "scalar" in outs and len(outs) >= 2, list(outs)
    base = outs["scalar"]
    for isa, o in outs.items():
        for k in ("th", "m", "v", "p"):
            assert np.array_equal(o[k].view(np.uint32 if o[k].dtype == np.float32 else np.uint16),
                                  base[k].view(np.uint32 if base[k].dtype == np.float32 else np.uint16)), (isa, k)
    # the non-finite gradients propagate as NaN / inf into the state, like on the GPU
    assert np.isnan(base["m"][2]) and np.isinf(base["v"][0])


@pytest.mark.parametrize("threads", [1, 2, 3, 0])
def test_thread_counts_give_the_same_bits(threads):
    n = 300_007
    g, th, m, v = state(n, 9)
    one = host_step(g, th, m, v, threads=1, step=4)
    got = host_step(g, th, m, v, threads=threads, step=4)
    for a, b in zip(got, one):
        assert np.array_equal(a, b)


def test_concurrent_callers():
    n = 200_003
    cases = [state(n, 20 + k) for k in range(4)]
    want = [host_step(*c, step=2) for c in cases]
    got = [None] * 4

    def run(k):
        got[k] = host_step(*cases[k], step=2)

    ts = [threading.Thread(target=run, args=(k,)) for k in range(4)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    for a, b in zip(got, want):
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


def test_no_param_copy():
    n = 1000
    g, th, m, v = state(n, 1)
    a = host_step(g, th, m, v, with_param=False, step=1)
    b = host_step(g, th, m, v, step=1)
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x, y)
    assert not a[3].any()


class _HP(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double), ("grad_scale", ctypes.c_double),
                ("step", ctypes.c_int64)]


def test_host_and_offload_validation():
    L = zr._lib
    hp = _HP(5e-5, 0.9, 0.999, 1e-8, 0.01, 1.0, 1)
    bad_hp = _HP(5e-5, 0.9, 0.999, 1e-8, 0.01, 1.0, 0)
    A = 0x7F0000000000
    g, th, m, v, p = A, A + 2**22, A + 2**23, A + 2**24, A + 2**25
    H = lambda *a: L.zr_host_adamw_step(*a)
    assert H(g, th, m, v, p, 16, None, 0) == zr.ZR_EINVAL
    assert H(g, th, m, v, p, 16, ctypes.byref(bad_hp), 0) == zr.ZR_EINVAL
    assert H(g, th, m, v, p, -1, ctypes.byref(hp), 0) == zr.ZR_EINVAL
    assert H(g, th, m, v, p, 16, ctypes.byref(hp), -1) == zr.ZR_EINVAL
    assert H(None, th, m, v, p, 16, ctypes.byref(hp), 0) == zr.ZR_EINVAL
    assert H(g + 1, th, m, v, p, 16, ctypes.byref(hp), 0) == zr.ZR_EALIGN
    assert H(g, th + 2, m, v, p, 16, ctypes.byref(hp), 0) == zr.ZR_EALIGN
    assert H(g, th, th + 32, v, p, 16, ctypes.byref(hp), 0) == zr.ZR_EINVAL   # m overlaps master
    assert H(g, th, m, v, v + 8, 16, ctypes.byref(hp), 0) == zr.ZR_EINVAL     # param overlaps v
    assert H(None, None, None, None, None, 0, ctypes.byref(hp), 0) == zr.ZR_OK
    st = A + 2**30
    O = lambda *a: L.zr_offload_adamw_step(*a)
    big = zr.ZR_OFFLOAD_MIN_STAGING
    assert O(g, th, m, v, p, 16, None, st, big, 0, None) == zr.ZR_EINVAL
    assert O(g, th, m, v, p, 16, ctypes.byref(hp), None, big, 0, None) == zr.ZR_EINVAL
    assert O(g, th, m, v, p, 16, ctypes.byref(hp), st, big - 1, 0, None) == zr.ZR_EINVAL
    assert O(g, th, m, v, p, 16, ctypes.byref(hp), st + 32, big, 0, None) == zr.ZR_EALIGN
    assert O(g, th, m, v, p, 16, ctypes.byref(hp), th - 64, big, 0, None) == zr.ZR_EINVAL  # staging over master
    assert O(g, th, m, v, g + 8, 16, ctypes.byref(hp), st, big, 0, None) == zr.ZR_EINVAL   # param over grad
    assert O(g, th, m, v, p, 16, ctypes.byref(hp), st, big, -2, None) == zr.ZR_EINVAL
    assert O(g + 1, th, m, v, p, 16, ctypes.byref(hp), st, big, 0, None) == zr.ZR_EALIGN
    assert O(g, th, m, v, p, 0, ctypes.byref(hp), st, big, 0, None) == zr.ZR_OK
    assert zr.zr_host_simd() in ("avx512", "avx2", "scalar")


def test_binding_checks_devices():
    t = torch.zeros(8)
    with pytest.raises(ValueError):
        zr.zr_offload_adamw_step(torch.zeros(8, dtype=torch.int16), t, t.clone(), t.clone(), None,
                                 torch.zeros(zr.ZR_OFFLOAD_MIN_STAGING, dtype=torch.uint8), step=1, **HP)
