"""Pins the oracle's floating-point steps (bf16 conversion, gradient mean,
AdamW) to the pages' worked example, exact arithmetic, closed forms and an
independent library implementation (torch.optim.AdamW run in float64)."""
import math
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def bf16(xs):
    return oracle.bf16_from_f32(np.asarray(xs, dtype=np.float32))


def f32_bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


# ------------------------------------------------------------------ bf16 ----

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # force exact ties and near ties on both parities
    bits[:1000] = (bits[:1000] & 0xFFFF0000) | 0x8000
    bits[1000:2000] = (bits[1000:2000] & 0xFFFF0000) | 0x7FFF
    bits[2000:3000] = (bits[2000:3000] & 0xFFFF0000) | 0x8001
    x = bits.view(np.float32)
    got = oracle.bf16_from_f32(x)
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], want[~nan])
    # NaN stays NaN with its sign
    g = got[nan]
    assert np.all((g & 0x7F80) == 0x7F80) and np.all((g & 0x007F) != 0)
    assert np.array_equal(g >> 15, (bits[nan] >> 31).astype(np.uint16))


def test_bf16_hand_cases():
    cases = {
        0x3F808000: 0x3F80,  # tie, even upper half -> down
        0x3F818000: 0x3F82,  # tie, odd upper half -> up
        0x3F808001: 0x3F81,  # above tie -> up
        0x3F807FFF: 0x3F80,  # below tie -> down
        0x7F7FFFFF: 0x7F80,  # rounds past max finite -> inf
        0x80000000: 0x8000,  # -0 kept
        0x00000001: 0x0000,  # smallest subnormal -> +0
        0x00008000: 0x0000,  # subnormal tie, even -> down
        0x00018000: 0x0002,  # subnormal tie, odd -> up
        0xFF800000: 0xFF80,  # -inf
    }
    x = np.array(list(cases), dtype=np.uint32).view(np.float32)
    assert list(oracle.bf16_from_f32(x)) == list(cases.values())


def test_bf16_widening_is_exact():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = oracle.f32_from_bf16(h)
    assert np.array_equal(f32_bits(f), h.astype(np.uint32) << 16)
    finite = ~np.isnan(f)
    assert np.array_equal(oracle.bf16_from_f32(f)[finite], h[finite])


# ---------------------------------------------------------------- reduce ----

def test_reduce_scatter_worked_example(golden):
    g = golden("reduce_scatter_example.txt")
    c0, c1 = bf16(g["contrib0"]), bf16(g["contrib1"])
    full = oracle.reduce([c0, c1])
    assert list(oracle.f32_from_bf16(full)) == g["allreduce_mean"]
    # rank r's ReduceScatter slice is slice r of the AllReduce result
    n_d = g["n_d"]
    per = len(c0) // n_d
    for r, key in enumerate(("rank0_slice", "rank1_slice")):
        sl = slice(r * per, (r + 1) * per)
        part = oracle.reduce([c0[sl].copy(), c1[sl].copy()])
        assert list(oracle.f32_from_bf16(part)) == g[key]
        assert np.array_equal(part, full[sl])


def _rne_bf16_of_fraction(q: Fraction) -> float:
    """Round an exact rational to the nearest bf16 value, ties to even (normal range)."""
    if q == 0:
        return 0.0
    s = -1 if q < 0 else 1
    a = abs(q)
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 7)          # 8 significant bits
    k = a / ulp
    lo = math.floor(k)
    rem = k - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return s * float(lo * ulp)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 7, 8, 64])
def test_reduce_is_rounded_exact_mean_for_exact_sums(n):
    # small-integer-scaled bf16 values: every fp32 partial sum is exact, so the
    # result is the exact mean rounded to bf16 (ties to even), except where the
    # fp32 quotient itself lands on a bf16 tie (double rounding)
    rng = random.Random(n)
    m = 300
    vals = [[rng.randrange(-255, 256) * 2.0 ** rng.randrange(-4, 3) for _ in range(m)] for _ in range(n)]
    contribs = [bf16(v) for v in vals]
    assert all(np.array_equal(oracle.f32_from_bf16(c), np.float32(v)) for c, v in zip(contribs, vals))
    out = oracle.f32_from_bf16(oracle.reduce(contribs))
    for i in range(m):
        exact = Fraction(sum(Fraction(v[i]) for v in vals), n)
        q32 = np.float32(exact.numerator) / np.float32(exact.denominator) if exact.denominator < 2**24 else None
        tie = q32 is not None and (int(f32_bits(q32)) & 0xFFFF) == 0x8000 and Fraction(float(q32)) != exact
        if not tie:
            assert out[i] == _rne_bf16_of_fraction(exact), (i, exact)


def test_reduce_within_error_bound_of_exact_mean():
    rng = np.random.default_rng(7)
    for n in (2, 4, 8, 64):
        contribs = [bf16(rng.normal(0, 1e-3, 4000)) for _ in range(n)]
        out = oracle.f32_from_bf16(oracle.reduce(contribs)).astype(np.float64)
        g = np.stack([oracle.f32_from_bf16(c).astype(np.float64) for c in contribs])
        exact = g.sum(0) / n                      # exact in float64 for these magnitudes
        abs_sum = np.abs(g).sum(0) / n
        u32 = 2.0 ** -24
        fp32_err = (n * u32) * abs_sum            # accumulation + division bound
        half_ulp_bf16 = np.maximum(np.abs(out), np.abs(exact)) * 2.0 ** -8
        assert np.all(np.abs(out - exact) <= fp32_err + half_ulp_bf16 + 1e-40)


def test_reduce_identities():
    rng = np.random.default_rng(3)
    c = [bf16(rng.normal(0, 1e-3, 1000)) for _ in range(5)]
    # n = 1: the mean of one contribution is that contribution, bit for bit
    assert np.array_equal(oracle.reduce([c[0]]), c[0])
    # in place on contribution 0
    ref = oracle.reduce(c)
    c0 = c[0].copy()
    oracle.reduce([c0] + c[1:], out=c0)
    assert np.array_equal(c0, ref)
    # ReduceScatter slice == AllReduce slice for every split
    for n_d in (2, 4, 8):
        per = 1000 // n_d
        for r in range(n_d):
            sl = slice(r * per, (r + 1) * per)
            assert np.array_equal(oracle.reduce([x[sl].copy() for x in c]), ref[sl])
    # contribution order is part of the definition: fp32 sum in ascending k
    big, one, neg = bf16([2.0 ** 25]), bf16([1.0]), bf16([-(2.0 ** 25)])
    assert oracle.f32_from_bf16(oracle.reduce([big, one, neg]))[0] == 0.0   # 2^25 + 1 rounds to 2^25
    third = oracle.f32_from_bf16(bf16([np.float32(1.0) / np.float32(3.0)]))[0]
    assert oracle.f32_from_bf16(oracle.reduce([big, neg, one]))[0] == third


def test_reduce_power_of_two_scaling_is_exact():
    rng = np.random.default_rng(11)
    x = bf16(rng.normal(0, 1e-3, 2000))
    for n in (2, 4, 8, 64):
        out = oracle.reduce([x] * n)
        assert np.array_equal(out, x)  # n equal terms: the mean is the term itself


# ----------------------------------------------------------------- AdamW ----

HP = dict(lr=5e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _state(rng, n, m_std, v_high):
    g = bf16(rng.normal(0, 1e-3, n))
    master = rng.normal(0, 0.02, n).astype(np.float32)
    m = (rng.normal(0, m_std, n) if m_std else np.zeros(n)).astype(np.float32)
    v = (rng.uniform(0, v_high, n) if v_high else np.zeros(n)).astype(np.float32)
    return g, master, m, v


def _torch_adamw(g, master, m, v, step, hp, grad_scale=1.0):
    """torch.optim.AdamW (float64, single-tensor path) from the same fp32 state."""
    p = torch.nn.Parameter(torch.from_numpy(master.astype(np.float64)))
    opt = torch.optim.AdamW([p], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"], foreach=False, fused=False)
    p.grad = torch.from_numpy(oracle.f32_from_bf16(g).astype(np.float64) * grad_scale)
    opt.state[p] = {"step": torch.tensor(float(step - 1), dtype=torch.float64),
                    "exp_avg": torch.from_numpy(m.astype(np.float64)),
                    "exp_avg_sq": torch.from_numpy(v.astype(np.float64))}
    opt.step()
    st = opt.state[p]
    return (p.detach().numpy().astype(np.float32), st["exp_avg"].numpy().astype(np.float32),
            st["exp_avg_sq"].numpy().astype(np.float32))


def _ulps(a, b):
    ai = a.view(np.int32).astype(np.int64)
    bi = b.view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7FFFFFFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFFFFFF), bi)
    return np.abs(ai - bi)


@pytest.mark.parametrize("step,m_std,v_high,scale,hp", [
    (1, 0.0, 0.0, 1.0, HP),
    (10, 1e-4, 1e-6, 1.0, HP),
    (1000, 1e-4, 1e-6, 1.0, dict(HP, lr=1e-4, weight_decay=0.1)),
    (3, 1e-4, 1e-6, 0.25, HP),
    (7, 1e-3, 1e-5, 1.0, dict(lr=1e-3, beta1=0.8, beta2=0.95, eps=1e-6, weight_decay=0.0)),
])
def test_adamw_matches_torch_float64(step, m_std, v_high, scale, hp):
    rng = np.random.default_rng(step)
    n = 20_000
    g, master, m, v = _state(rng, n, m_std, v_high)
    want = _torch_adamw(g, master, m, v, step, hp, scale)
    p = np.empty(n, dtype=np.uint16)
    oracle.adamw(g, master, m, v, p, step=step, grad_scale=scale, **hp)
    for got, ref in zip((master, m, v), want):
        d = _ulps(got, ref)
        assert d.max() <= 1
        # near-ties: (9 m + g) / 10 often sits within one fp64 ulp of an fp32
        # midpoint, where fp64 rounding order decides; so <= 1 ulp, mostly 0
        assert np.mean(d == 0) > 0.99
    assert np.array_equal(p, oracle.bf16_from_f32(master))


def test_adamw_step_one_closed_form():
    # m = v = 0, t = 1: the bias-corrected moments are g and g^2, so
    # th' = th (1 - lr wd) - lr g / (|g| + eps)
    rng = np.random.default_rng(5)
    n = 10_000
    g, master, m, v = _state(rng, n, 0, 0)
    th0 = master.astype(np.float64)
    gd = oracle.f32_from_bf16(g).astype(np.float64)
    oracle.adamw(g, master, m, v, None, step=1, **HP)
    lr, wd, eps = HP["lr"], HP["weight_decay"], HP["eps"]
    closed = th0 * (1 - lr * wd) - lr * gd / (np.abs(gd) + eps)
    assert _ulps(master, closed.astype(np.float32)).max() <= 1
    assert _ulps(m, ((1 - HP["beta1"]) * gd).astype(np.float32)).max() <= 1
    assert _ulps(v, ((1 - HP["beta2"]) * gd * gd).astype(np.float32)).max() <= 1


def test_adamw_zero_gradient_is_pure_decay():
    rng = np.random.default_rng(9)
    n = 5000
    _, master, m, v = _state(rng, n, 0, 0)
    g = np.zeros(n, dtype=np.uint16)
    th0 = master.astype(np.float64)
    for step in (1, 2, 50):
        oracle.adamw(g, master, m, v, None, step=step, **HP)
        th0 = (th0.astype(np.float32).astype(np.float64)) * (1 - HP["lr"] * HP["weight_decay"])
        assert np.array_equal(master, th0.astype(np.float32))
        assert not m.any() and not v.any()


def test_adamw_shards_concatenate_to_unsharded_step():
    # each element's update uses only its own gradient and state, so N_d
    # independent shard updates concatenate to the one unsharded update
    rng = np.random.default_rng(13)
    n = 4096 + 37
    g, master, m, v = _state(rng, n, 1e-4, 1e-6)
    whole = [a.copy() for a in (master, m, v)]
    pw = np.empty(n, dtype=np.uint16)
    oracle.adamw(g, *whole, pw, step=10, **HP)
    for n_d in (2, 3, 4, 64):
        cuts = np.linspace(0, n, n_d + 1).astype(int)
        parts = [a.copy() for a in (master, m, v)]
        pp = np.empty(n, dtype=np.uint16)
        for b, e in zip(cuts[:-1], cuts[1:]):
            sub = [a[b:e].copy() for a in parts]
            ps = np.empty(e - b, dtype=np.uint16)
            oracle.adamw(g[b:e].copy(), *sub, ps, step=10, **HP)
            for a, s in zip(parts, sub):
                a[b:e] = s
            pp[b:e] = ps
        for a, w in zip(parts, whole):
            assert np.array_equal(a.view(np.uint32), w.view(np.uint32))
        assert np.array_equal(pp, pw)


def test_adamw_moment_decay_special_case():
    # beta1 = beta2 = 0: m = g, v = g^2 at every step, and bias correction is 1
    rng = np.random.default_rng(17)
    n = 3000
    g, master, m, v = _state(rng, n, 1e-4, 1e-6)
    th0 = master.astype(np.float64)
    gd = oracle.f32_from_bf16(g).astype(np.float64)
    hp = dict(HP, beta1=0.0, beta2=0.0)
    oracle.adamw(g, master, m, v, None, step=5, **hp)
    assert np.array_equal(m, gd.astype(np.float32))
    closed = th0 * (1 - hp["lr"] * hp["weight_decay"]) - hp["lr"] * gd / (np.abs(gd) + hp["eps"])
    assert _ulps(master, closed.astype(np.float32)).max() <= 1
