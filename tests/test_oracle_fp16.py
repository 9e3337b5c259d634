"""Pins the oracle's fp16 path (fp16 conversions, fp16 gradient mean, overflow
check, loss-scaled AdamW, dynamic loss scale) to the tutorial's fp16 config,
numpy's IEEE half-precision casts, exact arithmetic and torch.optim.AdamW."""
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

HP = dict(lr=5e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def f16(xs):
    return oracle.f16_from_f32(np.asarray(xs, dtype=np.float32))


# ----------------------------------------------------------- conversions ----

def test_f16_rounding_matches_numpy():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, size=300_000, dtype=np.uint64).astype(np.uint32)
    # concentrate on the fp16 range, its subnormals and the overflow boundary
    e = rng.integers(100, 145, size=bits.size).astype(np.uint32)
    bits[:200_000] = (bits[:200_000] & 0x807FFFFF) | (e[:200_000] << 23)
    bits[:2000] = (bits[:2000] & 0xFFFFE000) | 0x1000      # exact ties of the 13 dropped bits
    bits[2000:4000] = (bits[2000:4000] & 0xFFFFE000) | 0x0FFF
    x = bits.view(np.float32)
    got = oracle.f16_from_f32(x)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all(got[nan] == ((bits[nan] >> 16) & 0x8000).astype(np.uint16) | 0x7E00)


def test_f16_boundaries():
    cases = {65504.0: 0x7BFF, 65519.0: 0x7BFF, 65520.0: 0x7C00, 1e10: 0x7C00, -65520.0: 0xFC00,
             2.0 ** -14: 0x0400, 2.0 ** -24: 0x0001, 2.0 ** -25: 0x0000, 3 * 2.0 ** -25: 0x0002,
             2.0 ** -14 - 2.0 ** -25: 0x0400, 1.0 + 2.0 ** -11: 0x3C00, 1.0 + 3 * 2.0 ** -11: 0x3C02,
             -0.0: 0x8000}
    got = oracle.f16_from_f32(np.array(list(cases), dtype=np.float32))
    assert [int(v) for v in got] == list(cases.values())


def test_f16_widening_is_exact():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f32_from_f16(h)
    want = h.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))
    assert np.all(np.isnan(got[nan]))
    finite = ~nan
    assert np.array_equal(oracle.f16_from_f32(got)[finite], h[finite])


# ---------------------------------------------------------------- reduce ----

def test_reduce_f16_worked_example(golden):
    g = golden("reduce_scatter_example.txt")
    out = oracle.reduce_f16([f16(g["contrib0"]), f16(g["contrib1"])])
    assert list(oracle.f32_from_f16(out)) == g["allreduce_mean"]


def _rne_f16_of_fraction(q: Fraction) -> float:
    """Exact rational -> nearest fp16 value, ties to even (normal range)."""
    if q == 0:
        return 0.0
    s = -1 if q < 0 else 1
    a = abs(q)
    e = 0
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 10)
    k = a / ulp
    lo = k.numerator // k.denominator
    rem = k - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return s * float(lo * ulp)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 7, 8, 64])
def test_reduce_f16_is_rounded_exact_mean(n):
    rng = random.Random(40 + n)
    m = 300
    vals = [[rng.randrange(-2047, 2048) * 2.0 ** rng.randrange(-8, 2) for _ in range(m)] for _ in range(n)]
    contribs = [f16(v) for v in vals]
    assert all(np.array_equal(oracle.f32_from_f16(c), np.float32(v)) for c, v in zip(contribs, vals))
    out = oracle.f32_from_f16(oracle.reduce_f16(contribs))
    for i in range(m):
        exact = Fraction(sum(Fraction(v[i]) for v in vals), n)
        q32 = np.float32(exact.numerator) / np.float32(exact.denominator)
        tie = (int(np.float32(q32).view(np.uint32)) & 0x1FFF) == 0x1000 and Fraction(float(q32)) != exact
        if not tie and abs(exact) >= Fraction(2) ** -14:
            assert out[i] == _rne_f16_of_fraction(exact), (i, exact)


def test_reduce_f16_extremes_and_identity():
    big = f16([60000.0, -60000.0, 1.0])
    out = oracle.reduce_f16([big, big])
    assert list(oracle.f32_from_f16(out)) == [60000.0, -60000.0, 1.0]
    # the fp32 sum of fp16 values cannot overflow, and their mean stays within fp16
    three = oracle.reduce_f16([f16([65504.0])] * 3)
    assert int(three[0]) == 0x7BFF
    # an inf contribution makes the mean inf (the overflow check then skips the step)
    inf = oracle.reduce_f16([f16([65504.0]), f16([np.inf])])
    assert int(inf[0]) == 0x7C00
    x = f16(np.random.default_rng(3).normal(0, 30, 1000))
    assert np.array_equal(oracle.reduce_f16([x]), x)


def test_found_inf():
    assert not oracle.found_inf_f16(f16([0.0, -65504.0, 65504.0, 2.0 ** -24]))
    assert oracle.found_inf_f16(f16([1.0, np.inf]))
    assert oracle.found_inf_f16(f16([-np.inf, 1.0]))
    assert oracle.found_inf_f16(f16([1.0, np.nan, 2.0]))
    assert not oracle.found_inf_f16(np.zeros(0, np.uint16))


# ------------------------------------------------------------ loss-scaled AdamW ----

def _ulps(a, b):
    ai = a.view(np.int32).astype(np.int64)
    bi = b.view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7FFFFFFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFFFFFF), bi)
    return np.abs(ai - bi)


@pytest.mark.parametrize("scale,step", [(2.0 ** 16, 1), (2.0 ** 12, 10), (1.0, 3), (2.0 ** 20, 1000)])
def test_adamw_f16_unscales_and_matches_torch(scale, step):
    rng = np.random.default_rng(int(scale) % 97 + step)
    n = 20_000
    g_true = rng.normal(0, 1e-3, n).astype(np.float32)
    grad = f16(g_true * np.float32(scale))               # the scaled gradient the backward produced
    g_used = oracle.f32_from_f16(grad).astype(np.float64) / scale
    master = rng.normal(0, 0.02, n).astype(np.float32)
    m = rng.normal(0, 1e-4, n).astype(np.float32)
    v = rng.uniform(0, 1e-6, n).astype(np.float32)
    p = torch.nn.Parameter(torch.from_numpy(master.astype(np.float64)))
    opt = torch.optim.AdamW([p], lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]), eps=HP["eps"],
                            weight_decay=HP["weight_decay"], foreach=False, fused=False)
    p.grad = torch.from_numpy(g_used)
    opt.state[p] = {"step": torch.tensor(float(step - 1), dtype=torch.float64),
                    "exp_avg": torch.from_numpy(m.astype(np.float64)),
                    "exp_avg_sq": torch.from_numpy(v.astype(np.float64))}
    opt.step()
    pout = np.zeros(n, np.uint16)
    oracle.adamw_f16(grad, master, m, v, pout, step=step, loss_scale=scale, **HP)
    want = (p.detach().numpy().astype(np.float32), opt.state[p]["exp_avg"].numpy().astype(np.float32),
            opt.state[p]["exp_avg_sq"].numpy().astype(np.float32))
    for got, ref in zip((master, m, v), want):
        assert _ulps(got, ref).max() <= 1
    assert np.array_equal(pout, oracle.f16_from_f32(master))


def test_adamw_f16_at_scale_one_equals_the_bf16_update():
    # gradients exactly representable in both 16-bit formats: the two updates coincide
    rng = np.random.default_rng(8)
    n = 5000
    g = (rng.integers(-127, 128, n) * 2.0 ** rng.integers(-20, -8, n)).astype(np.float32)
    gb, gh = oracle.bf16_from_f32(g), f16(g)
    assert np.array_equal(oracle.f32_from_bf16(gb), g) and np.array_equal(oracle.f32_from_f16(gh), g)
    st = [rng.normal(0, 0.02, n).astype(np.float32), rng.normal(0, 1e-4, n).astype(np.float32),
          rng.uniform(0, 1e-6, n).astype(np.float32)]
    a = [x.copy() for x in st]
    b = [x.copy() for x in st]
    oracle.adamw(gb, *a, None, step=7, **HP)
    oracle.adamw_f16(gh, *b, None, step=7, loss_scale=1.0, **HP)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


# ------------------------------------------------------------ loss scale ----

def test_loss_scale_config(golden):
    g = golden("fp16_loss_scale_config.txt")
    assert g["loss_scale"] == 0                          # 0 selects the dynamic scale
    s = oracle.LossScale()
    assert s.scale == 2.0 ** g["initial_scale_power"] and s.window == g["loss_scale_window"]


def test_loss_scale_growth_and_backoff_closed_forms():
    s = oracle.LossScale()
    for k in range(1, 3501):
        s.update(False)
        assert s.scale == 2.0 ** (16 + k // 1000)        # doubles after every 1000 clean steps
    s.update(True)                                       # overflow: halve, restart the window
    assert s.scale == 2.0 ** 18 and s.good_steps == 0 and s.skipped == 1
    for _ in range(999):
        s.update(False)
    assert s.scale == 2.0 ** 18
    s.update(False)
    assert s.scale == 2.0 ** 19
    t = oracle.LossScale(initial=4.0)
    for _ in range(5):
        t.update(True)
    assert t.scale == 1.0 and t.skipped == 5             # never below the floor


def test_step_f16_skips_an_overflowing_step_bit_for_bit():
    rng = np.random.default_rng(21)
    n = 4096
    scaler = oracle.LossScale()
    contribs = [f16(rng.normal(0, 1e-3, n) * scaler.scale) for _ in range(4)]
    contribs[2][100] = 0x7C00                            # one overflowed gradient value
    st = [rng.normal(0, 0.02, n).astype(np.float32), rng.normal(0, 1e-4, n).astype(np.float32),
          rng.uniform(0, 1e-6, n).astype(np.float32)]
    before = [x.copy() for x in st]
    param = np.full(n, 0x1234, np.uint16)
    oracle.step_f16(contribs, *st, param, scaler, step=1, **HP)
    for x, y in zip(st, before):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    assert np.all(param == 0x1234)
    assert scaler.scale == 2.0 ** 15 and scaler.skipped == 1
    contribs[2][100] = f16([0.5])[0]
    oracle.step_f16(contribs, *st, param, scaler, step=1, **HP)
    assert not np.array_equal(st[0], before[0]) and scaler.good_steps == 1
