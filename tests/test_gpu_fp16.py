"""GPU parity of the fp16 path with dynamic loss scaling against the oracle:
fp16 gradient mean (bit-exact) with its overflow flag, the standalone finite
check, the loss-scaled AdamW step (and its skip), the device-side scale rule,
and whole multi-step sequences with planted overflows."""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_optimizer_zr_amd as zr
from gpu_util import Placed, assert_bits_equal, assert_fp32_exact, device, say

pytestmark = pytest.mark.gpu

HP = dict(lr=5e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
S0 = 2.0 ** 16


def f16(x):
    return oracle.f16_from_f32(np.asarray(x, dtype=np.float32))


def record(scale=S0):
    ls = zr.loss_scale_record(device())
    zr.zr_loss_scale_init(ls, scale)
    return ls


def read_record(ls):
    torch.cuda.synchronize()
    r = ls.cpu()
    return float(r.view(torch.float32)[0]), int(r[1]), int(r[2]), int(r[3])


def assert_f16_within_1ulp(got, ref, what):
    def key(h):
        h = h.astype(np.int64)
        return np.where(h & 0x8000, -(h & 0x7FFF), h)
    d = np.abs(key(got) - key(ref))
    assert (d <= 1).all(), f"{what}: {int((d > 1).sum())} beyond 1 fp16 ulp"
    # the copy is rounded from a master that equals the oracle's bit for bit
    assert_bits_equal(np.ascontiguousarray(got, np.uint16), np.ascontiguousarray(ref, np.uint16), f"{what} (bits)")


def assert_f16_equal(got, ref, what):
    """Bit-exact, except that NaNs only have to be NaNs."""
    nan_g = ((got & 0x7C00) == 0x7C00) & ((got & 0x3FF) != 0)
    nan_r = ((ref & 0x7C00) == 0x7C00) & ((ref & 0x3FF) != 0)
    assert np.array_equal(nan_g, nan_r), f"{what}: NaN positions differ"
    assert_bits_equal(got[~nan_r], ref[~nan_r], what)


def scaled_contribs(n, size, seed, scale=S0):
    rng = np.random.default_rng(seed)
    return [f16(rng.normal(0, 1e-3, size) * scale) for _ in range(n)]


# ------------------------------------------------------------- fp16 mean ----

@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 8, 9, 64])
def test_reduce_f16_bit_exact(n):
    device()
    say("reduce f16 n =", n)
    size = 20_000 + n
    contribs = scaled_contribs(n, size, n)
    ref = oracle.reduce_f16(contribs)
    # aligned; a common 16-byte phase; mixed phases; heads of 48 and 3 elements to the
    # output's 128-byte line
    for offs, oo in (([0] * n, 0), ([3] * n, 3), ([k % 5 for k in range(n)], 1), ([16] * n, 16), ([61] * n, 61)):
        placed = [Placed(c, o) for c, o in zip(contribs, offs)]
        out = Placed(np.zeros(size, np.uint16), oo)
        ls = record()
        zr.zr_reduce_slice_f16([p.view for p in placed], out.view, ls)
        assert out.guards_intact()
        assert_f16_equal(out.host(), ref, f"reduce f16 n={n} offsets {offs[:3]}")
        assert read_record(ls)[2] == 0


@pytest.mark.parametrize("n", [3, 8])   # 8: the 4-elements-per-lane kernel
def test_reduce_f16_extremes_subnormals_and_flag(n):
    device()
    rng = np.random.default_rng(4 + n)
    size = 9000
    # magnitudes across the whole fp16 range (below its largest value, planted
    # next), including subnormal means and 65504
    vals = [rng.choice([-1, 1], size) * 2.0 ** rng.uniform(-26, 15.99, size) for _ in range(n)]
    vals[0][:8] = [65504, -65504, 65504, 2.0 ** -24, -(2.0 ** -24), 0.0, -0.0, 2.0 ** -14]
    contribs = [f16(v) for v in vals]
    ls = record()
    out = torch.empty(size, dtype=torch.int16, device=device())
    zr.zr_reduce_slice_f16([torch.from_numpy(c.view(np.int16)).to(device()) for c in contribs], out, ls)
    assert_f16_equal(out.cpu().numpy().view(np.uint16), oracle.reduce_f16(contribs), "reduce f16 extremes")
    assert read_record(ls)[2] == 0
    # inf, -inf and NaN contributions at the head, the middle and the tail
    for pos, val in ((0, 0x7C00), (4444, 0xFC00), (size - 1, 0x7E01), (4445, 0x7C00)):
        bad = [c.copy() for c in contribs]
        bad[1][pos] = val
        ls = record()
        zr.zr_reduce_slice_f16([torch.from_numpy(c.view(np.int16)).to(device()) for c in bad], out, ls)
        ref = oracle.reduce_f16(bad)
        assert_f16_equal(out.cpu().numpy().view(np.uint16), ref, f"reduce f16 with {val:#x} at {pos}")
        assert read_record(ls)[2] == int(oracle.found_inf_f16(ref)) == 1


@pytest.mark.parametrize("size,pos", [(1, 0), (7, 6), (8, 3), (4099, 0), (4099, 4098), (4099, 2000),
                                      (100_003, 77_777)])
def test_check_finite(size, pos):
    device()
    g = f16(np.random.default_rng(size).normal(0, 100, size))
    for off in (0, 3, 40, 61):
        p = Placed(g, off)
        ls = record()
        zr.zr_check_finite_f16(p.view, ls)
        assert read_record(ls)[2] == 0
        bad = g.copy()
        bad[pos] = 0xFE00
        p = Placed(bad, off)
        zr.zr_check_finite_f16(p.view, ls)
        assert read_record(ls)[2] == 1


# ---------------------------------------------------------- scaled AdamW ----

def _state(n, seed):
    rng = np.random.default_rng(seed)
    return [rng.normal(0, 0.02, n).astype(np.float32), rng.normal(0, 1e-4, n).astype(np.float32),
            rng.uniform(0, 1e-6, n).astype(np.float32)]


@pytest.mark.parametrize("scale,step,offs", [(S0, 1, (0, 0)), (2.0 ** 10, 10, (0, 0)), (1.0, 3, (3, 1)),
                                             (2.0 ** 20, 1000, (1, 1)), (S0, 2, (2, 0)),
                                             # element offsets from a 128-byte line (heads up to 63)
                                             (S0, 4, (8, 8)), (S0, 5, (40, 40)), (S0, 6, (61, 61)),
                                             (S0, 7, (12, 8))])
def test_adamw_f16_matches_oracle(scale, step, offs):
    device()
    n = 50_003
    grad = scaled_contribs(1, n, int(scale) % 91 + step, scale)[0]
    st = _state(n, step)
    ref = [x.copy() for x in st]
    rp = np.zeros(n, np.uint16)
    oracle.adamw_f16(grad, *ref, rp, step=step, loss_scale=scale, **HP)
    go, so = offs
    pg, pp = Placed(grad, go), Placed(np.zeros(n, np.uint16), go)
    ps = [Placed(x, so) for x in st]
    ls = record(scale)
    zr.zr_adamw_step_f16(pg.view, *[p.view for p in ps], pp.view, ls, step=step, **HP)
    torch.cuda.synchronize()
    for name, p, want in zip(("master", "m", "v"), ps, ref):
        assert p.guards_intact()
        assert_fp32_exact(p.host(), want, f"adamw f16 {name} scale {scale}")
    assert_f16_within_1ulp(pp.host(), rp, "adamw f16 param")


def test_adamw_f16_skips_when_flagged():
    device()
    n = 10_007
    grad = scaled_contribs(1, n, 5)[0]
    st = _state(n, 5)
    ps = [Placed(x, 0) for x in st]
    pp = Placed(np.full(n, 0x1234, np.uint16), 0)
    ls = record()
    bad = torch.tensor([0x7C00], dtype=torch.int16, device=device())
    zr.zr_check_finite_f16(bad, ls)                       # set the flag
    zr.zr_adamw_step_f16(Placed(grad, 0).view, *[p.view for p in ps], pp.view, ls, step=1, **HP)
    torch.cuda.synchronize()
    for p, x in zip(ps, st):
        assert np.array_equal(p.host().view(np.uint32), x.view(np.uint32))
    assert np.all(pp.host() == 0x1234)


# ------------------------------------------------------------ scale rule ----

def test_loss_scale_rule_matches_oracle():
    device()
    window = 5
    ls = record(2.0 ** 4)
    ref = oracle.LossScale(initial=2.0 ** 4, window=window)
    bad = torch.tensor([0x7C00], dtype=torch.int16, device=device())
    pattern = [0, 0, 1, 0, 0, 0, 0, 0, 0, 0, 0, 0, 1, 1, 1, 1, 1, 0, 0, 0, 0, 0, 0] + [0] * 20
    for k, overflow in enumerate(pattern):
        if overflow:
            zr.zr_check_finite_f16(bad, ls)
        zr.zr_loss_scale_update(ls, window=window)
        ref.update(bool(overflow))
        scale, good, flag, skipped = read_record(ls)
        assert (scale, good, flag, skipped) == (ref.scale, ref.good_steps, 0, ref.skipped), k


def test_loss_scale_default_window_long_run():
    device()
    ls = record()
    ref = oracle.LossScale()
    bad = torch.tensor([0x7C00], dtype=torch.int16, device=device())
    for k in range(2600):
        overflow = k in (777, 1900)
        if overflow:
            zr.zr_check_finite_f16(bad, ls)
        zr.zr_loss_scale_update(ls)
        ref.update(overflow)
    scale, good, flag, skipped = read_record(ls)
    assert (scale, good, skipped) == (ref.scale, ref.good_steps, ref.skipped) == (2.0 ** 16 / 2 / 2 * 2, 699, 2)


# ------------------------------------------------------- whole sequences ----

def test_fp16_step_count_is_the_callers_after_a_skip():
    """The bias corrections use the step the caller passes: a skipped step
    does not move them by itself.  Clean step 1, an overflowed call 2 (skipped),
    then the third call twice from the same state: with step = 2, the count of
    applied steps (calls made minus the record's skipped count: the rule
    dynamic loss scaling usually follows, the optimizer step not advancing on a
    skip), and with step = 3, the count of calls.  Each equals the oracle's
    update with that step, and the two differ."""
    dev = device()
    n, size = 4, 30_001
    st = _state(size, 91)
    gpu = [torch.from_numpy(x.copy()).to(dev) for x in st]
    ref = [x.copy() for x in st]
    grad = torch.empty(size, dtype=torch.int16, device=dev)
    ls = record()
    scaler = oracle.LossScale()
    for call in (1, 2):
        contribs = scaled_contribs(n, size, 2000 + call, scaler.scale)
        if call == 2:
            contribs[1][7] = 0x7C00
        zr.zr_reduce_slice_f16([torch.from_numpy(c.view(np.int16)).to(dev) for c in contribs], grad, ls)
        zr.zr_adamw_step_f16(grad, *gpu, None, ls, step=call, **HP)
        zr.zr_loss_scale_update(ls)
        oracle.step_f16(contribs, *ref, None, scaler, step=call, **HP)
    _, _, _, skipped = read_record(ls)
    assert skipped == 1
    contribs = scaled_contribs(n, size, 2003, scaler.scale)
    results = {}
    for step in (3 - skipped, 3):
        g2 = [x.clone() for x in gpu]
        r2 = [x.copy() for x in ref]
        zr.zr_reduce_slice_f16([torch.from_numpy(c.view(np.int16)).to(dev) for c in contribs], grad, ls)
        zr.zr_adamw_step_f16(grad, *g2, None, ls, step=step, **HP)
        oracle.step_f16(contribs, *r2, None, oracle.LossScale(scaler.scale), step=step, **HP)
        for name, g, want in zip(("master", "m", "v"), g2, r2):
            assert_fp32_exact(g.cpu().numpy(), want, f"third call, step {step}: {name}")
        results[step] = g2[0].cpu().numpy()
    assert not np.array_equal(results[2], results[3])


def test_fp16_steps_with_planted_overflow_match_oracle():
    dev = device()
    n, size, steps = 4, 60_001, 7
    st = _state(size, 77)
    gpu = [torch.from_numpy(x.copy()).to(dev) for x in st]
    ref = [x.copy() for x in st]
    param = torch.zeros(size, dtype=torch.int16, device=dev)
    rparam = np.zeros(size, np.uint16)
    grad = torch.empty(size, dtype=torch.int16, device=dev)
    ls = record()
    scaler = oracle.LossScale()
    for t in range(1, steps + 1):
        contribs = scaled_contribs(n, size, 1000 + t, scaler.scale)
        if t == 3:
            contribs[2][size // 2] = 0x7C00               # an overflowed backward on one rank
        say("fp16 step", t, "scale", scaler.scale)
        zr.zr_reduce_slice_f16([torch.from_numpy(c.view(np.int16)).to(dev) for c in contribs], grad, ls)
        zr.zr_adamw_step_f16(grad, *gpu, param, ls, step=t, **HP)
        zr.zr_loss_scale_update(ls)
        o_grad = oracle.step_f16(contribs, *ref, rparam, scaler, step=t, **HP)
        assert_f16_equal(grad.cpu().numpy().view(np.uint16), o_grad, f"step {t} mean")
        for name, g, want in zip(("master", "m", "v"), gpu, ref):
            assert_fp32_exact(g.cpu().numpy(), want, f"step {t} {name}")
        assert_f16_within_1ulp(param.cpu().numpy().view(np.uint16), rparam, f"step {t} param")
        scale, good, flag, skipped = read_record(ls)
        assert (scale, good, skipped) == (scaler.scale, scaler.good_steps, scaler.skipped)
    assert scaler.skipped == 1 and scaler.scale == S0 / 2
