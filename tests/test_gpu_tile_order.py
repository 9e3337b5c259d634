"""The streaming kernels take their tiles in runs per XCD: a launch of G
workgroups works in rounds of G tiles, and within a round, groups of 8R
consecutive tiles go to the 8 XCDs R at a time (XCD x takes tiles xR ...
xR + R - 1 of each group, or for the means of up to 8 contributions the slot
rotated by the group's index); the round's last, partial group is in launch
order.  The sizes here span several full groups and a ragged partial one for
each kernel that uses such runs (AdamW, the means of up to 8 contributions,
the fused reduce + AdamW, the fp16 mean, finite check and AdamW, the
quantizers and dequantizers), so every part of the order runs: each output
must equal the oracle's bit for bit, and stay the same with the grid capped at
one full group plus a few workgroups (rounds that mix both parts, and rounds
of launch order only), with nothing written outside the buffers."""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_optimizer_zr_amd as zr
from gpu_util import Placed, assert_bits_equal, device, say
from zr_workloads import synth

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)

# Tiles per workgroup: AdamW, the 4-per-lane means and the fused kernel take
# 1024 elements, the 8-per-lane means and the finite check 2048, the
# quantizers 4 x 2048.  Runs of 256 (64 for the quantizers) make groups of
# 2048 (512) workgroups.
N_1024 = 2 * 2048 * 1024 + 777 * 1024 + 333  # two full groups, a partial one, a ragged tail
N_2048 = 2 * 2048 * 2048 + 300 * 2048 + 5
N_QUANT = 2 * 512 * 8192 + 123 * 8192 + 4321
CAPS = ["2056", "520"]  # one group of 2048 (or 4 of 512) plus 8 workgroups; one of 512 plus 8


def bf16(n, std, seed):
    return synth.normal_bf16(n, std, seed).view(torch.int16).numpy().view(np.uint16).copy()


def f32(n, std, seed):
    return synth.normal_f32(n, std, seed).numpy().copy()


def outputs(placed):
    torch.cuda.synchronize()
    for p in placed:
        assert p.guards_intact(), "write outside the buffer"
    return [p.host() for p in placed]


def full_and_capped(monkeypatch, run, refs, what):
    """run() -> host arrays; equal to refs with the full grid and with each cap."""
    monkeypatch.delenv("ZR_MAX_GRID", raising=False)
    for cap in [None] + CAPS:
        if cap is not None:
            monkeypatch.setenv("ZR_MAX_GRID", cap)
        say(what, "grid cap", cap)
        got = run()
        for k, (a, b) in enumerate(zip(got, refs)):
            assert_bits_equal(a, b, f"{what} output {k} (grid cap {cap})")
    monkeypatch.delenv("ZR_MAX_GRID", raising=False)


def _adamw_case(n, seed):
    g = bf16(n, 1e-3, seed)
    th, m = f32(n, 0.02, seed + 1), f32(n, 1e-4, seed + 2)
    v = np.abs(f32(n, 1e-6, seed + 3))
    return g, th, m, v


def test_adamw_runs(monkeypatch):
    device()
    n = N_1024
    g, th, m, v = _adamw_case(n, 100)
    rt, rm, rv, rp = th.copy(), m.copy(), v.copy(), np.zeros(n, np.uint16)
    oracle.adamw(g, rt, rm, rv, rp, step=7, **HP)

    def run():
        pg, pt, pm, pv = Placed(g, 0), Placed(th, 0), Placed(m, 0), Placed(v, 0)
        pp = Placed(np.zeros(n, np.uint16), 0)
        zr.zr_adamw_step(pg.view, pt.view, pm.view, pv.view, pp.view, step=7, **HP)
        return outputs([pt, pm, pv, pp])

    full_and_capped(monkeypatch, run, [rt, rm, rv, rp], "adamw")


@pytest.mark.parametrize("n_contrib,size", [(4, N_2048), (6, N_2048), (8, N_1024), (7, N_1024 + 1)])
def test_reduce_runs(monkeypatch, n_contrib, size):
    device()
    cs = [bf16(size, 1e-3, 200 + k) for k in range(n_contrib)]
    ref = oracle.reduce(cs)

    def run():
        pc = [Placed(c, 0) for c in cs]
        out = Placed(np.zeros(size, np.uint16), 0)
        zr.zr_reduce_slice([p.view for p in pc], out.view)
        return outputs([out])

    full_and_capped(monkeypatch, run, [ref], f"reduce n={n_contrib}")


@pytest.mark.parametrize("n_contrib", [4, 16])
def test_fused_runs(monkeypatch, n_contrib):
    device()
    n = N_1024
    cs = [bf16(n, 1e-3, 300 + k) for k in range(n_contrib)]
    _, th, m, v = _adamw_case(n, 310)
    mean = oracle.reduce(cs)
    rt, rm, rv, rp = th.copy(), m.copy(), v.copy(), np.zeros(n, np.uint16)
    oracle.adamw(mean, rt, rm, rv, rp, step=3, **HP)

    def run():
        pc = [Placed(c, 0) for c in cs]
        pt, pm, pv = Placed(th, 0), Placed(m, 0), Placed(v, 0)
        pp, pg = Placed(np.zeros(n, np.uint16), 0), Placed(np.zeros(n, np.uint16), 0)
        zr.zr_reduce_adamw_step([p.view for p in pc], pt.view, pm.view, pv.view, pp.view, pg.view, step=3, **HP)
        return outputs([pt, pm, pv, pp, pg])

    full_and_capped(monkeypatch, run, [rt, rm, rv, rp, mean], f"fused n={n_contrib}")


def _f16(n, std, seed):
    return synth.normal_f32(n, std, seed).to(torch.float16).view(torch.int16).numpy().view(np.uint16).copy()


@pytest.mark.parametrize("n_contrib,size", [(4, N_2048), (8, N_1024)])
def test_fp16_mean_and_adamw_runs(monkeypatch, n_contrib, size):
    dev = device()
    scale = 2.0 ** 12
    cs = [_f16(size, 1e-3 * scale, 400 + k) for k in range(n_contrib)]
    mean = oracle.reduce_f16(cs)
    assert not oracle.found_inf_f16(mean)
    _, th, m, v = _adamw_case(size, 410)
    rt, rm, rv, rp = th.copy(), m.copy(), v.copy(), np.zeros(size, np.uint16)
    oracle.adamw_f16(mean, rt, rm, rv, rp, step=5, loss_scale=scale, **HP)

    def run():
        ls = zr.loss_scale_record(dev)
        zr.zr_loss_scale_init(ls, scale)
        pc = [Placed(c, 0) for c in cs]
        g = Placed(np.zeros(size, np.uint16), 0)
        pt, pm, pv = Placed(th, 0), Placed(m, 0), Placed(v, 0)
        pp = Placed(np.zeros(size, np.uint16), 0)
        zr.zr_reduce_slice_f16([p.view for p in pc], g.view, ls)
        zr.zr_check_finite_f16(g.view, ls)
        zr.zr_adamw_step_f16(g.view, pt.view, pm.view, pv.view, pp.view, ls, step=5, **HP)
        out = outputs([g, pt, pm, pv, pp])
        assert int(ls.cpu()[2]) == 0, "overflow flag set on finite data"
        return out

    full_and_capped(monkeypatch, run, [mean, rt, rm, rv, rp], f"fp16 n={n_contrib}")


@pytest.mark.parametrize("where", ["full group", "partial group", "tail"])
def test_check_finite_runs(monkeypatch, where):
    """One inf in a tile of a full run group, of the partial group, or in the
    element-wise tail: the flag is set every time, whatever the grid."""
    dev = device()
    n = N_2048
    x = _f16(n, 1.0, 500)
    pos = {"full group": 2048 * 2048 + 5 * 2048 + 77, "partial group": 2 * 2048 * 2048 + 299 * 2048 + 1,
           "tail": n - 2}[where]
    x[pos] = 0x7C00
    monkeypatch.delenv("ZR_MAX_GRID", raising=False)
    for cap in [None] + CAPS:
        if cap is not None:
            monkeypatch.setenv("ZR_MAX_GRID", cap)
        ls = zr.loss_scale_record(dev)
        zr.zr_loss_scale_init(ls, 1.0)
        g = Placed(x, 0)
        zr.zr_check_finite_f16(g.view, ls)
        torch.cuda.synchronize()
        assert int(ls.cpu()[2]) == 1, f"inf at {pos} ({where}) not flagged with grid cap {cap}"
    monkeypatch.delenv("ZR_MAX_GRID", raising=False)


@pytest.mark.parametrize("bits", [8, 4])
def test_quantize_dequantize_runs(monkeypatch, bits):
    device()
    n, block = N_QUANT, 2048
    x = bf16(n, 0.02, 600 + bits)
    nb = -(-n // block)
    if bits == 8:
        rq, rs = oracle.quantize_int8(x, block)
        rback = oracle.dequantize_int8(rq, rs, block)
    else:
        rq, rs = oracle.quantize_int4(x, block)
        rback = oracle.dequantize_int4(rq, rs, n, block)

    def run():
        src = Placed(x, 0)
        q = Placed(np.zeros(n if bits == 8 else -(-n // 2), np.int8 if bits == 8 else np.uint8), 0)
        sc = Placed(np.zeros(nb, np.float32), 0)
        back = Placed(np.zeros(n, np.uint16), 0)
        if bits == 8:
            zr.zr_quantize_int8(src.view, q.view, sc.view, block=block)
            zr.zr_dequantize_int8(q.view, sc.view, back.view, block=block)
        else:
            zr.zr_quantize_int4(src.view, q.view, sc.view, block=block)
            zr.zr_dequantize_int4(q.view, sc.view, back.view, block=block)
        return outputs([q, sc, back])

    full_and_capped(monkeypatch, run, [rq, rs, rback], f"int{bits} codec")
