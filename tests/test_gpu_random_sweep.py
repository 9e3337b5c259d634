"""Seeded random sweep: sizes from 1 to 3e5 elements, and every buffer placed
at its own element offset (0 to 63), so each case mixes 128-byte line phases
and 16-, 8- and 4-byte alignments the way slices of larger buffers do.  For
AdamW, the mean, the fused reduce + AdamW, the fp16 mean and AdamW, and the
int8 and int4 codecs, every output must equal the oracle's bit for bit (the
vector body, the line-head peel and the element-wise fallback all give the same
bits), and nothing may be written outside the buffers.  Each case names its
seed, size and offsets before it runs."""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_optimizer_zr_amd as zr
from gpu_util import Placed, assert_bits_equal, device, say
from zr_workloads import synth

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
SEEDS = range(24)


def _size(rng):
    return int(np.exp(rng.uniform(0.0, np.log(3e5))))


def _offs(rng, k):
    return [int(x) for x in rng.integers(0, 64, k)]


def _bf16(n, std, seed):
    return synth.normal_bf16(n, std, seed).view(torch.int16).numpy().view(np.uint16).copy()


def _f16(n, std, seed):
    return synth.normal_f32(n, std, seed).to(torch.float16).view(torch.int16).numpy().view(np.uint16).copy()


def _state(n, seed):
    th = synth.normal_f32(n, 0.02, seed).numpy().copy()
    m = synth.normal_f32(n, 1e-4, seed + 1).numpy().copy()
    v = np.abs(synth.normal_f32(n, 1e-6, seed + 2).numpy()).copy()
    return th, m, v


def _outputs(placed):
    torch.cuda.synchronize()
    for p in placed:
        assert p.guards_intact(), "write outside the buffer"
    return [p.host() for p in placed]


def _check(got, refs, what):
    for k, (a, b) in enumerate(zip(got, refs)):
        assert_bits_equal(a, b, f"{what}: output {k}")


@pytest.mark.parametrize("seed", SEEDS)
def test_adamw_random(seed):
    device()
    rng = np.random.default_rng(1000 + seed)
    n, o = _size(rng), _offs(rng, 5)
    step = int(rng.integers(1, 2000))
    say("adamw seed", seed, "n", n, "offsets", o, "step", step)
    g = _bf16(n, 1e-3, 10 * seed)
    th, m, v = _state(n, 10 * seed + 1)
    rt, rm, rv, rp = th.copy(), m.copy(), v.copy(), np.zeros(n, np.uint16)
    oracle.adamw(g, rt, rm, rv, rp, step=step, **HP)
    pg, pt, pm, pv = Placed(g, o[0]), Placed(th, o[1]), Placed(m, o[2]), Placed(v, o[3])
    pp = Placed(np.zeros(n, np.uint16), o[4])
    zr.zr_adamw_step(pg.view, pt.view, pm.view, pv.view, pp.view, step=step, **HP)
    _check(_outputs([pt, pm, pv, pp, pg]), [rt, rm, rv, rp, g], f"adamw seed {seed}")


@pytest.mark.parametrize("seed", SEEDS)
def test_reduce_random(seed):
    device()
    rng = np.random.default_rng(2000 + seed)
    n = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 16, 33, 64]))
    size, o = _size(rng), _offs(rng, n + 1)
    say("reduce seed", seed, "n", n, "size", size, "offsets", o)
    cs = [_bf16(size, 1e-3, 100 * seed + k) for k in range(n)]
    ref = oracle.reduce(cs)
    pc = [Placed(c, o[k]) for k, c in enumerate(cs)]
    out = Placed(np.zeros(size, np.uint16), o[n])
    zr.zr_reduce_slice([p.view for p in pc], out.view)
    _check(_outputs(pc + [out]), cs + [ref], f"reduce seed {seed}")


@pytest.mark.parametrize("seed", SEEDS)
def test_fused_random(seed):
    device()
    rng = np.random.default_rng(3000 + seed)
    n = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 9, 16, 24, 25, 40]))
    size, o = _size(rng), _offs(rng, n + 5)
    step = int(rng.integers(1, 500))
    say("fused seed", seed, "n", n, "size", size, "offsets", o, "step", step)
    cs = [_bf16(size, 1e-3, 200 * seed + k) for k in range(n)]
    th, m, v = _state(size, 200 * seed + 100)
    mean = oracle.reduce(cs)
    rt, rm, rv, rp = th.copy(), m.copy(), v.copy(), np.zeros(size, np.uint16)
    oracle.adamw(mean, rt, rm, rv, rp, step=step, **HP)
    pc = [Placed(c, o[k]) for k, c in enumerate(cs)]
    pt, pm, pv = Placed(th, o[n]), Placed(m, o[n + 1]), Placed(v, o[n + 2])
    pp, pg = Placed(np.zeros(size, np.uint16), o[n + 3]), Placed(np.zeros(size, np.uint16), o[n + 4])
    zr.zr_reduce_adamw_step([p.view for p in pc], pt.view, pm.view, pv.view, pp.view, pg.view, step=step, **HP)
    _check(_outputs([pt, pm, pv, pp, pg]), [rt, rm, rv, rp, mean], f"fused seed {seed}")


@pytest.mark.parametrize("seed", SEEDS)
def test_fp16_mean_and_adamw_random(seed):
    dev = device()
    rng = np.random.default_rng(4000 + seed)
    n = int(rng.choice([1, 2, 4, 5, 7, 8, 9, 16]))
    size, o = _size(rng), _offs(rng, n + 5)
    scale = float(2.0 ** int(rng.integers(0, 17)))
    step = int(rng.integers(1, 500))
    say("fp16 seed", seed, "n", n, "size", size, "offsets", o, "scale", scale, "step", step)
    cs = [_f16(size, 1e-3 * min(scale, 2.0 ** 12), 300 * seed + k) for k in range(n)]
    mean = oracle.reduce_f16(cs)
    inf = oracle.found_inf_f16(mean)
    th, m, v = _state(size, 300 * seed + 100)
    rt, rm, rv, rp = th.copy(), m.copy(), v.copy(), np.zeros(size, np.uint16)
    if not inf:
        oracle.adamw_f16(mean, rt, rm, rv, rp, step=step, loss_scale=scale, **HP)
    ls = zr.loss_scale_record(dev)
    zr.zr_loss_scale_init(ls, scale)
    pc = [Placed(c, o[k]) for k, c in enumerate(cs)]
    pg = Placed(np.zeros(size, np.uint16), o[n])
    pt, pm, pv = Placed(th, o[n + 1]), Placed(m, o[n + 2]), Placed(v, o[n + 3])
    pp = Placed(np.zeros(size, np.uint16), o[n + 4])
    zr.zr_reduce_slice_f16([p.view for p in pc], pg.view, ls)
    zr.zr_adamw_step_f16(pg.view, pt.view, pm.view, pv.view, pp.view, ls, step=step, **HP)
    got = _outputs([pg, pt, pm, pv, pp])
    assert int(ls.cpu()[2]) == int(inf), "overflow flag differs from the oracle's"
    _check(got, [mean, rt, rm, rv, rp], f"fp16 seed {seed}")


@pytest.mark.parametrize("seed", SEEDS)
def test_codecs_random(seed):
    device()
    rng = np.random.default_rng(5000 + seed)
    bits = 8 if seed % 2 == 0 else 4
    block = int(rng.choice([256, 512, 1024, 2048]))
    n, o = _size(rng), _offs(rng, 4)
    say("codec seed", seed, "int", bits, "block", block, "n", n, "offsets", o)
    x = _bf16(n, float(np.exp(rng.uniform(np.log(1e-4), np.log(10.0)))), 400 * seed)
    nb = -(-n // block)
    if bits == 8:
        rq, rs = oracle.quantize_int8(x, block)
        rb = oracle.dequantize_int8(rq, rs, block)
        q = Placed(np.zeros(n, np.int8), o[1])
    else:
        rq, rs = oracle.quantize_int4(x, block)
        rb = oracle.dequantize_int4(rq, rs, n, block)
        q = Placed(np.zeros(-(-n // 2), np.uint8), o[1])
    src = Placed(x, o[0])
    sc = Placed(np.zeros(nb, np.float32), o[2])
    back = Placed(np.zeros(n, np.uint16), o[3])
    if bits == 8:
        zr.zr_quantize_int8(src.view, q.view, sc.view, block=block)
        zr.zr_dequantize_int8(q.view, sc.view, back.view, block=block)
    else:
        zr.zr_quantize_int4(src.view, q.view, sc.view, block=block)
        zr.zr_dequantize_int4(q.view, sc.view, back.view, block=block)
    _check(_outputs([q, sc, back, src]), [rq, rs, rb, x], f"int{bits} codec seed {seed}")
