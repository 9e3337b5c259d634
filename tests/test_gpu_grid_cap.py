"""Results do not depend on the grid: with ZR_MAX_GRID capping every launch at
a few workgroups, each kernel loops over the work its grid does not cover and
must give the same bits as with a full grid, and write nothing outside its
buffers.  The full-grid results are checked against the oracle by the other
GPU tests; here every kernel family runs both ways on the same inputs: AdamW
(vector and element-wise paths), the reduce (XCD-ordered n <= 8, default order
n > 8, element-wise), the fused reduce + AdamW, the fp16 mean, finite check and
AdamW, the int8 and int4 quantizers and dequantizers (vector and element-wise), the
dequantize-on-unpack of both and the pack/unpack copy kernel."""
import numpy as np
import pytest
import torch

import zero_sharded_optimizer_zr_amd as zr
from gpu_util import Placed, assert_bits_equal, device, say
from zr_workloads import synth

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
CAPS = ["8", "24"]


def both_ways(monkeypatch, run):
    """run() -> list of host arrays; once with the full grid, then with each cap."""
    monkeypatch.delenv("ZR_MAX_GRID", raising=False)
    full = run()
    for cap in CAPS:
        monkeypatch.setenv("ZR_MAX_GRID", cap)
        say("grid cap", cap)
        got = run()
        for k, (a, b) in enumerate(zip(got, full)):
            assert_bits_equal(a, b, f"output {k} with ZR_MAX_GRID={cap}")
    monkeypatch.delenv("ZR_MAX_GRID", raising=False)


def bf16(n, std, seed):
    return synth.normal_bf16(n, std, seed).view(torch.int16).numpy().view(np.uint16).copy()


def f32(n, std, seed):
    return synth.normal_f32(n, std, seed).numpy().copy()


def outputs(placed):
    torch.cuda.synchronize()
    for p in placed:
        assert p.guards_intact(), "write outside the buffer"
    return [p.host() for p in placed]


@pytest.mark.parametrize("off", [0, 1])  # 1: inconsistent phases, the element-wise kernel
def test_adamw(monkeypatch, off):
    device()
    n = 1_000_003
    g, th, m = bf16(n, 1e-3, 1), f32(n, 0.02, 2), f32(n, 1e-4, 3)
    v = np.abs(f32(n, 1e-6, 4))

    def run():
        pg, pt, pm, pv = Placed(g, 0), Placed(th, off), Placed(m, 0), Placed(v, 0)
        pp = Placed(np.zeros(n, np.uint16), 0)
        zr.zr_adamw_step(pg.view, pt.view, pm.view, pv.view, pp.view, step=5, **HP)
        return outputs([pt, pm, pv, pp])

    both_ways(monkeypatch, run)


@pytest.mark.parametrize("n_contrib,off", [(4, 0), (8, 0), (9, 0), (4, 1)])
def test_reduce(monkeypatch, n_contrib, off):
    device()
    n = 700_001
    cs = [bf16(n, 1e-3, 10 + k) for k in range(n_contrib)]

    def run():
        pc = [Placed(c, off if k == 1 else 0) for k, c in enumerate(cs)]
        out = Placed(np.zeros(n, np.uint16), 0)
        zr.zr_reduce_slice([p.view for p in pc], out.view)
        return outputs([out])

    both_ways(monkeypatch, run)


@pytest.mark.parametrize("n_contrib", [4, 9, 33])
def test_fused(monkeypatch, n_contrib):
    device()
    n = 600_007
    cs = [bf16(n, 1e-3, 20 + k) for k in range(n_contrib)]
    th, m = f32(n, 0.02, 30), f32(n, 1e-4, 31)
    v = np.abs(f32(n, 1e-6, 32))

    def run():
        pc = [Placed(c, 0) for c in cs]
        pt, pm, pv = Placed(th, 0), Placed(m, 0), Placed(v, 0)
        pp, pg = Placed(np.zeros(n, np.uint16), 0), Placed(np.zeros(n, np.uint16), 0)
        zr.zr_reduce_adamw_step([p.view for p in pc], pt.view, pm.view, pv.view, pp.view, pg.view, step=2, **HP)
        return outputs([pt, pm, pv, pp, pg])

    both_ways(monkeypatch, run)


def test_fp16_path(monkeypatch):
    dev = device()
    n = 500_009
    scale = 2.0 ** 12
    cs = [(synth.normal_f32(n, 1e-3 * scale, 40 + k).to(torch.float16)).view(torch.int16).numpy().view(np.uint16).copy()
          for k in range(4)]
    th, m = f32(n, 0.02, 41), f32(n, 1e-4, 42)
    v = np.abs(f32(n, 1e-6, 43))

    def run():
        ls = zr.loss_scale_record(dev)
        zr.zr_loss_scale_init(ls, scale)
        pc = [Placed(c, 0) for c in cs]
        g = Placed(np.zeros(n, np.uint16), 0)
        pt, pm, pv = Placed(th, 0), Placed(m, 0), Placed(v, 0)
        pp = Placed(np.zeros(n, np.uint16), 0)
        zr.zr_reduce_slice_f16([p.view for p in pc], g.view, ls)
        zr.zr_check_finite_f16(g.view, ls)
        zr.zr_adamw_step_f16(g.view, pt.view, pm.view, pv.view, pp.view, ls, step=4, **HP)
        torch.cuda.synchronize()
        return outputs([g, pt, pm, pv, pp]) + [ls.cpu().numpy().view(np.uint32).copy()]

    both_ways(monkeypatch, run)


@pytest.mark.parametrize("block,off", [(256, 0), (2048, 0), (512, 1)])  # off 1: element-wise kernels
def test_int8_codec(monkeypatch, block, off):
    device()
    n = 900_001
    x = bf16(n, 0.02, 50)
    nb = -(-n // block)

    def run():
        src = Placed(x, off)
        q = Placed(np.zeros(n, np.int8), off)
        sc = Placed(np.zeros(nb, np.float32), 0)
        zr.zr_quantize_int8(src.view, q.view, sc.view, block=block)
        back = Placed(np.zeros(n, np.uint16), off)
        zr.zr_dequantize_int8(q.view, sc.view, back.view, block=block)
        return outputs([q, sc, back])

    both_ways(monkeypatch, run)


@pytest.mark.parametrize("block,off", [(256, 0), (2048, 0), (512, 2)])  # off 2: element-wise kernels
def test_int4_codec(monkeypatch, block, off):
    device()
    n = 900_001
    x = bf16(n, 0.02, 51)
    nb = -(-n // block)

    def run():
        src = Placed(x, off)
        q = Placed(np.zeros(-(-n // 2), np.uint8), off)
        sc = Placed(np.zeros(nb, np.float32), 0)
        zr.zr_quantize_int4(src.view, q.view, sc.view, block=block)
        back = Placed(np.zeros(n, np.uint16), off)
        zr.zr_dequantize_int4(q.view, sc.view, back.view, block=block)
        return outputs([q, sc, back])

    both_ways(monkeypatch, run)


def _many_tensors():
    """30 tensors, two of them persistent: 30 descriptors in one unpack launch
    (the int4 unpack's launch-order kernel)."""
    numels = [int(x) for x in np.random.default_rng(64).integers(100_001, 160_000, 30)]
    numels[5], numels[11] = 7, 99_999
    return numels


@pytest.mark.parametrize("numels", [[300_001, 7, 250_013, 123_457, 99_999, 400_003], _many_tensors()],
                         ids=["six_tensors", "thirty_tensors"])
def test_copy_and_unpack_int8(monkeypatch, numels):
    dev = device()
    lay = zr.zr_layout_create(numels, 3, 100_000)
    info = zr.zr_layout_query(lay)
    psi_pad, S = info["psi_pad"], info["shard"]
    views_host = [synth.random_bits16(x, 60 + t).numpy().view(np.uint16).copy() for t, x in enumerate(numels)]
    block = 1024
    per_rank = -(-S // block)
    codes = np.random.default_rng(61).integers(-127, 128, psi_pad).astype(np.int8)
    scales = np.abs(np.random.default_rng(62).normal(0, 1e-3, 3 * per_rank)).astype(np.float32)
    persistent = [zr.zr_layout_tensor(lay, t)[0] for t in range(len(numels))]
    codes4 = np.random.default_rng(63).integers(0, 256, 3 * -(-S // 2)).astype(np.uint8)
    codes4[(codes4 & 0xF) == 8] ^= 1                     # no -8 codes
    codes4[(codes4 >> 4) == 8] ^= 0x10

    def run():
        views = [None if persistent[t] else Placed(views_host[t], t % 3) for t in range(len(numels))]
        flat = Placed(np.zeros(psi_pad, np.uint16), 5)
        zr.zr_pack(lay, [None if p is None else p.view for p in views], flat.view, 0, psi_pad)
        back = [None if persistent[t] else Placed(np.zeros(numels[t], np.uint16), 1) for t in range(len(numels))]
        zr.zr_unpack(lay, flat.view, 0, psi_pad, [None if p is None else p.view for p in back])
        deq = [None if persistent[t] else Placed(np.zeros(numels[t], np.uint16), 2) for t in range(len(numels))]
        q = torch.from_numpy(codes).to(dev)
        sc = torch.from_numpy(scales).to(dev)
        zr.zr_unpack_int8(lay, q, sc, 0, psi_pad, [None if p is None else p.view for p in deq], block=block)
        deq4 = [None if persistent[t] else Placed(np.zeros(numels[t], np.uint16), 3) for t in range(len(numels))]
        q4 = torch.from_numpy(codes4).to(dev)
        zr.zr_unpack_int4(lay, q4, sc, 0, psi_pad, [None if p is None else p.view for p in deq4], block=block)
        return outputs([flat] + [p for p in back + deq + deq4 if p is not None])

    both_ways(monkeypatch, run)
