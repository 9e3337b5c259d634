"""GPU parity of each kernel against the oracle through the C ABI, at sizes the
oracle finishes in seconds: several tiles, ragged tails, odd base offsets
(head/tail peel and the unaligned fallback), guard bands, in-place use, and
the invariants (shard concatenation, ReduceScatter slice = AllReduce slice,
bit-identical results on every code path)."""
import random

import numpy as np
import pytest
import torch

import oracle
import zero_sharded_optimizer_zr_amd as zr
from gpu_util import (Placed, assert_bf16_exact, assert_bits_equal, assert_fp32_exact, device, f32, say,
                      u16)
from zr_workloads import TINY_MLP, synth

pytestmark = pytest.mark.gpu

HP = dict(lr=5e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _bits(x: torch.Tensor) -> np.ndarray:
    return x.view(torch.int16).numpy().view(np.uint16).copy()


def _adamw_inputs(n, seed, m_std=1e-4, v_high=1e-6):
    g = _bits(synth.normal_bf16(n, 1e-3, seed))
    master = synth.normal_f32(n, 0.02, seed + 1).numpy()
    m = synth.normal_f32(n, m_std, seed + 2).numpy()
    v = synth.uniform_f32(n, v_high, seed + 3).numpy()
    return g, master, m, v


def _adamw_gpu(g, master, m, v, step, offsets=(0, 0, 0, 0, 0), with_param=True, hp=HP, grad_scale=1.0):
    pg = Placed(g, offsets[0])
    pt, pm, pv = Placed(master, offsets[1]), Placed(m, offsets[2]), Placed(v, offsets[3])
    pp = Placed(np.zeros(g.size, np.uint16), offsets[4]) if with_param else None
    zr.zr_adamw_step(pg.view, pt.view, pm.view, pv.view, pp.view if pp else None, step=step,
                     grad_scale=grad_scale, **hp)
    torch.cuda.synchronize()
    for p in (pg, pt, pm, pv, pp):
        assert p is None or p.guards_intact(), "write outside the buffer"
    assert np.array_equal(pg.host(), g), "gradient modified"
    return pt.host(), pm.host(), pv.host(), (pp.host() if pp else None)


def _adamw_ref(g, master, m, v, step, with_param=True, hp=HP, grad_scale=1.0):
    t, mm, vv = master.copy(), m.copy(), v.copy()
    p = np.zeros(g.size, np.uint16) if with_param else None
    oracle.adamw(g, t, mm, vv, p, step=step, grad_scale=grad_scale, **hp)
    return t, mm, vv, p


def _check_adamw(got, ref, what):
    for name, a, b in zip(("master", "exp_avg", "exp_avg_sq"), got[:3], ref[:3]):
        assert_fp32_exact(a, b, f"{what} {name}")
    if ref[3] is not None:
        assert_bf16_exact(got[3], ref[3], f"{what} param")


# ------------------------------------------------------------------ AdamW ----

@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 255, 2048 + 13, 300_001])
def test_adamw_sizes(n):
    device()
    say("adamw n =", n)
    g, master, m, v = _adamw_inputs(n, 100 + n)
    got = _adamw_gpu(g, master, m, v, step=10)
    _check_adamw(got, _adamw_ref(g, master, m, v, 10), f"adamw n={n}")


def _cancellation_inputs(n, seed):
    """Step-1 inputs whose update nearly cancels the decayed master: theta *
    (1 - lr wd) equals lr * g / (|g| + eps) up to ~1e-12, so the new master is
    within a few 1e-10 of zero.  An fp32 evaluation of the update is off by
    many bf16 ulps there; the kernels' double evaluation is exact."""
    rng = np.random.default_rng(seed)
    g = oracle.bf16_from_f32(rng.choice([-1.0, 1.0], n).astype(np.float32) * np.float32(1e-3))
    gf = oracle.f32_from_bf16(g).astype(np.float64)
    target = HP["lr"] * gf / (np.abs(gf) + HP["eps"]) / (1.0 - HP["lr"] * HP["weight_decay"])
    master = (target + rng.normal(0, 1e-12, n)).astype(np.float32)
    return g, master, np.zeros(n, np.float32), np.zeros(n, np.float32)


def test_adamw_near_total_cancellation():
    device()
    g, master, m, v = _cancellation_inputs(65_536 + 5, 9)
    ref = _adamw_ref(g, master, m, v, 1)
    assert np.median(np.abs(ref[0])) < 1e-9
    for offsets in ((0, 0, 0, 0, 0), (1, 0, 0, 0, 1)):     # vector body; element-wise fallback
        _check_adamw(_adamw_gpu(g, master, m, v, step=1, offsets=offsets), ref, f"cancellation {offsets}")
    # the fused call, one contribution equal to g (its mean is g itself), and 33
    # (the two-pass schedule)
    for n in (1, 4, 33):
        pc = [Placed(g, 0) for _ in range(n)]
        pt, pm, pv = Placed(master, 0), Placed(m, 0), Placed(v, 0)
        pp = Placed(np.zeros(g.size, np.uint16), 0)
        zr.zr_reduce_adamw_step([p.view for p in pc], pt.view, pm.view, pv.view, pp.view, step=1, **HP)
        torch.cuda.synchronize()
        _check_adamw((pt.host(), pm.host(), pv.host(), pp.host()), ref, f"fused cancellation n={n}")


# (grad, master, m, v, param) element offsets: aligned; consistent head peel;
# inconsistent phases that force the element-wise fallback
OFFSETS = [(0, 0, 0, 0, 0), (3, 3, 3, 3, 3), (5, 1, 1, 1, 5), (1, 0, 0, 0, 1), (0, 1, 2, 3, 0), (0, 0, 0, 0, 4),
           (7, 3, 7, 11, 15)]


def test_adamw_every_path_gives_the_same_bits():
    device()
    n = 50_000 + 11
    g, master, m, v = _adamw_inputs(n, 7)
    ref = _adamw_ref(g, master, m, v, 3)
    base = None
    for off in OFFSETS:
        say("adamw offsets", off)
        got = _adamw_gpu(g, master, m, v, step=3, offsets=off)
        _check_adamw(got, ref, f"adamw offsets {off}")
        if base is None:
            base = got
        else:
            for a, b, name in zip(got, base, ("master", "m", "v", "param")):
                assert_bits_equal(a, b, f"path {off} vs aligned: {name}")


# (grad, master, m, v, param) element offsets from a 128-byte line: every array
# sliced at one offset (heads of 56, 24 or 20 elements that put the fp32 and the
# bf16 arrays on lines together, and 61 that puts them on lines at 3), and bf16
# arrays at another phase than the fp32 ones (the head follows master alone).
LINE_OFFSETS = [(8, 8, 8, 8, 8), (12, 12, 12, 12, 12), (40, 40, 40, 40, 40), (61, 61, 61, 61, 61),
                (12, 8, 8, 8, 12), (4, 24, 24, 24, 36)]


@pytest.mark.parametrize("n", [1, 50, 63, 64, 65, 200, 4099, 50_011])
def test_adamw_line_heads(n):
    """The vector body starts where master (and, when one index does both, the
    gradient) starts a 128-byte line: heads of up to 63 elements, done
    element-wise with the tail, at every length from all-element-wise up."""
    device()
    g, master, m, v = _adamw_inputs(n, 41 + n)
    ref = _adamw_ref(g, master, m, v, 6)
    for off in LINE_OFFSETS:
        _check_adamw(_adamw_gpu(g, master, m, v, step=6, offsets=off), ref, f"adamw n={n} offsets {off}")


@pytest.mark.parametrize("step,hp,scale,m_std,v_high", [
    (1, HP, 1.0, 0.0, 0.0),
    (1000, dict(HP, lr=1e-4, weight_decay=0.1), 1.0, 1e-4, 1e-6),
    (4, HP, 0.125, 1e-4, 1e-6),
    (9, dict(lr=1e-3, beta1=0.0, beta2=0.0, eps=1e-6, weight_decay=0.0), 1.0, 1e-4, 1e-6),
    (3, dict(HP, lr=0.0), 1.0, 1e-4, 1e-6),                                # no update, no decay
    (10**9, HP, 1.0, 1e-4, 1e-6),                                          # bias corrections at 1
    (2, dict(HP, beta1=0.999, beta2=0.999999), 1.0, 1e-4, 1e-6),          # long averages
    (5, HP, -2.0, 1e-4, 1e-6),                                             # negative gradient scale
    (5, HP, 0.0, 1e-4, 1e-6),                                              # zero gradient scale
    (7, dict(HP, eps=1.0, weight_decay=1.0), 1.0, 1e-4, 1e-6),            # large eps and decay
])
def test_adamw_hyperparameters(step, hp, scale, m_std, v_high):
    device()
    say("adamw step", step, "scale", scale)
    g, master, m, v = _adamw_inputs(100_003, step, m_std, v_high)
    got = _adamw_gpu(g, master, m, v, step=step, hp=hp, grad_scale=scale)
    _check_adamw(got, _adamw_ref(g, master, m, v, step, hp=hp, grad_scale=scale), f"adamw step {step}")


def test_adamw_without_param_copy():
    device()
    g, master, m, v = _adamw_inputs(4099, 3)
    got = _adamw_gpu(g, master, m, v, step=2, with_param=False)
    _check_adamw(got, _adamw_ref(g, master, m, v, 2, with_param=False), "adamw no param")


def test_adamw_shards_concatenate_bit_exactly():
    device()
    n = 4 * 65_536 + 20
    g, master, m, v = _adamw_inputs(n, 21)
    whole = _adamw_gpu(g, master, m, v, step=10)
    for n_d in (2, 4, 7):
        cuts = np.linspace(0, n, n_d + 1).astype(int)
        parts = [np.empty_like(x) for x in whole]
        for b, e in zip(cuts[:-1], cuts[1:]):
            sub = _adamw_gpu(g[b:e].copy(), master[b:e].copy(), m[b:e].copy(), v[b:e].copy(), step=10)
            for dst, s in zip(parts, sub):
                dst[b:e] = s
        for a, w, name in zip(parts, whole, ("master", "m", "v", "param")):
            assert_bits_equal(a, w, f"{n_d} shards vs whole: {name}")


def test_adamw_tiny_mlp_shard_and_persistent_region():
    dev = device()
    w = TINY_MLP
    lay = oracle.Layout(w.numels, w.n_d)
    b, e = lay.rank_range(w.rank)
    for what, n in (("shard", e - b), ("persistent", lay.psi_persist)):
        st = synth.shard_state(w, n, salt=0 if what == "shard" else 1)
        g = _bits(synth.contributions(w, n, salt=0 if what == "shard" else 1)[0])
        master, m, v = (st[k].numpy() for k in ("master", "exp_avg", "exp_avg_sq"))
        got = _adamw_gpu(g, master, m, v, step=1)
        _check_adamw(got, _adamw_ref(g, master, m, v, 1), f"tiny mlp {what}")
    assert dev.type == "cuda"


# ----------------------------------------------------------------- reduce ----

def _reduce_gpu(contribs, offsets, out_offset=0, in_place=False):
    placed = [Placed(c, o) for c, o in zip(contribs, offsets)]
    if in_place:
        out = placed[0]
    else:
        out = Placed(np.zeros(contribs[0].size, np.uint16), out_offset)
    zr.zr_reduce_slice([p.view for p in placed], out.view)
    torch.cuda.synchronize()
    for p in placed + [out]:
        assert p.guards_intact()
    if not in_place:
        for p, c in zip(placed, contribs):
            assert np.array_equal(p.host(), c), "contribution modified"
    return out.host()


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 7, 8, 9, 63, 64, 65, 256])
def test_reduce_bit_exact(n):
    device()
    rng = np.random.default_rng(n)
    size = 20_000 + n
    say("reduce n =", n)
    contribs = [_bits(synth.normal_bf16(size, 1e-3, 1000 * n + k)) for k in range(n)]
    ref = oracle.reduce(contribs)
    assert_bits_equal(_reduce_gpu(contribs, [0] * n), ref, f"reduce n={n} aligned")
    offs = [int(x) for x in rng.integers(0, 8, n)]
    assert_bits_equal(_reduce_gpu(contribs, offs, int(rng.integers(0, 8))), ref, f"reduce n={n} offsets")
    assert_bits_equal(_reduce_gpu(contribs, [3] * n, 3), ref, f"reduce n={n} common phase")


@pytest.mark.parametrize("off", [8, 16, 40, 61, 63])
def test_reduce_line_heads(off):
    """Contributions and output at one element offset from a 128-byte line: the
    vector body starts on the output's line (a head of up to 63 elements)."""
    device()
    for size in (1, 63, 64, 65, 130, 5003):
        contribs = [_bits(synth.normal_bf16(size, 1e-3, 700 + 7 * off + k)) for k in range(4)]
        ref = oracle.reduce(contribs)
        assert_bits_equal(_reduce_gpu(contribs, [off] * 4, off), ref, f"reduce size {size} offset {off}")


@pytest.mark.parametrize("size", [0, 1, 5, 8, 17, 2048, 2049 * 8 + 3])
def test_reduce_sizes_and_in_place(size):
    device()
    contribs = [_bits(synth.normal_bf16(size, 1e-3, 50 + k)) for k in range(4)]
    ref = oracle.reduce(contribs)
    assert_bits_equal(_reduce_gpu(contribs, [0, 0, 0, 0]), ref, f"reduce size {size}")
    assert_bits_equal(_reduce_gpu(contribs, [1, 1, 1, 1], in_place=True), ref, f"reduce in place size {size}")


def test_reduce_special_values():
    device()
    rng = np.random.default_rng(5)
    n = 4096
    # finite bf16 patterns across the whole exponent range, plus infinities and signed zeros
    pats = rng.integers(0, 65536, size=(3, n)).astype(np.uint16)
    pats[(pats & 0x7F80) == 0x7F80] &= 0xBFFF  # no NaN/inf from the random draw
    pats[0, :16] = [0x7F80, 0xFF80, 0x8000, 0x0000, 0x0001, 0x8001, 0x7F7F, 0xFF7F] * 2
    contribs = [pats[k].copy() for k in range(3)]
    assert_bits_equal(_reduce_gpu(contribs, [0, 0, 0]), oracle.reduce(contribs), "reduce special values")


def test_reduce_worked_example_and_slices(golden):
    device()
    gld = golden("reduce_scatter_example.txt")
    c = [oracle.bf16_from_f32(np.array(gld["contrib0"], np.float32)),
         oracle.bf16_from_f32(np.array(gld["contrib1"], np.float32))]
    full = _reduce_gpu(c, [0, 0])
    assert list(oracle.f32_from_bf16(full)) == gld["allreduce_mean"]
    for r, key in enumerate(("rank0_slice", "rank1_slice")):
        part = _reduce_gpu([x[r:r + 1].copy() for x in c], [0, 0])
        assert list(oracle.f32_from_bf16(part)) == gld[key]
    # ReduceScatter slice r == slice r of the AllReduce, for a bigger buffer
    contribs = [_bits(synth.normal_bf16(64 * 1000, 1e-3, 900 + k)) for k in range(8)]
    whole = _reduce_gpu(contribs, [0] * 8)
    for r in range(0, 64, 9):
        sl = slice(r * 1000, (r + 1) * 1000)
        assert_bits_equal(_reduce_gpu([x[sl].copy() for x in contribs], [0] * 8), whole[sl], f"slice {r}")


# ------------------------------------------------------------ pack/unpack ----

def _random_layout(rng):
    numels = [rng.choice([0, 1, 2, 3, 5, 7, 8, 9, 15, 16, 17, 100, 1000, rng.randrange(0, 40_000)])
              for _ in range(rng.randrange(1, 12))]
    return numels, rng.randrange(1, 9), rng.choice([0, 4, 20, 100])


@pytest.mark.parametrize("seed", range(24))
def test_pack_unpack_bit_exact(seed):
    device()
    rng = random.Random(seed)
    numels, n_d, thr = _random_layout(rng)
    ref = oracle.Layout(numels, n_d, thr)
    lay = zr.zr_layout_create(numels, n_d, thr)
    say("pack/unpack seed", seed, "numels", numels, "n_d", n_d, "thr", thr)
    host_views, placed = [], []
    for t, x in enumerate(numels):
        if ref.persistent[t]:
            host_views.append(None)
            placed.append(None)
            continue
        bits = _bits(synth.random_bits16(x, 10_000 * seed + t))
        host_views.append((bits, 0))
        placed.append(Placed(bits, rng.randrange(0, 8)))
    ranges = [(0, ref.psi_pad), ref.rank_range(rng.randrange(n_d))]
    b = rng.randrange(0, ref.psi_pad + 1)
    ranges.append((b, rng.randrange(b, ref.psi_pad + 1)))
    for b, e in ranges:
        want = oracle.pack(ref, host_views, b, e)
        flat = Placed(np.full(e - b, 0xFFFF, np.uint16), rng.randrange(0, 8))
        zr.zr_pack(lay, [None if p is None else p.view for p in placed], flat.view, b, e)
        torch.cuda.synchronize()
        assert flat.guards_intact()
        assert_bits_equal(flat.host(), want, f"pack [{b}, {e})")
        # unpack a fresh random flat range into sentinel-filled views
        src = _bits(synth.random_bits16(e - b, 77 + seed))
        expect = [None if v is None else (v[0].copy(), 0) for v in host_views]
        oracle.unpack(ref, src, b, e, expect)
        outs = [None if v is None else Placed(v[0], rng.randrange(0, 8)) for v in host_views]
        srcp = Placed(src, rng.randrange(0, 8))
        zr.zr_unpack(lay, srcp.view, b, e, [None if p is None else p.view for p in outs])
        torch.cuda.synchronize()
        for t, (p, x) in enumerate(zip(outs, expect)):
            if p is not None:
                assert p.guards_intact()
                assert_bits_equal(p.host(), x[0], f"unpack [{b}, {e}) tensor {t}")


def test_pack_with_window_views():
    device()
    numels = [1000, 37, 5000]
    ref = oracle.Layout(numels, 3, 0)
    lay = zr.zr_layout_create(numels, 3, 0)
    b, e = ref.rank_range(1)
    frs = ref.fragments(b, e)
    full = [_bits(synth.random_bits16(x, 31 + t)) for t, x in enumerate(numels)]
    views, host_views = [None] * 3, [None] * 3
    for t, toff, _, n in frs:
        first = max(0, toff - 3)
        last = min(numels[t], toff + n + 5)
        views[t] = (Placed(full[t][first:last].copy(), 1).view, first)
        host_views[t] = (full[t][first:last].copy(), first)
    flat = torch.empty(e - b, dtype=torch.int16, device=device())
    zr.zr_pack(lay, views, flat, b, e)
    assert_bits_equal(u16(flat), oracle.pack(ref, host_views, b, e), "pack with windows")


def test_gather_example_on_gpu(golden):
    device()
    gld = golden("gather_example.txt")
    lay = zr.zr_layout_create([2], 2, 0)
    shards = [oracle.bf16_from_f32(np.array(gld[k], np.float32)) for k in ("rank0_updated", "rank1_updated")]
    gathered = torch.from_numpy(np.concatenate(shards).view(np.int16)).to(device())
    w = torch.from_numpy(oracle.bf16_from_f32(np.array(gld["before"], np.float32)).view(np.int16)).to(device())
    zr.zr_unpack(lay, gathered, 0, 2, [w])
    assert list(oracle.f32_from_bf16(u16(w))) == gld["gathered"]


# ------------------------------------------------------ fused reduce+AdamW ----

def _fused_vs_separate(n, size, offsets, seed, with_param=True, with_grad=True, in_place=False, step=3,
                       hp=HP):
    """The fused call against zr_reduce_slice then zr_adamw_step on copies of the
    same inputs: every output bit-identical; both within the oracle's bar."""
    contribs = [_bits(synth.normal_bf16(size, 1e-3, seed + k)) for k in range(n)]
    _, master, m, v = _adamw_inputs(size, seed + 100)
    co, so = offsets
    # separate path
    pc = [Placed(c, co) for c in contribs]
    grad = Placed(np.zeros(size, np.uint16), co)
    zr.zr_reduce_slice([p.view for p in pc], grad.view)
    pt, pm, pv = Placed(master, so), Placed(m, so), Placed(v, so)
    pp = Placed(np.zeros(size, np.uint16), co) if with_param else None
    zr.zr_adamw_step(grad.view, pt.view, pm.view, pv.view, pp.view if pp else None, step=step, **hp)
    # fused path
    fc = [Placed(c, co) for c in contribs]
    ft, fm, fv = Placed(master, so), Placed(m, so), Placed(v, so)
    fp = Placed(np.zeros(size, np.uint16), co) if with_param else None
    if in_place:
        fg = fc[0]
    else:
        fg = Placed(np.zeros(size, np.uint16), co) if with_grad else None
    zr.zr_reduce_adamw_step([p.view for p in fc], ft.view, fm.view, fv.view, fp.view if fp else None,
                            fg.view if fg else None, step=step, **hp)
    torch.cuda.synchronize()
    for p in fc + [ft, fm, fv, fp, fg]:
        assert p is None or p.guards_intact()
    for a, b, name in ((ft, pt, "master"), (fm, pm, "m"), (fv, pv, "v")):
        assert_bits_equal(a.host(), b.host(), f"fused {name} n={n} size={size} offsets={offsets}")
    if with_param:
        assert_bits_equal(fp.host(), pp.host(), f"fused param n={n}")
    if fg is not None:
        assert_bits_equal(fg.host(), grad.host(), f"fused grad_out n={n}")
    # and the composition of the oracle's two steps
    o_grad = oracle.reduce(contribs)
    ref = _adamw_ref(o_grad, master, m, v, step, with_param=with_param, hp=hp)
    _check_adamw((ft.host(), fm.host(), fv.host(), fp.host() if fp else None), ref, f"fused vs oracle n={n}")


@pytest.mark.parametrize("n,size", [(4, 65), (4, 5003), (8, 200), (8, 5003), (33, 5003)])
@pytest.mark.parametrize("offsets", [(8, 8), (12, 12), (40, 40), (61, 61), (12, 8)])
def test_fused_line_heads(n, size, offsets):
    """(contribution, state) element offsets from a 128-byte line, as in the
    AdamW line-head test: the fused call (one pass, and two passes above 24
    contributions) equals the two calls and the oracle."""
    device()
    _fused_vs_separate(n, size, offsets, 900 + n + size)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 8, 9, 24, 25, 64, 65])
def test_fused_matches_separate_calls(n):
    device()
    say("fused n =", n)
    _fused_vs_separate(n, 30_000 + 7 * n + 3, (0, 0), 300 + n)


# (contribution / copy / mean offset, state offset) in elements: aligned; a head
# peel that keeps every buffer vector-aligned ((1,1), (2,2), (3,3)); phases that
# force the element-wise fallback ((1,0), (0,2), (2,1), (3,1))
@pytest.mark.parametrize("size,offsets", [(0, (0, 0)), (1, (0, 0)), (3, (1, 1)), (4, (0, 0)), (5, (2, 1)),
                                          (4099, (3, 3)), (4099, (1, 0)), (4099, (0, 2)), (65_537, (2, 2)),
                                          (65_537, (3, 1))])
def test_fused_sizes_and_paths(size, offsets):
    device()
    _fused_vs_separate(4, size, offsets, 7 + size)


def test_fused_optional_outputs_and_in_place():
    device()
    _fused_vs_separate(4, 10_001, (0, 0), 11, with_param=False, with_grad=False)
    _fused_vs_separate(8, 10_001, (0, 0), 12, with_param=True, with_grad=False)
    _fused_vs_separate(8, 10_001, (0, 0), 13, with_param=False, with_grad=True)
    _fused_vs_separate(4, 10_001, (2, 1), 14, in_place=True)
    _fused_vs_separate(3, 10_001, (0, 0), 15, step=1000, hp=dict(HP, lr=1e-4, weight_decay=0.1))


def test_fused_two_pass_schedule_outputs_and_paths():
    """Above 24 contributions the call runs the mean and AdamW as two passes,
    with the mean in grad_out, or in param_out when only the copy is asked for
    (AdamW then overwrites it in place), and the one-pass kernel when neither
    output is given: every combination, both sides of the threshold, aligned,
    head-peeled and element-wise placements, equal the separate calls bit for bit."""
    device()
    for n in (24, 25, 33):
        _fused_vs_separate(n, 10_001, (0, 0), 20 + n, with_param=True, with_grad=False)
        _fused_vs_separate(n, 10_001, (0, 0), 21 + n, with_param=False, with_grad=True)
        _fused_vs_separate(n, 10_001, (0, 0), 22 + n, with_param=False, with_grad=False)
        _fused_vs_separate(n, 10_001, (2, 1), 23 + n, in_place=True)
        _fused_vs_separate(n, 4099, (3, 3), 24 + n, with_param=True, with_grad=False)
        _fused_vs_separate(n, 4099, (1, 0), 25 + n, with_param=True, with_grad=False)
    _fused_vs_separate(256, 3001, (0, 0), 26, with_param=True, with_grad=False)
