"""GPU parity of the int8 block quantization of a bf16 shard (the quantized
weight AllGather) against the oracle, through the C ABI: codes, scales and the
rebuilt bf16 values bit-exact, for every block size, ragged lengths (short last
blocks, lengths that are not a multiple of 4), both the vector and the
element-wise paths (misaligned buffers), all-zero blocks, subnormal blocks,
exact ties and, at the real size of a 7e9-parameter shard over 4 ranks, sampled
blocks (blocks are independent, so the oracle recomputes each sampled block on
its own)."""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_optimizer_zr_amd as zr
from gpu_util import Placed, assert_bf16_equal_nan_as_class, assert_bits_equal, device, say
from zr_workloads import FLAT_7B, synth

pytestmark = pytest.mark.gpu

BLOCKS = [256, 512, 1024, 2048]


def bf16(x):
    return oracle.bf16_from_f32(np.asarray(x, dtype=np.float32))


def run_gpu(x, block, offs=(0, 0, 0, 0)):
    """Quantize and dequantize through the C ABI with src, q, scales and dst
    placed at the given element offsets; returns host copies."""
    n = x.size
    nb = -(-n // block)
    so, qo, sco, do = offs
    src = Placed(x, so)
    q = Placed(np.zeros(n, np.int8), qo)
    sc = Placed(np.zeros(nb, np.float32), sco)
    dst = Placed(np.zeros(n, np.uint16), do)
    zr.zr_quantize_int8(src.view, q.view, sc.view, block=block)
    zr.zr_dequantize_int8(q.view, sc.view, dst.view, block=block)
    torch.cuda.synchronize()
    for p in (src, q, sc, dst):
        assert p.guards_intact()
    return q.host(), sc.host(), dst.host()


def check(x, block, offs=(0, 0, 0, 0), what=""):
    q, s, back = run_gpu(x, block, offs)
    rq, rs = oracle.quantize_int8(x, block)
    rb = oracle.dequantize_int8(rq, rs, block)
    assert_bits_equal(s, rs, f"scales {what} block {block} offs {offs}")
    assert_bits_equal(q, rq, f"codes {what} block {block} offs {offs}")
    assert_bits_equal(back, rb, f"dequantized {what} block {block} offs {offs}")


@pytest.mark.parametrize("block", BLOCKS)
@pytest.mark.parametrize("n", [1, 3, 255, 256, 257, 2047, 2048 * 5 + 3, 100_003])
def test_int8_matches_oracle_vector_path(block, n):
    device()
    say("int8 vector path block", block, "n", n)
    x = bf16(np.random.default_rng(n + block).normal(0, 0.02, n))
    check(x, block, what=f"n={n}")


@pytest.mark.parametrize("block", BLOCKS)
@pytest.mark.parametrize("offs", [(1, 0, 0, 0), (0, 1, 0, 0), (0, 0, 0, 3), (2, 3, 1, 1)])
def test_int8_matches_oracle_elementwise_path(block, offs):
    device()
    say("int8 element-wise path block", block, "offsets", offs)
    n = 3 * block + 77
    x = bf16(np.random.default_rng(block + sum(offs)).normal(0, 1.0, n))
    check(x, block, offs, "misaligned")


@pytest.mark.parametrize("block", [256, 2048])
def test_int8_zero_subnormal_and_outlier_blocks(block):
    device()
    rng = np.random.default_rng(9)
    nb = 6
    x = rng.normal(0, 0.02, nb * block - 5).astype(np.float32)
    x[0:block] = 0.0                                         # all-zero block: s == 0, q == 0
    x[block: 2 * block] = rng.normal(0, 1e-39, block)        # subnormal block (s subnormal)
    x[2 * block: 3 * block] = rng.normal(0, 1e-30, block)
    x[3 * block + 17] = 300.0                                # one outlier dominates its block
    x[4 * block: 5 * block] *= -1e4
    xb = bf16(x)
    xb[block + 5] = 0x8000                                   # -0.0
    for offs in ((0, 0, 0, 0), (1, 1, 0, 1)):
        check(xb, block, offs, "zero/subnormal/outlier")


def test_int8_exact_ties_round_to_even():
    """Blocks whose amax is 127 * 2^e hold elements at exact half steps: the
    codes must round to even (1.5 -> 2, 2.5 -> 2, -0.5 -> -0)."""
    device()
    block = 256
    rng = np.random.default_rng(3)
    nb = 8
    k = rng.integers(-126, 126, size=(nb, block)) + 0.5
    k[:, 0] = 127.0
    e = rng.integers(-10, 2, size=nb)
    x = bf16((k * (2.0 ** e)[:, None]).ravel())
    q, _, _ = run_gpu(x, block)
    kk = k.ravel()
    want = np.where(np.abs(kk) >= 127, np.sign(kk) * 127, np.round(kk)).astype(np.int8)  # numpy rounds half to even
    exact = oracle.f32_from_bf16(x) == (k * (2.0 ** e)[:, None]).ravel().astype(np.float32)
    assert exact.mean() > 0.9
    assert np.array_equal(q[exact], want[exact])
    check(x, block, what="ties")


def near_half_step_blocks(block, nb, seed):
    """Blocks of elements whose fp32 quotients x / s lie within 2^-11 of a
    half-integer: exact ties, quotients off a tie by less than 2^-14 and ones a
    little further off, where a quotient taken any other way than one correctly
    rounded division could round the other way.  Returns the bf16 bits and the
    count of non-tie elements within 2^-14 of a half-integer."""
    rng = np.random.default_rng(seed)
    every = oracle.f32_from_bf16(np.arange(0x10000, dtype=np.uint32).astype(np.uint16))
    every = every[np.isfinite(every)]
    out, close = [], 0
    while len(out) < nb:
        amax = np.float32(rng.uniform(0.5, 2.0) * 2.0 ** rng.integers(-20, 10))
        amax = oracle.f32_from_bf16(bf16([amax]))[0]
        s = np.float32(amax / np.float32(127))
        cand = every[np.abs(every) <= amax]
        t = cand / s
        d = np.abs(np.abs(t - np.floor(t)) - 0.5)
        near, dn = cand[d < 2.0 ** -11], d[d < 2.0 ** -11]
        if not (dn > 0).any():
            continue
        w = np.where(dn > 0, 4.0, 1.0)
        pick = rng.choice(near.size, block, p=w / w.sum())
        x = near[pick]
        close += int(((dn[pick] > 0) & (dn[pick] < 2.0 ** -14)).sum())
        x[rng.integers(0, block)] = amax * rng.choice([-1, 1])
        out.append(x)
    return bf16(np.concatenate(out)), close


@pytest.mark.parametrize("block", BLOCKS)
def test_int8_near_half_steps(block):
    device()
    x, close = near_half_step_blocks(block, 24, block)
    assert close > 0
    check(x, block, what="near half steps")
    check(x, block, (1, 1, 0, 1), "near half steps, element-wise")


def test_int8_full_shard_sampled_blocks():
    """A 7e9-parameter model over 4 ranks: the rank's 1.75e9-element bf16
    shard (3.5 GB) quantized and rebuilt on the GPU; about 2000 random blocks
    plus the first and last ones are recomputed by the oracle."""
    dev = device()
    w = FLAT_7B
    n = w.numels[0] // w.n_d
    block = 2048
    nb = -(-n // block)
    say("int8 full shard n", n, "block", block)
    x = synth.normal_bf16(n, 0.02, synth.seed_of(w.seed, 40), device=dev)
    q = torch.empty(n, dtype=torch.int8, device=dev)
    sc = torch.empty(nb, dtype=torch.float32, device=dev)
    back = torch.empty(n, dtype=torch.int16, device=dev)
    zr.zr_quantize_int8(x, q, sc, block=block)
    zr.zr_dequantize_int8(q, sc, back, block=block)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    picks = np.unique(np.concatenate([rng.integers(0, nb, 2000), [0, 1, nb - 2, nb - 1]]))
    for b in picks:
        lo, hi = int(b) * block, min(n, (int(b) + 1) * block)
        xs = x.view(torch.int16)[lo:hi].cpu().numpy().view(np.uint16).copy()
        rq, rs = oracle.quantize_int8(xs, block)
        assert_bits_equal(sc[b:b + 1].cpu().numpy(), rs, f"scale of block {b}")
        assert_bits_equal(q[lo:hi].cpu().numpy(), rq, f"codes of block {b}")
        assert_bits_equal(back[lo:hi].cpu().numpy().view(np.uint16), oracle.dequantize_int8(rq, rs, block),
                          f"dequantized block {b}")
    del x, q, sc, back
    torch.cuda.empty_cache()


def test_int8_empty_is_noop():
    dev = device()
    e16 = torch.empty(0, dtype=torch.int16, device=dev)
    e8 = torch.empty(0, dtype=torch.int8, device=dev)
    ef = torch.empty(0, dtype=torch.float32, device=dev)
    zr.zr_quantize_int8(e16, e8, ef, block=256)
    zr.zr_dequantize_int8(e8, ef, e16, block=256)
    torch.cuda.synchronize()


# ------------------------------------------------- dequantize-on-unpack ----

def _gathered_case(numels, n_d, block, seed, threshold=100_000):
    lay = oracle.Layout(numels, n_d, threshold)
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 1, lay.psi_pad)
    x *= 2.0 ** rng.integers(-12, 12, size=lay.psi_pad // 64 + 1).repeat(64)[: lay.psi_pad]
    x[lay.psi_part:] = 0.0
    flat = bf16(x)
    q, s = oracle.quantize_gathered(lay, flat, block)
    return lay, q, s


def _unpack_int8_both(lay, q, s, block, begin, end, q_off=0, view_off=3):
    """GPU (through the C ABI, codes at byte offset q_off, views at element
    offset view_off) and oracle results of the dequantize-on-unpack of
    [begin, end); returns (gpu views, oracle views) as host arrays."""
    g0 = int(oracle.gathered_block(lay, np.array([begin]), block)[0])
    qs = np.ascontiguousarray(q[begin:end])
    ss = np.ascontiguousarray(s[g0:])
    placed_views, ref_views = [], []
    for t, n in enumerate(lay.numels):
        if lay.persistent[t]:
            placed_views.append(None)
            ref_views.append(None)
            continue
        init = np.full(n, 0x7777, np.uint16)
        placed_views.append(Placed(init, view_off + t % 5))
        ref_views.append((init.copy(), 0))
    pq = Placed(qs, q_off)
    ps = Placed(ss, 0)
    glay = zr.zr_layout_create(lay.numels, lay.n_d, lay.threshold)
    zr.zr_unpack_int8(glay, pq.view, ps.view, begin, end, [p.view if p else None for p in placed_views], block=block)
    torch.cuda.synchronize()
    oracle.unpack_int8(lay, qs, ss, block, begin, end, ref_views)
    assert pq.guards_intact() and ps.guards_intact()
    got = []
    for p in placed_views:
        if p is not None:
            assert p.guards_intact()
        got.append(None if p is None else p.host())
    return got, [None if v is None else v[0] for v in ref_views]


@pytest.mark.parametrize("block", BLOCKS)
@pytest.mark.parametrize("n_d", [1, 3, 4])
def test_unpack_int8_full_range_matches_oracle(block, n_d):
    device()
    numels = [200_003, 7, 150_001, 99_999, 130_000, 5, 311_111]
    say("unpack_int8 full range block", block, "n_d", n_d)
    lay, q, s = _gathered_case(numels, n_d, block, block + n_d)
    got, ref = _unpack_int8_both(lay, q, s, block, 0, lay.psi_pad)
    for t, (g, r) in enumerate(zip(got, ref)):
        if g is not None:
            assert_bits_equal(g, r, f"tensor {t} block {block} n_d {n_d}")


@pytest.mark.parametrize("count,n_d,q_off,view_off", [(30, 3, 0, 0), (68, 2, 3, 5)])
def test_unpack_int8_many_tensors(count, n_d, q_off, view_off):
    """A model's tensors: 30 descriptors in one launch, and 67 (a launch of 64,
    then one of 3).  Bit-exact against the oracle, also with codes and views at
    odd offsets."""
    device()
    rng = np.random.default_rng(count + n_d)
    numels = [int(x) for x in rng.integers(100_001, 160_000, count)]
    numels[5], numels[11] = 7, 99_999
    block = 512
    lay, q, s = _gathered_case(numels, n_d, block, count)
    nd = sum(len(lay.fragments(*lay.rank_range(r))) for r in range(lay.n_d))
    assert nd > 8 and (count < 60 or 64 < nd <= 72), nd
    say("unpack_int8 many tensors", count, "descriptors", nd)
    got, ref = _unpack_int8_both(lay, q, s, block, 0, lay.psi_pad, q_off, view_off)
    for t, (g, r) in enumerate(zip(got, ref)):
        if g is not None:
            assert_bits_equal(g, r, f"tensor {t} of {count}, {nd} descriptors, offsets {q_off}/{view_off}")


# Scale values the unpack may be handed.  The quantizer makes finite ones >= 0,
# but the call takes any fp32: NaN, infinities, signed zeros, subnormals, values
# whose products overflow, negative scales.
ANY_SCALES = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 1e-45, -3e-42, 1e-39, 1.1754942e-38, 2.0 ** 100,
                       3.4e38, -3.4e38, 0.0123, -7.5, 1.0, 2.0 ** -126], np.float32)


@pytest.mark.parametrize("view_off,begin", [(0, 0), (3, 0), (0, 5), (1, 2)])
def test_unpack_int8_any_scale_values(view_off, begin):
    """Random code bytes and scales drawn from ANY_SCALES, unpacked with
    tensor windows whose first 8-element chunk starts on (view offset 0,
    range from 0: one scale per chunk) and off (the other cases: a chunk may
    straddle two blocks) a multiple of 8 in the block grid.  Bit-exact against
    the oracle, NaN results compared as NaN."""
    device()
    numels = [120_017, 50_003, 170_001]
    block = 256
    lay, q, s = _gathered_case(numels, 3, block, 21)
    rng = np.random.default_rng(22 + view_off + begin)
    q = rng.integers(-128, 128, q.size).astype(np.int8)
    s = ANY_SCALES[rng.integers(0, ANY_SCALES.size, s.size)]
    with np.errstate(over="ignore", invalid="ignore"):  # products that overflow, 0 * inf
        got, ref = _unpack_int8_both(lay, q, s, block, begin, lay.psi_pad - begin, 0, view_off)
    for t, (g, r) in enumerate(zip(got, ref)):
        if g is not None:
            assert_bf16_equal_nan_as_class(g, r, f"tensor {t} view offset {view_off} range from {begin}")


@pytest.mark.parametrize("q_off,view_off", [(0, 0), (1, 0), (5, 3), (7, 1), (4, 4)])
def test_unpack_int8_misaligned_codes_and_views(q_off, view_off):
    device()
    numels = [120_017, 50_003, 170_001]
    block = 512
    lay, q, s = _gathered_case(numels, 3, block, 11)
    got, ref = _unpack_int8_both(lay, q, s, block, 0, lay.psi_pad, q_off, view_off)
    for t, (g, r) in enumerate(zip(got, ref)):
        if g is not None:
            assert_bits_equal(g, r, f"tensor {t} offsets {q_off}/{view_off}")


def test_unpack_int8_subranges_and_short_shard_blocks():
    device()
    block = 256
    # shard = 113_335 elements: 442 full blocks and a last block of 183 per shard
    numels = [200_003, 150_001, 90_000, 13]
    lay, q, s = _gathered_case(numels, 4, block, 3, threshold=50)
    S = lay.shard
    for begin, end in [(0, 1000), (S - 300, S + 300), (S + 100, 2 * S + 7), (777, lay.psi_pad),
                       (2 * S - 1, 2 * S + 1), (3 * S - 183, 3 * S - 180), (5, 6), (0, lay.psi_part)]:
        got, ref = _unpack_int8_both(lay, q, s, block, begin, end)
        for t, (g, r) in enumerate(zip(got, ref)):
            if g is not None:
                assert_bits_equal(g, r, f"tensor {t} range [{begin}, {end})")


def test_unpack_int8_equals_dequantize_then_unpack_on_gpu():
    """The fused path gives the same bits as dequantizing each rank's shard
    into a flat bf16 buffer and unpacking it."""
    dev = device()
    numels = [300_001, 70_003, 250_000]
    block = 1024
    lay, q, s = _gathered_case(numels, 4, block, 21)
    S, per_rank = lay.shard, -(-lay.shard // block)
    qd = torch.from_numpy(q).to(dev)
    sd = torch.from_numpy(s).to(dev)
    flat = torch.empty(lay.psi_pad, dtype=torch.int16, device=dev)
    for r in range(4):
        zr.zr_dequantize_int8(qd[r * S:(r + 1) * S], sd[r * per_rank:(r + 1) * per_rank],
                              flat[r * S:(r + 1) * S], block=block)
    glay = zr.zr_layout_create(numels, 4)
    a = [torch.full((n,), 0x1234, dtype=torch.int16, device=dev) for n in numels]
    b = [torch.full((n,), 0x1234, dtype=torch.int16, device=dev) for n in numels]
    zr.zr_unpack(glay, flat, 0, lay.psi_pad, a)
    zr.zr_unpack_int8(glay, qd, sd, 0, lay.psi_pad, b, block=block)
    torch.cuda.synchronize()
    for t in range(3):
        assert torch.equal(a[t], b[t]), t


def test_unpack_int8_full_size_7b_over_4_ranks_sampled():
    """The gathered codes of a 7e9-parameter tensor over 4 ranks (7 GB of codes,
    14 GB of bf16 output) rebuilt in one call; sampled windows are recomputed by
    the oracle from the same codes and scales."""
    dev = device()
    w = FLAT_7B
    block = 2048
    lay = oracle.Layout(w.numels, w.n_d)
    S, per_rank = lay.shard, -(-lay.shard // block)
    say("unpack_int8 full size psi_pad", lay.psi_pad, "shard", S)
    g = torch.Generator(device=dev)
    g.manual_seed(77)
    qd = torch.randint(-127, 128, (lay.psi_pad,), dtype=torch.int8, device=dev, generator=g)
    sd = torch.rand(w.n_d * per_rank, dtype=torch.float32, device=dev, generator=g) * 1e-3
    out = torch.empty(w.numels[0], dtype=torch.int16, device=dev)
    glay = zr.zr_layout_create(w.numels, w.n_d)
    zr.zr_unpack_int8(glay, qd, sd, 0, lay.psi_pad, [out], block=block)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    starts = np.concatenate([rng.integers(0, lay.psi_part - 4096, 300), [0, S - 2000, 2 * S - 7, lay.psi_part - 4096]])
    sh = sd.cpu().numpy()
    for b0 in starts:
        b0 = int(b0)
        b1 = b0 + 4096
        g0 = int(oracle.gathered_block(lay, np.array([b0]), block)[0])
        ref = (np.full(4096, 0, np.uint16), b0)
        oracle.unpack_int8(lay, qd[b0:b1].cpu().numpy(), sh[g0:g0 + 8].copy(), block, b0, b1, [ref])
        assert_bits_equal(out[b0:b1].cpu().numpy().view(np.uint16), ref[0], f"window at {b0}")
    del qd, sd, out
    torch.cuda.empty_cache()


@pytest.mark.slow
@pytest.mark.parametrize("block", [256, 2048])
def test_unpack_int8_full_size_llama_layout_sampled(block):
    """The whole gathered buffer of the Llama-7B layout over 64 ranks (6.7e9
    codes, 291 tensors, 65 of them persistent) rebuilt in one call; windows on
    every tensor boundary, every shard boundary and at random places are
    recomputed by the oracle from the same codes and scales."""
    from zr_workloads import LLAMA_7B
    dev = device()
    w = LLAMA_7B
    lay = oracle.Layout(w.numels, w.n_d, w.threshold)
    S, per_rank = lay.shard, -(-lay.shard // block)
    say("unpack_int8 llama layout psi_pad", lay.psi_pad, "block", block)
    g = torch.Generator(device=dev)
    g.manual_seed(91 + block)
    qd = torch.randint(-127, 128, (lay.psi_pad,), dtype=torch.int8, device=dev, generator=g)
    sd = torch.rand(w.n_d * per_rank, dtype=torch.float32, device=dev, generator=g) * 1e-2
    views = [None if lay.persistent[t] else torch.full((n,), 0x7777, dtype=torch.int16, device=dev)
             for t, n in enumerate(w.numels)]
    glay = zr.zr_layout_create(w.numels, w.n_d, w.threshold)
    zr.zr_unpack_int8(glay, qd, sd, 0, lay.psi_pad, views, block=block)
    torch.cuda.synchronize()
    sh = sd.cpu().numpy()
    rng = np.random.default_rng(block)
    starts = [lay.offset[t] for t in range(len(w.numels)) if not lay.persistent[t]]
    starts += [r * S for r in range(1, w.n_d)]
    starts = sorted({max(0, min(lay.psi_pad - 3000, x - 1500)) for x in starts} |
                    {int(x) for x in rng.integers(0, lay.psi_pad - 3000, 200)})
    for b0 in starts:
        b1 = b0 + 3000
        g0 = int(oracle.gathered_block(lay, np.array([b0]), block)[0])
        frags = lay.fragments(b0, b1)
        ref = [None] * len(w.numels)
        for t, toff, foff, n in frags:
            ref[t] = (np.zeros(n, np.uint16), toff)
        oracle.unpack_int8(lay, qd[b0:b1].cpu().numpy(), sh[g0:g0 + 32].copy(), block, b0, b1, ref)
        for t, toff, foff, n in frags:
            got = views[t][toff:toff + n].cpu().numpy().view(np.uint16)
            assert_bits_equal(got, ref[t][0], f"tensor {t} window at {b0}")
    # the padding writes nowhere, and persistent tensors are not touched
    assert all(v is None for v, p in zip(views, lay.persistent) if p)
    del qd, sd, views
    torch.cuda.empty_cache()
