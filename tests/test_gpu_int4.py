"""GPU parity of the int4 block quantization (the qwZ AllGather with int4
codes, two per byte) against the oracle, through the C ABI: packed codes,
scales and rebuilt bf16 values bit-exact for every block size, odd and ragged
lengths, both the vector and the element-wise paths (misaligned buffers),
all-zero and subnormal blocks and exact ties; the dequantize-on-unpack of the
gathered codes (packing and blocks restarting at every shard, odd shard sizes,
sub-ranges starting on odd elements, misaligned codes and views) against the
oracle; and the gathered codes of a 7e9-parameter tensor over 4 ranks at full
size, on sampled windows."""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_optimizer_zr_amd as zr
from gpu_util import Placed, assert_bf16_equal_nan_as_class, assert_bits_equal, device, say
from zr_workloads import FLAT_7B

pytestmark = pytest.mark.gpu

BLOCKS = [256, 512, 1024, 2048]


def bf16(x):
    return oracle.bf16_from_f32(np.asarray(x, dtype=np.float32))


def run_gpu(x, block, offs=(0, 0, 0, 0)):
    """Quantize and dequantize through the C ABI with src, q4, scales and dst
    placed at the given element (byte, for q4) offsets; returns host copies."""
    n = x.size
    nb = -(-n // block)
    so, qo, sco, do = offs
    src = Placed(x, so)
    q = Placed(np.zeros(-(-n // 2), np.uint8), qo)
    sc = Placed(np.zeros(nb, np.float32), sco)
    dst = Placed(np.zeros(n, np.uint16), do)
    zr.zr_quantize_int4(src.view, q.view, sc.view, block=block)
    zr.zr_dequantize_int4(q.view, sc.view, dst.view, block=block)
    torch.cuda.synchronize()
    for p in (src, q, sc, dst):
        assert p.guards_intact()
    return q.host(), sc.host(), dst.host()


def check(x, block, offs=(0, 0, 0, 0), what=""):
    q, s, back = run_gpu(x, block, offs)
    rq, rs = oracle.quantize_int4(x, block)
    rb = oracle.dequantize_int4(rq, rs, x.size, block)
    assert_bits_equal(s, rs, f"scales {what} block {block} offs {offs}")
    assert_bits_equal(q, rq, f"codes {what} block {block} offs {offs}")
    assert_bits_equal(back, rb, f"dequantized {what} block {block} offs {offs}")


@pytest.mark.parametrize("block", BLOCKS)
@pytest.mark.parametrize("n", [1, 2, 3, 255, 256, 257, 2047, 2048 * 5 + 3, 100_003, 100_004])
def test_int4_matches_oracle_vector_path(block, n):
    device()
    say("int4 vector path block", block, "n", n)
    x = bf16(np.random.default_rng(n + block).normal(0, 0.02, n))
    check(x, block, what=f"n={n}")


@pytest.mark.parametrize("block", BLOCKS)
@pytest.mark.parametrize("offs", [(1, 0, 0, 0), (0, 1, 0, 0), (0, 2, 0, 0), (0, 0, 0, 3), (2, 3, 1, 1)])
def test_int4_matches_oracle_elementwise_path(block, offs):
    device()
    say("int4 element-wise path block", block, "offs", offs)
    x = bf16(np.random.default_rng(sum(offs) + block).normal(0, 1.0, 20_001))
    check(x, block, offs, what="element-wise")


@pytest.mark.parametrize("block", [256, 2048])
def test_int4_zero_subnormal_and_outlier_blocks(block):
    device()
    rng = np.random.default_rng(block)
    x = rng.normal(0, 1e-3, 8 * block).astype(np.float32)
    x[:block] = 0.0                                           # an all-zero block
    x[block:2 * block] = rng.normal(0, 1e-39, block)          # subnormal bf16 values (scale below 2^-100)
    x[2 * block + 17] = 3e4                                   # one outlier
    x[3 * block:4 * block] *= 2.0 ** -110                     # tiny but normal
    check(bf16(x), block, what="special blocks")


def test_int4_exact_ties_round_to_even():
    device()
    for e in (0, 7, 30):
        vals = np.array([7, 0.5, 1.5, 2.5, -2.5, 6.5, -0.5, 3.5] * 32, np.float64) * 2.0 ** -e
        check(bf16(vals), 256, what=f"ties 2^-{e}")


@pytest.mark.parametrize("block", BLOCKS)
def test_int4_near_half_steps(block):
    """Values whose quotients sit next to half steps, where a plain reciprocal
    product would round some codes the other way."""
    device()
    rng = np.random.default_rng(block + 3)
    k = rng.integers(-7, 7, 40 * block) + 0.5
    amax = 7.0 * 2.0 ** rng.integers(-20, 10, 40)
    x = (k.reshape(40, block) * (amax / 7.0)[:, None] * (1 + rng.normal(0, 2 ** -9, (40, block)))).ravel()
    x.reshape(40, block)[:, 0] = amax
    check(bf16(x), block, what="near half steps")


def test_int4_empty_is_noop():
    dev = device()
    e16 = torch.empty(0, dtype=torch.int16, device=dev)
    e8 = torch.empty(0, dtype=torch.uint8, device=dev)
    ef = torch.empty(0, dtype=torch.float32, device=dev)
    zr.zr_quantize_int4(e16, e8, ef, block=256)
    zr.zr_dequantize_int4(e8, ef, e16, block=256)
    torch.cuda.synchronize()


# ------------------------------------------------- dequantize-on-unpack ----

def _gathered_case(numels, n_d, block, seed, threshold=100_000):
    lay = oracle.Layout(numels, n_d, threshold)
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 1, lay.psi_pad)
    x *= 2.0 ** rng.integers(-12, 12, size=lay.psi_pad // 64 + 1).repeat(64)[: lay.psi_pad]
    x[lay.psi_part:] = 0.0
    flat = bf16(x)
    q4, s = oracle.quantize_gathered_int4(lay, flat, block)
    return lay, q4, s


def _unpack_int4_both(lay, q4, s, block, begin, end, q_off=0, view_off=3):
    """GPU (codes at byte offset q_off, views at element offset view_off) and
    oracle results of the int4 dequantize-on-unpack of [begin, end)."""
    b0 = int(oracle.gathered_code_byte(lay, np.array([begin]))[0])
    b1 = int(oracle.gathered_code_byte(lay, np.array([end - 1]))[0]) + 1
    g0 = int(oracle.gathered_block(lay, np.array([begin]), block)[0])
    qs = np.ascontiguousarray(q4[b0:b1])
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
    zr.zr_unpack_int4(glay, pq.view, ps.view, begin, end, [p.view if p else None for p in placed_views], block=block)
    torch.cuda.synchronize()
    oracle.unpack_int4(lay, qs, ss, block, begin, end, ref_views)
    assert pq.guards_intact() and ps.guards_intact()
    got = []
    for p in placed_views:
        if p is not None:
            assert p.guards_intact()
        got.append(None if p is None else p.host())
    return got, [None if v is None else v[0] for v in ref_views]


@pytest.mark.parametrize("block", BLOCKS)
@pytest.mark.parametrize("numels,n_d", [([200_003, 7, 150_001, 99_999, 130_000, 5, 311_111], 3),   # S even
                                        ([200_003, 7, 150_002, 99_999, 130_002], 3),               # S odd
                                        ([300_000, 50, 211_000], 4), ([123_457], 1)])
def test_unpack_int4_full_range_matches_oracle(block, numels, n_d):
    device()
    say("unpack_int4 full range block", block, "n_d", n_d)
    lay, q4, s = _gathered_case(numels, n_d, block, block + n_d)
    got, ref = _unpack_int4_both(lay, q4, s, block, 0, lay.psi_pad)
    for t, (g, r) in enumerate(zip(got, ref)):
        if g is not None:
            assert_bits_equal(g, r, f"tensor {t} block {block} n_d {n_d} S {lay.shard}")


def _many_tensor_numels(count, seed):
    """`count` tensors of 100,001-159,999 elements, two of them persistent."""
    rng = np.random.default_rng(seed)
    numels = [int(x) for x in rng.integers(100_001, 160_000, count)]
    numels[5], numels[11] = 7, 99_999
    return numels


def _descriptors(lay):
    """Tensor pieces of the whole flat buffer split at shard boundaries: the
    descriptors the unpack launches over (batches of at most 64)."""
    return sum(len(lay.fragments(*lay.rank_range(r))) for r in range(lay.n_d))


@pytest.mark.parametrize("count,n_d,q_off,view_off", [(30, 3, 0, 0), (30, 3, 1, 3), (68, 2, 0, 0), (68, 2, 2, 5)])
def test_unpack_int4_many_tensors(count, n_d, q_off, view_off):
    """A model's tensors: more than 8 descriptors in one launch (four chunks
    per lane in launch order), and more than 64 (64 of them, then a second
    launch of the few left: two chunks per lane in XCD runs).  Bit-exact
    against the oracle, also with codes and views at odd offsets."""
    device()
    numels = _many_tensor_numels(count, count + n_d)
    block = 512
    lay, q4, s = _gathered_case(numels, n_d, block, count)
    nd = _descriptors(lay)
    assert nd > 8 and (count < 60 or 64 < nd <= 72), nd
    say("unpack_int4 many tensors", count, "descriptors", nd, "offsets", q_off, view_off)
    got, ref = _unpack_int4_both(lay, q4, s, block, 0, lay.psi_pad, q_off, view_off)
    for t, (g, r) in enumerate(zip(got, ref)):
        if g is not None:
            assert_bits_equal(g, r, f"tensor {t} of {count}, {nd} descriptors, offsets {q_off}/{view_off}")


# Scale values the unpack may be handed.  The quantizer makes finite ones >= 0,
# but the call takes any fp32: NaN, infinities, signed zeros, subnormals, values
# whose products overflow, negative scales.
ANY_SCALES = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 1e-45, -3e-42, 1e-39, 1.1754942e-38, 2.0 ** 100,
                       3.4e38, -3.4e38, 0.0123, -7.5, 1.0, 2.0 ** -126], np.float32)


@pytest.mark.parametrize("view_off,begin,many", [(0, 0, False), (3, 0, False), (0, 5, False), (1, 2, False),
                                                (0, 0, True), (3, 1, True)])
def test_unpack_int4_any_scale_values(view_off, begin, many):
    """Random code bytes and scales drawn from ANY_SCALES, unpacked with
    tensor windows whose first 8-element chunk starts on (view offset 0,
    range from 0: one scale per chunk) and off (the other cases: a chunk may
    straddle two blocks) a multiple of 8 in the block grid, for a few tensors
    and for a model's many.  Bit-exact against the oracle, NaN results
    compared as NaN."""
    device()
    numels = _many_tensor_numels(30, 9) if many else [120_017, 50_003, 170_002]
    block = 256
    lay, q4, s = _gathered_case(numels, 3, block, 21)
    rng = np.random.default_rng(22 + view_off + begin)
    q4 = rng.integers(0, 256, q4.size).astype(np.uint8)
    s = ANY_SCALES[rng.integers(0, ANY_SCALES.size, s.size)]
    with np.errstate(over="ignore", invalid="ignore"):  # products that overflow, 0 * inf
        got, ref = _unpack_int4_both(lay, q4, s, block, begin, lay.psi_pad - begin, 0, view_off)
    for t, (g, r) in enumerate(zip(got, ref)):
        if g is not None:
            assert_bf16_equal_nan_as_class(g, r, f"tensor {t} view offset {view_off} range from {begin}")


@pytest.mark.parametrize("q_off,view_off", [(0, 0), (1, 0), (2, 3), (3, 1), (4, 4)])
def test_unpack_int4_misaligned_codes_and_views(q_off, view_off):
    device()
    numels = [120_017, 50_003, 170_002]   # S odd
    block = 512
    lay, q4, s = _gathered_case(numels, 3, block, 11)
    got, ref = _unpack_int4_both(lay, q4, s, block, 0, lay.psi_pad, q_off, view_off)
    for t, (g, r) in enumerate(zip(got, ref)):
        if g is not None:
            assert_bits_equal(g, r, f"tensor {t} offsets {q_off}/{view_off}")


@pytest.mark.parametrize("numels,threshold", [([200_003, 150_001, 90_000, 13], 50),      # S = 110_002 (even)
                                              ([200_003, 150_002, 90_000, 13], 50)])     # S = 110_003 (odd)
def test_unpack_int4_subranges(numels, threshold):
    device()
    block = 256
    lay, q4, s = _gathered_case(numels, 4, block, 3, threshold=threshold)
    S = lay.shard
    for begin, end in [(0, 1000), (1, 1000), (S - 301, S + 300), (S + 101, 2 * S + 7), (777, lay.psi_pad),
                       (2 * S - 1, 2 * S + 1), (3 * S - 183, 3 * S - 180), (5, 6), (6, 7), (0, lay.psi_part)]:
        got, ref = _unpack_int4_both(lay, q4, s, block, begin, end)
        for t, (g, r) in enumerate(zip(got, ref)):
            if g is not None:
                assert_bits_equal(g, r, f"tensor {t} range [{begin}, {end}) S {S}")


def test_unpack_int4_equals_dequantize_then_unpack_on_gpu():
    dev = device()
    numels = [300_001, 70_003, 250_000]
    block = 1024
    lay, q4, s = _gathered_case(numels, 4, block, 21)
    S, per_rank, nbytes = lay.shard, -(-lay.shard // block), -(-lay.shard // 2)
    qd = torch.from_numpy(q4).to(dev)
    sd = torch.from_numpy(s).to(dev)
    flat = torch.empty(lay.psi_pad, dtype=torch.int16, device=dev)
    for r in range(4):
        zr.zr_dequantize_int4(qd[r * nbytes:(r + 1) * nbytes], sd[r * per_rank:(r + 1) * per_rank],
                              flat[r * S:(r + 1) * S], block=block)
    glay = zr.zr_layout_create(numels, 4)
    a = [torch.full((n,), 0x1234, dtype=torch.int16, device=dev) for n in numels]
    b = [torch.full((n,), 0x1234, dtype=torch.int16, device=dev) for n in numels]
    zr.zr_unpack(glay, flat, 0, lay.psi_pad, a)
    zr.zr_unpack_int4(glay, qd, sd, 0, lay.psi_pad, b, block=block)
    torch.cuda.synchronize()
    for t in range(3):
        assert torch.equal(a[t], b[t]), t


def test_int4_full_shard_and_gather_7b_over_4_ranks_sampled():
    """A 1.75e9-element shard quantized in one call, and the gathered int4
    codes of the 7e9-parameter tensor over 4 ranks (3.5 GB of codes, 14 GB of
    bf16 output) rebuilt in one call; sampled blocks and windows are recomputed
    by the oracle."""
    dev = device()
    w = FLAT_7B
    block = 2048
    lay = oracle.Layout(w.numels, w.n_d)
    S, per_rank, nbytes = lay.shard, -(-lay.shard // block), -(-lay.shard // 2)
    say("int4 full size shard", S)
    g = torch.Generator(device=dev)
    g.manual_seed(78)
    x = (torch.randn(S, generator=g, device=dev) * 0.02).to(torch.bfloat16)
    q4 = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sc = torch.empty(per_rank, dtype=torch.float32, device=dev)
    zr.zr_quantize_int4(x, q4, sc, block=block)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    for blk in np.unique(np.concatenate([rng.integers(0, per_rank, 200), [0, per_rank - 1]])):
        lo, hi = int(blk) * block, min(S, (int(blk) + 1) * block)
        xs = x[lo:hi].view(torch.int16).cpu().numpy().view(np.uint16).copy()
        rq, rs = oracle.quantize_int4(xs, block)
        assert_bits_equal(q4[lo // 2:(hi + 1) // 2].cpu().numpy(), rq, f"codes of block {blk}")
        assert_bits_equal(sc[blk:blk + 1].cpu().numpy(), rs, f"scale of block {blk}")
    del x, q4, sc
    torch.cuda.empty_cache()
    # the gather
    qd = torch.randint(0, 256, (w.n_d * nbytes,), dtype=torch.uint8, device=dev, generator=g)
    qd = torch.where((qd & 0xf) == 8, qd ^ 0x1, qd)              # no -8 codes
    qd = torch.where((qd >> 4) == 8, qd ^ 0x10, qd)
    sd = torch.rand(w.n_d * per_rank, dtype=torch.float32, device=dev, generator=g) * 1e-3
    out = torch.empty(w.numels[0], dtype=torch.int16, device=dev)
    glay = zr.zr_layout_create(w.numels, w.n_d)
    zr.zr_unpack_int4(glay, qd, sd, 0, lay.psi_pad, [out], block=block)
    torch.cuda.synchronize()
    starts = np.concatenate([rng.integers(0, lay.psi_part - 4096, 300), [0, 1, S - 2001, 2 * S - 7, lay.psi_part - 4096]])
    sh = sd.cpu().numpy()
    for b0 in starts:
        b0 = int(b0)
        b1 = b0 + 4096
        c0 = int(oracle.gathered_code_byte(lay, np.array([b0]))[0])
        c1 = int(oracle.gathered_code_byte(lay, np.array([b1 - 1]))[0]) + 1
        g0 = int(oracle.gathered_block(lay, np.array([b0]), block)[0])
        ref = (np.full(4096, 0, np.uint16), b0)
        oracle.unpack_int4(lay, qd[c0:c1].cpu().numpy(), sh[g0:g0 + 8].copy(), block, b0, b1, [ref])
        assert_bits_equal(out[b0:b1].cpu().numpy().view(np.uint16), ref[0], f"window at {b0}")
    del qd, sd, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("bits", [8, 4])
def test_dequantize_past_2_31_elements_sampled(bits):
    """The flat dequantizers over 2^31 + 4099 elements (random codes, random
    scales, block 2048, a ragged last tile): sampled blocks, among them those
    around element 2^31 and the last, recomputed by the oracle."""
    dev = device()
    n, block = 2 ** 31 + 4099, 2048
    nb = -(-n // block)
    say("dequantize past 2^31, int", bits, "n", n)
    g = torch.Generator(device=dev)
    g.manual_seed(90 + bits)
    if bits == 8:
        q = torch.randint(-127, 128, (n,), dtype=torch.int8, device=dev, generator=g)
    else:
        q = torch.randint(0, 256, ((n + 1) // 2,), dtype=torch.uint8, device=dev, generator=g)
        q = torch.where((q & 0xf) == 8, q ^ 0x1, q)              # no -8 codes
        q = torch.where((q >> 4) == 8, q ^ 0x10, q)
    sc = torch.rand(nb, dtype=torch.float32, device=dev, generator=g) * 1e-3
    out = torch.empty(n, dtype=torch.int16, device=dev)
    if bits == 8:
        zr.zr_dequantize_int8(q, sc, out, block=block)
    else:
        zr.zr_dequantize_int4(q, sc, out, block=block)
    torch.cuda.synchronize()
    rng = np.random.default_rng(91)
    edge = 2 ** 31 // block
    picks = np.unique(np.concatenate([rng.integers(0, nb, 200), [0, edge - 1, edge, edge + 1, nb - 2, nb - 1]]))
    sh = sc.cpu().numpy()
    for b in picks:
        lo, hi = int(b) * block, min(n, (int(b) + 1) * block)
        if bits == 8:
            ref = oracle.dequantize_int8(q[lo:hi].cpu().numpy(), sh[b:b + 1].copy(), block)
        else:
            ref = oracle.dequantize_int4(q[lo // 2:(hi + 1) // 2].cpu().numpy(), sh[b:b + 1].copy(), hi - lo, block)
        assert_bits_equal(out[lo:hi].cpu().numpy().view(np.uint16), ref, f"int{bits} block {b}")
    del q, sc, out
    torch.cuda.empty_cache()
