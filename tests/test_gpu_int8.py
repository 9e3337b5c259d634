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
from gpu_util import Placed, assert_bits_equal, device, say
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
