"""Pins the oracle's symmetric block-wise int4 quantization (the ZeRO++ qwZ
sentence names int4 beside int8; the reading is the int8 rule with 7 for 127
and two codes per byte, low four bits first): a worked block written out by
hand, exactness on representable blocks, symmetry, the absmax element, the
per-element error bound, zero and short blocks, block independence, the
nibble packing (read back bit by bit here), the per-shard restart of blocks and
packing in the gather, and sub-range unpacks."""
import numpy as np
import pytest

import oracle


def bf16(xs):
    return oracle.bf16_from_f32(np.asarray(xs, dtype=np.float32))


def codes_of(q4, n):
    """The n signed 4-bit codes of packed bytes, read with Python integers."""
    out = []
    for i in range(n):
        v = (int(q4[i // 2]) >> (4 * (i % 2))) & 0xF
        out.append(v - 16 if v >= 8 else v)
    return np.array(out, dtype=np.int64)


def rt(x, block):
    q4, s = oracle.quantize_int4(x, block)
    return q4, s, oracle.dequantize_int4(q4, s, x.size, block)


def test_worked_block():
    # amax 14 -> s = 2; 14/2 = 7, -7/2 = -3.5 (tie, to even: -4), 1/2 = 0.5 (tie: 0),
    # 3/2 = 1.5 (tie: 2), -2/2 = -1; nibbles 7, 0xC, 0, 2, 0xF; odd count pads a zero nibble
    q4, s, back = rt(bf16([14, -7, 1, 3, -2]), 256)
    assert list(s) == [2.0]
    assert [int(b) for b in q4] == [0xC7, 0x20, 0x0F]
    assert list(oracle.f32_from_bf16(back)) == [14.0, -8.0, 0.0, 4.0, -2.0]


@pytest.mark.parametrize("block", [4, 256, 1024])
def test_representable_blocks_round_trip_exactly(block):
    rng = np.random.default_rng(block)
    nb = 6
    k = rng.integers(-7, 8, size=(nb, block))
    k[:, 0] = rng.choice([-7, 7], nb)                  # every block reaches +-7
    e = rng.integers(-20, 4, size=nb)
    x = (k * (2.0 ** e)[:, None]).astype(np.float32).ravel()
    xb = bf16(x)
    assert np.array_equal(oracle.f32_from_bf16(xb), x)
    q4, s, back = rt(xb, block)
    assert np.array_equal(codes_of(q4, x.size).reshape(nb, block), k)
    assert np.array_equal(s, (2.0 ** e).astype(np.float32))
    assert np.array_equal(back, xb)


def test_symmetry_and_absmax():
    rng = np.random.default_rng(2)
    x = bf16(rng.normal(0, 0.02, 4096))
    q4, s, _ = rt(x, 256)
    qn4, sn, _ = rt(x ^ np.uint16(0x8000), 256)        # negate every element
    q, qn = codes_of(q4, x.size), codes_of(qn4, x.size)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    xf = oracle.f32_from_bf16(x).reshape(16, 256)
    amax_pos = np.abs(xf).argmax(axis=1)
    qq = q.reshape(16, 256)
    assert np.all(np.abs(qq[np.arange(16), amax_pos]) == 7)
    assert np.all(np.abs(qq) <= 7)                     # -8 never occurs


@pytest.mark.parametrize("block,std", [(256, 0.02), (512, 1e-3), (2048, 5.0), (256, 1e-30)])
def test_round_trip_error_bound(block, std):
    rng = np.random.default_rng(int(block + 1e3 * std) % 1000)
    x = bf16(rng.normal(0, std, 50_001))
    q4, s, back = rt(x, block)
    xf = oracle.f32_from_bf16(x).astype(np.float64)
    bf = oracle.f32_from_bf16(back).astype(np.float64)
    sc = np.repeat(s.astype(np.float64), block)[: x.size]
    # half a quantization step (plus the fp32 quotient's rounding) and half a bf16 ulp of the result
    bound = sc * (0.5 + 1e-5) + np.abs(bf) * 2.0 ** -8 + 1e-45
    assert np.all(np.abs(bf - xf) <= bound)
    assert np.all(sc == np.repeat([np.float32(np.abs(xf[b:b + block]).max()) / np.float32(7)
                                   for b in range(0, x.size, block)], block)[: x.size])


def test_zero_block_short_tail_and_odd_count():
    x = np.zeros(701, dtype=np.uint16)
    x[512:] = bf16(np.linspace(-3, 3, 189))
    q4, s, back = rt(x, 256)
    assert q4.size == 351 and s.size == 3 and s[0] == 0 and s[1] == 0 and s[2] > 0
    assert not q4[:256].any() and not back[:512].any()
    assert int(q4[-1]) >> 4 == 0                       # the pad nibble of the odd count
    # the short tail block is quantized on its own (512 is even: its packing starts on a byte)
    q3, s3, _ = rt(x[512:].copy(), 256)
    assert np.array_equal(q3, q4[256:]) and s3[0] == s[2]


def test_blocks_are_independent():
    rng = np.random.default_rng(9)
    a = bf16(rng.normal(0, 1, 512))
    b = bf16(rng.normal(0, 1e-3, 768))
    qa, sa, _ = rt(a, 256)
    qb, sb, _ = rt(b, 256)
    qab, sab, _ = rt(np.concatenate([a, b]), 256)
    assert np.array_equal(qab, np.concatenate([qa, qb])) and np.array_equal(sab, np.concatenate([sa, sb]))


def test_int4_codes_are_the_int8_rule_at_a_coarser_step():
    # with s8 = amax / 127 and s4 = amax / 7 of the same block, both codes are the
    # nearest multiples: |x - q4 s4| <= s4 / 2 and |x - q8 s8| <= s8 / 2, so they agree
    # to within the coarser step
    rng = np.random.default_rng(4)
    x = bf16(rng.normal(0, 0.3, 8192))
    q4, s4, _ = rt(x, 512)
    q8, s8 = oracle.quantize_int8(x, 512)
    c4 = codes_of(q4, x.size).astype(np.float64) * np.repeat(s4.astype(np.float64), 512)
    c8 = q8.astype(np.float64) * np.repeat(s8.astype(np.float64), 512)
    assert np.all(np.abs(c4 - c8) <= np.repeat(s4.astype(np.float64), 512) * (0.5 + 1e-5)
                  + np.repeat(s8.astype(np.float64), 512) * (0.5 + 1e-5))


def test_payload_is_about_a_quarter_of_bf16():
    # half a byte per element plus one fp32 scale per block
    for block in (256, 512, 1024, 2048):
        n = 116_465_664
        q_bytes = n // 2 + 4 * -(-n // block)
        assert q_bytes / (2 * n) == pytest.approx(0.25 + 2 / block, rel=1e-6)


def test_exact_ties_round_to_even():
    # s = 2^-e exactly (amax = 7 * 2^-e); (k + 1/2) * 2^-e divides to an exact tie
    for e in (0, 7, 30):
        vals = np.array([7, 0.5, 1.5, 2.5, -2.5, 6.5, -0.5, 3.5], np.float64) * 2.0 ** -e
        x = bf16(vals)
        assert np.array_equal(oracle.f32_from_bf16(x).astype(np.float64), vals)
        q4, s, _ = rt(x, 8)
        assert s[0] == np.float32(2.0 ** -e)
        assert list(codes_of(q4, 8)) == [7, 0, 2, 2, -2, 6, 0, 4]


# ------------------------------------------- the gathered, per-shard blocks ----

def _flat_with_block_magnitudes(layout, seed):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 1, layout.psi_pad)
    x *= 2.0 ** rng.integers(-12, 12, size=layout.psi_pad // 64 + 1).repeat(64)[: layout.psi_pad]
    x[layout.psi_part:] = 0.0
    return bf16(x)


def test_gathered_packing_restarts_at_every_shard():
    lay = oracle.Layout([200_003, 7, 150_002], n_d=3)  # S odd: a shard's last byte holds one code
    block = 512
    S = lay.shard
    assert S % 2 == 1 and S % block != 0
    flat = _flat_with_block_magnitudes(lay, 2)
    q4, s = oracle.quantize_gathered_int4(lay, flat, block)
    per_rank = -(-S // block)
    nbytes = -(-S // 2)
    assert q4.size == 3 * nbytes and s.size == 3 * per_rank
    for r in range(3):
        mine, ms = oracle.quantize_int4(np.ascontiguousarray(flat[r * S:(r + 1) * S]), block)
        assert np.array_equal(q4[r * nbytes:(r + 1) * nbytes], mine)
        assert np.array_equal(s[r * per_rank:(r + 1) * per_rank], ms)
        assert int(q4[(r + 1) * nbytes - 1]) >> 4 == 0   # the odd shard's pad nibble
    i = np.array([0, S - 1, S, S + 1, 2 * S - 1, 2 * S, 3 * S - 1])
    assert list(oracle.gathered_code_byte(lay, i)) == [0, (S - 1) // 2, nbytes, nbytes, nbytes + (S - 1) // 2,
                                                       2 * nbytes, 2 * nbytes + (S - 1) // 2]


def _views_for(lay, fill=0x7777):
    return [None if lay.persistent[t] else (np.full(n, fill, np.uint16), 0) for t, n in enumerate(lay.numels)]


@pytest.mark.parametrize("numels,n_d,block", [([200_003, 7, 150_002, 99_999, 130_000], 3, 256),
                                              ([300_000, 50, 211_000], 4, 2048)])
def test_unpack_int4_is_dequantize_of_each_shard(numels, n_d, block):
    lay = oracle.Layout(numels, n_d)
    S = lay.shard
    flat = _flat_with_block_magnitudes(lay, block)
    q4, s = oracle.quantize_gathered_int4(lay, flat, block)
    views = _views_for(lay)
    oracle.unpack_int4(lay, q4, s, block, 0, lay.psi_pad, views)
    back = oracle.pack(lay, views, 0, lay.psi_pad)
    per_rank, nbytes = -(-S // block), -(-S // 2)
    want = np.concatenate([oracle.dequantize_int4(q4[r * nbytes:(r + 1) * nbytes], s[r * per_rank:(r + 1) * per_rank],
                                                  S, block) for r in range(n_d)])
    assert np.array_equal(back[: lay.psi_part], want[: lay.psi_part])
    xf = oracle.f32_from_bf16(flat[: lay.psi_part]).astype(np.float64)
    bf = oracle.f32_from_bf16(back[: lay.psi_part]).astype(np.float64)
    sc = s[oracle.gathered_block(lay, np.arange(lay.psi_part), block)].astype(np.float64)
    assert np.all(np.abs(bf - xf) <= sc * (0.5 + 1e-5) + np.abs(bf) * 2.0 ** -8)


def test_unpack_int4_subranges_match_the_full_range():
    lay = oracle.Layout([200_003, 7, 150_002, 99_999, 130_002], n_d=3)   # S odd
    block = 256
    S = lay.shard
    assert S % 2 == 1
    flat = _flat_with_block_magnitudes(lay, 5)
    q4, s = oracle.quantize_gathered_int4(lay, flat, block)
    full = _views_for(lay, 0)
    oracle.unpack_int4(lay, q4, s, block, 0, lay.psi_pad, full)
    for begin, end in [(0, 1000), (1, 1000), (S - 301, S + 300), (S + 101, 2 * S + 7), (777, lay.psi_pad),
                       (2 * S - 1, 2 * S + 1)]:
        part = _views_for(lay, 0)
        b0 = int(oracle.gathered_code_byte(lay, np.array([begin]))[0])
        g0 = int(oracle.gathered_block(lay, np.array([begin]), block)[0])
        oracle.unpack_int4(lay, q4[b0:].copy(), s[g0:].copy(), block, begin, end, part)
        for t, toff, foff, n in lay.fragments(begin, end):
            assert np.array_equal(part[t][0][toff:toff + n], full[t][0][toff:toff + n]), (begin, end, t)
        touched = {t for t, *_ in lay.fragments(begin, end)}
        for t, v in enumerate(part):
            if v is not None and t not in touched:
                assert np.all(v[0] == 0)
