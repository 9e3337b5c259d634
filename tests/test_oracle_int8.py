"""Pins the oracle's symmetric block-wise int8 quantization (the quantized
weight AllGather, ZeRO++ qwZ): exactness on representable blocks, symmetry,
the absmax element, the per-element error bound, zero and short blocks, and
block independence."""
import numpy as np
import pytest

import oracle


def bf16(xs):
    return oracle.bf16_from_f32(np.asarray(xs, dtype=np.float32))


def rt(x, block):
    q, s = oracle.quantize_int8(x, block)
    return q, s, oracle.dequantize_int8(q, s, block)


@pytest.mark.parametrize("block", [4, 256, 1024])
def test_representable_blocks_round_trip_exactly(block):
    rng = np.random.default_rng(block)
    nb = 6
    k = rng.integers(-127, 128, size=(nb, block))
    k[:, 0] = rng.choice([-127, 127], nb)              # every block reaches +-127
    e = rng.integers(-20, 4, size=nb)
    x = (k * (2.0 ** e)[:, None]).astype(np.float32).ravel()
    xb = bf16(x)
    assert np.array_equal(oracle.f32_from_bf16(xb), x)
    q, s, back = rt(xb, block)
    assert np.array_equal(q.reshape(nb, block), k)
    assert np.array_equal(s, (2.0 ** e).astype(np.float32))
    assert np.array_equal(back, xb)


def test_symmetry_and_absmax():
    rng = np.random.default_rng(2)
    x = bf16(rng.normal(0, 0.02, 4096))
    q, s, _ = rt(x, 256)
    qn, sn, _ = rt(x ^ np.uint16(0x8000), 256)         # negate every element
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    xf = oracle.f32_from_bf16(x).reshape(16, 256)
    amax_pos = np.abs(xf).argmax(axis=1)
    qq = q.reshape(16, 256)
    assert np.all(np.abs(qq[np.arange(16), amax_pos]) == 127)
    assert np.all(np.abs(qq) <= 127)


@pytest.mark.parametrize("block,std", [(256, 0.02), (512, 1e-3), (2048, 5.0), (256, 1e-30)])
def test_round_trip_error_bound(block, std):
    rng = np.random.default_rng(int(block + 1e3 * std) % 1000)
    x = bf16(rng.normal(0, std, 50_000))
    q, s, back = rt(x, block)
    xf = oracle.f32_from_bf16(x).astype(np.float64)
    bf = oracle.f32_from_bf16(back).astype(np.float64)
    sc = np.repeat(s.astype(np.float64), block)[: x.size]
    # half a quantization step (plus the fp32 quotient's rounding) and half a bf16 ulp of the result
    bound = sc * (0.5 + 1e-5) + np.abs(bf) * 2.0 ** -8 + 1e-45
    assert np.all(np.abs(bf - xf) <= bound)


def test_zero_block_and_short_tail():
    x = np.zeros(700, dtype=np.uint16)
    x[512:] = bf16(np.linspace(-3, 3, 188))
    q, s, back = rt(x, 256)
    assert s.size == 3 and s[0] == 0 and s[1] == 0 and s[2] > 0
    assert not q[:512].any() and not back[:512].any()
    # the short tail block is quantized on its own
    q3, s3, _ = rt(x[512:].copy(), 256)
    assert np.array_equal(q3, q[512:]) and s3[0] == s[2]


def test_blocks_are_independent():
    rng = np.random.default_rng(9)
    a = bf16(rng.normal(0, 1, 512))
    b = bf16(rng.normal(0, 1e-3, 768))
    qa, sa, _ = rt(a, 256)
    qb, sb, _ = rt(b, 256)
    qab, sab, _ = rt(np.concatenate([a, b]), 256)
    assert np.array_equal(qab, np.concatenate([qa, qb])) and np.array_equal(sab, np.concatenate([sa, sb]))


def test_payload_is_about_half_of_bf16():
    # the quantized AllGather carries 1 byte per element plus one fp32 scale per block
    for block in (256, 512, 1024, 2048):
        n = 116_465_664
        q_bytes = n + 4 * -(-n // block)
        assert q_bytes / (2 * n) == pytest.approx(0.5 + 2 / block, rel=1e-6)


def test_exact_ties_round_to_even():
    # s = 2^-e exactly (amax = 127 * 2^-e); (k + 1/2) * 2^-e divides to an exact tie
    for e in (0, 7, 30):
        vals = np.array([127, 0.5, 1.5, 2.5, -2.5, 126.5, -0.5, 3.5], np.float64) * 2.0 ** -e
        x = bf16(vals)
        assert np.array_equal(oracle.f32_from_bf16(x).astype(np.float64), vals)
        q, s, _ = rt(x, 8)
        assert s[0] == np.float32(2.0 ** -e)
        assert list(q) == [127, 0, 2, 2, -2, 126, 0, 4]


# ------------------------------------------- the gathered, per-shard blocks ----

def _flat_with_block_magnitudes(layout, block, seed):
    """bf16 flat buffer whose blocks (of the shard-relative grid) have very
    different magnitudes, so that a wrong scale for an element shows."""
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 1, layout.psi_pad)
    x *= 2.0 ** rng.integers(-12, 12, size=layout.psi_pad // 64 + 1).repeat(64)[: layout.psi_pad]
    x[layout.psi_part:] = 0.0                          # the padding is zero
    return bf16(x)


def test_gathered_equals_one_grid_when_block_divides_shard():
    lay = oracle.Layout([300_000, 50, 211_000, 120_000], n_d=4)
    block = 256
    pad = (-lay.psi_part) % (4 * block)                # make S a multiple of the block
    lay = oracle.Layout([300_000, 50, 211_000, 120_000 + pad], n_d=4)
    assert lay.shard % block == 0
    flat = _flat_with_block_magnitudes(lay, block, 1)
    q, s = oracle.quantize_gathered(lay, flat, block)
    q1, s1 = oracle.quantize_int8(flat, block)
    assert np.array_equal(q, q1) and np.array_equal(s, s1)


def test_gathered_blocks_restart_at_every_shard():
    lay = oracle.Layout([200_003, 7, 150_001], n_d=3)
    block = 512
    S = lay.shard
    assert S % block != 0
    flat = _flat_with_block_magnitudes(lay, block, 2)
    q, s = oracle.quantize_gathered(lay, flat, block)
    per_rank = -(-S // block)
    assert s.size == 3 * per_rank and q.size == lay.psi_pad
    xf = np.abs(oracle.f32_from_bf16(flat))
    for r in range(3):
        for j in (0, 1, per_rank - 2, per_rank - 1):
            lo, hi = r * S + j * block, min(r * S + (j + 1) * block, (r + 1) * S)
            assert s[r * per_rank + j] == np.float32(xf[lo:hi].max()) / np.float32(127)
    assert S - (per_rank - 1) * block < block           # every shard ends with a short block


def _views_for(lay, seed, fill=0x7777):
    rng = np.random.default_rng(seed)
    views = []
    for t, n in enumerate(lay.numels):
        if lay.persistent[t]:
            views.append(None)
        else:
            views.append((np.full(n, fill, np.uint16), 0))
    return views


@pytest.mark.parametrize("block", [256, 2048])
def test_unpack_int8_error_bound_per_element(block):
    lay = oracle.Layout([200_003, 7, 150_001, 99_999, 130_000], n_d=3)
    flat = _flat_with_block_magnitudes(lay, block, block)
    q, s = oracle.quantize_gathered(lay, flat, block)
    views = _views_for(lay, 0)
    oracle.unpack_int8(lay, q, s, block, 0, lay.psi_pad, views)
    back = oracle.pack(lay, views, 0, lay.psi_pad)
    i = np.arange(lay.psi_part)
    sc = s[oracle.gathered_block(lay, i, block)].astype(np.float64)
    xf = oracle.f32_from_bf16(flat[: lay.psi_part]).astype(np.float64)
    bf = oracle.f32_from_bf16(back[: lay.psi_part]).astype(np.float64)
    assert np.all(np.abs(bf - xf) <= sc * (0.5 + 1e-5) + np.abs(bf) * 2.0 ** -8)
    # and the scale really is the block's own: each rebuilt element is a code times it
    qq = q[: lay.psi_part].astype(np.float64)
    assert np.array_equal(back[: lay.psi_part], bf16((qq * sc).astype(np.float32)))


def test_unpack_int8_subranges_match_the_full_range():
    lay = oracle.Layout([200_003, 7, 150_001, 99_999, 130_000], n_d=3)
    block = 256
    S = lay.shard
    flat = _flat_with_block_magnitudes(lay, block, 5)
    q, s = oracle.quantize_gathered(lay, flat, block)
    full = _views_for(lay, 0)
    oracle.unpack_int8(lay, q, s, block, 0, lay.psi_pad, full)
    for begin, end in [(0, 1000), (S - 300, S + 300), (S + 100, 2 * S + 7), (777, lay.psi_pad), (2 * S - 1, 2 * S + 1)]:
        part = _views_for(lay, 0)
        g0 = int(oracle.gathered_block(lay, np.array([begin]), block)[0])
        oracle.unpack_int8(lay, q[begin:end].copy(), s[g0:].copy(), block, begin, end, part)
        for t, toff, foff, n in lay.fragments(begin, end):
            assert np.array_equal(part[t][0][toff:toff + n], full[t][0][toff:toff + n]), (begin, end, t)
        # nothing outside the range is written
        touched = {t for t, *_ in lay.fragments(begin, end)}
        for t, v in enumerate(part):
            if v is not None and t not in touched:
                assert np.all(v[0] == 0x7777)
