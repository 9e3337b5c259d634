"""Pins the oracle's partition layout and pack/unpack against the pages'
examples and a per-element brute force (explicit enumeration, no interval
arithmetic)."""
import random

import numpy as np
import pytest

import oracle
from oracle import Layout


def brute_force(numels, n_d, threshold):
    """Enumerate every partitioned element in list order as (tensor, index),
    pad with None to a multiple of n_d, deal consecutive runs to the ranks."""
    flat = []
    for t, x in enumerate(numels):
        if x < threshold:
            continue
        for i in range(x):
            flat.append((t, i))
    while len(flat) % n_d:
        flat.append(None)
    per = len(flat) // n_d
    ranks = [flat[r * per:(r + 1) * per] for r in range(n_d)]
    persistent = [t for t, x in enumerate(numels) if x < threshold]
    return flat, ranks, persistent


def expand(fragments):
    out = []
    for t, toff, foff, n in fragments:
        for i in range(n):
            out.append((foff + i, (t, toff + i)))
    return out


def test_eight_params_on_four_gpus(golden):
    g = golden("partition_8params.txt")
    lay = Layout([g["numel"]], g["n_d"], g["threshold"])
    for r in range(g["n_d"]):
        b, e = lay.rank_range(r)
        assert list(range(b, e)) == g[f"rank{r}"]
        assert lay.fragments(b, e) == [(0, g[f"rank{r}"][0], b, 2)]
    # rank 0 holds the first psi / n_d elements, rank 1 the next (tutorial section 2.1)
    assert lay.rank_range(0) == (0, lay.psi // lay.n_d)
    assert lay.rank_range(1)[0] == lay.rank_range(0)[1]


def test_persistence_threshold(golden):
    g = golden("persistence_threshold.txt")
    thr = g["default_threshold"]
    lay = Layout([thr - 1, thr, thr + 1, 1, 0], 4)
    assert lay.threshold == thr == oracle.DEFAULT_PERSIST_THRESHOLD
    assert lay.persistent == [True, False, False, True, True]
    assert lay.psi_persist == thr - 1 + 1
    assert lay.psi_part == 2 * thr + 1
    # persistent tensors never appear in any rank's fragments
    frag_tensors = {f[0] for f in lay.fragments(0, lay.psi_pad)}
    assert frag_tensors == {1, 2}
    # persistent region: list order, contiguous
    assert lay.offset[0] == 0 and lay.offset[3] == thr - 1 and lay.offset[4] == thr


@pytest.mark.parametrize("seed", range(40))
def test_layout_against_brute_force(seed):
    rng = random.Random(seed)
    numels = [rng.choice([0, 1, 2, 3, 5, 8, 13, rng.randrange(0, 50)]) for _ in range(rng.randrange(0, 9))]
    n_d = rng.randrange(1, 10)
    threshold = rng.choice([0, 1, 5, 10**9])
    lay = Layout(numels, n_d, threshold)
    flat, ranks, persistent = brute_force(numels, n_d, threshold)
    assert lay.psi_pad == len(flat)
    assert lay.psi_part == sum(1 for x in flat if x is not None)
    assert [t for t in range(len(numels)) if lay.persistent[t]] == persistent
    # whole-buffer fragments reproduce the enumeration element by element
    whole = dict(expand(lay.fragments(0, lay.psi_pad)))
    assert whole == {j: x for j, x in enumerate(flat) if x is not None}
    for r in range(n_d):
        b, e = lay.rank_range(r)
        got = expand(lay.fragments(b, e))
        want = [(b + i, x) for i, x in enumerate(ranks[r]) if x is not None]
        assert got == want
        for j in range(b, e):
            assert lay.owner(j) == r
    # arbitrary sub-ranges
    for _ in range(10):
        b = rng.randrange(0, lay.psi_pad + 1)
        e = rng.randrange(b, lay.psi_pad + 1)
        got = expand(lay.fragments(b, e))
        want = [(j, flat[j]) for j in range(b, e) if flat[j] is not None]
        assert got == want


def _views(lay, rng, windows=False):
    """Random 16-bit content for every partitioned tensor; optionally as a
    window [first, first+count) that still covers the whole tensor."""
    views = []
    for t, x in enumerate(lay.numels):
        if lay.persistent[t]:
            views.append(None)
            continue
        first = 0
        arr = np.array([rng.randrange(0, 65536) for _ in range(x)], dtype=np.uint16)
        views.append((arr, first))
    return views


@pytest.mark.parametrize("seed", range(30))
def test_pack_unpack_against_brute_force(seed):
    rng = random.Random(1000 + seed)
    numels = [rng.randrange(0, 40) for _ in range(rng.randrange(1, 7))]
    n_d = rng.randrange(1, 8)
    threshold = rng.choice([0, 3, 10])
    lay = Layout(numels, n_d, threshold)
    flat_enum, _, _ = brute_force(numels, n_d, threshold)
    views = _views(lay, rng)
    b = rng.randrange(0, lay.psi_pad + 1)
    e = rng.randrange(b, lay.psi_pad + 1)
    got = oracle.pack(lay, views, b, e)
    want = np.array([0 if flat_enum[j] is None else views[flat_enum[j][0]][0][flat_enum[j][1]]
                     for j in range(b, e)], dtype=np.uint16)
    assert got.dtype == np.uint16 and np.array_equal(got, want)
    # unpack into fresh (sentinel-filled) views writes exactly the covered elements
    sentinel = np.uint16(0xA5A5)
    fresh = [None if v is None else (np.full_like(v[0], sentinel), 0) for v in views]
    oracle.unpack(lay, got, b, e, fresh)
    covered = {flat_enum[j] for j in range(b, e) if flat_enum[j] is not None}
    for t, v in enumerate(views):
        if v is None:
            continue
        for i in range(len(v[0])):
            expect = v[0][i] if (t, i) in covered else sentinel
            assert fresh[t][0][i] == expect


def test_pack_window_views():
    # a view may hold only a window [first, first+count) of its tensor
    lay = Layout([10, 6], 4, 0)
    t0 = np.arange(100, 110, dtype=np.uint16)
    t1 = np.arange(200, 206, dtype=np.uint16)
    b, e = lay.rank_range(2)  # psi_pad = 16, shard 4 -> [8, 12)
    assert (b, e) == (8, 12)
    views = [(t0[8:], 8), (t1[:2], 0)]
    assert list(oracle.pack(lay, views, b, e)) == [108, 109, 200, 201]


def test_gather_example(golden):
    g = golden("gather_example.txt")
    to_bf16 = lambda xs: oracle.bf16_from_f32(np.array(xs, dtype=np.float32))
    lay = Layout([len(g["before"])], g["n_d"], 0)
    shards = [to_bf16(g["rank0_updated"]), to_bf16(g["rank1_updated"])]
    # the AllGather result is the shards in rank order; unpacking it rebuilds W
    gathered = np.concatenate(shards)
    w = to_bf16(g["before"])
    oracle.unpack(lay, gathered, 0, lay.psi_pad, [(w, 0)])
    assert list(oracle.f32_from_bf16(w)) == g["gathered"]
    # and packing each rank's own slice of the updated W gives back its shard
    for r in range(g["n_d"]):
        b, e = lay.rank_range(r)
        assert np.array_equal(oracle.pack(lay, [(w, 0)], b, e), shards[r])


def test_padding_is_zero_and_roundtrip_keeps_bits():
    lay = Layout([7, 3, 11], 4, 0)   # 21 -> padded to 24
    assert lay.psi_pad == 24 and lay.shard == 6
    patterns = [0x7FC1, 0xFFFF, 0x8000, 0x0001, 0x7F80, 0xFF80, 0x0000]
    views = [(np.array((patterns * 3)[:x], dtype=np.uint16), 0) for x in lay.numels]
    flat = oracle.pack(lay, views, 0, lay.psi_pad)
    assert list(flat[21:]) == [0, 0, 0]
    back = [(np.zeros_like(v[0]), 0) for v in views]
    oracle.unpack(lay, flat, 0, lay.psi_pad, back)
    for v, w in zip(views, back):
        assert np.array_equal(v[0], w[0])


def test_large_offsets_are_exact():
    from zr_workloads import FLAT_1T, LLAMA_7B
    lay = Layout(FLAT_1T.numels, FLAT_1T.n_d)
    assert lay.shard == 1_953_125_000
    b, e = lay.rank_range(511)
    assert (b, e) == (511 * 1_953_125_000, 10**12) and b > 2**32
    assert lay.fragments(b, e) == [(0, b, b, 1_953_125_000)]
    llama = Layout(LLAMA_7B.numels, LLAMA_7B.n_d)
    assert llama.psi == 6_738_415_616 and llama.psi_persist == 65 * 4096
    assert llama.psi_pad == llama.psi_part  # 64 divides it: no padding
    frs = llama.fragments(*llama.rank_range(17))
    assert sum(f[3] for f in frs) == llama.shard
    # the shard starts inside one tensor and ends inside another
    first, last = frs[0], frs[-1]
    assert first[1] > 0 and last[1] + last[3] < llama.numels[last[0]]


def test_llama_rank17_fragments_exact():
    """The Llama-style 7B list over 64 ranks, worked out by hand from its
    dimensions (hidden 4096, FFN 11008, vocab 32000, 32 layers; HF
    registration order: embed, then per layer q, k, v, o, gate, up, down and
    two 4096-element norms, then the final norm and the untied head).  The
    norms (4096 < 1e5) are persistent; a tensor may straddle rank edges (blog
    111qqz.com, "ZeRO-3: why parameters can be sharded too": one layer's
    parameters split over GPUs; tutorial cnhsyj.com 2.1: rank r owns the r-th
    contiguous 1/N_d of the flat buffer).

    By hand: embed = 32000*4096 = 131,072,000; one layer's partitioned
    tensors = 4*4096^2 + 3*11008*4096 = 202,375,168; Psi_part = 131,072,000 +
    32*202,375,168 + 131,072,000 = 6,738,149,376, which 64 divides, so
    S = 105,283,584 and rank 17 owns [1,789,820,928, 1,895,104,512).  Layer 8
    starts at 131,072,000 + 8*202,375,168 = 1,750,073,344 (tensor 1 + 9*8 =
    73 is its q): v (74 + 1 = tensor 75) starts at 1,783,627,776, so the shard
    begins 6,193,152 elements into v; o (76) and gate (77) lie inside; up (78)
    starts at 1,862,270,976 and is cut after 32,833,536 of its 45,088,768."""
    from zr_workloads import LLAMA_7B
    lay = Layout(LLAMA_7B.numels, LLAMA_7B.n_d, 100_000)
    assert lay.rank_range(17) == (1_789_820_928, 1_895_104_512)
    assert lay.fragments(*lay.rank_range(17)) == [
        (75, 6_193_152, 1_789_820_928, 10_584_064),
        (76, 0, 1_800_404_992, 16_777_216),
        (77, 0, 1_817_182_208, 45_088_768),
        (78, 0, 1_862_270_976, 32_833_536),
    ]
    # the whole buffer: one fragment per partitioned tensor (291 - 65 norms)
    full = lay.fragments(0, lay.psi_pad)
    assert len(full) == 226 and all(f[1] == 0 and f[3] == lay.numels[f[0]] for f in full)
    # over all 64 ranks: of the 63 interior rank edges, 62 fall strictly
    # inside a tensor and cut it into two partial fragments (edge 32, at
    # 32*S = 3,369,074,688 = 131,072,000 + 16*202,375,168, is the start of
    # layer 16's q), so 124 fragments are partial; no rank holds more than 6
    assert 32 * lay.shard == 131_072_000 + 16 * 202_375_168
    partial, most = 0, 0
    for r in range(lay.n_d):
        frs = lay.fragments(*lay.rank_range(r))
        most = max(most, len(frs))
        partial += sum(1 for t, toff, _, n in frs if toff > 0 or n < lay.numels[t])
    assert (partial, most) == (124, 6)
