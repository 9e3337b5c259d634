"""Property tests (hypothesis) of libzr's partition layout against a
per-element brute force, on the CPU (the layout is host code): for any tensor
list, rank count and persistence threshold, every rank's fragments, every
sub-range's fragments, the per-tensor offsets and the stage-3 ledger follow
from enumerating the partitioned elements one by one."""
from hypothesis import given, settings, strategies as st

import zero_sharded_optimizer_zr_amd as zr
from test_oracle_layout import brute_force, expand

lists = st.lists(st.one_of(st.integers(0, 3), st.integers(0, 60)), min_size=0, max_size=10)


@settings(max_examples=300, deadline=None)
@given(numels=lists, n_d=st.integers(1, 9), threshold=st.sampled_from([0, 1, 2, 5, 17, 10**12]),
       cut=st.tuples(st.floats(0, 1), st.floats(0, 1)))
def test_library_layout_equals_the_element_enumeration(numels, n_d, threshold, cut):
    flat, ranks, persistent = brute_force(numels, n_d, threshold)
    lay = zr.zr_layout_create(numels, n_d, threshold)
    info = zr.zr_layout_query(lay)
    assert info["psi_pad"] == len(flat)
    assert info["psi_part"] == sum(1 for x in flat if x is not None)
    assert info["psi_persist"] == sum(numels[t] for t in persistent)
    assert info["shard"] * n_d == len(flat)
    # per-tensor placement: first element's flat index, or the persistent region in list order
    region = 0
    for t, x in enumerate(numels):
        is_persistent, offset = zr.zr_layout_tensor(lay, t)
        assert is_persistent == (t in persistent)
        if is_persistent:
            assert offset == region
            region += x
        elif x > 0:
            assert offset == flat.index((t, 0))
    # every rank's fragments, element by element
    for r in range(n_d):
        b, e = zr.zr_layout_rank_range(lay, r)
        assert (b, e) == (r * info["shard"], (r + 1) * info["shard"])
        want = [(b + i, x) for i, x in enumerate(ranks[r]) if x is not None]
        assert expand(zr.zr_layout_fragments(lay, b, e)) == want
    # an arbitrary sub-range
    lo, hi = sorted(int(c * len(flat)) for c in cut)
    assert expand(zr.zr_layout_fragments(lay, lo, hi)) == [(j, flat[j]) for j in range(lo, hi) if flat[j] is not None]
    # stage 3 keeps 16 bytes per owned element (padding included) plus the replicated persistent state
    assert zr.zr_layout_ledger_bytes(lay, 3) == 16 * info["shard"] + 16 * info["psi_persist"]
