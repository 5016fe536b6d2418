"""The expert calls of the offloaded layer with pinned experts (host logic,
no GPU): every expert in exactly one call, offloaded groups of at most G
unpinned experts, resident runs maximal and mapped onto consecutive rows of
the pinned weights; and the choice of the most-routed experts."""
import random

import pytest

from mixture_experts_layer_permute_amd.layer import OffloadedMoELayer, offload_groups


@pytest.mark.parametrize("seed", range(40))
def test_offload_groups_cover_every_expert_once(seed):
    r = random.Random(seed)
    E = r.randint(1, 70)
    G = r.randint(1, 9)
    pinned = sorted(r.sample(range(E), r.randint(0, E)))
    groups, resident = offload_groups(E, G, pinned)
    seen = []
    for e0, ne in groups:
        assert 1 <= ne <= G
        assert not set(range(e0, e0 + ne)) & set(pinned)
        seen += range(e0, e0 + ne)
    for e0, ne, p0 in resident:
        assert pinned[p0:p0 + ne] == list(range(e0, e0 + ne))
        assert e0 - 1 not in pinned and e0 + ne not in pinned      # maximal runs
        seen += range(e0, e0 + ne)
    assert sorted(seen) == list(range(E))
    # offloaded groups are cut only at G or at a pinned expert
    for (a0, an), (b0, _) in zip(groups, groups[1:]):
        if b0 == a0 + an:
            assert an == G


def test_offload_groups_without_pins_is_plain_grouping():
    assert offload_groups(8, 3, []) == ([(0, 3), (3, 3), (6, 2)], [])
    assert offload_groups(5, 2, list(range(5))) == ([], [(0, 5, 0)])


def test_most_routed():
    counts = [5, 0, 9, 9, 1, 3, 7, 2]
    assert OffloadedMoELayer.most_routed(counts, 0.25) == [2, 3]
    assert OffloadedMoELayer.most_routed(counts, 0.5) == [0, 2, 3, 6]
    assert OffloadedMoELayer.most_routed([4, 4, 4], 0.3) == [0]       # ties: lower index
    assert OffloadedMoELayer.most_routed(counts, 0.0) == []
    assert OffloadedMoELayer.most_routed(counts, 1.0) == list(range(8))
