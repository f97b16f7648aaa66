"""One GPU's share of a data-parallel Muon step: whole matrices dealt out round-robin within
each size group. The ownership rule must partition the matrices, balance each size group and
give the shapes the share workloads declare."""
from collections import Counter

import pytest

import seeded_inputs as si


@pytest.mark.parametrize("world", [1, 2, 3, 4, 8])
def test_owned_indices_partition_and_balance(world):
    shapes = si.WORKLOADS["gpt2_124m"].shapes
    parts = [si.owned_indices(shapes, world, r) for r in range(world)]
    flat = [i for p in parts for i in p]
    assert sorted(flat) == list(range(len(shapes)))          # every matrix owned exactly once
    for numel in {r * c for r, c in shapes}:
        counts = [sum(1 for i in p if shapes[i][0] * shapes[i][1] == numel) for p in parts]
        assert max(counts) - min(counts) <= 1                  # each size group balanced


def test_owned_indices_rejects_bad_rank():
    with pytest.raises(ValueError):
        si.owned_indices([(2, 2)], 2, 2)


def test_share_workloads():
    full = si.WORKLOADS["gpt2_124m"]
    for world in (2, 4, 8):
        wl = si.WORKLOADS[f"gpt2_124m_share{world}"]
        assert wl.n == full.n // world
        # 48 square and 24 of the 768 x 3072 size group split evenly; rank 0 draws the fc
        # matrices (3072 x 768) of the interleaved fc / proj order
        assert Counter(wl.shapes) == Counter({(768, 768): 48 // world, (3072, 768): 24 // world})
        assert abs(wl.ns_flops_per_step() * world - full.ns_flops_per_step()) < 1.0
    assert si.WORKLOADS["gpt2_124m_share8"].labels[:5] == ("l0.q", "l0.fc", "l2.q", "l4.q",
                                                          "l4.fc")
