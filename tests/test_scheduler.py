"""Properties of the split-KV partition (CPU reference of the scheduler)."""

import numpy as np
import pytest

from oracle.schedule import blocks_per_unit, schedule, segments


def check_partition(nb, P, pen=2):
    sched, splits = schedule(nb, P, pen)
    U = len(nb)
    seen = {}
    per_part_cost = []
    for p, row in enumerate(sched):
        segs = segments(nb, row)
        cost = 0
        for (u, k0, k1, s) in segs:
            for k in range(k0, k1):
                assert (u, k) not in seen, "block assigned twice"
                seen[(u, k)] = (p, s)
            cost += (k1 - k0) + pen
        per_part_cost.append(cost)
    assert len(seen) == sum(nb), "some block was not assigned"
    for u in range(U):
        n = splits[u + 1] - splits[u]
        if nb[u] == 0:
            assert n == 0
            continue
        parts = sorted({seen[(u, k)][0] for k in range(nb[u])})
        assert n == len(parts)
        # split indices enumerate the unit's segments 0..n-1 in order
        idx = [seen[(u, k)][1] for k in range(nb[u])]
        assert sorted(set(idx)) == list(range(n))
        assert all(np.diff(idx) >= 0)
    T = sched[0][5]
    total = sum(c + pen for c in nb if c > 0)
    assert T == max(1, -(-total // P))
    # each part's block count is within the budget
    for p, row in enumerate(sched):
        blocks = sum(k1 - k0 for (_, k0, k1, _) in segments(nb, row))
        assert blocks <= T
    return sched, splits


@pytest.mark.parametrize("seed", range(20))
def test_random_partitions(seed):
    rng = np.random.default_rng(seed)
    U = int(rng.integers(1, 60))
    nb = [int(x) for x in rng.integers(0, 40, size=U)]
    P = int(rng.integers(1, 300))
    check_partition(nb, P)


def test_edge_partitions():
    check_partition([0, 0, 0], 4)
    check_partition([1], 1)
    check_partition([1], 256)
    check_partition([5, 0, 2], 256)
    check_partition([64] * 128, 128)
    check_partition([100] * 3, 7)


def test_uniform_units_one_per_part():
    """128 equal units on 128 parts: no unit is split."""
    sched, splits = check_partition([64] * 128, 128)
    assert splits[-1] == 128


def test_blocks_per_unit():
    assert blocks_per_unit([0, 1, 64, 65], 1, 0) == [0, 1, 1, 2]
    assert blocks_per_unit([10, 10], 2, 100) == [2, 2, 2, 2]
