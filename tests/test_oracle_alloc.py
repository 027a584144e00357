"""Pins of the slot-pool model (no GPU): hand-stepped sequences and invariants."""
import numpy as np

from oracle.alloc import SlotPoolModel, OFF_NONE, run_granules

C = [60, 60, 60, 60]          # four compressed blocks -> 12 granules
R1 = [60, 255, 60, 60]        # one raw block -> 13 granules
R4 = [255, 255, 255, 255]     # 16 granules


def test_run_sizes():
    """768 B = 3 granules per compressed block, 1024 B = 4 per raw block."""
    assert [run_granules(k) for k in range(5)] == [12, 13, 14, 15, 16]


def test_hand_stepped_frontier_and_bins():
    p = SlotPoolModel(100)
    assert p.alloc([C, R1, C]) == [0, 12, 25]
    assert p.frontier == 37
    p.free([(12, R1), (0, C)])
    assert p.bins[1] == [12] and p.bins[0] == [0]
    # LIFO per bin in item order; a size class with an empty bin goes to the frontier
    p.free([(25, C)])
    assert p.alloc([C, C, C, R4]) == [25, 0, 37, 49]
    assert p.frontier == 65
    assert p.live_runs == 4 and p.live_granules == 12 * 3 + 16


def test_frontier_requests_are_served_as_a_prefix():
    p = SlotPoolModel(40)
    # 12 + 16 = 28 fits, 28 + 16 = 44 does not, and no later frontier request of the call fits
    assert p.alloc([C, R4, R4, C]) == [0, 12, OFF_NONE, OFF_NONE]
    assert p.frontier == 28 and p.enospc == 2
    assert p.alloc([C]) == [28]
    assert p.alloc([C]) == [OFF_NONE]


def test_free_skips_unplaced_groups():
    p = SlotPoolModel(12)
    offs = p.alloc([C, C])
    p.free([(offs[0], C), (offs[1], C)])
    assert p.bins[0] == [0] and p.live_runs == 0


def test_random_churn_invariants():
    rng = np.random.default_rng(7)
    cap = 5000
    p = SlotPoolModel(cap)
    live = {}
    for step in range(400):
        n = int(rng.integers(0, 12))
        reqs = []
        for _ in range(n):
            k = int(rng.integers(0, 5))
            reqs.append([255] * k + [10] * (4 - k))
        offs = p.alloc(reqs)
        for off, tags in zip(offs, reqs):
            if off != OFF_NONE:
                assert off not in live
                live[off] = tags
        if live and rng.random() < 0.6:
            keys = list(live.keys())
            pick = rng.choice(len(keys), size=int(rng.integers(1, len(keys) + 1)), replace=False)
            victims = [(keys[i], live.pop(keys[i])) for i in pick]
            p.free(victims)
        # no overlap, inside the arena
        spans = sorted((off, off + run_granules(sum(t == 255 for t in tags)))
                       for off, tags in live.items())
        for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
            assert a1 <= b0
        assert all(0 <= a and b <= cap for a, b in spans)
        # conservation: live + binned + unused frontier = capacity
        assert p.live_granules + p.binned_granules() + (cap - p.frontier) == cap
        assert p.live_runs == len(live)
