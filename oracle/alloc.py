"""CPU model of the two-size-class slot pool.

TEST INFRASTRUCTURE ONLY (see oracle/codec.py for who may import it).

What it follows:
  * "GAAC: Lossless KV Compression for Bandwidth-Efficient LLM Inference on Personal Devices",
    section "Block-Wise Compression Scheduling": fixed-capacity slots in two storage classes
    (compressed slots and raw BF16 blocks); a block that does not fit keeps its BF16 form.
  * "ZipFusion ...", section "How it works": the memory manager frees chunks in one layer for
    reuse by another; a group's blocks are located from the first block's offset plus prefix-
    summed sizes, so the four blocks of a group are one contiguous run.

Readings: slots are 768 B (3 granules of 256 B) and 1024 B (4 granules);
a group takes one contiguous run of 12 + n_raw granules.  Free runs are kept in five LIFO bins
keyed by n_raw.  Allocation, in item order: pop the bin for that n_raw if it is not empty;
otherwise take the run from the frontier.  Frontier requests of one call are served as a
prefix: request r (in item order among the call's frontier requests) succeeds iff
F + (sum of the sizes of frontier requests up to and including r) <= capacity, and then sits at
F + (sum of the sizes before it); failures return OFF_NONE.  Free, in item order: push the run
on the bin for its n_raw.

Pins (tests/test_oracle_alloc.py): hand-stepped sequences, and invariants checked after random
churn - live runs never overlap, every run is inside [0, capacity), and live + binned + unused
frontier granules equal the capacity.
"""
from __future__ import annotations

OFF_NONE = 0xFFFFFFFF
RAW_TAG = 0xFF
N_BINS = 5


def run_granules(k: int) -> int:
    """Granules of a group run with k raw blocks: 3 per compressed block, 4 per raw block."""
    return 3 * (4 - k) + 4 * k


def n_raw_of(tags) -> int:
    return sum(1 for t in tags if int(t) == RAW_TAG)


class SlotPoolModel:
    def __init__(self, capacity_granules: int):
        self.capacity = int(capacity_granules)
        self.frontier = 0
        self.bins = [[] for _ in range(N_BINS)]
        self.enospc = 0
        self.live_runs = 0
        self.live_granules = 0
        self.raw_blocks = 0

    def alloc(self, tag_list):
        """tag_list: sequence of 4-tag groups, in item order.  Returns a list of offsets."""
        offs = []
        pending = 0                      # sizes of this call's frontier requests so far
        granted = 0                      # granules granted from the frontier in this call
        for tags in tag_list:
            k = n_raw_of(tags)
            size = run_granules(k)
            if self.bins[k]:
                off = self.bins[k].pop()
            else:
                start = self.frontier + pending
                pending += size
                if self.frontier + pending <= self.capacity:
                    off = start
                    granted += size
                else:
                    off = OFF_NONE
            if off == OFF_NONE:
                self.enospc += 1
            else:
                self.live_runs += 1
                self.live_granules += size
                self.raw_blocks += k
            offs.append(off)
        self.frontier += granted
        return offs

    def free(self, metas):
        """metas: sequence of (off, tags) in item order.  Runs with off == OFF_NONE are skipped."""
        for off, tags in metas:
            if int(off) == OFF_NONE:
                continue
            k = n_raw_of(tags)
            self.bins[k].append(int(off))
            self.live_runs -= 1
            self.live_granules -= run_granules(k)
            self.raw_blocks -= k

    def binned_granules(self) -> int:
        return sum(len(self.bins[k]) * run_granules(k) for k in range(N_BINS))
