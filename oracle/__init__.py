"""CPU oracle for the exponent-coded KV formats (12-bit BF16 pages, group-adaptive BF16 and FP8
tiles), the slot-pool model, and decode attention over them.

TEST INFRASTRUCTURE ONLY.  Imported by tests/, by the smoke check in __graft_entry__ and by
the CPU-baseline leg of bench.py; never by the HIP library or its binding, and it imports
neither.  Every function is a plain, slow statement of what the pages define; see the module
headers for the passages followed and the pins that check each part.
"""
from . import codec, alloc, cache, attention, gaac, fp8  # noqa: F401
