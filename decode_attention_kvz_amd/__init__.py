"""Lossless exponent-coded KV pages (12-bit BF16 pages, group-adaptive BF16 and FP8 tiles) and
fused paged decode attention for MI355X.

Submodules:
  kvz    - ctypes binding of libkvz.so (the C-ABI declared in include/kvz.h); importing it
           fails loudly when the library has not been built
  paged  - host-side glue: slot arenas (BF16 and FP8 pools), metadata tables, encode items,
           calibration calls, the uncompressed BF16 / FP8 page stores
  synth  - seeded synthetic KV pages (BF16, and FP8 by conversion) and queries
  build  - hipcc build of libkvz.so
"""
