"""Lossless 12-bit exponent-coded BF16 KV pages and fused paged decode attention for MI355X.

Submodules:
  kvz    - ctypes binding of libkvz.so (the C-ABI declared in include/kvz.h); importing it
           fails loudly when the library has not been built
  paged  - host-side glue: slot arena, metadata tables, encode items, baseline page store
  synth  - seeded synthetic KV pages and queries
  build  - hipcc build of libkvz.so
"""
