"""CPU model of page-completion encoding into a slot arena, and of reading a group back.

TEST INFRASTRUCTURE ONLY (see oracle/codec.py for who may import it).

Follows "GAAC: ..." section "Block-Wise Compression Scheduling" (a completed page is encoded
once; its compressed segments become the cache representation; the block table records where
and how each block is stored) and the "How it works" metadata paragraph of "ZipFusion: ...".
Composes oracle.codec (the format) and oracle.alloc (the slot pool model) in item order;
GaacOracleCache does the same with oracle.gaac, whose tiles take runs of 12 or 16 granules of
the same pool.
"""
from __future__ import annotations

import numpy as np

from . import codec, fp8, gaac
from .alloc import SlotPoolModel, OFF_NONE


def pool_capacity_granules(arena_bytes: int) -> int:
    """Usable granules of an arena: whole 256-byte granules, minus one kept as a guard."""
    return max(int(arena_bytes) // codec.GRANULE_BYTES - 1, 0)


class OracleCache:
    """An arena of `arena_bytes` bytes plus a slot pool model, filled by encode()."""

    def __init__(self, arena_bytes: int):
        self.arena = np.zeros(int(arena_bytes), dtype=np.uint8)
        self.pool = SlotPoolModel(pool_capacity_granules(arena_bytes))

    def encode(self, pages, kinds, force_raw: bool = False):
        """Encode groups in item order.

        pages: uint16 [n, 16, 128] natural-order K or V pages; kinds: n values in {0, 1}.
        Returns metas: list of (off, tags) with off == OFF_NONE where the pool had no room
        (that page then keeps its BF16 form and is not written).
        """
        pages = np.asarray(pages, dtype=np.uint16).reshape(-1, codec.PAGE_TOKENS, codec.HEAD_DIM)
        encoded = [codec.encode_group(pages[n], int(kinds[n]), force_raw=force_raw)
                   for n in range(pages.shape[0])]
        offs = self.pool.alloc([tags for tags, _ in encoded])
        metas = []
        for (tags, rec), off in zip(encoded, offs):
            if off != OFF_NONE:
                at = off * codec.GRANULE_BYTES
                self.arena[at:at + rec.size] = rec
            metas.append((off, [int(t) for t in tags]))
        return metas

    def free(self, metas):
        self.pool.free(metas)

    def page(self, meta, kind: int) -> np.ndarray:
        off, tags = meta
        assert off != OFF_NONE
        return codec.decode_group(self.arena, off, tags, kind)


def metas_to_array(metas) -> np.ndarray:
    """List of (off, tags) -> uint8 [n, 8] in the 8-byte metadata layout."""
    out = np.zeros((len(metas), 8), dtype=np.uint8)
    for n, (off, tags) in enumerate(metas):
        out[n] = np.frombuffer(codec.meta_bytes(off, tags), dtype=np.uint8)
    return out


class GaacOracleCache(OracleCache):
    """The same arena and pool model, filled with group-adaptive tiles."""

    def encode_gaac(self, pages, kinds, bases, force_raw: bool = False):
        """pages: uint16 [n, 16, 128]; kinds: n values; bases: n pairs (b3 [128], b4 [128]).
        Returns metas: list of (off, tags) with tags 00x4 (compressed) or FFx4 (raw)."""
        pages = np.asarray(pages, dtype=np.uint16).reshape(-1, codec.PAGE_TOKENS, codec.HEAD_DIM)
        encoded = [gaac.encode_tile(pages[n], int(kinds[n]), bases[n][0], bases[n][1], force_raw)
                   for n in range(pages.shape[0])]
        offs = self.pool.alloc([gaac.tags_of(raw) for raw, _ in encoded])
        metas = []
        for (raw, rec), off in zip(encoded, offs):
            if off != OFF_NONE:
                at = off * codec.GRANULE_BYTES
                self.arena[at:at + rec.size] = rec
            metas.append((off, gaac.tags_of(raw)))
        return metas

    def gaac_page(self, meta, kind: int, b3, b4) -> np.ndarray:
        off, tags = meta
        assert off != OFF_NONE
        raw = tags == gaac.TAGS_RAW
        at = off * codec.GRANULE_BYTES
        size = gaac.RAW_TILE_BYTES if raw else gaac.SLOT_BYTES
        return gaac.decode_tile(self.arena[at:at + size], raw, kind, b3, b4)


class Fp8OracleCache:
    """An arena of FP8 tiles: the same slot pool model over 128-byte granules (a compressed
    E4M3 / E5M2 tile takes 15 / 13 granules, a raw tile 16; see oracle/fp8.py)."""

    def __init__(self, arena_bytes: int, fk: int):
        self.fk = fk
        self.arena = np.zeros(int(arena_bytes), dtype=np.uint8)
        self.pool = SlotPoolModel(max(int(arena_bytes) // fp8.GRANULE_BYTES - 1, 0))

    def encode(self, pages, kinds, bases, force_raw: bool = False):
        """pages: uint8 [n, 16, 128] FP8 tiles; kinds: n values; bases: n pairs (b3, b4).
        Returns metas: list of (off, tags), off == OFF_NONE where the pool had no room."""
        pages = np.asarray(pages, dtype=np.uint8).reshape(-1, fp8.TILE_TOKENS, fp8.HEAD_DIM)
        encoded = [fp8.encode_tile(pages[n], int(kinds[n]), self.fk, bases[n][0], bases[n][1],
                                   force_raw) for n in range(pages.shape[0])]
        offs = self.pool.alloc([fp8.tags_of(raw, self.fk) for raw, _ in encoded])
        metas = []
        for (raw, rec), off in zip(encoded, offs):
            if off != OFF_NONE:
                at = off * fp8.GRANULE_BYTES
                self.arena[at:at + rec.size] = rec
            metas.append((off, fp8.tags_of(raw, self.fk)))
        return metas

    def free(self, metas):
        self.pool.free(metas)

    def page(self, meta, kind: int, b3, b4) -> np.ndarray:
        off, tags = meta
        assert off != OFF_NONE
        raw = list(tags) == fp8.TAGS_RAW
        at = off * fp8.GRANULE_BYTES
        size = fp8.RAW_TILE_BYTES if raw else fp8.slot_bytes(self.fk)
        return fp8.decode_tile(self.arena[at:at + size], raw, kind, self.fk, b3, b4)
