"""Host-side glue for a paged, exponent-coded KV cache built on the C-ABI.

Owns device buffers (torch tensors): the slot arena and pool state shared by all layers, one
8-byte-metadata table per layer, and the baseline's BF16 page store.  Every operation on the data
is a library call; this module only lays out records and pointers.
"""
from __future__ import annotations

import numpy as np
import torch

from . import kvz

PAGE = 16
HEAD_DIM = 128
GROUP_ELEMS = PAGE * HEAD_DIM


class SlotArena:
    """A pool arena plus its device state (one per device, shared by every layer).  fp8=True
    makes a pool of FP8 tiles (128-byte granules, kvz_fp8_pool_init)."""

    def __init__(self, arena_bytes: int, device="cuda", fp8: bool = False):
        arena_bytes = (int(arena_bytes) + 255) // 256 * 256
        self.device = torch.device(device)
        self.fp8 = fp8
        self.granule = kvz.FP8_GRANULE if fp8 else kvz.GRANULE
        self.arena = torch.zeros(arena_bytes, dtype=torch.uint8, device=self.device)
        state_bytes = (kvz.kvz_fp8_pool_state_bytes if fp8 else kvz.kvz_pool_state_bytes)(arena_bytes)
        self.state = torch.zeros(state_bytes, dtype=torch.uint8, device=self.device)
        self.pool = (kvz.kvz_fp8_pool_init if fp8 else kvz.kvz_pool_init)(self.arena, self.state)

    def stats(self) -> dict:
        return kvz.kvz_pool_stats(self.pool)

    def close(self):
        if self.pool is not None:
            kvz.kvz_pool_destroy(self.pool)
            self.pool = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def new_meta_table(n_phys: int, n_kv: int, device="cuda") -> torch.Tensor:
    """[n_phys, Hkv, 2 (K,V), 8] uint8 metadata, every group marked 'not stored'."""
    t = torch.zeros((n_phys, n_kv, 2, 8), dtype=torch.uint8, device=device)
    t[..., :4] = 0xFF
    return t


def page_items(pages: torch.Tensor, page_ids, meta: torch.Tensor, phys_ids) -> np.ndarray:
    """kvz_encode_item records for pages[s, p] (natural [n_seq, n_pages, 2, Hkv, 16, 128] bf16,
    or uint8 FP8 pages) stored as physical page phys_ids[k] for (s, p) = page_ids[k].  The row
    stride is 128 elements (bytes for FP8).

    Item order: page_ids order, then KV head, then K before V."""
    n_kv = pages.shape[3]
    n_pages = pages.shape[1]
    assert pages.is_contiguous() and meta.is_contiguous()
    sp = np.asarray(page_ids, dtype=np.int64).reshape(-1, 2)
    phys = np.asarray(phys_ids, dtype=np.int64).reshape(-1)
    h = np.arange(n_kv, dtype=np.int64)
    kind = np.arange(2, dtype=np.int64)
    src_group = (((sp[:, 0:1, None] * n_pages + sp[:, 1:2, None]) * 2 + kind[None, None, :])
                 * n_kv + h[None, :, None])                               # [n, Hkv, 2]
    dst_group = (phys[:, None, None] * n_kv + h[None, :, None]) * 2 + kind[None, None, :]
    src = pages.data_ptr() + src_group.reshape(-1) * (GROUP_ELEMS * pages.element_size())
    dst = meta.data_ptr() + dst_group.reshape(-1) * 8
    kinds = np.broadcast_to(kind[None, None, :], src_group.shape).reshape(-1)
    return kvz.encode_items(src.astype(np.uint64), dst.astype(np.uint64), HEAD_DIM, kinds)


def encode(arena: SlotArena, items: np.ndarray, flags: int = 0, stream=None) -> torch.Tensor:
    """Copy the item records to the device and run kvz_encode_pages; returns the device copy
    (keep it alive until the stream has consumed it)."""
    d = torch.from_numpy(np.ascontiguousarray(items)).to(arena.device)
    n = items.size // kvz.ENCODE_ITEM_DTYPE.itemsize
    kvz.kvz_encode_pages(arena.pool, d, n, flags, stream)
    return d


def meta_pointers(meta: torch.Tensor, groups) -> torch.Tensor:
    """Device int64 tensor of pointers to the metadata records with flat indices `groups`."""
    g = np.asarray(groups, dtype=np.int64)
    return torch.from_numpy(meta.data_ptr() + g * 8).to(meta.device)


def meta_host(meta: torch.Tensor) -> np.ndarray:
    """Metadata table as a host structured view: off uint32, tags uint8[4]."""
    raw = meta.detach().cpu().contiguous().numpy().reshape(-1, 8)
    return raw


def pack_bf16_pages(pages_by_phys: torch.Tensor) -> torch.Tensor:
    """Baseline page store [n_phys, 2, Hkv, 4, 1024] uint8 from natural pages
    [n_phys, 2, Hkv, 16, 128] bf16 (kvz_bf16_pack_pages)."""
    n, _, hkv = pages_by_phys.shape[:3]
    dst = torch.empty((n, 2, hkv, 4, 1024), dtype=torch.uint8, device=pages_by_phys.device)
    kvz.kvz_bf16_pack_pages(pages_by_phys.contiguous(), dst)
    return dst


def gaac_page_items(pages: torch.Tensor, page_ids, meta: torch.Tensor, phys_ids,
                    bases: torch.Tensor) -> np.ndarray:
    """kvz_gaac_item records, in page_items order; bases: [Hkv, 2 (K,V), 2 (b3,b4), 128] uint8
    of this layer (device)."""
    rec = page_items(pages, page_ids, meta, phys_ids).view(kvz.ENCODE_ITEM_DTYPE)
    n_kv = pages.shape[3]
    assert bases.is_contiguous() and tuple(bases.shape) == (n_kv, 2, 2, HEAD_DIM)
    n = rec.shape[0]
    h = np.tile(np.repeat(np.arange(n_kv, dtype=np.int64), 2), n // (2 * n_kv))
    kind = rec["kind"].astype(np.int64)
    bases_ptr = bases.data_ptr() + (h * 2 + kind) * 256
    return kvz.gaac_items(rec["src"], rec["dst"], HEAD_DIM, kind, bases_ptr.astype(np.uint64))


def gaac_calibrate(pages: torch.Tensor, device="cuda") -> torch.Tensor:
    """Bases [Hkv, 2, 2, 128] uint8 from calibration pages [n_seq, n_pages, 2, Hkv, 16, 128] bf16
    (device): one kvz_gaac_calibrate call per (K|V, KV head)."""
    n_kv = pages.shape[3]
    assert pages.is_contiguous()
    bases = torch.zeros((n_kv, 2, 2, HEAD_DIM), dtype=torch.uint8, device=device)
    hist = torch.empty(128 * 256, dtype=torch.int32, device=device)
    n_pg = pages.shape[0] * pages.shape[1]
    keep = []
    for h in range(n_kv):
        for kind in range(2):
            g = (np.arange(n_pg, dtype=np.int64) * 2 + kind) * n_kv + h
            src = pages.data_ptr() + g * (GROUP_ELEMS * 2)
            items = torch.from_numpy(kvz.encode_items(src.astype(np.uint64), np.zeros(n_pg, np.uint64),
                                                      HEAD_DIM, np.full(n_pg, kind))).to(device)
            keep.append(items)
            kvz.kvz_gaac_calibrate(items, n_pg, hist, bases[h, kind])
    torch.cuda.synchronize()
    return bases


def gaac_encode(arena: SlotArena, items: np.ndarray, flags: int = 0, stream=None) -> torch.Tensor:
    d = torch.from_numpy(np.ascontiguousarray(items)).to(arena.device)
    n = items.size // kvz.GAAC_ITEM_DTYPE.itemsize
    kvz.kvz_gaac_encode_pages(arena.pool, d, n, flags, stream)
    return d


def gaac_decompress_pages(arena: SlotArena, meta: torch.Tensor, bases: torch.Tensor,
                          out: torch.Tensor | None = None) -> torch.Tensor:
    n, hkv = meta.shape[0], meta.shape[1]
    if out is None:
        out = torch.empty((n, 2, hkv, 4, 1024), dtype=torch.uint8, device=meta.device)
    kvz.kvz_gaac_decompress_pages(arena.arena, meta, bases, out)
    return out


def decompress_pages(arena: "SlotArena", meta: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Decompress-first: every group of the meta table [n_phys, Hkv, 2, 8] rebuilt into the
    baseline page store [n_phys, 2, Hkv, 4, 1024] uint8 (kvz_decompress_pages)."""
    n, hkv = meta.shape[0], meta.shape[1]
    if out is None:
        out = torch.empty((n, 2, hkv, 4, 1024), dtype=torch.uint8, device=meta.device)
    kvz.kvz_decompress_pages(arena.arena, meta, out)
    return out


def workspace(batch: int, num_q_heads: int, num_kv_heads: int, max_pages: int, splits: int = 0,
              device="cuda") -> torch.Tensor:
    nbytes = kvz.kvz_attn_workspace_bytes(batch, num_q_heads, num_kv_heads, max_pages, splits)
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)   # the merge counters start at 0


# ---------------------------------------------------------------------------------------------
# FP8 tiles
# ---------------------------------------------------------------------------------------------
def fp8_page_items(pages: torch.Tensor, page_ids, meta: torch.Tensor, phys_ids,
                   bases: torch.Tensor) -> np.ndarray:
    """kvz_fp8_item records for uint8 FP8 pages [n_seq, n_pages, 2, Hkv, 16, 128], in
    page_items order; bases [Hkv, 2, 2, 128] uint8 of this layer (device)."""
    assert pages.dtype == torch.uint8
    return gaac_page_items(pages, page_ids, meta, phys_ids, bases)


def fp8_encode(arena: SlotArena, items: np.ndarray, fmt: int, flags: int = 0,
               stream=None) -> torch.Tensor:
    assert arena.fp8, "FP8 tiles need an FP8 pool"
    d = torch.from_numpy(np.ascontiguousarray(items)).to(arena.device)
    n = items.size // kvz.FP8_ITEM_DTYPE.itemsize
    kvz.kvz_fp8_encode_pages(arena.pool, d, n, fmt, flags, stream)
    return d


def fp8_calibrate(pages: torch.Tensor, fmt: int, device="cuda") -> torch.Tensor:
    """Bases [Hkv, 2, 2, 128] uint8 from FP8 calibration pages [n_seq, n_pages, 2, Hkv, 16, 128]
    uint8 (device): one kvz_fp8_calibrate call per (K|V, KV head)."""
    n_kv = pages.shape[3]
    assert pages.is_contiguous() and pages.dtype == torch.uint8
    bases = torch.zeros((n_kv, 2, 2, HEAD_DIM), dtype=torch.uint8, device=device)
    hist = torch.empty(128 * 32, dtype=torch.int32, device=device)
    n_pg = pages.shape[0] * pages.shape[1]
    keep = []
    for h in range(n_kv):
        for kind in range(2):
            g = (np.arange(n_pg, dtype=np.int64) * 2 + kind) * n_kv + h
            src = pages.data_ptr() + g * GROUP_ELEMS
            items = torch.from_numpy(kvz.gaac_items(src.astype(np.uint64), np.zeros(n_pg, np.uint64),
                                                    HEAD_DIM, np.full(n_pg, kind),
                                                    np.zeros(n_pg, np.uint64))).to(device)
            keep.append(items)
            kvz.kvz_fp8_calibrate(items, n_pg, fmt, hist, bases[h, kind])
    torch.cuda.synchronize()
    return bases


def fp8_decompress_pages(arena: SlotArena, meta: torch.Tensor, bases: torch.Tensor, fmt: int,
                         out: torch.Tensor | None = None) -> torch.Tensor:
    """Every tile of the meta table [n_phys, Hkv, 2, 8] rebuilt into uncompressed FP8 pages
    [n_phys, 2, Hkv, 2048] uint8 (kvz_fp8_decompress_pages)."""
    n, hkv = meta.shape[0], meta.shape[1]
    if out is None:
        out = torch.empty((n, 2, hkv, 2048), dtype=torch.uint8, device=meta.device)
    kvz.kvz_fp8_decompress_pages(arena.arena, meta, bases, fmt, out)
    return out


def pack_fp8_pages(pages_by_phys: torch.Tensor) -> torch.Tensor:
    """Uncompressed FP8 pages [n_phys, 2, Hkv, 2048] uint8 (the FP8 chunk layout) from natural
    FP8 pages [n_phys, 2, Hkv, 16, 128] uint8 (kvz_fp8_pack_pages)."""
    n, _, hkv = pages_by_phys.shape[:3]
    dst = torch.empty((n, 2, hkv, 2048), dtype=torch.uint8, device=pages_by_phys.device)
    kvz.kvz_fp8_pack_pages(pages_by_phys.contiguous(), dst)
    return dst
