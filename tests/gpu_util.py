"""Shared pieces of the GPU parity tests (imported by test_gpu_*.py; not a test module)."""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

from decode_attention_kvz_amd import kvz, paged, synth
from oracle import codec
from oracle.alloc import OFF_NONE

MAX_REL = 2e-3   # per output row: max_d |o - r| / max_d |r|


def announce(msg: str):
    print(f"[gpu-test] {msg}", flush=True)


@dataclass
class Layer:
    """One layer of a paged compressed cache on the GPU plus what the oracle needs."""
    pages: torch.Tensor          # natural [B, n_pages_total, 2, Hkv, 16, 128] bf16 (device)
    meta: torch.Tensor           # [n_phys, Hkv, 2, 8] uint8 (device)
    block_table: torch.Tensor    # [B, max_pages] int32 (device)
    seq_lens: torch.Tensor       # [B] int32
    n_comp: torch.Tensor         # [B] int32
    tail: torch.Tensor | None    # [B, 2, Hkv, 16, 128] bf16
    items: torch.Tensor          # device copy of the encode items (kept alive)
    phys_of: np.ndarray          # [B, max_pages] host copy of the block table


def build_layer(arena: paged.SlotArena, pages: torch.Tensor, seq_lens, n_comp, *, seed: int,
                flags: int = 0, with_tail: bool = True, gaac_bases=None) -> Layer:
    """Encode pages [b, p] for p < n_comp[b] into the arena (physical pages in a seeded random
    order) and return the layer.  The tail of sequence b is pages[b, n_comp[b]].  With
    gaac_bases ([Hkv, 2, 2, 128] uint8, device) the pages are encoded in the group-adaptive
    format instead."""
    bsz, n_total, _, hkv = pages.shape[:4]
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    n_comp = np.asarray(n_comp, dtype=np.int64)
    max_pages = max(int(n_comp.max()) if bsz else 0, 1)
    n_phys = int(n_comp.sum())
    rng = np.random.default_rng(seed)
    perm = rng.permutation(max(n_phys, 1))
    block_table = np.zeros((bsz, max_pages), dtype=np.int32)
    page_ids, phys_ids = [], []
    used = 0
    for b in range(bsz):
        for p in range(int(n_comp[b])):
            block_table[b, p] = perm[used]
            page_ids.append((b, p))
            phys_ids.append(perm[used])
            used += 1
    meta = paged.new_meta_table(max(n_phys, 1), hkv, device=pages.device)
    if gaac_bases is None:
        items = paged.page_items(pages, page_ids, meta, phys_ids) if page_ids else None
        d_items = paged.encode(arena, items, flags) if items is not None else None
    else:
        items = paged.gaac_page_items(pages, page_ids, meta, phys_ids, gaac_bases) if page_ids else None
        d_items = paged.gaac_encode(arena, items, flags) if items is not None else None
    tail = None
    if with_tail:
        idx = torch.as_tensor(np.minimum(n_comp, n_total - 1), device=pages.device)
        tail = pages[torch.arange(bsz, device=pages.device), idx].contiguous()
    dev = pages.device
    return Layer(pages=pages, meta=meta,
                 block_table=torch.from_numpy(block_table).to(dev),
                 seq_lens=torch.from_numpy(seq_lens.astype(np.int32)).to(dev),
                 n_comp=torch.from_numpy(n_comp.astype(np.int32)).to(dev),
                 tail=tail, items=d_items, phys_of=block_table)


def run_fused(layer: Layer, arena: paged.SlotArena, q: torch.Tensor, sm_scale: float,
              splits: int = 0) -> torch.Tensor:
    bsz, hq, _ = q.shape
    hkv = layer.meta.shape[1]
    out = torch.empty((bsz, hq, 128), dtype=torch.float32, device=q.device)
    ws = paged.workspace(bsz, hq, hkv, layer.block_table.shape[1], splits, device=q.device)
    kvz.kvz_decode_attention(q, out, arena.arena, layer.meta, layer.block_table, layer.seq_lens,
                             layer.n_comp, layer.tail, sm_scale, ws, splits)
    return out


def run_gaac(layer: Layer, arena: paged.SlotArena, bases: torch.Tensor, q: torch.Tensor,
             sm_scale: float, splits: int = 0) -> torch.Tensor:
    bsz, hq, _ = q.shape
    hkv = layer.meta.shape[1]
    out = torch.empty((bsz, hq, 128), dtype=torch.float32, device=q.device)
    ws = paged.workspace(bsz, hq, hkv, layer.block_table.shape[1], splits, device=q.device)
    kvz.kvz_gaac_decode_attention(q, out, arena.arena, layer.meta, bases, layer.block_table,
                                  layer.seq_lens, layer.n_comp, layer.tail, sm_scale, ws, splits)
    return out


def run_bf16(layer: Layer, q: torch.Tensor, sm_scale: float, splits: int = 0) -> torch.Tensor:
    """Baseline over the same pages, packed by physical page id."""
    bsz, hq, _ = q.shape
    hkv = layer.meta.shape[1]
    n_phys = layer.meta.shape[0]
    nat = torch.zeros((n_phys, 2, hkv, 16, 128), dtype=torch.bfloat16, device=q.device)
    for b in range(bsz):
        nc = int(layer.n_comp[b])
        if nc:
            phys = torch.as_tensor(layer.phys_of[b, :nc], device=q.device, dtype=torch.long)
            nat[phys] = layer.pages[b, :nc]
    store = paged.pack_bf16_pages(nat)
    out = torch.empty((bsz, hq, 128), dtype=torch.float32, device=q.device)
    ws = paged.workspace(bsz, hq, hkv, layer.block_table.shape[1], splits, device=q.device)
    kvz.kvz_bf16_decode_attention(q, out, store, layer.block_table, layer.seq_lens, layer.n_comp,
                                  layer.tail, sm_scale, ws, hkv, splits)
    return out


def _sequence_kv(pages, seq_lens, n_comp, b):
    """K and V of sequence b in token order [T, Hkv, 128] (bit patterns) from the natural pages:
    its compressed pages, then its tail tokens."""
    nc = int(n_comp[b])
    nt = int(seq_lens[b]) - 16 * nc
    hkv = pages.shape[3]
    k = pages[b, :nc, 0].transpose(0, 2, 1, 3).reshape(16 * nc, hkv, 128)
    v = pages[b, :nc, 1].transpose(0, 2, 1, 3).reshape(16 * nc, hkv, 128)
    if nt > 0:
        k = np.concatenate([k, pages[b, nc, 0, :, :nt].transpose(1, 0, 2)])
        v = np.concatenate([v, pages[b, nc, 1, :, :nt].transpose(1, 0, 2)])
    return k, v


def oracle_attention_rows(layer: Layer, q: torch.Tensor, sm_scale: float, batch_indices,
                          effective: dict | None = None):
    """Oracle output for the listed sequences, computed from the natural pages (the values the
    encoder received), not from anything the GPU wrote.  With `effective` (a dict), also the
    number of keys each query head's softmax spreads over, 1 / sum_t w_t^2 (1 for a one-hot
    softmax, T for a uniform one), per sequence: effective[b] = [Hq] array."""
    from oracle import attention
    pages = synth.bits(layer.pages)                         # [B, P, 2, Hkv, 16, 128]
    qb = synth.bits(q)
    seq_lens = layer.seq_lens.cpu().numpy()
    n_comp = layer.n_comp.cpu().numpy()
    out = {}
    for b in batch_indices:
        k, v = _sequence_kv(pages, seq_lens, n_comp, b)
        out[b] = attention.attention_fp64(qb[b], k, v, sm_scale)
        if effective is not None:
            w = attention.softmax_weights_fp64(qb[b], k, sm_scale)
            effective[b] = 1.0 / np.sum(w * w, axis=1) if w.shape[1] else np.zeros(w.shape[0])
    return out


def report_effective(effective: dict, what: str) -> float:
    """Print the smallest and median effective key count over the checked rows; return the
    smallest."""
    allv = np.concatenate([np.asarray(v) for v in effective.values()]) if effective else np.zeros(1)
    announce(f"  {what}: effective keys per head min {allv.min():.1f} median "
             f"{np.median(allv):.1f} over {len(effective)} sequences")
    return float(allv.min())


def scaled_queries(q: torch.Tensor, log2_scale: int) -> torch.Tensor:
    """q times 2**log2_scale (exact in BF16 for these magnitudes): a broader softmax."""
    return (q.float() * (2.0 ** log2_scale)).to(torch.bfloat16) if log2_scale else q


def check_rows(got: np.ndarray, ref: np.ndarray, tol: float = MAX_REL, what: str = ""):
    """Per row max|o - r| / max|r| <= tol; non-finite positions must agree."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    fin_g, fin_r = np.isfinite(got), np.isfinite(ref)
    assert (fin_g == fin_r).all(), f"{what}: non-finite positions differ"
    worst = 0.0
    for row in range(got.shape[0]):
        m = fin_r[row]
        if not m.any():
            continue
        den = np.max(np.abs(ref[row][m]))
        err = np.max(np.abs(got[row][m] - ref[row][m]))
        rel = err / den if den > 0 else err
        worst = max(worst, rel)
    assert worst <= tol, f"{what}: max relative row error {worst:.3e} > {tol}"
    return worst


def sm_scale():
    return 1.0 / math.sqrt(128.0)
