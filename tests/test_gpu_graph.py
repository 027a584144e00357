"""The library's launches captured in HIP graphs: every replay equals the eager result.

The benchmark replays graphs of the attention calls and of page completion (encode + free), so
both are checked here over several replays with eager work and synchronization in between.
"""
import math

import numpy as np
import pytest
import torch

from decode_attention_kvz_amd import kvz, paged, synth
from oracle.alloc import SlotPoolModel
from oracle.cache import pool_capacity_granules

from gpu_util import announce, build_layer, run_fused

pytestmark = pytest.mark.gpu


def test_attention_graph_replays_match_eager():
    announce("graph replay: attention")
    pages = synth.kv_pages(4, 33, 8, seed=31, forced_frac=0.05, device="cuda")
    q = synth.queries(4, 32, seed=31, device="cuda")
    seq_lens, n_comp = [16 * 32 + 9, 16 * 20, 16 * 32 + 16, 7], [32, 20, 32, 0]
    arena = paged.SlotArena(int(pages.numel() * 2 * 1.05) + (1 << 20))
    layer = build_layer(arena, pages, seq_lens, n_comp, seed=31)
    eager = run_fused(layer, arena, q, 1 / math.sqrt(128)).clone()
    out = torch.zeros_like(eager)
    ws = paged.workspace(4, 32, 8, layer.block_table.shape[1])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kvz.kvz_decode_attention(q, out, arena.arena, layer.meta, layer.block_table,
                                 layer.seq_lens, layer.n_comp, layer.tail, 1 / math.sqrt(128), ws)
    for rep in range(4):
        out.fill_(float("nan"))
        _ = (q.float() * 2).sum()          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"


def test_encode_and_free_graph_replays_follow_the_pool_model():
    announce("graph replay: encode + free")
    pages = synth.kv_pages(2, 6, 4, seed=32, forced_frac=0.3, device="cuda")
    arena = paged.SlotArena(1 << 20)
    n_items = 2 * 6 * 4 * 2
    meta = paged.new_meta_table(12, 4)
    ids = [(b, p) for b in range(2) for p in range(6)]
    items = torch.from_numpy(paged.page_items(pages, ids, meta, list(range(12)))).cuda()
    ptrs = paged.meta_pointers(meta, np.arange(n_items))
    torch.cuda.synchronize()
    g_enc, g_free = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_enc):
        kvz.kvz_encode_pages(arena.pool, items, n_items)
    with torch.cuda.graph(g_free):
        kvz.kvz_slot_free(arena.pool, ptrs)
    # tags of every item, from the first (eager) encode
    kvz.kvz_encode_pages(arena.pool, items, n_items)
    torch.cuda.synchronize()
    first = meta.cpu().numpy().reshape(-1, 8)
    tags = [list(first[i, 4:]) for i in range(n_items)]
    model = SlotPoolModel(pool_capacity_granules(arena.arena.numel()))
    offs = model.alloc(tags)
    np.testing.assert_array_equal(first[:, :4].copy().view("<u4")[:, 0], np.asarray(offs, np.uint32))
    live = list(zip(offs, tags))
    for rep in range(4):
        _ = pages.float().abs().sum()      # eager work between replays
        torch.cuda.synchronize()
        g_free.replay()
        model.free(live)
        torch.cuda.synchronize()
        cleared = meta.cpu().numpy().reshape(-1, 8)
        assert (cleared[:, :4] == 0xFF).all() and (cleared[:, 4:] == 0).all(), f"free {rep}"
        g_enc.replay()
        offs = model.alloc(tags)
        live = list(zip(offs, tags))
        torch.cuda.synchronize()
        got = meta.cpu().numpy().reshape(-1, 8)
        np.testing.assert_array_equal(got[:, :4].copy().view("<u4")[:, 0],
                                      np.asarray(offs, np.uint32), err_msg=f"encode {rep}")
        assert [list(got[i, 4:]) for i in range(n_items)] == tags
        st = arena.stats()
        assert st["live_runs"] == model.live_runs == n_items
        assert st["free_runs"] == [len(model.bins[k]) for k in range(5)]
        assert st["frontier_granules"] == model.frontier


def test_gaac_attention_graph_replays_match_eager():
    announce("graph replay: GAAC attention")
    cal = synth.kv_pages(2, 8, 8, seed=33, forced_frac=0.05, sample=1, device="cuda")
    bases = paged.gaac_calibrate(cal)
    pages = synth.kv_pages(4, 33, 8, seed=33, forced_frac=0.05, device="cuda")
    q = synth.queries(4, 32, seed=33, device="cuda")
    seq_lens, n_comp = [16 * 32 + 9, 16 * 20, 16 * 32 + 16, 7], [32, 20, 32, 0]
    arena = paged.SlotArena(int(pages.numel() * 2 * 1.05) + (1 << 20))
    layer = build_layer(arena, pages, seq_lens, n_comp, seed=33, gaac_bases=bases)
    ws = paged.workspace(4, 32, 8, layer.block_table.shape[1])
    eager = torch.empty((4, 32, 128), dtype=torch.float32, device="cuda")
    kvz.kvz_gaac_decode_attention(q, eager, arena.arena, layer.meta, bases, layer.block_table,
                                  layer.seq_lens, layer.n_comp, layer.tail, 1 / math.sqrt(128), ws)
    out = torch.zeros_like(eager)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kvz.kvz_gaac_decode_attention(q, out, arena.arena, layer.meta, bases, layer.block_table,
                                      layer.seq_lens, layer.n_comp, layer.tail, 1 / math.sqrt(128), ws)
    for rep in range(4):
        out.fill_(float("nan"))
        _ = (q.float() * 2).sum()          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
