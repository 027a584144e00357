"""Decompress-first pipeline: kvz_decompress_pages rebuilds whole pages into the uncompressed
layout (bit-exact against the oracle's raw group records of the input pages), and attention
over the rebuilt pages equals the fused attention over the compressed ones."""
import numpy as np
import pytest
import torch

from decode_attention_kvz_amd import kvz, paged, synth
from oracle import codec

from gpu_util import (announce, build_layer, check_rows, oracle_attention_rows, run_fused,
                      sm_scale)

pytestmark = pytest.mark.gpu


def _natural_by_phys(layer):
    """Host natural pages indexed by physical page: [n_phys, 2, Hkv, 16, 128] uint16."""
    nat = synth.bits(layer.pages)                     # [B, P, 2, Hkv, 16, 128]
    n_phys = layer.meta.shape[0]
    out = np.zeros((n_phys,) + nat.shape[2:], dtype=np.uint16)
    n_comp = layer.n_comp.cpu().numpy()
    for b in range(nat.shape[0]):
        for p in range(int(n_comp[b])):
            out[layer.phys_of[b, p]] = nat[b, p]
    return out


def _oracle_raw_store(nat_phys, groups):
    """Expected bytes of the listed groups (phys, kind, kvh): the oracle's all-raw record of the
    natural page, i.e. the uncompressed chunk layout."""
    return {g: codec.encode_group(nat_phys[g[0], g[1], g[2]], g[1], force_raw=True)[1]
            for g in groups}


@pytest.mark.parametrize("stress", [False, True])
def test_decompress_pages_bit_exact_against_oracle(stress):
    announce(f"decompress pages: 3 sequences, 4 KV heads, stress={stress}")
    pages = synth.kv_pages(3, 21, 4, seed=51, forced_frac=0.15, stress=stress, device="cuda")
    arena = paged.SlotArena(3 * 21 * 4 * 2 * 4096 + (1 << 20))
    layer = build_layer(arena, pages, [16 * 20 + 3, 16 * 13, 16 * 20], [20, 13, 20], seed=51)
    store = paged.decompress_pages(arena, layer.meta)
    torch.cuda.synchronize()
    got = store.cpu().numpy()                          # [n_phys, 2, Hkv, 4, 1024]
    nat = _natural_by_phys(layer)
    n_phys, hkv = layer.meta.shape[0], layer.meta.shape[1]
    groups = [(p, k, h) for p in range(n_phys) for k in range(2) for h in range(hkv)]
    want = _oracle_raw_store(nat, groups)
    for (p, k, h), rec in want.items():
        np.testing.assert_array_equal(got[p, k, h].reshape(-1), rec, err_msg=f"group {(p, k, h)}")
    # the same bytes as packing the natural pages directly
    packed = paged.pack_bf16_pages(torch.from_numpy(nat.view(np.int16)).cuda().view(torch.bfloat16))
    assert torch.equal(store, packed)
    tags = layer.meta.cpu().numpy()[..., 4:]
    announce(f"decompress pages: raw block fraction {(tags == 0xFF).mean():.3f}")
    if stress:     # zeros, subnormals and Inf/NaN in nearly every block: all raw
        assert (tags == 0xFF).mean() > 0.99
    else:
        assert 0 < (tags == 0xFF).mean() < 1


def test_decompress_pages_unstored_and_out_of_arena_groups_are_zero():
    announce("decompress pages: unstored / out-of-arena groups")
    pages = synth.kv_pages(1, 4, 2, seed=52, forced_frac=0.1, device="cuda")
    arena = paged.SlotArena(1 << 20)
    layer = build_layer(arena, pages, [64], [4], seed=52, with_tail=False)
    meta = layer.meta.clone()
    m = meta.cpu().numpy()
    m[0, 0, 0, :4] = 0xFF                                            # not stored
    m[1, 1, 1, :4] = np.frombuffer(np.uint32(arena.arena.numel() // 256 - 1).tobytes(), np.uint8)
    meta.copy_(torch.from_numpy(m))                                  # runs past the arena end
    store = paged.decompress_pages(arena, meta).cpu().numpy()
    assert (store[0, 0, 0] == 0).all() and (store[1, 1, 1] == 0).all()
    nat = _natural_by_phys(layer)
    rec = codec.encode_group(nat[2, 1, 0], 1, force_raw=True)[1]
    np.testing.assert_array_equal(store[2, 1, 0].reshape(-1), rec)


def test_decompress_first_attention_equals_fused():
    """Decompress + uncompressed attention gives the fused kernel's output bit for bit (same
    arithmetic after a bit-exact restore), and both meet the tolerance against the oracle."""
    announce("decompress-first attention vs fused")
    bsz, hkv, hq = 4, 8, 32
    pages = synth.kv_pages(bsz, 40, hkv, seed=53, forced_frac=0.05, device="cuda")
    q = synth.queries(bsz, hq, seed=53, device="cuda")
    arena = paged.SlotArena(bsz * 40 * hkv * 2 * 4096 + (1 << 20))
    seq_lens, n_comp = [16 * 39 + 7, 16 * 25 + 16, 16 * 39, 5], [39, 25, 39, 0]
    layer = build_layer(arena, pages, seq_lens, n_comp, seed=53)
    fused = run_fused(layer, arena, q, sm_scale())
    store = paged.decompress_pages(arena, layer.meta)
    out = torch.empty_like(fused)
    ws = paged.workspace(bsz, hq, hkv, layer.block_table.shape[1])
    kvz.kvz_bf16_decode_attention(q, out, store, layer.block_table, layer.seq_lens, layer.n_comp,
                                  layer.tail, sm_scale(), ws, hkv)
    torch.cuda.synchronize()
    assert torch.equal(out, fused)
    ref = oracle_attention_rows(layer, q, sm_scale(), range(bsz))
    got = out.cpu().numpy()
    for b in range(bsz):
        check_rows(got[b], ref[b], what=f"decompress-first seq {b}")


def test_decompress_full_size_qwen8k_layer_sampled():
    """The 8K workload's layer (16 x 511 pages, 8 KV heads, u~U[-5,5], 5% forced): every group
    equals packing the input pages; 256 sampled groups equal the oracle's raw records."""
    announce("decompress pages: full 8K layer")
    bsz, n_comp, hkv = 16, 511, 8
    pages = synth.kv_pages(bsz, n_comp + 1, hkv, seed=2, u_max=5.0, forced_frac=0.05, device="cuda")
    arena = paged.SlotArena(bsz * n_comp * hkv * 2 * 4096 + (16 << 20))
    layer = build_layer(arena, pages, [16 * n_comp + 16] * bsz, [n_comp] * bsz, seed=2)
    store = paged.decompress_pages(arena, layer.meta)
    inv = torch.as_tensor(np.argsort(layer.phys_of.reshape(-1)), device="cuda")
    nat_phys = pages[:, :n_comp].reshape(bsz * n_comp, 2, hkv, 16, 128)[inv]
    assert torch.equal(store, paged.pack_bf16_pages(nat_phys))
    rng = np.random.default_rng(54)
    n_phys = bsz * n_comp
    pick = rng.choice(n_phys * 2 * hkv, 256, replace=False)
    nat_h = synth.bits(nat_phys)
    got = store.cpu().numpy()
    for g in pick:
        p, k, h = int(g // (2 * hkv)), int((g // hkv) % 2), int(g % hkv)
        rec = codec.encode_group(nat_h[p, k, h], k, force_raw=True)[1]
        np.testing.assert_array_equal(got[p, k, h].reshape(-1), rec, err_msg=f"group {(p, k, h)}")
