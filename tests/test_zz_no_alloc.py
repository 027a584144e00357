"""The allocation-free attention call (kvz_decode_attention_noalloc) against the workspace call
(kvz_decode_attention), through the C-ABI: the same kernels and split counts, so the outputs
must be bit-identical.  Two calls in a row with the second on a smaller input (the scratch keeps
the first call's contents), at split counts that write directly (1), merge inside the attention
kernel (2, 3) and merge in the combine kernel (8), plus the automatic count; and the size limit
is rejected with an error before anything is launched."""
import numpy as np
import pytest
import torch

from decode_attention_kvz_amd import kvz, paged, synth

from gpu_util import announce, build_layer, check_rows, oracle_attention_rows, sm_scale

pytestmark = pytest.mark.gpu


def _layer(bsz, n_pages, hkv, seed, tails):
    pages = synth.kv_pages(bsz, n_pages + 1, hkv, seed=seed, forced_frac=0.05, forced_exp=-16.0,
                           device="cuda")
    n_comp = [max(1, n_pages - 3 * b) for b in range(bsz)]
    seq_lens = [16 * n + tails[b % len(tails)] for b, n in enumerate(n_comp)]
    arena = paged.SlotArena(bsz * (n_pages + 1) * hkv * 2 * 4096 + (1 << 20))
    return arena, build_layer(arena, pages, seq_lens, n_comp, seed=seed)


def _both(arena, layer, q, splits):
    bsz, hq, _ = q.shape
    hkv = layer.meta.shape[1]
    ws = paged.workspace(bsz, hq, hkv, layer.block_table.shape[1], splits, device="cuda")
    ref = torch.empty((bsz, hq, 128), dtype=torch.float32, device="cuda")
    kvz.kvz_decode_attention(q, ref, arena.arena, layer.meta, layer.block_table, layer.seq_lens,
                             layer.n_comp, layer.tail, sm_scale(), ws, splits)
    got = torch.full((bsz, hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    kvz.kvz_decode_attention_noalloc(q, got, arena.arena, layer.meta, layer.block_table,
                                     layer.seq_lens, layer.n_comp, layer.tail, sm_scale(), splits)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("splits", [0, 1, 2, 3, 8])
def test_noalloc_equals_workspace_call_twice_with_smaller_second(splits):
    announce(f"allocation-free attention, splits={splits}")
    # first call: 6 ragged sequences, 32/8 heads; second: 3 shorter sequences, 16/4 heads
    arena1, layer1 = _layer(6, 40, 8, seed=31, tails=[5, 0, 16, 9])
    q1 = synth.queries(6, 32, seed=31, device="cuda")
    ref1, got1 = _both(arena1, layer1, q1, splits)
    assert torch.equal(ref1, got1)
    arena2, layer2 = _layer(3, 12, 4, seed=32, tails=[3, 11])
    q2 = synth.queries(3, 16, seed=32, device="cuda")
    ref2, got2 = _both(arena2, layer2, q2, splits)
    assert torch.equal(ref2, got2)
    # and against the oracle (tolerance of the method)
    want = oracle_attention_rows(layer2, q2, sm_scale(), range(3))
    g = got2.cpu().numpy()
    for b in range(3):
        check_rows(g[b], want[b], what=f"seq {b}")
    # the first shape again after the smaller one: nothing left over changes it
    _, again = _both(arena1, layer1, q1, splits)
    assert torch.equal(again, ref1)
    # every merge counter of the scratch was consistent
    assert kvz.kvz_attn_workspace_status(None) == 0


def test_noalloc_rejects_sizes_beyond_its_scratch():
    announce("allocation-free attention: size limits")
    bsz, hq, hkv = 4100, 8, 4          # 16,400 (sequence, KV head) pairs > 16,384
    q = torch.zeros((bsz, hq, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((bsz, hq, 128), dtype=torch.float32, device="cuda")
    meta = paged.new_meta_table(1, hkv)
    bt = torch.zeros((bsz, 1), dtype=torch.int32, device="cuda")
    lens = torch.zeros((bsz,), dtype=torch.int32, device="cuda")
    arena = torch.zeros((8192,), dtype=torch.uint8, device="cuda")
    with pytest.raises(kvz.KvzError) as e:
        kvz.kvz_decode_attention_noalloc(q, out, arena, meta, bt, lens, lens, None, sm_scale(), 1)
    assert e.value.code == kvz.KVZ_EINVAL and "16384" in str(e.value)
    # partial results too large: 64 sequences x 64 KV heads x 16 splits x 4 heads x 520 B = 17 MB
    bsz, hq, hkv = 64, 256, 64
    q = torch.zeros((bsz, hq, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((bsz, hq, 128), dtype=torch.float32, device="cuda")
    meta = paged.new_meta_table(1, hkv)
    bt = torch.zeros((bsz, 1), dtype=torch.int32, device="cuda")
    lens = torch.zeros((bsz,), dtype=torch.int32, device="cuda")
    with pytest.raises(kvz.KvzError) as e:
        kvz.kvz_decode_attention_noalloc(q, out, arena, meta, bt, lens, lens, None, sm_scale(), 16)
    assert e.value.code == kvz.KVZ_EINVAL and "bytes" in str(e.value)
    assert (out == 0).all()
