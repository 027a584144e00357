"""Online page completion over 4,096 decode steps (the churn workload: 64 sequences, 32 layers,
8 KV heads, staggered phases so that 4 sequences complete a page every step, 2,048 groups per
step; a sequence that reaches its target length frees every group and restarts), against the
oracle pool model and the oracle's classification after every step, then every live group
decoded again.

The bookkeeping is vectorized (numpy arrays of the live offsets and tags) so that the 4,096
steps fit in about a minute.  At the end every stored group of every layer is rebuilt by the
library's decompress-first kernel and compared with its source page bit for bit (that kernel is
itself checked against the oracle's decoder in tests/test_gpu_decompress.py), and a sample of
groups is also decoded by the oracle from the arena bytes."""
import numpy as np
import pytest
import torch

from decode_attention_kvz_amd import kvz, paged, synth
from oracle import codec
from oracle.alloc import SlotPoolModel, OFF_NONE
from oracle.cache import pool_capacity_granules

from gpu_util import announce

pytestmark = pytest.mark.gpu

STEPS = 4096
N_SEQ, N_LAYERS, HKV, BANK, MAX_PAGES = 64, 32, 8, 16, 8


def _tags_of(groups, kinds):
    """Oracle classification of natural groups [n, 16, 128] (uint16): [n, 4] tags."""
    tags = np.zeros((groups.shape[0], 4), dtype=np.uint8)
    for j in range(4):
        blk = groups[:, :, 32 * j:32 * j + 32].reshape(groups.shape[0], 512)
        b, ok = codec.base_and_eligible(codec.fields(blk)[1])
        tags[:, j] = np.where(ok, b // 2, 0xFF)
    return tags


def test_online_churn_4096_steps():
    announce(f"online churn, {STEPS} steps")
    rng = np.random.default_rng(11)
    bank = synth.kv_pages(N_SEQ, BANK, HKV, seed=11, forced_frac=0.10, device="cuda")
    bank_h = synth.bits(bank)                              # [S, BANK, 2, Hkv, 16, 128]
    # the oracle's tags of every bank group, once: [S, BANK, 2, Hkv, 4]
    bank_tags = _tags_of(bank_h.reshape(-1, 16, 128), None).reshape(N_SEQ, BANK, 2, HKV, 4)
    arena = paged.SlotArena(1 << 30)
    model = SlotPoolModel(pool_capacity_granules(arena.arena.numel()))
    # one metadata table per layer, [N_SEQ * MAX_PAGES, Hkv, 2, 8] each, in one tensor
    metas = torch.empty((N_LAYERS, N_SEQ * MAX_PAGES, HKV, 2, 8), dtype=torch.uint8, device="cuda")
    metas.view(-1, 8)[:, :4] = 0xFF
    metas.view(-1, 8)[:, 4:] = 0
    meta_base = metas.data_ptr()
    bank_base = bank.data_ptr()
    # live state: offset and tags of every (layer, s, p, h, kind)
    live_off = np.full((N_LAYERS, N_SEQ, MAX_PAGES, HKV, 2), OFF_NONE, dtype=np.int64)
    live_tags = np.zeros((N_LAYERS, N_SEQ, MAX_PAGES, HKV, 2, 4), dtype=np.uint8)
    live_page = np.zeros((N_SEQ, MAX_PAGES), dtype=bool)
    length = (np.arange(N_SEQ) * 3) % 16
    target = rng.integers(32, 16 * MAX_PAGES + 1, size=N_SEQ)
    L, H, K = np.meshgrid(np.arange(N_LAYERS), np.arange(HKV), np.arange(2), indexing="ij")
    L, H, K = L.reshape(-1), H.reshape(-1), K.reshape(-1)   # item order per page: layer, head, K/V
    encoded = freed = reused_steps = 0
    for step in range(STEPS):
        done = np.nonzero(length >= target)[0]
        if done.size:
            ptrs, recs = [], []
            for s in done:
                for p in range(int(length[s]) // 16):
                    gi = (s * MAX_PAGES + p)
                    ptrs.append(meta_base + (((L * N_SEQ * MAX_PAGES + gi) * HKV + H) * 2 + K) * 8)
                    recs.append((live_off[L, s, p, H, K], live_tags[L, s, p, H, K]))
                    live_off[:, s, p] = OFF_NONE
                    live_page[s, p] = False
                length[s] = 0
                target[s] = rng.integers(32, 16 * MAX_PAGES + 1)
            ptrs = np.concatenate(ptrs)
            kvz.kvz_slot_free(arena.pool, torch.from_numpy(ptrs.astype(np.int64)).cuda())
            model.free([(int(o), t) for offs, tags in recs for o, t in zip(offs, tags)])
            freed += ptrs.size
        length += 1
        completing = np.nonzero(length % 16 == 0)[0]
        if completing.size:
            src, dst, kinds, keys = [], [], [], []
            for s in completing:
                p = int(length[s]) // 16 - 1
                bp = (p + L) % BANK
                src.append(bank_base + ((((s * BANK + bp) * 2 + K) * HKV + H) * 2048) * 2)
                dst.append(meta_base + (((L * N_SEQ * MAX_PAGES + s * MAX_PAGES + p) * HKV + H) * 2 + K) * 8)
                kinds.append(K)
                keys.append((s, p, bp))
            src, dst, kinds = np.concatenate(src), np.concatenate(dst), np.concatenate(kinds)
            items = kvz.encode_items(src.tolist(), dst.tolist(), 128, kinds.tolist())
            kvz.kvz_encode_pages(arena.pool, torch.from_numpy(items).cuda(), src.size)
            want_tags = np.concatenate([bank_tags[s, bp, K, H] for s, p, bp in keys])
            offs = np.asarray(model.alloc(want_tags.tolist()), dtype=np.int64)
            # this step's records, gathered on the device
            gi = torch.from_numpy((dst - meta_base) // 8).cuda()
            got = metas.view(-1, 8)[gi].cpu().numpy()
            got_off = got[:, :4].copy().view(np.uint32).reshape(-1).astype(np.int64)
            assert np.array_equal(got_off, offs), step
            assert np.array_equal(got[:, 4:], want_tags), step
            k = 0
            for s, p, bp in keys:
                n = L.size
                live_off[L, s, p, H, K] = offs[k:k + n]
                live_tags[L, s, p, H, K] = want_tags[k:k + n]
                live_page[s, p] = True
                k += n
            encoded += src.size
        st = arena.stats()
        assert st["frontier_granules"] == model.frontier, step
        assert st["free_runs"] == [len(model.bins[k]) for k in range(5)], step
        assert st["live_runs"] == model.live_runs, step
        assert st["live_granules"] == model.live_granules, step
        assert st["enospc"] == model.enospc == 0, step
        reused_steps += int(any(model.bins))
    assert freed > 0 and reused_steps > 0, "the churn should free and reuse runs"
    announce(f"   {encoded} groups encoded, {freed} freed, {int(live_page.sum())} live pages at the end")

    # every live group of every layer, decoded again and compared with its source page
    s_idx, p_idx = np.nonzero(live_page)
    bp = (p_idx[None, :] + np.arange(N_LAYERS)[:, None]) % BANK          # [L, n]
    n_checked = 0
    for layer in range(N_LAYERS):
        out = paged.decompress_pages(arena, metas[layer])                   # [S*MAX_PAGES, 2, Hkv, 4, 1024]
        rows = torch.from_numpy(s_idx * MAX_PAGES + p_idx).cuda()
        got = out[rows]
        want = paged.pack_bf16_pages(bank[torch.from_numpy(s_idx).cuda(), torch.from_numpy(bp[layer]).cuda()])
        stored = torch.from_numpy(live_off[layer, s_idx, p_idx] != OFF_NONE).cuda()   # [n, Hkv, 2]
        stored = stored.permute(0, 2, 1)[..., None, None].expand_as(got)              # [n, 2, Hkv, 4, 1024]
        assert torch.equal(got[stored], want[stored]), layer
        n_checked += int(stored[:, :, :, 0, 0].sum())
    assert n_checked == int((live_off != OFF_NONE).sum())
    # a sample decoded by the oracle from the arena bytes
    arena_h = arena.arena.cpu().numpy()
    live_idx = np.argwhere(live_off != OFF_NONE)
    for layer, s, p, h, kind in live_idx[rng.choice(len(live_idx), size=min(64, len(live_idx)), replace=False)]:
        np.testing.assert_array_equal(
            codec.decode_group(arena_h, int(live_off[layer, s, p, h, kind]),
                               live_tags[layer, s, p, h, kind].tolist(), int(kind)),
            bank_h[s, (p + layer) % BANK, kind, h])
    announce(f"   {n_checked} live groups decoded again")
