"""GPU parity of the encoder, block decoder and slot pool against the CPU oracle (bit-exact)."""
import numpy as np
import pytest
import torch

from decode_attention_kvz_amd import kvz, paged, synth
from oracle import codec
from oracle.alloc import SlotPoolModel, OFF_NONE, n_raw_of
from oracle.cache import OracleCache, pool_capacity_granules

from gpu_util import announce, build_layer

pytestmark = pytest.mark.gpu


def _meta_items(meta_host, phys_ids, hkv):
    """(off, tags) per item in item order (page, KV head, K/V) from a host meta table."""
    out = []
    m = meta_host.reshape(-1, hkv, 2, 8)
    for ph in phys_ids:
        for h in range(hkv):
            for kind in range(2):
                rec = m[ph, h, kind]
                out.append((int.from_bytes(rec[:4].tobytes(), "little"), [int(x) for x in rec[4:]]))
    return out


@pytest.mark.parametrize("force_raw", [False, True])
def test_encode_tiny_config_matches_oracle_bytes(force_raw):
    """1 sequence, 16 pages, 2 KV heads, 10% forced-raw blocks, seed 0: whole arena, every
    metadata record and the pool counters equal the oracle's."""
    announce(f"encode tiny config force_raw={force_raw}")
    pages = synth.kv_pages(1, 16, 2, seed=0, forced_frac=0.10)
    arena_bytes = 320 * 1024     # 64 all-raw groups (1024 granules) plus room
    arena = paged.SlotArena(arena_bytes)
    layer = build_layer(arena, pages.cuda(), [256], [16], seed=0,
                        flags=kvz.KVZ_ENC_FORCE_RAW if force_raw else 0, with_tail=False)
    torch.cuda.synchronize()
    phys = [int(layer.phys_of[0, p]) for p in range(16)]
    got = _meta_items(layer.meta.cpu().numpy(), phys, 2)

    oc = OracleCache(arena_bytes)
    nat = synth.bits(pages)[0]                                # [16, 2, 2, 16, 128]
    flat = nat.transpose(0, 2, 1, 3, 4).reshape(-1, 16, 128)  # item order (page, head, K/V)
    kinds = [n % 2 for n in range(flat.shape[0])]
    want = oc.encode(flat, kinds, force_raw=force_raw)
    assert got == want
    np.testing.assert_array_equal(arena.arena.cpu().numpy(), oc.arena)
    st = arena.stats()
    assert st["frontier_granules"] == oc.pool.frontier
    assert st["live_runs"] == oc.pool.live_runs == 64
    assert st["live_raw_blocks"] == oc.pool.raw_blocks
    assert st["enospc"] == 0
    if force_raw:
        assert oc.pool.raw_blocks == 256
    else:
        assert 0 < oc.pool.raw_blocks < 256


@pytest.mark.parametrize("stride,shift", [(136, 0), (131, 1)])
def test_encode_from_strided_sources_matches_oracle(stride, shift):
    """Items whose token rows are `stride` elements apart, the first one `shift` elements past a
    16-byte boundary: the 16-byte path with a row stride other than 128 (136) and the
    element-wise path (odd stride, misaligned base) both give the oracle's records."""
    announce(f"encode strided sources stride={stride} shift={shift}")
    pages = synth.kv_pages(1, 8, 2, seed=21, forced_frac=0.10)
    nat = synth.bits(pages)[0]                                # [8, 2, 2, 16, 128]
    flat = nat.transpose(0, 2, 1, 3, 4).reshape(-1, 16, 128)  # item order (page, head, K/V)
    n = flat.shape[0]
    buf = np.zeros((n, 16, stride), dtype=np.uint16)
    buf[:, :, :128] = flat
    dev = torch.zeros(shift + buf.size + 8, dtype=torch.int16, device="cuda")
    dev[shift:shift + buf.size] = torch.from_numpy(buf.reshape(-1).view(np.int16)).cuda()
    base = dev.data_ptr() + 2 * shift
    meta = paged.new_meta_table(8, 2)
    kinds = [i % 2 for i in range(n)]
    items = torch.from_numpy(kvz.encode_items([base + 2 * i * 16 * stride for i in range(n)],
                                              [meta.data_ptr() + 8 * i for i in range(n)],
                                              stride, kinds)).cuda()
    arena = paged.SlotArena(256 * 1024)
    kvz.kvz_encode_pages(arena.pool, items, n, 0)
    torch.cuda.synchronize()
    oc = OracleCache(256 * 1024)
    assert _meta_items(meta.cpu().numpy(), range(8), 2) == oc.encode(flat, kinds)
    np.testing.assert_array_equal(arena.arena.cpu().numpy(), oc.arena)


def test_encode_rows_farther_apart_than_32bit_offsets():
    """A row stride whose 16 rows span more than 2 GiB (beyond the 32-bit offsets of the
    buffer-load path) takes the element-wise path and still gives the oracle's records."""
    announce("encode with a 2.2 GB row span")
    stride = 72 * 1024 * 1024                                 # elements, a multiple of 8
    pages = synth.kv_pages(1, 1, 1, seed=23, forced_frac=0.0)
    nat = synth.bits(pages)[0, 0]                             # [2 (K,V), 1, 16, 128]
    flat = nat[:, 0]                                          # items K, V
    span = 15 * stride + 128
    dev = torch.zeros(2 * span, dtype=torch.int16, device="cuda")
    for i in range(2):
        for t in range(16):
            at = i * span + t * stride
            dev[at:at + 128] = torch.from_numpy(flat[i, t].view(np.int16)).cuda()
    meta = paged.new_meta_table(1, 1)
    items = torch.from_numpy(kvz.encode_items([dev.data_ptr() + 2 * i * span for i in range(2)],
                                              [meta.data_ptr() + 8 * i for i in range(2)],
                                              stride, [0, 1])).cuda()
    arena = paged.SlotArena(64 * 1024)
    kvz.kvz_encode_pages(arena.pool, items, 2, 0)
    torch.cuda.synchronize()
    del dev
    oc = OracleCache(64 * 1024)
    assert _meta_items(meta.cpu().numpy(), range(1), 1) == oc.encode(flat, [0, 1])
    np.testing.assert_array_equal(arena.arena.cpu().numpy(), oc.arena)


def test_decode_block_bit_exact_and_matches_oracle():
    announce("decode_block tiny config")
    pages = synth.kv_pages(1, 16, 2, seed=0, forced_frac=0.10)
    arena = paged.SlotArena(256 * 1024)
    layer = build_layer(arena, pages.cuda(), [256], [16], seed=0, with_tail=False)
    n_groups = 16 * 2 * 2
    meta_ptrs, blocks, kinds = [], [], []
    for ph in range(16):
        for h in range(2):
            for kind in range(2):
                for j in range(4):
                    meta_ptrs.append(layer.meta.data_ptr() + ((ph * 2 + h) * 2 + kind) * 8)
                    blocks.append(j)
                    kinds.append(kind)
    refs = torch.from_numpy(kvz.block_refs(meta_ptrs, blocks, kinds)).cuda()
    out = torch.empty((n_groups * 4, 16, 32), dtype=torch.int16, device="cuda")
    kvz.kvz_decode_block(arena.arena, refs, n_groups * 4, out)
    got = out.cpu().numpy().view(np.uint16)
    nat = synth.bits(pages)[0]
    inv = np.argsort(layer.phys_of[0, :16])
    arena_h = arena.arena.cpu().numpy()
    meta_h = layer.meta.cpu().numpy().reshape(16, 2, 2, 8)
    n = 0
    for ph in range(16):
        p = int(inv[ph])
        for h in range(2):
            for kind in range(2):
                page = nat[p, kind, h]
                off = int.from_bytes(meta_h[ph, h, kind, :4].tobytes(), "little")
                tags = list(meta_h[ph, h, kind, 4:])
                orc = codec.decode_group(arena_h, off, tags, kind)
                np.testing.assert_array_equal(orc, page)
                for j in range(4):
                    np.testing.assert_array_equal(got[n], page[:, 32 * j:32 * j + 32])
                    n += 1


def _oracle_tags(nat_groups, kinds, force_raw=False):
    """Tags of many groups by the oracle's own classification, in chunks."""
    tags = np.zeros((nat_groups.shape[0], 4), dtype=np.uint8)
    for a in range(0, nat_groups.shape[0], 4096):
        g = nat_groups[a:a + 4096]
        for j in range(4):
            blk = g[:, :, 32 * j:32 * j + 32].reshape(g.shape[0], 512)
            b, ok = codec.base_and_eligible(codec.fields(blk)[1])
            if force_raw:
                ok = np.zeros_like(ok)
            tags[a:a + 4096, j] = np.where(ok, b // 2, 0xFF)
    return tags


def test_long_context_stress_round_trips_every_block():
    """131072 tokens, 8 KV heads, stress values (zeros, subnormals, Inf/NaN) on top of the
    tiny-config distribution: every block decodes to its input bit for bit; every group's tags
    and offset equal the oracle's (tags by the oracle's classification, offsets by its pool
    model); a sample of records equals the oracle's bytes."""
    announce("long-context stress round trip: generate")
    n_pages, hkv = 8192, 8
    pages = synth.kv_pages(1, n_pages, hkv, seed=4, forced_frac=0.10, stress=True, device="cuda")
    arena_bytes = n_pages * hkv * 2 * 4096 + (1 << 20)
    arena = paged.SlotArena(arena_bytes)
    announce("long-context stress round trip: encode")
    layer = build_layer(arena, pages, [n_pages * 16], [n_pages], seed=4, with_tail=False)
    n_groups = n_pages * hkv * 2
    announce("long-context stress round trip: decode every block")
    meta_base = layer.meta.data_ptr()
    g = np.arange(n_groups, dtype=np.int64)
    ptrs = np.repeat(meta_base + g * 8, 4)
    blocks = np.tile(np.arange(4), n_groups)
    kinds = np.repeat(g % 2, 4)
    refs = torch.from_numpy(kvz.block_refs(ptrs, blocks, kinds)).cuda()
    out = torch.empty((n_groups * 4, 16, 32), dtype=torch.int16, device="cuda")
    kvz.kvz_decode_block(arena.arena, refs, n_groups * 4, out)
    # expected: natural pages by physical id, split into blocks [group][block][16][32]
    inv = torch.as_tensor(np.argsort(layer.phys_of[0, :n_pages]), device="cuda")
    nat = pages[0][inv]                                         # [phys, 2, Hkv, 16, 128]
    nat = nat.permute(0, 2, 1, 3, 4).contiguous()               # [phys, Hkv, 2, 16, 128]
    want = nat.view(torch.int16).reshape(n_groups, 16, 4, 32).permute(0, 2, 1, 3)
    assert torch.equal(out.view(n_groups, 4, 16, 32), want.contiguous())
    announce("long-context stress round trip: oracle tags and offsets")
    nat_h = nat.cpu().view(torch.int16).numpy().view(np.uint16).reshape(n_groups, 16, 128)
    meta_h = layer.meta.cpu().numpy().reshape(n_groups, 8)
    got_tags = meta_h[:, 4:]
    want_tags = _oracle_tags(nat_h, g % 2)
    np.testing.assert_array_equal(got_tags, want_tags)
    # item order was (logical page, head, K/V); map to physical order for the offsets
    model = SlotPoolModel(pool_capacity_granules(arena.arena.numel()))
    phys_order = layer.phys_of[0, :n_pages]
    item_groups = ((phys_order[:, None, None] * hkv + np.arange(hkv)[None, :, None]) * 2
                   + np.arange(2)[None, None, :]).reshape(-1)
    offs = model.alloc([want_tags[k].tolist() for k in item_groups])
    got_off = meta_h[:, :4].copy().view("<u4")[:, 0]
    np.testing.assert_array_equal(got_off[item_groups], np.asarray(offs, dtype=np.uint32))
    arena_h = arena.arena.cpu().numpy()
    rng = np.random.default_rng(44)
    for k in rng.choice(n_groups, 64, replace=False):
        tags, rec = codec.encode_group(nat_h[k], int(k % 2))
        off = int(got_off[k])
        np.testing.assert_array_equal(arena_h[off * 256: off * 256 + rec.size], rec)
    raw_frac = float((want_tags == 0xFF).mean())
    announce(f"long-context stress: raw block fraction {raw_frac:.4f}")
    assert raw_frac > 0.99


def test_slot_alloc_free_churn_matches_model():
    """kvz_slot_alloc / kvz_slot_free over random calls equal the pool model call by call,
    including exhaustion (OFF_NONE) and bin reuse."""
    announce("slot alloc/free churn")
    rng = np.random.default_rng(21)
    arena = paged.SlotArena(64 * 1024 * 256 // 64)  # 1024 granules minus guard
    cap = arena.stats()["capacity_granules"]
    model = SlotPoolModel(cap)
    live = []   # (off, tags)
    meta = torch.zeros((4096, 8), dtype=torch.uint8, device="cuda")
    for step in range(60):
        n = int(rng.integers(1, 40))
        tags = np.full((n, 4), 7, dtype=np.uint8)
        for i in range(n):
            tags[i, :int(rng.integers(0, 5))] = 0xFF
            rng.shuffle(tags[i])
        d_tags = torch.from_numpy(tags).cuda()
        d_off = torch.empty(n, dtype=torch.int32, device="cuda")
        kvz.kvz_slot_alloc(arena.pool, d_tags, d_off)
        got = d_off.cpu().numpy().view(np.uint32)
        want = model.alloc([t.tolist() for t in tags])
        np.testing.assert_array_equal(got, np.asarray(want, dtype=np.uint32))
        for i in range(n):
            if want[i] != OFF_NONE:
                live.append((want[i], tags[i].tolist()))
        if live and rng.random() < 0.7:
            k = int(rng.integers(1, len(live) + 1))
            pick = sorted(rng.choice(len(live), k, replace=False).tolist())
            victims = [live[i] for i in pick]
            live = [x for i, x in enumerate(live) if i not in set(pick)]
            host = np.zeros((len(victims), 8), dtype=np.uint8)
            for i, (off, t) in enumerate(victims):
                host[i, :4] = np.frombuffer(int(off).to_bytes(4, "little"), dtype=np.uint8)
                host[i, 4:] = t
            meta[:len(victims)] = torch.from_numpy(host).cuda()
            ptrs = torch.from_numpy(meta.data_ptr() + np.arange(len(victims), dtype=np.int64) * 8).cuda()
            kvz.kvz_slot_free(arena.pool, ptrs)
            model.free(victims)
            cleared = meta[:len(victims)].cpu().numpy()
            assert (cleared[:, :4] == 0xFF).all() and (cleared[:, 4:] == 0).all()
        st = arena.stats()
        assert st["frontier_granules"] == model.frontier
        assert st["free_runs"] == [len(model.bins[k]) for k in range(5)]
        assert st["live_runs"] == model.live_runs
        assert st["live_granules"] == model.live_granules
        assert st["enospc"] == model.enospc
    assert model.enospc > 0, "the churn should have exhausted the pool at least once"


@pytest.mark.parametrize("forced,n_layers,fused", [(0.0, 4, False), (0.10, 4, False), (0.50, 4, False),
                                                   (0.10, 32, False), (0.10, 4, True), (0.10, 32, True)])
def test_online_page_completion_churn(forced, n_layers, fused):
    """Online encode at page completion with frees and reuse across layers (64 sequences,
    8 KV heads, 4 layers with a small arena that runs out, or all 32 layers of the online
    workload with room for every page, staggered phases): offsets and tags equal the oracle
    pool model and classification after every step; live groups decode to their source pages.
    fused: each step's free and encode are one kvz_complete_pages call."""
    announce(f"online churn forced={forced} layers={n_layers} fused={fused}")
    rng = np.random.default_rng(int(forced * 100) + 3)
    n_seq, hkv, page_bank = 64, 8, 16
    bank = synth.kv_pages(n_seq, page_bank, hkv, seed=3, forced_frac=forced, device="cuda")
    bank_h = synth.bits(bank)                                  # [S, 16, 2, Hkv, 16, 128]
    max_pages = 64
    arena_bytes = (96 << 20) if n_layers == 4 else (1 << 30)
    arena = paged.SlotArena(arena_bytes)
    model = SlotPoolModel(pool_capacity_granules(arena.arena.numel()))
    metas = [paged.new_meta_table(n_seq * max_pages, hkv) for _ in range(n_layers)]
    length = (np.arange(n_seq) * 3) % 16                       # staggered phases
    target = rng.integers(32, 128, size=n_seq)
    live = {}   # (layer, s, p) -> list of (off, tags) per (h, kind)
    for step in range(160):
        # sequences that reached their target free every group and restart
        done = [s for s in range(n_seq) if length[s] >= target[s]]
        d_free = None
        if done:
            ptrs, model_metas = [], []
            for s in done:
                for layer in range(n_layers):
                    for p in range(int(length[s]) // 16):
                        for h in range(hkv):
                            for kind in range(2):
                                gi = ((s * max_pages + p) * hkv + h) * 2 + kind
                                ptrs.append(metas[layer].data_ptr() + gi * 8)
                        model_metas.extend(live.pop((layer, s, p)))
                length[s] = 0
                target[s] = rng.integers(32, 128)
            d_free = torch.from_numpy(np.asarray(ptrs, dtype=np.int64)).cuda()
            if not fused:
                kvz.kvz_slot_free(arena.pool, d_free)
            model.free(model_metas)
        length += 1
        # pages that completed with this token: encode them in all layers
        completing = [s for s in range(n_seq) if length[s] % 16 == 0]
        src, dst, kinds, want_tags, keys = [], [], [], [], []
        for s in completing:
            p = int(length[s]) // 16 - 1
            for layer in range(n_layers):
                bp = (p + layer) % page_bank
                for h in range(hkv):
                    for kind in range(2):
                        gi = ((s * max_pages + p) * hkv + h) * 2 + kind
                        src.append(bank.data_ptr() + ((((s * page_bank + bp) * 2 + kind) * hkv + h) * 2048) * 2)
                        dst.append(metas[layer].data_ptr() + gi * 8)
                        kinds.append(kind)
                        want_tags.append(bank_h[s, bp, kind, h])
                keys.append((layer, s, p))
        if fused and d_free is not None and not src:
            kvz.kvz_complete_pages(arena.pool, d_free, None, 0)
        if src:
            items = kvz.encode_items(src, dst, 128, kinds)
            d_items = torch.from_numpy(items).cuda()
            if fused:
                kvz.kvz_complete_pages(arena.pool, d_free, d_items, len(src))
            else:
                kvz.kvz_encode_pages(arena.pool, d_items, len(src))
            tags = _oracle_tags(np.stack(want_tags), kinds)
            offs = model.alloc([t.tolist() for t in tags])
            got = np.stack([m.cpu().numpy().reshape(-1, 8) for m in metas])   # [L, groups, 8]
            k = 0
            for layer, s, p in keys:
                recs = []
                for h in range(hkv):
                    for kind in range(2):
                        gi = ((s * max_pages + p) * hkv + h) * 2 + kind
                        rec = got[layer, gi]
                        off = int.from_bytes(rec[:4].tobytes(), "little")
                        assert off == offs[k], (step, layer, s, p, h, kind)
                        assert list(rec[4:]) == tags[k].tolist()
                        recs.append((off, tags[k].tolist()))
                        k += 1
                live[(layer, s, p)] = recs
        st = arena.stats()
        assert st["frontier_granules"] == model.frontier
        assert st["free_runs"] == [len(model.bins[k]) for k in range(5)]
        assert st["live_runs"] == model.live_runs
    assert sum(len(b) for b in model.bins) > 0, "the churn should have reused freed runs"
    # live groups decode to their source pages
    arena_h = arena.arena.cpu().numpy()
    for (layer, s, p), recs in list(live.items())[:40]:
        bp = (p + layer) % page_bank
        i = 0
        for h in range(hkv):
            for kind in range(2):
                off, tags = recs[i]
                i += 1
                if off == OFF_NONE:
                    continue
                np.testing.assert_array_equal(codec.decode_group(arena_h, off, tags, kind),
                                              bank_h[s, bp, kind, h])


def test_tiny_arena_reports_no_room_and_leaves_pages_unstored():
    announce("tiny arena ENOSPC")
    pages = synth.kv_pages(1, 4, 2, seed=5, forced_frac=0.0)
    arena = paged.SlotArena(256 * 60)              # 59 usable granules: fits 4 runs of 12
    layer = build_layer(arena, pages.cuda(), [64], [4], seed=5, with_tail=False)
    torch.cuda.synchronize()
    meta = layer.meta.cpu().numpy().reshape(-1, 8)
    offs = meta[:, :4].copy().view("<u4")[:, 0]
    placed = offs != OFF_NONE
    assert placed.sum() == 4 and (~placed).sum() == 12
    st = arena.stats()
    assert st["enospc"] == 12 and st["live_runs"] == 4


def _alloc_and_check(arena, model, tags):
    d_tags = torch.from_numpy(np.ascontiguousarray(tags)).cuda()
    d_off = torch.empty(tags.shape[0], dtype=torch.int32, device="cuda")
    kvz.kvz_slot_alloc(arena.pool, d_tags, d_off)
    got = d_off.cpu().numpy().view(np.uint32)
    want = np.asarray(model.alloc(tags.tolist()), dtype=np.uint32)
    np.testing.assert_array_equal(got, want)
    return want


def _free(arena, model, victims):
    host = np.zeros((len(victims), 8), dtype=np.uint8)
    offs = np.asarray([v[0] for v in victims], dtype=np.uint32)
    host[:, :4] = offs.view(np.uint8).reshape(-1, 4)
    host[:, 4:] = np.asarray([v[1] for v in victims], dtype=np.uint8)
    meta = torch.from_numpy(host).cuda()
    ptrs = torch.from_numpy(meta.data_ptr() + np.arange(len(victims), dtype=np.int64) * 8).cuda()
    kvz.kvz_slot_free(arena.pool, ptrs)
    model.free(victims)
    cleared = meta.cpu().numpy()
    assert (cleared[:, :4] == 0xFF).all() and (cleared[:, 4:] == 0).all()


def _check_stats(arena, model):
    st = arena.stats()
    assert st["frontier_granules"] == model.frontier
    assert st["free_runs"] == [len(model.bins[k]) for k in range(5)]
    assert st["live_runs"] == model.live_runs
    assert st["live_granules"] == model.live_granules
    assert st["live_raw_blocks"] == model.raw_blocks
    assert st["enospc"] == model.enospc


def _random_tags(rng, n, p_raw):
    tags = np.full((n, 4), 60, dtype=np.uint8)
    tags[rng.random((n, 4)) < p_raw] = 0xFF
    return tags


def test_slot_pool_calls_spanning_many_tiles_match_model():
    """Calls of many 1024-item tiles: frontier offsets, bin pops that run out part-way,
    exhaustion in a later tile, and frees spanning tiles all equal the pool model."""
    announce("slot pool: multi-tile calls")
    rng = np.random.default_rng(61)
    cap_target = 20000 * 14
    arena = paged.SlotArena((cap_target + 1) * 256)
    model = SlotPoolModel(arena.stats()["capacity_granules"])
    tags = _random_tags(rng, 3 * 4096 + 777, 0.2)
    offs = _alloc_and_check(arena, model, tags)
    _check_stats(arena, model)
    live = [(int(o), t.tolist()) for o, t in zip(offs, tags)]
    order = rng.permutation(len(live))
    victims = [live[i] for i in order[:6000]]
    live = [live[i] for i in order[6000:]]
    _free(arena, model, victims)
    _check_stats(arena, model)
    # pops of every class across tiles, some bins run dry, then the frontier runs out
    tags2 = _random_tags(rng, 5 * 4096 + 100, 0.35)
    offs2 = _alloc_and_check(arena, model, tags2)
    _check_stats(arena, model)
    assert model.enospc > 0 and (offs2 != OFF_NONE).sum() > 6000


@pytest.mark.parametrize("small,big", [(1024, 1025), (4096, 4097)])
def test_slot_pool_one_workgroup_and_tiled_calls_at_the_boundary(small, big):
    """Calls of up to 1,024 items run in one workgroup with 2 items per thread, up to 4,096 with
    8, larger ones in tiles: calls on both sides of each switch, alternating, for allocation
    (bin pops that run out, frontier) and free, all equal the pool model."""
    announce(f"slot pool: call sizes {small} / {big}")
    rng = np.random.default_rng(63 + small)
    arena = paged.SlotArena((35 * small + 1) * 256)
    model = SlotPoolModel(arena.stats()["capacity_granules"])
    ta, tb = _random_tags(rng, small, 0.15), _random_tags(rng, big, 0.3)
    a = _alloc_and_check(arena, model, ta)
    b = _alloc_and_check(arena, model, tb)
    _check_stats(arena, model)
    assert (a != OFF_NONE).all() and (b != OFF_NONE).all()
    live_a = [(int(o), t.tolist()) for o, t in zip(a, ta)]
    live_b = [(int(o), t.tolist()) for o, t in zip(b, tb)]
    _free(arena, model, live_a + live_b[:1])           # `big` records
    _check_stats(arena, model)
    _free(arena, model, live_b[1:])                    # `small` records
    _check_stats(arena, model)
    _alloc_and_check(arena, model, _random_tags(rng, small, 0.5))   # pops, bins run dry
    _check_stats(arena, model)
    _alloc_and_check(arena, model, _random_tags(rng, big, 0.05))
    _check_stats(arena, model)


def test_slot_alloc_call_larger_than_one_chunk_matches_model():
    """One call of 1 Mi + 5000 items (two chunks of the tiled allocator: 1024 tiles of 1024
    items each): bin state and the frontier's request prefix carry into the second chunk."""
    announce("slot pool: call of more than one chunk")
    rng = np.random.default_rng(62)
    arena = paged.SlotArena(400_001 * 256)
    model = SlotPoolModel(arena.stats()["capacity_granules"])
    # fill bins 0 and 4
    seed_tags = np.concatenate([_random_tags(rng, 3000, 0.0), np.full((500, 4), 0xFF, np.uint8)])
    offs = _alloc_and_check(arena, model, seed_tags)
    _free(arena, model, [(int(o), t.tolist()) for o, t in zip(offs, seed_tags)])
    n = 1024 * 1024 + 5000
    tags = np.full((n, 4), 60, dtype=np.uint8)
    tags[rng.random(n) < 0.3, 0] = 0xFF             # classes 0 and 1 only ...
    late = 1024 * 1024 + rng.choice(5000, 300, replace=False)
    tags[late] = 0xFF                                # ... until the second chunk: class 4
    _alloc_and_check(arena, model, tags)
    _check_stats(arena, model)
    assert len(model.bins[4]) == 200                 # 300 of the 500 class-4 runs popped late


def test_guaranteed_capacity_always_fits():
    """After churn that leaves free runs in several bins, as many all-raw groups as the capacity
    report guarantees are all placed (the worst case for the frontier), and the report's free
    granules match the pool model."""
    announce("pool capacity guarantee")
    rng = np.random.default_rng(63)
    arena = paged.SlotArena(5001 * 256)
    model = SlotPoolModel(arena.stats()["capacity_granules"])
    tags = _random_tags(rng, 250, 0.3)
    offs = _alloc_and_check(arena, model, tags)
    _free(arena, model, [(int(o), t.tolist()) for o, t in zip(offs[:120], tags[:120])])
    st = arena.stats()
    cap = kvz.kvz_pool_capacity(st, 1, 1)
    free_model = (model.capacity - model.frontier
                  + sum(len(model.bins[k]) * (12 + k) for k in range(5)))
    assert cap["free_granules"] == free_model
    g = cap["guaranteed_groups"]
    assert g > 100
    raw = np.full((g, 4), 0xFF, dtype=np.uint8)
    got = _alloc_and_check(arena, model, raw)
    assert (got != OFF_NONE).all()
