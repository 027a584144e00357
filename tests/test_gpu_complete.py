"""The encoder on both sides of the one-pass limit, and the fused step call.

* Into a pool whose bins hold freed runs: 16,384 groups (the largest one-pass call: two rounds
  of tiles), then a bulk call of 140,000 groups (classify, multi-pass allocation, pack): every
  offset and tag equals the oracle pool model and classification, the pool counters equal the
  model's, and a sample of groups decoded by the oracle from the arena bytes equals its source.
* kvz_complete_pages against kvz_slot_free followed by kvz_encode_pages on a second pool: the
  same records, arena bytes and counters after every step, for frees of one to twelve free tiles
  (up to 512 groups each), frees that include the records the encode then rewrites, a call of
  20,000 groups (above the one-pass limit), and an arena that runs out.
* A captured kvz_complete_pages replayed with new item records each time equals eager calls.
* A one-pass launch whose wait gives up (forced from the host) stores and frees nothing and
  halts the one-pass encoder until kvz_pool_init; bulk calls are not affected.
* 17,000 steady-state steps of both paths cross the free tiles' 14-bit launch tag and agree.
"""
import numpy as np
import pytest
import torch

from decode_attention_kvz_amd import kvz, paged, synth
from oracle import codec
from oracle.alloc import SlotPoolModel, OFF_NONE
from oracle.cache import pool_capacity_granules

from gpu_util import announce

pytestmark = pytest.mark.gpu

BANK_SEQ, BANK_PAGES, HKV = 8, 32, 8      # 8 x 32 pages x 8 heads x K|V = 4,096 source groups


def _bank(seed, forced):
    bank = synth.kv_pages(BANK_SEQ, BANK_PAGES, HKV, seed=seed, forced_frac=forced, device="cuda")
    nat = synth.bits(bank).reshape(-1, 16, 128)               # [(s, p, kind, h), 16, 128]
    tags = np.zeros((nat.shape[0], 4), dtype=np.uint8)
    for j in range(4):
        blk = nat[:, :, 32 * j:32 * j + 32].reshape(nat.shape[0], 512)
        b, ok = codec.base_and_eligible(codec.fields(blk)[1])
        tags[:, j] = np.where(ok, b // 2, 0xFF)
    return bank, nat, tags


def _items(bank, src_ids, meta, dst_ids):
    """Items encoding bank groups src_ids (flat (s, p, kind, h) index) into meta slots dst_ids."""
    src_ids = np.asarray(src_ids, dtype=np.int64)
    kinds = ((src_ids // HKV) % 2).tolist()
    src = (bank.data_ptr() + src_ids * 2048 * 2).tolist()
    dst = (meta.data_ptr() + np.asarray(dst_ids, dtype=np.int64) * 8).tolist()
    return torch.from_numpy(kvz.encode_items(src, dst, 128, kinds)).cuda()


def _records(meta, ids):
    m = meta.view(-1, 8)[torch.from_numpy(np.asarray(ids, dtype=np.int64)).cuda()].cpu().numpy()
    return m[:, :4].copy().view(np.uint32).reshape(-1).astype(np.int64), m[:, 4:]


def _check_stats(arena, model, what):
    st = arena.stats()
    assert st["frontier_granules"] == model.frontier, what
    assert st["free_runs"] == [len(model.bins[k]) for k in range(5)], what
    assert st["live_runs"] == model.live_runs, what
    assert st["live_granules"] == model.live_granules, what
    assert st["enospc"] == model.enospc, what


def test_largest_one_pass_and_bulk_encode_match_model():
    announce("encode of 16,384 (one pass) and 140,000 groups (bulk), bins holding freed runs")
    rng = np.random.default_rng(5)
    bank, nat, tags = _bank(seed=5, forced=0.10)
    n0, n_free, n1, n2 = 20000, 9000, 16384, 140000
    arena = paged.SlotArena(768 << 20)
    model = SlotPoolModel(pool_capacity_granules(arena.arena.numel()))
    meta = torch.empty((n0 + n1 + n2, 8), dtype=torch.uint8, device="cuda")
    meta[:, :4] = 0xFF
    meta[:, 4:] = 0
    # a first call, then frees scattered over it (the bins then hold runs of every class)
    src0 = rng.integers(0, nat.shape[0], size=n0)
    kvz.kvz_encode_pages(arena.pool, _items(bank, src0, meta, np.arange(n0)), n0)
    want0 = model.alloc([t.tolist() for t in tags[src0]])
    got0, _ = _records(meta, np.arange(n0))
    np.testing.assert_array_equal(got0, np.asarray(want0, dtype=np.int64))
    victims = np.sort(rng.choice(n0, size=n_free, replace=False))
    kvz.kvz_slot_free(arena.pool, torch.from_numpy(meta.data_ptr() + victims * 8).cuda())
    model.free([(want0[i], tags[src0[i]].tolist()) for i in victims])
    _check_stats(arena, model, "after the free")
    assert sum(len(b) for b in model.bins) == n_free
    arena_h = None
    for n, base, what in ((n1, n0, "one pass"), (n2, n0 + n1, "bulk")):
        src = rng.integers(0, nat.shape[0], size=n)
        ids = base + np.arange(n)
        kvz.kvz_encode_pages(arena.pool, _items(bank, src, meta, ids), n)
        want = np.asarray(model.alloc([t.tolist() for t in tags[src]]), dtype=np.int64)
        got, gtags = _records(meta, ids)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"{what}: {bad.size} offsets differ, first at item {bad[:5]}"
        np.testing.assert_array_equal(gtags, tags[src])
        _check_stats(arena, model, f"after the {what} call")
        # a sample decoded by the oracle from the arena bytes
        arena_h = arena.arena.cpu().numpy()
        for i in rng.choice(n, 48, replace=False):
            g = src[i]
            np.testing.assert_array_equal(
                codec.decode_group(arena_h, int(want[i]), tags[g].tolist(), int((g // HKV) % 2)), nat[g])
    assert sum(len(b) for b in model.bins) == 0, "the calls should have popped every freed run"


@pytest.mark.parametrize("arena_mb", [256, 24])
def test_complete_pages_equals_free_then_encode(arena_mb):
    """Two pools driven by the same steps: one with kvz_slot_free + kvz_encode_pages, the other
    with kvz_complete_pages.  Records, stored bytes and counters agree after every step; the
    first pool is also checked against the oracle model."""
    announce(f"complete_pages vs free + encode, {arena_mb} MiB arena")
    rng = np.random.default_rng(arena_mb)
    bank, nat, tags = _bank(seed=7, forced=0.10)
    n_slots = 40000
    pools = [paged.SlotArena(arena_mb << 20) for _ in range(2)]
    metas = []
    for _ in range(2):
        m = torch.empty((n_slots, 8), dtype=torch.uint8, device="cuda")
        m[:, :4] = 0xFF
        m[:, 4:] = 0
        metas.append(m)
    model = SlotPoolModel(pool_capacity_granules(pools[0].arena.numel()))
    live = {}                                   # slot -> source group
    live_off = {}                               # slot -> offset (the model's)
    free_slots = list(range(n_slots))
    # (groups freed, groups encoded): one to twelve free tiles, small and multi-tile encodes, and a
    # call above the one-pass limit (the free, then the bulk path)
    plan = [(0, 3000), (700, 2048), (1024, 1025), (2500, 4096), (6000, 9216), (5000, 100),
            (300, 5000), (4000, 4000), (1, 64), (3000, 20000)]
    for step, (nf, ne) in enumerate(plan):
        nf = min(nf, len(live))
        victims = sorted(rng.choice(sorted(live), size=nf, replace=False).tolist()) if nf else []
        # some of this step's encodes go to the slots just freed (their records are read by the
        # free before the encode rewrites them)
        reuse = victims[:ne // 2]
        fresh_n = ne - len(reuse)
        fresh = [free_slots.pop() for _ in range(min(fresh_n, len(free_slots)))]
        dst = reuse + fresh
        src = rng.integers(0, nat.shape[0], size=len(dst))
        freed_recs = [(live_off[v], tags[live[v]].tolist()) for v in victims] if nf else []
        for i, pool in enumerate(pools):
            d_free = (torch.from_numpy(metas[i].data_ptr() + np.asarray(victims, dtype=np.int64) * 8).cuda()
                      if nf else None)
            d_items = _items(bank, src, metas[i], dst)
            if i == 0:
                if nf:
                    kvz.kvz_slot_free(pool.pool, d_free)
                kvz.kvz_encode_pages(pool.pool, d_items, len(dst))
            else:
                kvz.kvz_complete_pages(pool.pool, d_free, d_items, len(dst))
        torch.cuda.synchronize()
        if nf:
            model.free(freed_recs)
        want = np.asarray(model.alloc([t.tolist() for t in tags[src]]), dtype=np.int64)
        for v in victims:
            del live[v]
        freed_not_reused = [v for v in victims if v not in set(reuse)]
        free_slots.extend(freed_not_reused)
        for d, g, off in zip(dst, src, want):
            live[d] = g
            live_off[d] = int(off)
        # records: both pools, and the model
        ra = metas[0].cpu().numpy()
        rb = metas[1].cpu().numpy()
        np.testing.assert_array_equal(ra, rb, err_msg=f"step {step}")
        got, _ = _records(metas[0], dst)
        np.testing.assert_array_equal(got, want, err_msg=f"step {step}")
        for v in freed_not_reused:
            assert (ra[v, :4] == 0xFF).all() and (ra[v, 4:] == 0).all(), (step, v)
        _check_stats(pools[0], model, f"step {step}")
        sa, sb = pools[0].stats(), pools[1].stats()
        assert sa == sb, (step, sa, sb)
        # the stored bytes of this step's groups are the same in both arenas
        for d, off in zip(dst, want):
            if off == OFF_NONE:
                continue
            n_raw = int((tags[live[d]] == 0xFF).sum())
            a0, a1 = int(off) * 256, (int(off) + 12 + n_raw) * 256
            assert torch.equal(pools[0].arena[a0:a1], pools[1].arena[a0:a1]), (step, d)
    if arena_mb == 24:
        assert model.enospc > 0, "the small arena should run out"


@pytest.mark.parametrize("n", [2048, 9216])
def test_graph_replays_with_new_items_match_eager_calls(n):
    """A captured kvz_complete_pages replayed with other item records each time (other source
    pages, so other size classes per tile) gives what eager calls on a second pool give: each
    launch numbers its records from the device, so a replay never takes the previous replay's
    records for its own."""
    announce(f"complete_pages graph replays with new items, {n} groups")
    rng = np.random.default_rng(n)
    bank, nat, tags = _bank(seed=9, forced=0.30)
    pools = [paged.SlotArena(256 << 20) for _ in range(2)]
    metas, ptrs, items = [], [], []
    src0 = rng.integers(0, nat.shape[0], size=n)
    for i in range(2):
        m = torch.empty((n, 8), dtype=torch.uint8, device="cuda")
        m[:, :4] = 0xFF
        m[:, 4:] = 0
        metas.append(m)
        ptrs.append(torch.from_numpy(m.data_ptr() + np.arange(n, dtype=np.int64) * 8).cuda())
        items.append(_items(bank, src0, m, np.arange(n)))
    # warm-up, capture (the captured call runs once more on replay)
    for _ in range(2):
        kvz.kvz_complete_pages(pools[0].pool, ptrs[0], items[0], n)
        kvz.kvz_complete_pages(pools[1].pool, ptrs[1], items[1], n)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kvz.kvz_complete_pages(pools[0].pool, ptrs[0], items[0], n)
    kvz.kvz_complete_pages(pools[1].pool, ptrs[1], items[1], n)   # the capture's turn, eagerly
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    for rep in range(6):
        src = rng.integers(0, nat.shape[0], size=n)
        items[0].copy_(_items(bank, src, metas[0], np.arange(n)))
        items[1].copy_(_items(bank, src, metas[1], np.arange(n)))
        torch.cuda.synchronize()
        g.replay()
        kvz.kvz_complete_pages(pools[1].pool, ptrs[1], items[1], n)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(metas[0].cpu().numpy(), metas[1].cpu().numpy(), err_msg=f"replay {rep}")
        got, gtags = _records(metas[0], np.arange(n))
        np.testing.assert_array_equal(gtags, tags[src])
        assert pools[0].stats() == pools[1].stats(), rep
        assert pools[0].stats()["enospc"] == 0


def test_a_wait_that_gives_up_halts_the_one_pass_encoder():
    """The failure path of the one-pass launch, forced from the host (KVZ_ENC_SIMULATE_GIVE_UP:
    every workgroup acts as if a wait had given up; every kernel still runs to its end).  That
    launch stores and frees nothing and empties the bins; it halts the one-pass encoder, so the
    next one-pass calls store and free nothing either; a bulk call still allocates as the model
    says; kvz_pool_init brings the one-pass encoder back."""
    announce("one-pass encoder: a wait that gives up (forced), then the halted state")
    rng = np.random.default_rng(13)
    bank, nat, tags = _bank(seed=13, forced=0.10)
    arena = paged.SlotArena(256 << 20)
    model = SlotPoolModel(pool_capacity_granules(arena.arena.numel()))
    n_slots = 40000
    meta = torch.empty((n_slots, 8), dtype=torch.uint8, device="cuda")
    meta[:, :4] = 0xFF
    meta[:, 4:] = 0

    def ptrs(ids):
        return torch.from_numpy(meta.data_ptr() + np.asarray(ids, dtype=np.int64) * 8).cuda()

    # a normal call, then a free of part of it (the bins hold runs)
    src0 = rng.integers(0, nat.shape[0], size=3000)
    kvz.kvz_encode_pages(arena.pool, _items(bank, src0, meta, np.arange(3000)), 3000)
    off0 = model.alloc([t.tolist() for t in tags[src0]])
    kvz.kvz_slot_free(arena.pool, ptrs(np.arange(0, 3000, 3)))
    model.free([(off0[i], tags[src0[i]].tolist()) for i in range(0, 3000, 3)])
    _check_stats(arena, model, "before")
    assert arena.stats()["encoder_halted"] == 0
    before = meta.cpu().numpy()

    # the forced give-up: frees of 1,000 live groups and 2,000 encodes into fresh slots
    victims = np.arange(1, 3000, 3)
    src1 = rng.integers(0, nat.shape[0], size=2000)
    ids1 = 3000 + np.arange(2000)
    kvz.kvz_complete_pages(arena.pool, ptrs(victims), _items(bank, src1, meta, ids1), 2000,
                           flags=kvz.KVZ_ENC_SIMULATE_GIVE_UP)
    got, gtags = _records(meta, ids1)
    assert (got == OFF_NONE).all()
    np.testing.assert_array_equal(gtags, tags[src1])
    np.testing.assert_array_equal(meta.cpu().numpy()[victims], before[victims])   # not freed
    st = arena.stats()
    assert st["encoder_halted"] == 1
    assert st["free_runs"] == [0] * 5 and st["frontier_granules"] == model.frontier
    assert st["enospc"] == model.enospc + 2000 and st["bad_frees"] == len(victims)
    assert st["live_runs"] == model.live_runs and st["live_granules"] == model.live_granules
    model.bins = [[] for _ in range(5)]            # the launch emptied the bins
    model.enospc += 2000

    # halted: a one-pass encode and a fused call store and free nothing
    for what in ("encode", "complete"):
        src2 = rng.integers(0, nat.shape[0], size=700)
        ids2 = (5000 if what == "encode" else 6000) + np.arange(700)
        items = _items(bank, src2, meta, ids2)
        if what == "encode":
            kvz.kvz_encode_pages(arena.pool, items, 700)
        else:
            kvz.kvz_complete_pages(arena.pool, ptrs(np.arange(2, 3000, 3)), items, 700)
        got, gtags = _records(meta, ids2)
        assert (got == OFF_NONE).all(), what
        np.testing.assert_array_equal(gtags, tags[src2])
        model.enospc += 700
        _check_stats(arena, model, f"halted {what}")
        assert arena.stats()["encoder_halted"] == 1
        assert arena.stats()["bad_frees"] == len(victims)
    np.testing.assert_array_equal(meta.cpu().numpy()[2:3000:3], before[2:3000:3])

    # a bulk call is not affected: it allocates from the frontier as the model does
    src3 = rng.integers(0, nat.shape[0], size=20000)
    ids3 = 8000 + np.arange(20000)
    kvz.kvz_encode_pages(arena.pool, _items(bank, src3, meta, ids3), 20000)
    want3 = np.asarray(model.alloc([t.tolist() for t in tags[src3]]), dtype=np.int64)
    got, _ = _records(meta, ids3)
    np.testing.assert_array_equal(got, want3)
    _check_stats(arena, model, "bulk while halted")

    # kvz_pool_init: empty pool, one-pass encoder working
    kvz.kvz_pool_destroy(arena.pool)
    arena.pool = kvz.kvz_pool_init(arena.arena, arena.state)
    model = SlotPoolModel(pool_capacity_granules(arena.arena.numel()))
    src4 = rng.integers(0, nat.shape[0], size=3000)
    ids4 = 30000 + np.arange(3000)
    kvz.kvz_complete_pages(arena.pool, None, _items(bank, src4, meta, ids4), 3000)
    want4 = np.asarray(model.alloc([t.tolist() for t in tags[src4]]), dtype=np.int64)
    got, _ = _records(meta, ids4)
    np.testing.assert_array_equal(got, want4)
    _check_stats(arena, model, "after kvz_pool_init")
    assert arena.stats()["encoder_halted"] == 0
    arena_h = arena.arena.cpu().numpy()
    for i in rng.choice(3000, 24, replace=False):
        g = src4[i]
        np.testing.assert_array_equal(
            codec.decode_group(arena_h, int(want4[i]), tags[g].tolist(), int((g // HKV) % 2)), nat[g])


def test_launch_numbers_across_the_short_tag_wrap():
    """17,000 steady-state steps (free the previous records, encode the same pages again) on one
    pool with kvz_complete_pages and on another with kvz_slot_free + kvz_encode_pages, captured
    100 steps per graph: both cross the free tiles' 14-bit launch tag (16,383 values), with two
    free tiles per step exchanging their counts.  The records, arena bytes and counters of the two
    pools agree, the counters are those of the step's groups, and a sample of groups decodes to
    its source."""
    announce("17,000 completion steps across the 14-bit launch tag")
    rng = np.random.default_rng(21)
    bank, nat, tags = _bank(seed=21, forced=0.10)
    n = 600                                    # two free tiles of up to 512 groups
    src = rng.integers(0, nat.shape[0], size=n)
    pools = [paged.SlotArena(64 << 20) for _ in range(2)]
    metas, items, ptrs = [], [], []
    for i in range(2):
        m = torch.empty((n, 8), dtype=torch.uint8, device="cuda")
        m[:, :4] = 0xFF
        m[:, 4:] = 0
        metas.append(m)
        items.append(_items(bank, src, m, np.arange(n)))
        ptrs.append(torch.from_numpy(m.data_ptr() + np.arange(n, dtype=np.int64) * 8).cuda())
        kvz.kvz_encode_pages(pools[i].pool, items[i], n)

    def step(i):
        if i == 0:
            kvz.kvz_complete_pages(pools[0].pool, ptrs[0], items[0], n)
        else:
            kvz.kvz_slot_free(pools[1].pool, ptrs[1])
            kvz.kvz_encode_pages(pools[1].pool, items[1], n)
    graphs = []
    for i in range(2):
        step(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(100):
                step(i)
        graphs.append(g)
    for _ in range(170):
        for g in graphs:
            g.replay()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(metas[0].cpu().numpy(), metas[1].cpu().numpy())
    sa, sb = pools[0].stats(), pools[1].stats()
    assert sa == sb, (sa, sb)
    assert sa["live_runs"] == n and sa["enospc"] == 0 and sa["bad_frees"] == 0
    assert sa["encoder_halted"] == 0
    assert sa["live_raw_blocks"] == int((tags[src] == 0xFF).sum())
    assert torch.equal(pools[0].arena, pools[1].arena)
    offs, gtags = _records(metas[0], np.arange(n))
    np.testing.assert_array_equal(gtags, tags[src])
    arena_h = pools[0].arena.cpu().numpy()
    for i in rng.choice(n, 32, replace=False):
        g = src[i]
        np.testing.assert_array_equal(
            codec.decode_group(arena_h, int(offs[i]), tags[g].tolist(), int((g // HKV) % 2)), nat[g])
