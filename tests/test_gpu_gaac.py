"""GPU parity of the group-adaptive additive exponent code (second page format) against the CPU
oracle: calibration, the encoded arena and metadata bit for bit, decompression, and the slot
pool shared with the first format."""
import numpy as np
import pytest
import torch

from decode_attention_kvz_amd import kvz, paged, synth
from oracle import codec, gaac
from oracle.alloc import OFF_NONE
from oracle.cache import GaacOracleCache

from gpu_util import announce, build_layer

pytestmark = pytest.mark.gpu


def _oracle_bases(cal_pages):
    """Oracle bases [Hkv, 2, 2, 128] from natural calibration pages [S, P, 2, Hkv, 16, 128]."""
    nat = synth.bits(cal_pages)
    hkv = nat.shape[3]
    out = np.zeros((hkv, 2, 2, 128), dtype=np.uint8)
    for h in range(hkv):
        for kind in range(2):
            b3, b4 = gaac.calibrate(nat[:, :, kind, h].reshape(-1, 16, 128), kind)
            out[h, kind, 0], out[h, kind, 1] = b3, b4
    return out


@pytest.mark.parametrize("u_max", [3.0, 5.0])
def test_calibration_matches_oracle(u_max):
    announce(f"gaac calibration u_max={u_max}")
    cal = synth.kv_pages(2, 12, 4, seed=70, u_max=u_max, forced_frac=0.05, device="cuda")
    got = paged.gaac_calibrate(cal).cpu().numpy()
    np.testing.assert_array_equal(got, _oracle_bases(cal))


def _encode_layer(pages, bases, arena, seed, flags=0):
    """Encode every page of `pages` (all sequences full) through kvz_gaac_encode_pages, physical
    pages in a seeded random order.  Returns (meta, block_table, items)."""
    bsz, n_pages, _, hkv = pages.shape[:4]
    rng = np.random.default_rng(seed)
    n_phys = bsz * n_pages
    block_table = rng.permutation(n_phys).reshape(bsz, n_pages).astype(np.int32)
    meta = paged.new_meta_table(n_phys, hkv)
    ids = [(b, p) for b in range(bsz) for p in range(n_pages)]
    items = paged.gaac_page_items(pages, ids, meta, block_table.reshape(-1), bases)
    d_items = paged.gaac_encode(arena, items, flags)
    torch.cuda.synchronize()
    return meta, block_table, d_items


def _oracle_encode(pages, bases_h, block_table, arena_bytes, force_raw=False):
    """The oracle's arena and metas for the same items in the same order."""
    nat = synth.bits(pages)
    bsz, n_pages, _, hkv = nat.shape[:4]
    tiles, kinds, bl = [], [], []
    for b in range(bsz):
        for p in range(n_pages):
            for h in range(hkv):
                for kind in range(2):
                    tiles.append(nat[b, p, kind, h])
                    kinds.append(kind)
                    bl.append((bases_h[h, kind, 0], bases_h[h, kind, 1]))
    oc = GaacOracleCache(arena_bytes)
    metas = oc.encode_gaac(np.stack(tiles), kinds, bl, force_raw=force_raw)
    return oc, metas


@pytest.mark.parametrize("force_raw,stress", [(False, False), (True, False), (False, True)])
def test_encode_matches_oracle_arena_and_meta(force_raw, stress):
    """2 sequences x 9 pages x 4 KV heads; bases calibrated on another sample of the same layer: the whole
    arena, every metadata record and the pool counters equal the oracle's."""
    announce(f"gaac encode force_raw={force_raw} stress={stress}")
    cal = synth.kv_pages(2, 6, 4, seed=72, u_max=3.0, forced_frac=0.0, sample=1, device="cuda")
    bases = paged.gaac_calibrate(cal)
    pages = synth.kv_pages(2, 9, 4, seed=72, u_max=3.0, forced_frac=0.2, stress=stress,
                           device="cuda")
    arena_bytes = 2 * 9 * 4 * 2 * 4096 + (64 << 10)
    arena = paged.SlotArena(arena_bytes)
    meta, block_table, _ = _encode_layer(pages, bases, arena, seed=72,
                                         flags=kvz.KVZ_ENC_FORCE_RAW if force_raw else 0)
    oc, metas = _oracle_encode(pages, bases.cpu().numpy(), block_table, arena_bytes, force_raw)
    # item k = (b, p, h, kind) -> meta record of physical page block_table[b, p]
    m = meta.cpu().numpy()
    k = 0
    for b in range(2):
        for p in range(9):
            for h in range(4):
                for kind in range(2):
                    rec = m[block_table[b, p], h, kind]
                    off = int.from_bytes(rec[:4].tobytes(), "little")
                    assert (off, [int(x) for x in rec[4:]]) == (metas[k][0], metas[k][1]), k
                    k += 1
    np.testing.assert_array_equal(arena.arena.cpu().numpy(), oc.arena)
    st = arena.stats()
    assert st["frontier_granules"] == oc.pool.frontier
    assert st["live_runs"] == oc.pool.live_runs
    n_raw_tiles = sum(1 for _, t in metas if t == gaac.TAGS_RAW)
    announce(f"gaac encode: {n_raw_tiles} of {len(metas)} tiles raw")
    if force_raw:
        assert n_raw_tiles == len(metas)
    elif stress:     # zeros, subnormals and Inf/NaN push most tiles past the escape slot
        assert len(metas) // 2 < n_raw_tiles
    else:
        assert n_raw_tiles < len(metas)


@pytest.mark.parametrize("stride,shift", [(136, 0), (131, 1)])
def test_encode_from_strided_sources_matches_oracle(stride, shift):
    """Items whose token rows are `stride` elements apart, the first one `shift` elements past a
    16-byte boundary: the buffer-load path with a row stride other than 128 (136) and the
    element-wise path (odd stride, misaligned base) both give the oracle's tiles and metadata."""
    announce(f"gaac encode strided sources stride={stride} shift={shift}")
    cal = synth.kv_pages(1, 6, 2, seed=74, u_max=3.0, forced_frac=0.0, sample=1, device="cuda")
    bases = paged.gaac_calibrate(cal)
    pages = synth.kv_pages(1, 8, 2, seed=74, u_max=3.0, forced_frac=0.2)
    nat = synth.bits(pages)[0]                                # [8, 2, 2, 16, 128]
    flat = nat.transpose(0, 2, 1, 3, 4).reshape(-1, 16, 128)  # item order (page, head, K/V)
    n = flat.shape[0]
    kinds = [i % 2 for i in range(n)]
    heads = [(i // 2) % 2 for i in range(n)]
    buf = np.zeros((n, 16, stride), dtype=np.uint16)
    buf[:, :, :128] = flat
    dev = torch.zeros(shift + buf.size + 8, dtype=torch.int16, device="cuda")
    dev[shift:shift + buf.size] = torch.from_numpy(buf.reshape(-1).view(np.int16)).cuda()
    base = dev.data_ptr() + 2 * shift
    meta = paged.new_meta_table(8, 2)
    items = torch.from_numpy(kvz.gaac_items(
        [base + 2 * i * 16 * stride for i in range(n)], [meta.data_ptr() + 8 * i for i in range(n)],
        stride, kinds, [bases.data_ptr() + (heads[i] * 2 + kinds[i]) * 256 for i in range(n)])).cuda()
    arena_bytes = 256 * 1024
    arena = paged.SlotArena(arena_bytes)
    kvz.kvz_gaac_encode_pages(arena.pool, items, n)
    torch.cuda.synchronize()
    bh = bases.cpu().numpy()
    oc = GaacOracleCache(arena_bytes)
    metas = oc.encode_gaac(flat, kinds, [(bh[heads[i], kinds[i], 0], bh[heads[i], kinds[i], 1])
                                         for i in range(n)])
    m = meta.cpu().numpy().reshape(-1, 8)
    for i in range(n):
        off = int.from_bytes(m[i, :4].tobytes(), "little")
        assert (off, [int(x) for x in m[i, 4:]]) == (metas[i][0], list(metas[i][1])), i
    np.testing.assert_array_equal(arena.arena.cpu().numpy(), oc.arena)


def test_decompress_matches_oracle_decode():
    """Decompress every tile of a layer (compressed and raw tiles, an unstored one) into the raw
    chunk layout: equal to the oracle's all-raw record of the input page."""
    announce("gaac decompress")
    cal = synth.kv_pages(1, 8, 2, seed=74, u_max=3.0, forced_frac=0.0, sample=1, device="cuda")
    bases = paged.gaac_calibrate(cal)
    pages = synth.kv_pages(3, 7, 2, seed=74, u_max=3.0, forced_frac=0.3, device="cuda")
    arena = paged.SlotArena(3 * 7 * 2 * 2 * 4096 + (64 << 10))
    rng = np.random.default_rng(74)
    block_table = rng.permutation(21).reshape(3, 7).astype(np.int32)
    meta = paged.new_meta_table(21, 2)
    keep = []
    for seqs, flags in (([0], kvz.KVZ_ENC_FORCE_RAW), ([1, 2], 0)):   # raw and compressed tiles
        ids = [(b, p) for b in seqs for p in range(7)]
        phys = [block_table[b, p] for b, p in ids]
        keep.append(paged.gaac_encode(arena, paged.gaac_page_items(pages, ids, meta, phys, bases),
                                      flags))
    torch.cuda.synchronize()
    meta2 = meta.clone()
    m = meta2.cpu().numpy()
    m[0, 0, 0, :4] = 0xFF                  # phys page 0, head 0, K: not stored -> zeros
    meta2.copy_(torch.from_numpy(m))
    store = paged.gaac_decompress_pages(arena, meta2, bases).cpu().numpy()
    nat = synth.bits(pages)
    tags = m[..., 4:]
    assert (tags == 0xFF).all(axis=-1).any() and (tags == 0).all(axis=-1).any()
    for b in range(3):
        for p in range(7):
            ph = block_table[b, p]
            for h in range(2):
                for kind in range(2):
                    got = store[ph, kind, h].reshape(-1)
                    if (ph, h, kind) == (0, 0, 0):
                        assert (got == 0).all()
                        continue
                    want = codec.encode_group(nat[b, p, kind, h], kind, force_raw=True)[1]
                    np.testing.assert_array_equal(got, want, err_msg=f"{(b, p, h, kind)}")


def test_full_size_qwen8k_layer_round_trip_and_ratio():
    """The 8K workload's layer (16 x 511 pages, 8 KV heads, u~U[-5,5], 5% forced), bases from
    another sample of the same layer: decompression returns every page bit for bit; sampled
    records equal the oracle's; the per-dim bases absorb the per-channel spread."""
    announce("gaac full 8K layer")
    bsz, n_comp, hkv = 16, 511, 8
    cal = synth.kv_pages(4, 32, hkv, seed=2, u_max=5.0, forced_frac=0.05, sample=1, device="cuda")
    bases = paged.gaac_calibrate(cal)
    pages = synth.kv_pages(bsz, n_comp, hkv, seed=2, u_max=5.0, forced_frac=0.05, device="cuda")
    arena = paged.SlotArena(bsz * n_comp * hkv * 2 * 4096 + (16 << 20))
    meta, block_table, _ = _encode_layer(pages, bases, arena, seed=2)
    st = arena.stats()
    n_tiles = bsz * n_comp * hkv * 2
    assert st["live_runs"] == n_tiles and st["enospc"] == 0
    tags = meta.cpu().numpy()[..., 4:]
    raw_frac = float((tags == 0xFF).all(axis=-1).mean())
    bytes_ratio = n_tiles * 4096 / (st["live_granules"] * 256)
    announce(f"gaac 8K layer: raw tiles {raw_frac:.4f}, storage ratio {bytes_ratio:.3f}")
    assert raw_frac < 0.5 and bytes_ratio > 1.1
    store = paged.gaac_decompress_pages(arena, meta, bases)
    inv = torch.as_tensor(np.argsort(block_table.reshape(-1)), device="cuda")
    nat_phys = pages.reshape(bsz * n_comp, 2, hkv, 16, 128)[inv]
    assert torch.equal(store, paged.pack_bf16_pages(nat_phys))
    arena_h = arena.arena.cpu().numpy()
    bases_h = bases.cpu().numpy()
    nat_h = synth.bits(nat_phys)
    m = meta.cpu().numpy()
    rng = np.random.default_rng(75)
    for g in rng.choice(n_tiles, 128, replace=False):
        ph, kind, h = int(g // (2 * hkv)), int((g // hkv) % 2), int(g % hkv)
        raw, rec = gaac.encode_tile(nat_h[ph, kind, h], kind, bases_h[h, kind, 0], bases_h[h, kind, 1])
        off = int.from_bytes(m[ph, h, kind, :4].tobytes(), "little")
        assert off != OFF_NONE
        assert list(m[ph, h, kind, 4:]) == gaac.tags_of(raw)
        np.testing.assert_array_equal(arena_h[off * 256: off * 256 + rec.size], rec)


# ---------------------------------------------------------------------------------------------
# fused attention over group-adaptive tiles
# ---------------------------------------------------------------------------------------------
from gpu_util import (check_rows, oracle_attention_rows, report_effective, run_bf16, run_gaac,  # noqa: E402
                      scaled_queries, sm_scale)


@pytest.mark.parametrize("hq,hkv", [(32, 8), (16, 2), (12, 4)])
def test_gaac_attention_matches_oracle_and_baseline(hq, hkv):
    """Ragged sequences (an empty one, a tail-only one, partial tails), some tiles raw: within
    the tolerance of the fp64 oracle, and bit for bit the uncompressed kernel's output at the
    same split count."""
    announce(f"gaac attention hq={hq} hkv={hkv}")
    bsz = 5
    cal = synth.kv_pages(2, 8, hkv, seed=80, u_max=3.0, forced_frac=0.05, sample=1, device="cuda")
    bases = paged.gaac_calibrate(cal)
    pages = synth.kv_pages(bsz, 41, hkv, seed=80, u_max=3.0, forced_frac=0.05, device="cuda")
    q = synth.queries(bsz, hq, seed=80, device="cuda")
    seq_lens, n_comp = [16 * 40 + 7, 16 * 23 + 16, 0, 9, 16 * 40], [40, 23, 0, 0, 40]
    arena = paged.SlotArena(bsz * 41 * hkv * 2 * 4096 + (1 << 20))
    layer = build_layer(arena, pages, seq_lens, n_comp, seed=80, gaac_bases=bases)
    tags = layer.meta.cpu().numpy()[..., 4:]
    assert (tags == 0).all(axis=-1).any()
    got = run_gaac(layer, arena, bases, q, sm_scale())
    # with the same split count the two kernels run the same arithmetic on the same values
    same = run_gaac(layer, arena, bases, q, sm_scale(), splits=5)
    base = run_bf16(layer, q, sm_scale(), splits=5)
    torch.cuda.synchronize()
    assert torch.equal(same, base)
    ref = oracle_attention_rows(layer, q, sm_scale(), range(bsz))
    g = got.cpu().numpy()
    for b in range(bsz):
        if seq_lens[b] == 0:
            assert (g[b] == 0).all()
        else:
            check_rows(g[b], ref[b], what=f"gaac seq {b}")


def test_gaac_attention_raw_and_compressed_tiles_agree_bitwise():
    """The same pages stored all raw (KVZ_ENC_FORCE_RAW) and compressed give identical output:
    the restore is exact."""
    announce("gaac attention storage-mode invariance")
    cal = synth.kv_pages(1, 8, 8, seed=81, u_max=5.0, forced_frac=0.05, sample=1, device="cuda")
    bases = paged.gaac_calibrate(cal)
    pages = synth.kv_pages(3, 30, 8, seed=81, u_max=5.0, forced_frac=0.05, device="cuda")
    q = synth.queries(3, 32, seed=81, device="cuda")
    outs = []
    for flags in (0, kvz.KVZ_ENC_FORCE_RAW):
        arena = paged.SlotArena(3 * 30 * 8 * 2 * 4096 + (1 << 20))
        layer = build_layer(arena, pages, [16 * 29 + 5] * 3, [29] * 3, seed=81, flags=flags,
                            gaac_bases=bases)
        outs.append(run_gaac(layer, arena, bases, q, sm_scale()).clone())
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("forced_exp,q_log2,min_eff", [
    pytest.param(12.0, 0, None, id="forced2^12"),
    pytest.param(-16.0, 0, None, id="forced2^-16"),
    pytest.param(-16.0, -3, 10.0, id="forced2^-16-broad"),
])
def test_gaac_attention_full_size_qwen8k_sampled(forced_exp, q_log2, min_eff):
    """The 8K workload's shape (16 x 511 compressed pages + the 16-token tail, u~U[-5,5]): rows
    of 8 sequences against the oracle, all rows bit for bit against the uncompressed kernel
    run with the same split count.  Forced elements as specified (one-hot softmax), tiny, and
    tiny with q scaled down (every checked head spreads over more than 10 keys)."""
    announce(f"gaac attention full 8K forced=2^{forced_exp:g} q x2^{q_log2}")
    bsz, n_comp, hkv, hq = 16, 511, 8, 32
    cal = synth.kv_pages(4, 32, hkv, seed=2, u_max=5.0, forced_frac=0.05, forced_exp=forced_exp,
                         sample=1, device="cuda")
    bases = paged.gaac_calibrate(cal)
    pages = synth.kv_pages(bsz, n_comp + 1, hkv, seed=2, u_max=5.0, forced_frac=0.05,
                           forced_exp=forced_exp, device="cuda")
    q = scaled_queries(synth.queries(bsz, hq, seed=2, device="cuda"), q_log2)
    arena = paged.SlotArena(bsz * n_comp * hkv * 2 * 4096 + (16 << 20))
    layer = build_layer(arena, pages, [16 * n_comp + 16] * bsz, [n_comp] * bsz, seed=2,
                        gaac_bases=bases)
    got = run_gaac(layer, arena, bases, q, sm_scale())
    same = run_gaac(layer, arena, bases, q, sm_scale(), splits=16)
    base = run_bf16(layer, q, sm_scale(), splits=16)
    torch.cuda.synchronize()
    assert torch.equal(same, base)
    samples = [0, 2, 5, 7, 9, 11, 13, 15]
    eff = {}
    ref = oracle_attention_rows(layer, q, sm_scale(), samples, eff)
    g = got.cpu().numpy()
    for b in samples:
        check_rows(g[b], ref[b], what=f"gaac 8K seq {b}")
    lo = report_effective(eff, "gaac 8K")
    if min_eff is not None:
        assert lo > min_eff


def test_gaac_attention_non_finite_values_propagate_like_the_oracle():
    """NaN / Inf in K and V: out of both windows, so their groups go raw inside compressed tiles;
    the non-finite output positions equal the oracle's."""
    announce("gaac attention non-finite propagation")
    cal = synth.kv_pages(2, 8, 2, seed=82, forced_frac=0.0, sample=1, device="cuda")
    bases = paged.gaac_calibrate(cal)
    pages = synth.kv_pages(4, 9, 2, seed=82, forced_frac=0.0, device="cuda")
    bits = pages.view(torch.int16)
    bits[0, 2, 1, 0, 3, 17] = 0x7FC0          # NaN in V: one output dim of head group 0
    bits[1, 4, 0, 1, 5, 3] = 0x7F80           # +Inf in K: scores of head group 1 go non-finite
    bits[2, 8, 1, 0, 2, 40] = -128            # -Inf (0xFF80) in V on the tail page
    q = synth.queries(4, 8, seed=82, device="cuda")
    seq_lens, n_comp = [16 * 8 + 4, 16 * 8 + 4, 16 * 8 + 4, 16 * 8], [8, 8, 8, 8]
    arena = paged.SlotArena(4 * 9 * 2 * 2 * 4096 + (1 << 20))
    layer = build_layer(arena, pages, seq_lens, n_comp, seed=82, gaac_bases=bases)
    tags = layer.meta.cpu().numpy()[..., 4:]
    assert (tags == 0).all()                  # every tile compressed (raw groups inside)
    got = run_gaac(layer, arena, bases, q, sm_scale()).cpu().numpy()
    ref = oracle_attention_rows(layer, q, sm_scale(), range(4))
    for b in range(4):
        check_rows(got[b], ref[b], what=f"gaac seq {b}")
    assert not np.isfinite(got[0]).all() and not np.isfinite(got[2]).all()
