"""GPU parity of the exponent code on FP8 KV (E4M3 and E5M2) against the CPU oracle: the
hardware FP8 -> BF16 conversion, calibration, the encoded arena and metadata bit for bit,
decompression and the uncompressed layout, and fused / uncompressed FP8 decode attention."""
import numpy as np
import pytest
import torch

from decode_attention_kvz_amd import kvz, paged, synth
from oracle import fp8
from oracle.alloc import SlotPoolModel
from oracle.cache import Fp8OracleCache

from gpu_util import announce, check_rows, sm_scale

pytestmark = pytest.mark.gpu
FORMATS = [kvz.KVZ_FP8_E4M3, kvz.KVZ_FP8_E5M2]
NAME = {kvz.KVZ_FP8_E4M3: "e4m3", kvz.KVZ_FP8_E5M2: "e5m2"}


def _oracle_bases(cal_pages, fmt):
    nat = cal_pages.cpu().numpy()
    hkv = nat.shape[3]
    out = np.zeros((hkv, 2, 2, 128), dtype=np.uint8)
    for h in range(hkv):
        for kind in range(2):
            out[h, kind, 0], out[h, kind, 1] = fp8.calibrate(nat[:, :, kind, h].reshape(-1, 16, 128), fmt)
    return out


class Fp8Layer:
    """Pages [B, P, 2, Hkv, 16, 128] uint8 encoded into an FP8 pool: sequence b has n_comp[b]
    compressed pages (physical ids in a seeded random order) and its tail is page n_comp[b]."""

    def __init__(self, pages, seq_lens, n_comp, fmt, bases, *, seed, flags=0, arena_extra=1 << 16):
        bsz, n_total, _, hkv = pages.shape[:4]
        self.pages, self.fmt, self.bases = pages, fmt, bases
        n_comp = np.asarray(n_comp, dtype=np.int64)
        self.n_phys = max(int(n_comp.sum()), 1)
        max_pages = max(int(n_comp.max()), 1)
        perm = np.random.default_rng(seed).permutation(self.n_phys)
        bt = np.zeros((bsz, max_pages), dtype=np.int32)
        ids, phys = [], []
        k = 0
        for b in range(bsz):
            for p in range(int(n_comp[b])):
                bt[b, p] = perm[k]
                ids.append((b, p))
                phys.append(perm[k])
                k += 1
        self.arena = paged.SlotArena(self.n_phys * hkv * 2 * 2048 + arena_extra, fp8=True)
        self.meta = paged.new_meta_table(self.n_phys, hkv)
        self.items = None
        if ids:
            items = paged.fp8_page_items(pages, ids, self.meta, phys, bases)
            self.items = paged.fp8_encode(self.arena, items, fmt, flags)
        idx = torch.as_tensor(np.minimum(n_comp, n_total - 1), device=pages.device)
        self.tail = pages[torch.arange(bsz, device=pages.device), idx].contiguous()
        dev = pages.device
        self.phys_of = bt
        self.block_table = torch.from_numpy(bt).to(dev)
        self.seq_lens = torch.as_tensor(np.asarray(seq_lens, dtype=np.int32), device=dev)
        self.n_comp = torch.as_tensor(n_comp.astype(np.int32), device=dev)
        self.hkv = hkv

    def fused(self, q, ks, vs, splits=0):
        out = torch.empty((q.shape[0], q.shape[1], 128), dtype=torch.float32, device=q.device)
        ws = paged.workspace(q.shape[0], q.shape[1], self.hkv, self.block_table.shape[1], splits)
        kvz.kvz_fp8_decode_attention(q, out, self.fmt, self.arena.arena, self.meta, self.bases,
                                     self.block_table, self.seq_lens, self.n_comp, self.tail,
                                     sm_scale(), ks, vs, ws, splits)
        return out

    def raw(self, q, ks, vs, splits=0):
        """The uncompressed FP8 kernel over the same pages, packed by physical id."""
        nat = torch.zeros((self.n_phys, 2, self.hkv, 16, 128), dtype=torch.uint8, device=q.device)
        for b in range(q.shape[0]):
            nc = int(self.n_comp[b])
            if nc:
                nat[torch.as_tensor(self.phys_of[b, :nc], device=q.device, dtype=torch.long)] = self.pages[b, :nc]
        store = paged.pack_fp8_pages(nat)
        out = torch.empty((q.shape[0], q.shape[1], 128), dtype=torch.float32, device=q.device)
        ws = paged.workspace(q.shape[0], q.shape[1], self.hkv, self.block_table.shape[1], splits)
        kvz.kvz_fp8_raw_decode_attention(q, out, self.fmt, store, self.block_table, self.seq_lens,
                                         self.n_comp, self.tail, sm_scale(), ks, vs, ws, self.hkv,
                                         splits)
        return out

    def oracle_rows(self, q, ks, vs, batch_indices):
        """Oracle attention from the input FP8 pages (what the encoder received)."""
        pages = self.pages.cpu().numpy()
        qb = synth.bits(q)
        out = {}
        for b in batch_indices:
            nc = int(self.n_comp[b])
            nt = int(self.seq_lens[b]) - 16 * nc
            k = pages[b, :nc, 0].transpose(0, 2, 1, 3).reshape(16 * nc, self.hkv, 128)
            v = pages[b, :nc, 1].transpose(0, 2, 1, 3).reshape(16 * nc, self.hkv, 128)
            if nt > 0:
                k = np.concatenate([k, pages[b, nc, 0, :, :nt].transpose(1, 0, 2)])
                v = np.concatenate([v, pages[b, nc, 1, :, :nt].transpose(1, 0, 2)])
            out[b] = fp8.attention_fp64(qb[b], k, v, self.fmt, sm_scale(), ks, vs)
        return out


@pytest.mark.parametrize("fmt", FORMATS)
def test_hardware_conversion_is_exact_for_every_byte(fmt):
    """One-token attention returns that token's V: every one of the 256 byte patterns placed in
    the V of a single-token sequence comes back as its exact value (non-finite where the value
    is NaN or Inf), through the uncompressed kernel's tail path and through a compressed page."""
    announce(f"fp8 {NAME[fmt]} conversion, all byte patterns")
    hkv = 2
    pages = torch.zeros((1, 2, 2, hkv, 16, 128), dtype=torch.uint8)
    pat = np.arange(256, dtype=np.uint8).reshape(hkv, 128)
    pages[0, 0, 1, :, 0, :] = torch.from_numpy(pat)     # V of token 0 of page 0 (the tail)
    pages = pages.cuda()
    bases = paged.fp8_calibrate(pages, fmt)
    lay = Fp8Layer(pages, [1], [0], fmt, bases, seed=1)
    q = synth.queries(1, 8, seed=3, device="cuda")
    want = fp8.to_f64(pat, fmt)                          # [hkv, 128]
    for name, got in (("tail", lay.raw(q, 1.0, 1.0)), ("fused-tail", lay.fused(q, 1.0, 1.0))):
        g = got.cpu().numpy().reshape(hkv, 4, 128)
        for h in range(hkv):
            for r in range(4):
                fin = np.isfinite(want[h])
                assert np.array_equal(np.isfinite(g[h, r]), fin), name
                assert np.array_equal(g[h, r][fin], want[h][fin].astype(np.float32)), name
    # the same values inside a compressed page: K zero everywhere except token 3, dim 0, where
    # q's one-hot query picks it with an overwhelming score (k_scale 4 for E4M3, 1/32 for E5M2:
    # ~229 in log2 units, so every other weight underflows to 0 and the scores stay on the
    # plain fp32 path), so the output is V of token 3
    pages2 = torch.zeros((1, 2, 2, hkv, 16, 128), dtype=torch.uint8)
    one = 0x38 if fmt == kvz.KVZ_FP8_E4M3 else 0x3C
    big = 0x7E if fmt == kvz.KVZ_FP8_E4M3 else 0x7B      # the largest finite value
    pages2[0, 0, 0, :, 3, 0] = big
    pages2[0, 0, 1, :, :, :] = one
    pages2[0, 0, 1, :, 3, :] = torch.from_numpy(pat)
    pages2 = pages2.cuda()
    for force in (0, kvz.KVZ_ENC_FORCE_RAW):
        lay2 = Fp8Layer(pages2, [16], [1], fmt, paged.fp8_calibrate(pages2, fmt), seed=2, flags=force)
        qh = torch.zeros((1, 8, 128), dtype=torch.bfloat16, device="cuda")
        qh[:, :, 0] = 1.0
        k_scale = 4.0 if fmt == kvz.KVZ_FP8_E4M3 else 1.0 / 32.0
        got = lay2.fused(qh, k_scale, 1.0).cpu().numpy().reshape(hkv, 4, 128)
        for h in range(hkv):
            fin = np.isfinite(want[h])
            for r in range(4):
                assert np.array_equal(np.isfinite(got[h, r]), fin)
                assert np.array_equal(got[h, r][fin], want[h][fin].astype(np.float32))
        # a score 250 times larger takes the float64 score path: the chosen token's weight is
        # then carried as bf16 hi + lo parts like any other (2^-17 relative)
        got = lay2.fused(qh, 250.0 * k_scale, 1.0).cpu().numpy().reshape(hkv, 4, 128)
        for h in range(hkv):
            fin = np.isfinite(want[h])
            for r in range(4):
                assert np.array_equal(np.isfinite(got[h, r]), fin)
                np.testing.assert_allclose(got[h, r][fin], want[h][fin], rtol=2.0 ** -16, atol=0)


@pytest.mark.parametrize("fmt", FORMATS)
def test_calibration_matches_oracle(fmt):
    announce(f"fp8 {NAME[fmt]} calibration")
    cal = synth.fp8_kv_pages(2, 10, 4, seed=80, fmt=fmt, device="cuda")
    np.testing.assert_array_equal(paged.fp8_calibrate(cal, fmt).cpu().numpy(), _oracle_bases(cal, fmt))


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("stride,shift", [(136, 0), (131, 1)])
def test_encode_from_strided_sources_matches_oracle(fmt, stride, shift):
    """Items whose token rows are `stride` bytes apart, the first one `shift` bytes past an
    8-byte boundary: the buffer-load path with a row stride other than 128 (136) and the
    byte-wise path (odd stride, misaligned base) both give the oracle's tiles and metadata."""
    announce(f"fp8 {NAME[fmt]} encode strided sources stride={stride} shift={shift}")
    cal = synth.fp8_kv_pages(1, 6, 2, seed=84, fmt=fmt, forced_frac=0.0, sample=1, device="cuda")
    bases = paged.fp8_calibrate(cal, fmt)
    pages = synth.fp8_kv_pages(1, 8, 2, seed=84, fmt=fmt, forced_frac=0.2)
    nat = pages.cpu().numpy()[0]                              # [8, 2, 2, 16, 128] uint8
    flat = nat.transpose(0, 2, 1, 3, 4).reshape(-1, 16, 128)  # item order (page, head, K/V)
    n = flat.shape[0]
    kinds = [i % 2 for i in range(n)]
    heads = [(i // 2) % 2 for i in range(n)]
    buf = np.zeros((n, 16, stride), dtype=np.uint8)
    buf[:, :, :128] = flat
    dev = torch.zeros(shift + buf.size + 8, dtype=torch.uint8, device="cuda")
    dev[shift:shift + buf.size] = torch.from_numpy(buf.reshape(-1)).cuda()
    base = dev.data_ptr() + shift
    meta = paged.new_meta_table(8, 2)
    items = torch.from_numpy(kvz.gaac_items(
        [base + i * 16 * stride for i in range(n)], [meta.data_ptr() + 8 * i for i in range(n)],
        stride, kinds, [bases.data_ptr() + (heads[i] * 2 + kinds[i]) * 256 for i in range(n)])).cuda()
    arena = paged.SlotArena(256 * 1024, fp8=True)
    kvz.kvz_fp8_encode_pages(arena.pool, items, n, fmt)
    torch.cuda.synchronize()
    bh = bases.cpu().numpy()
    oc = Fp8OracleCache(arena.arena.numel(), fmt)
    metas = oc.encode(flat, kinds, [(bh[heads[i], kinds[i], 0], bh[heads[i], kinds[i], 1])
                                    for i in range(n)])
    m = meta.cpu().numpy().reshape(-1, 8)
    for i in range(n):
        off = int.from_bytes(m[i, :4].tobytes(), "little")
        assert (off, [int(x) for x in m[i, 4:]]) == (metas[i][0], list(metas[i][1])), i
    np.testing.assert_array_equal(arena.arena.cpu().numpy(), oc.arena)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("force_raw,stress", [(False, False), (True, False), (False, True)])
def test_encode_matches_oracle_arena_and_meta(fmt, force_raw, stress):
    """2 sequences x 9 pages x 4 KV heads, bases from another sample of the layer: the whole
    arena, every metadata record and the pool counters equal the oracle's."""
    announce(f"fp8 {NAME[fmt]} encode force_raw={force_raw} stress={stress}")
    cal = synth.fp8_kv_pages(2, 6, 4, seed=82, fmt=fmt, forced_frac=0.0, sample=1, device="cuda")
    bases = paged.fp8_calibrate(cal, fmt)
    pages = synth.fp8_kv_pages(2, 9, 4, seed=82, fmt=fmt, forced_frac=0.2, stress=stress,
                               device="cuda")
    lay = Fp8Layer(pages, [16 * 9] * 2, [9, 9], fmt, bases, seed=82,
                   flags=kvz.KVZ_ENC_FORCE_RAW if force_raw else 0)
    torch.cuda.synchronize()
    nat = pages.cpu().numpy()
    bh = bases.cpu().numpy()
    tiles, kinds, bl = [], [], []
    for b in range(2):
        for p in range(9):
            for h in range(4):
                for kind in range(2):
                    tiles.append(nat[b, p, kind, h])
                    kinds.append(kind)
                    bl.append((bh[h, kind, 0], bh[h, kind, 1]))
    oc = Fp8OracleCache(lay.arena.arena.numel(), fmt)
    metas = oc.encode(np.stack(tiles), kinds, bl, force_raw=force_raw)
    m = lay.meta.cpu().numpy()
    k = 0
    for b in range(2):
        for p in range(9):
            for h in range(4):
                for kind in range(2):
                    rec = m[lay.phys_of[b, p], h, kind]
                    off = int.from_bytes(rec[:4].tobytes(), "little")
                    assert (off, [int(x) for x in rec[4:]]) == (metas[k][0], list(metas[k][1])), k
                    k += 1
    np.testing.assert_array_equal(lay.arena.arena.cpu().numpy(), oc.arena)
    st = lay.arena.stats()
    assert st["frontier_granules"] == oc.pool.frontier
    assert st["live_runs"] == oc.pool.live_runs
    n_raw = sum(1 for _, t in metas if list(t) == fp8.TAGS_RAW)
    announce(f"fp8 {NAME[fmt]} encode: {n_raw} of {len(metas)} tiles uncompressed")
    if force_raw:
        assert n_raw == len(metas)
    elif not stress:
        assert n_raw < len(metas) // 4


@pytest.mark.parametrize("fmt", FORMATS)
def test_decompress_and_pack_match_oracle_layout(fmt):
    """Every tile (compressed, uncompressed, one not stored) rebuilt into the FP8 chunk layout
    equals the oracle's layout of the input page; kvz_fp8_pack_pages writes the same bytes."""
    announce(f"fp8 {NAME[fmt]} decompress")
    cal = synth.fp8_kv_pages(1, 8, 2, seed=84, fmt=fmt, sample=1, device="cuda")
    bases = paged.fp8_calibrate(cal, fmt)
    pages = synth.fp8_kv_pages(3, 7, 2, seed=84, fmt=fmt, forced_frac=0.3, stress=True,
                               device="cuda")
    lay = Fp8Layer(pages, [16 * 7] * 3, [7, 7, 7], fmt, bases, seed=84)
    m = lay.meta.clone()
    m[5, 1, 0, :4] = 0xFF                                   # one tile not stored
    out = paged.fp8_decompress_pages(lay.arena, m, bases, fmt).cpu().numpy()
    nat = pages.cpu().numpy()
    by_phys = np.zeros((lay.n_phys, 2, 2, 16, 128), dtype=np.uint8)
    for b in range(3):
        for p in range(7):
            by_phys[lay.phys_of[b, p]] = nat[b, p]
    for ph in range(lay.n_phys):
        for kind in range(2):
            for h in range(2):
                want = (np.zeros(2048, np.uint8) if (ph, h, kind) == (5, 1, 0)
                        else fp8.raw_tile(by_phys[ph, kind, h], kind))
                np.testing.assert_array_equal(out[ph, kind, h], want, err_msg=f"{ph} {kind} {h}")
    packed = paged.pack_fp8_pages(torch.from_numpy(by_phys).cuda()).cpu().numpy()
    for ph in range(lay.n_phys):
        for kind in range(2):
            for h in range(2):
                np.testing.assert_array_equal(packed[ph, kind, h], fp8.raw_tile(by_phys[ph, kind, h], kind))


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("hq,hkv", [(8, 2), (32, 8), (16, 2)])
def test_attention_matches_oracle(fmt, hq, hkv):
    """Ragged batch (tails of 0..16 tokens, an empty sequence, a single-page one), fused and
    uncompressed FP8 kernels, dequantization scales != 1."""
    announce(f"fp8 {NAME[fmt]} attention hq={hq} hkv={hkv}")
    cal = synth.fp8_kv_pages(1, 8, hkv, seed=86, fmt=fmt, sample=1, device="cuda")
    bases = paged.fp8_calibrate(cal, fmt)
    pages = synth.fp8_kv_pages(5, 12, hkv, seed=86, fmt=fmt, forced_exp=-12.0, device="cuda")
    n_comp = [11, 5, 0, 1, 7]
    seq_lens = [11 * 16 + 9, 5 * 16, 0, 16 + 16, 7 * 16 + 1]
    lay = Fp8Layer(pages, seq_lens, n_comp, fmt, bases, seed=86)
    q = synth.queries(5, hq, seed=87, device="cuda")
    ks, vs = 0.75, 1.5
    ref = lay.oracle_rows(q, ks, vs, range(5))
    for name, got in (("fused", lay.fused(q, ks, vs)), ("raw", lay.raw(q, ks, vs)),
                      ("fused S=3", lay.fused(q, ks, vs, splits=3))):
        g = got.cpu().numpy()
        for b in range(5):
            if seq_lens[b] == 0:
                assert not g[b].any(), name
                continue
            w = check_rows(g[b], ref[b], what=f"{name} b={b}")
            announce(f"  {name} b={b} worst row error {w:.2e}")


@pytest.mark.parametrize("fmt", FORMATS)
def test_fused_equals_uncompressed_bitwise(fmt):
    """Lossless: the fused kernel over compressed tiles, over the same pages stored uncompressed
    (KVZ_ENC_FORCE_RAW) and the uncompressed FP8 kernel give bit-identical outputs."""
    announce(f"fp8 {NAME[fmt]} storage-mode invariance")
    cal = synth.fp8_kv_pages(1, 8, 8, seed=88, fmt=fmt, sample=1, device="cuda")
    bases = paged.fp8_calibrate(cal, fmt)
    pages = synth.fp8_kv_pages(4, 20, 8, seed=88, fmt=fmt, device="cuda")
    seq_lens, n_comp = [19 * 16 + 5, 10 * 16, 16 * 16 + 16, 3], [19, 10, 16, 0]
    q = synth.queries(4, 32, seed=89, device="cuda")
    a = Fp8Layer(pages, seq_lens, n_comp, fmt, bases, seed=88)
    b = Fp8Layer(pages, seq_lens, n_comp, fmt, bases, seed=88, flags=kvz.KVZ_ENC_FORCE_RAW)
    o1, o2, o3 = a.fused(q, 0.5, 2.0), b.fused(q, 0.5, 2.0), a.raw(q, 0.5, 2.0)
    assert torch.equal(o1, o2) and torch.equal(o1, o3)


@pytest.mark.parametrize("fmt", FORMATS)
def test_non_finite_values_propagate_like_the_oracle(fmt):
    announce(f"fp8 {NAME[fmt]} non-finite propagation")
    cal = synth.fp8_kv_pages(1, 6, 2, seed=90, fmt=fmt, sample=1, device="cuda")
    bases = paged.fp8_calibrate(cal, fmt)
    pages = synth.fp8_kv_pages(3, 6, 2, seed=90, fmt=fmt, device="cuda")
    p = pages.cpu().numpy()
    nan = 0x7F if fmt == kvz.KVZ_FP8_E4M3 else 0x7E
    p[1, 2, 1, 0, 7, 33] = nan          # a NaN in V of sequence 1, KV head 0
    p[2, 4, 0, 1, 3, 100] = nan         # a NaN in K of sequence 2, KV head 1
    pages = torch.from_numpy(p).cuda()
    lay = Fp8Layer(pages, [5 * 16 + 3] * 3, [5] * 3, fmt, bases, seed=90)
    q = synth.queries(3, 8, seed=91, device="cuda")
    ref = lay.oracle_rows(q, 1.0, 1.0, range(3))
    for got in (lay.fused(q, 1.0, 1.0), lay.raw(q, 1.0, 1.0)):
        g = got.cpu().numpy()
        for b in range(3):
            check_rows(g[b], ref[b], what=f"b={b}")
        assert not np.isfinite(g[1, 0:4]).all() and np.isfinite(g[1, 4:8]).all()


@pytest.mark.parametrize("fmt", FORMATS)
def test_full_size_qwen8k_layer_sampled(fmt):
    """The 8K-context Qwen3-8B-shaped layer (16 sequences x 511 compressed pages + a 16-token
    tail, 32/8 heads) at the automatic split count, two sequences checked against the oracle, and
    the storage ratio reported."""
    announce(f"fp8 {NAME[fmt]} full-size 8K layer")
    cal = synth.fp8_kv_pages(1, 64, 8, seed=92, fmt=fmt, sample=1, device="cuda")
    bases = paged.fp8_calibrate(cal, fmt)
    pages = synth.fp8_kv_pages(16, 512, 8, seed=92, fmt=fmt, device="cuda")
    lay = Fp8Layer(pages, [8192] * 16, [511] * 16, fmt, bases, seed=92)
    st = lay.arena.stats()
    ratio = (16 * 511 * 8 * 2 * 2048) / (st["live_granules"] * 128)
    announce(f"fp8 {NAME[fmt]} storage ratio vs FP8: {ratio:.4f}")
    assert ratio > (1.05 if fmt == kvz.KVZ_FP8_E4M3 else 1.2)
    q = synth.queries(16, 32, seed=93, device="cuda")
    ref = lay.oracle_rows(q, 0.5, 2.0, [0, 13])
    got = lay.fused(q, 0.5, 2.0).cpu().numpy()
    for b in (0, 13):
        check_rows(got[b], ref[b], what=f"b={b}")


def test_churn_reuses_freed_runs_like_the_pool_model():
    """Encode FP8 tiles of both formats into one FP8 pool, free a random subset, encode more:
    the freed 13-, 15- and 16-granule runs are reused from their bins exactly as the oracle's
    pool model says, the records are byte-identical to the oracle's, and every stored tile
    decodes back to its input (decompress-first into the FP8 chunk layout)."""
    announce("fp8 pool churn")
    rng = np.random.default_rng(94)
    arena = paged.SlotArena(600 * 128 * 16, fp8=True)
    model = SlotPoolModel(arena.stats()["capacity_granules"])   # one pool for both formats
    live = []                            # (fmt, meta row on device, page, kind, bases)
    for rnd in range(3):
        for fmt in FORMATS:
            pages = synth.fp8_kv_pages(1, 6, 2, seed=95 + 10 * rnd + fmt, fmt=fmt,
                                       forced_frac=0.6 if rnd == 1 else 0.05, device="cuda")
            if rnd == 2:                 # a few tiles too wide for the escape slot
                p = pages.cpu().numpy()
                p[0, 0, :, :] = rng.integers(0, 0x70, p[0, 0].shape)
                pages = torch.from_numpy(p).cuda()
            bases = paged.fp8_calibrate(pages, fmt)
            meta = paged.new_meta_table(6, 2)
            items = paged.fp8_page_items(pages, [(0, p) for p in range(6)], meta, list(range(6)), bases)
            d = paged.fp8_encode(arena, items, fmt)
            torch.cuda.synchronize()
            nat, bh = pages.cpu().numpy(), bases.cpu().numpy()
            tiles = [(p, h, kind) for p in range(6) for h in range(2) for kind in range(2)]
            enc = [fp8.encode_tile(nat[0, p, kind, h], kind, fmt, bh[h, kind, 0], bh[h, kind, 1])
                   for p, h, kind in tiles]
            offs = model.alloc([fp8.tags_of(raw, fmt) for raw, _ in enc])
            m = meta.cpu().numpy()
            arena_h = arena.arena.cpu().numpy()
            for (p, h, kind), (raw, rec), off in zip(tiles, enc, offs):
                got_off = int.from_bytes(m[p, h, kind, :4].tobytes(), "little")
                assert got_off == off and list(m[p, h, kind, 4:]) == fp8.tags_of(raw, fmt)
                np.testing.assert_array_equal(arena_h[off * 128: off * 128 + rec.size], rec)
                live.append((fmt, meta, (p, h, kind), nat[0, p, kind, h], bases, off,
                             fp8.tags_of(raw, fmt)))
            del d
            st = arena.stats()
            assert st["frontier_granules"] == model.frontier
            assert st["free_runs"] == [len(model.bins[k]) for k in range(5)]
            assert st["live_runs"] == model.live_runs and st["live_granules"] == model.live_granules
        # free a random half of what is live
        order = rng.permutation(len(live))
        victims = [live[i] for i in order[: len(live) // 2]]
        live = [live[i] for i in order[len(live) // 2:]]
        ptrs = torch.from_numpy(np.asarray(
            [v[1].data_ptr() + ((v[2][0] * 2 + v[2][1]) * 2 + v[2][2]) * 8 for v in victims],
            dtype=np.int64)).cuda()
        kvz.kvz_slot_free(arena.pool, ptrs)
        model.free([(v[5], v[6]) for v in victims])
        torch.cuda.synchronize()
    assert any(len(model.bins[k]) for k in (1, 3, 4))
    # every live tile still decodes to its input
    for fmt, meta, (p, h, kind), page, bases, off, tags in live:
        out = paged.fp8_decompress_pages(arena, meta, bases, fmt).cpu().numpy()
        np.testing.assert_array_equal(out[p, kind, h], fp8.raw_tile(page, kind))


@pytest.mark.parametrize("fmt", FORMATS)
def test_graph_replays_match_eager(fmt):
    """Fused and uncompressed FP8 attention captured in HIP graphs: every replay, with eager work
    and synchronization in between, equals the eager call."""
    announce(f"fp8 {NAME[fmt]} graph replay")
    cal = synth.fp8_kv_pages(1, 8, 8, seed=96, fmt=fmt, sample=1, device="cuda")
    bases = paged.fp8_calibrate(cal, fmt)
    pages = synth.fp8_kv_pages(4, 33, 8, seed=96, fmt=fmt, device="cuda")
    lay = Fp8Layer(pages, [16 * 32 + 9, 16 * 20, 16 * 32 + 16, 7], [32, 20, 32, 0], fmt, bases,
                   seed=96)
    q = synth.queries(4, 32, seed=97, device="cuda")
    for fused in (True, False):
        eager = (lay.fused if fused else lay.raw)(q, 0.5, 2.0).clone()
        out = torch.zeros_like(eager)
        ws = paged.workspace(4, 32, 8, lay.block_table.shape[1])
        store = None
        if not fused:
            nat = torch.zeros((lay.n_phys, 2, 8, 16, 128), dtype=torch.uint8, device="cuda")
            for b in range(4):
                nc = int(lay.n_comp[b])
                if nc:
                    nat[torch.as_tensor(lay.phys_of[b, :nc], device="cuda", dtype=torch.long)] = pages[b, :nc]
            store = paged.pack_fp8_pages(nat)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            if fused:
                kvz.kvz_fp8_decode_attention(q, out, fmt, lay.arena.arena, lay.meta, bases,
                                             lay.block_table, lay.seq_lens, lay.n_comp, lay.tail,
                                             sm_scale(), 0.5, 2.0, ws)
            else:
                kvz.kvz_fp8_raw_decode_attention(q, out, fmt, store, lay.block_table, lay.seq_lens,
                                                 lay.n_comp, lay.tail, sm_scale(), 0.5, 2.0, ws, 8)
        for rep in range(4):
            out.fill_(float("nan"))
            _ = (q.float() * 2).sum()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager), f"fused={fused} replay {rep}"
