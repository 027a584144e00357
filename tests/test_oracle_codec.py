"""Pins of the CPU codec oracle against what the pages fix (no GPU).

Each test checks oracle/codec.py against something other than itself: hand-worked bytes,
the ExANS field split, a brute-force window search, the page's register-restore description,
the MFMA operand layout, or exhaustive/closed-form properties.
"""
import json
import os

import numpy as np
import pytest

from oracle import codec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "codec_worked_examples.json")


def _hex(s):
    return np.array([int(x, 16) for x in s.split()], dtype=np.uint8)


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_worked_examples(case):
    """Hand-worked records (ZipFusion "How it works", steps 2-4)."""
    kind = codec.KIND_K if case["kind"] == "K" else codec.KIND_V
    page = np.full((16, 128), int(case["default"], 16), dtype=np.uint16)
    for t, d, w in case["set"]:
        page[t, d] = int(w, 16)
    tags, rec = codec.encode_group(page, kind)
    assert [int(t) for t in tags] == case["tags"]
    assert rec.size == case["group_bytes"]
    expect = []
    for blk in case["blocks"]:
        dflt = _hex(blk["default_chunk"])
        for c in range(64):
            expect.append(_hex(blk["chunks"][str(c)]) if str(c) in blk["chunks"] else dflt)
    np.testing.assert_array_equal(rec, np.concatenate(expect))
    arena = np.zeros(8192, dtype=np.uint8)
    arena[256:256 + rec.size] = rec
    np.testing.assert_array_equal(codec.decode_group(arena, 1, tags, kind), page)


def test_field_split_matches_exans_formulas():
    """ExANS "Encoding/Decoding Pipeline": E = (w>>7)&0xff, SF = ((w>>8)&0x80)|(w&0x7f),
    word = ((SF&0x80)<<8)|(E<<7)|(SF&0x7f).  The kept low byte is the fraction plus the
    exponent's LSB (ZipFusion step 3)."""
    w = np.arange(65536, dtype=np.uint32)
    s, e, lo = codec.fields(w.astype(np.uint16))
    E = (w >> 7) & 0xFF
    SF = ((w >> 8) & 0x80) | (w & 0x7F)
    np.testing.assert_array_equal(e, E)
    np.testing.assert_array_equal((s << 7) | (lo & 0x7F), SF)
    np.testing.assert_array_equal(lo >> 7, E & 1)
    np.testing.assert_array_equal(((SF & 0x80) << 8) | (E << 7) | (SF & 0x7F), w)


def test_bf16_value_formula():
    """BF16 normal value = (-1)^s * 2^(e-127) * (1 + f/128) (ExANS "Under the hood")."""
    rng = np.random.default_rng(1)
    w = rng.integers(0, 65536, 4096).astype(np.uint16)
    s, e, lo = codec.fields(w)
    normal = (e > 0) & (e < 255)
    f = (w.astype(np.int64) & 0x7F)
    val = np.where(s == 1, -1.0, 1.0) * np.exp2(e.astype(np.float64) - 127) * (1 + f / 128.0)
    np.testing.assert_array_equal(codec.bf16_bits_to_f64(w)[normal], val[normal])


def _brute_eligible(e):
    """Some even b' in [0, 254] with every exponent inside [b', b'+15]."""
    return any(all(b <= x <= b + 15 for x in e) for b in range(0, 256, 2))


def test_eligibility_equals_brute_force_window_search():
    rng = np.random.default_rng(2)
    for trial in range(3000):
        lo_e = int(rng.integers(0, 256))
        span = int(rng.integers(0, 20))
        e = rng.integers(lo_e, min(lo_e + span, 255) + 1, size=int(rng.integers(1, 40)))
        b, ok = codec.base_and_eligible(e)
        assert bool(ok) == _brute_eligible(e.tolist()), e
        assert b % 2 == 0 and b <= e.min() and e.min() - b <= 1
        if ok:
            d = (e - b) // 2
            assert d.min() >= 0 and d.max() <= 7


def test_window_edges():
    assert bool(codec.base_and_eligible(np.arange(126, 142))[1])       # 126..141
    assert not bool(codec.base_and_eligible(np.arange(127, 143))[1])   # odd min -> b = 126
    assert not bool(codec.base_and_eligible(np.array([0, 127]))[1])
    assert bool(codec.base_and_eligible(np.array([254, 255]))[1])
    assert codec.base_and_eligible(np.array([255]))[0] == 254


def test_all_bf16_patterns_round_trip_compressed_and_raw():
    """Every one of the 65,536 BF16 patterns survives the compressed path (blocks holding all
    patterns with e in {2k, 2k+1}, which always fit a window) and the raw path (shuffled)."""
    w = np.arange(65536, dtype=np.uint32)
    e = (w >> 7) & 0xFF
    blocks = [w[(e >> 1) == k].astype(np.uint16) for k in range(128)]
    assert all(bl.size == 512 for bl in blocks)
    tags, recs = codec.encode_blocks(np.stack(blocks))
    assert all(r.size == 768 for r in recs)
    assert list(tags) == list(range(128))
    for k in range(128):
        np.testing.assert_array_equal(codec.decode_block(int(tags[k]), recs[k]), blocks[k])
    perm = np.random.default_rng(3).permutation(65536).astype(np.uint16)
    tags, recs = codec.encode_blocks(perm.reshape(128, 512))
    for k in range(128):
        assert recs[k].size == (1024 if tags[k] == 0xFF else 768)
        np.testing.assert_array_equal(codec.decode_block(int(tags[k]), recs[k]),
                                      perm.reshape(128, 512)[k])


def test_force_raw_keeps_words_in_storage_order():
    rng = np.random.default_rng(4)
    words = rng.integers(0x3C00, 0x4000, size=(3, 512)).astype(np.uint16)
    tags, recs = codec.encode_blocks(words, force_raw=True)
    assert list(tags) == [255, 255, 255]
    for k in range(3):
        assert recs[k].size == 1024
        np.testing.assert_array_equal(recs[k].view("<u2"), words[k])


def test_register_restore_described_on_the_page():
    """ZipFusion: code bytes pair (x0,x4)..(x3,x7); a mask on one branch and an unpack on the
    other each give four high bytes after one 32-bit add of b/2 replicated per byte, with no
    carry.  Checked on bytes written by the oracle for random eligible blocks."""
    rng = np.random.default_rng(5)
    for _ in range(200):
        b = int(rng.integers(0, 128)) * 2
        e = rng.integers(b, min(b + 15, 255) + 1, size=512)
        s = rng.integers(0, 2, size=512)
        f = rng.integers(0, 128, size=512)
        words = ((s << 15) | (e << 7) | f).astype(np.uint16)
        tags, recs = codec.encode_blocks(words[None])
        assert tags[0] == codec.base_and_eligible(e)[0] // 2
        ch = recs[0].reshape(64, 12)
        C = ch[:, 8:12].copy().view("<u4")[:, 0].astype(np.uint64)
        B = int(tags[0]) * 0x01010101
        mask_branch = ((C & 0x87878787) + B) & 0xFFFFFFFF
        unpack_branch = ((((C >> 4) | (C << 28)) & 0x87878787) + B) & 0xFFFFFFFF
        hi = (words.reshape(64, 8) >> 8).astype(np.uint64)
        for k in range(4):
            np.testing.assert_array_equal((mask_branch >> (8 * k)) & 0xFF, hi[:, k])
            np.testing.assert_array_equal((unpack_branch >> (8 * k)) & 0xFF, hi[:, k + 4])
        np.testing.assert_array_equal(ch[:, :8], (words.reshape(64, 8) & 0xFF).astype(np.uint8))


def test_blocks_partition_the_page():
    for kind in (codec.KIND_K, codec.KIND_V):
        seen = np.zeros((16, 128), dtype=np.int64)
        for j in range(4):
            t, d = codec.storage_coords(kind, j)
            assert set(d.tolist()) == set(range(32 * j, 32 * j + 32))
            np.add.at(seen, (t, d), 1)
        assert (seen == 1).all()


def test_storage_order_is_the_mfma_operand_order():
    """CDNA3/CDNA4 ISA operand layouts of the bf16 MFMAs with 8 values per lane:
    v_mfma_f32_16x16x32_bf16 row operand - lane l holds row l%16, k = 8*(l//16) + i;
    v_mfma_f32_32x32x16_bf16 column operand - lane l holds column l%32, k = 8*(l//32) + i.
    K feeds the first with rows = tokens and k = dims of the block; V feeds the second with
    columns = dims of the block and k = tokens."""
    for j in range(4):
        t, d = codec.storage_coords(codec.KIND_K, j)
        for l in range(64):
            for i in range(8):
                n = 8 * l + i
                assert t[n] == l % 16 and d[n] == 32 * j + 8 * (l // 16) + i
        t, d = codec.storage_coords(codec.KIND_V, j)
        for l in range(64):
            for i in range(8):
                n = 8 * l + i
                assert d[n] == 32 * j + l % 32 and t[n] == 8 * (l // 32) + i


def test_group_sizes_and_meta_layout():
    """768 / 1024 bytes per block, 8 bytes of metadata per group; later blocks are located
    by summing the sizes of the blocks before them (ZipFusion metadata paragraph)."""
    tags = [60, 255, 7, 255]
    assert codec.group_bytes(tags) == 768 + 1024 + 768 + 1024
    assert codec.group_granules(tags) == 14
    assert [codec.block_offset_bytes(5, tags, j) for j in range(4)] == [1280, 2048, 3072, 3840]
    m = codec.meta_bytes(0x01020304, tags)
    assert m == bytes([4, 3, 2, 1, 60, 255, 7, 255]) and len(m) == 8
    assert codec.parse_meta(np.frombuffer(m, dtype=np.uint8)) == (0x01020304, tags)


def test_random_pages_round_trip_and_sizes():
    rng = np.random.default_rng(6)
    for trial in range(50):
        kind = trial % 2
        scale = rng.uniform(-5, 5, size=128)
        x = rng.standard_normal((16, 128)) * np.exp2(scale)
        page = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        tags, rec = codec.encode_group(page, kind)
        assert rec.size == 3072 + 256 * sum(1 for t in tags if t == 255)
        arena = np.zeros(rec.size + 512, dtype=np.uint8)
        arena[512:] = rec
        np.testing.assert_array_equal(codec.decode_group(arena, 2, tags, kind), page)
