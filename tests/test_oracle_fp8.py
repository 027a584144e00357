"""Pins of the FP8 exponent-code oracle (oracle/fp8.py) to facts outside itself.

"GAAC: Lossless KV Compression for Bandwidth-Efficient LLM Inference on Personal Devices",
appendix "Relation to FP8 KV" (Table 7), with the code of section "Lossless KV Compression" and
the slots of section "Block-Wise Compression Scheduling"; FP8 values as defined by the OCP 8-bit
formats (checked against torch's float8 types)."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import attention, cache, codec, fp8

HERE = os.path.dirname(os.path.abspath(__file__))
KINDS = [fp8.E4M3, fp8.E5M2]
TORCH_DTYPE = {fp8.E4M3: torch.float8_e4m3fn, fp8.E5M2: torch.float8_e5m2}


def _byte(s, e, m, fk):
    return (s << 7) | (e << fp8.FRAC_BITS[fk]) | m


@pytest.mark.parametrize("fk", KINDS)
def test_values_match_torch_float8(fk):
    """All 256 byte patterns decode to exactly what torch's float8 type holds (NaN positions
    included): zeros, subnormals, the largest finite values, Inf (E5M2) and NaN."""
    x = np.arange(256, dtype=np.uint8)
    mine = fp8.to_f64(x, fk)
    ref = torch.from_numpy(x.copy()).view(TORCH_DTYPE[fk]).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    # a few values known by heart: 1.0, the largest finite value, the smallest subnormal
    one = 0x38 if fk == fp8.E4M3 else 0x3C
    top = 0x7E if fk == fp8.E4M3 else 0x7B
    assert fp8.to_f64(np.array([one, top, 0x01]), fk).tolist() == (
        [1.0, 448.0, 2.0 ** -9] if fk == fp8.E4M3 else [1.0, 57344.0, 2.0 ** -16])


def test_hand_worked_bytes():
    with open(os.path.join(HERE, "golden", "fp8_worked_example.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        fk = fp8.E4M3 if case["format"] == "e4m3" else fp8.E5M2
        page = np.full((16, 128), int(case["default"], 16), dtype=np.uint8)
        for t, d, w in case["set"]:
            page[t, d] = int(w, 16)
        b3 = np.full(128, case["b3"], dtype=np.uint8)
        b4 = np.full(128, case["b4"], dtype=np.uint8)
        raw, rec = fp8.encode_tile(page, codec.KIND_K, fk, b3, b4)
        assert not raw
        assert rec.size == case["record_bytes"]
        for at, byte in case["expect"]:
            assert rec[at] == int(byte, 16), f"{case['format']} byte {at}"
        np.testing.assert_array_equal(fp8.decode_tile(rec, False, codec.KIND_K, fk, b3, b4), page)


@pytest.mark.parametrize("fk,bits,ratio", [(fp8.E4M3, 7.25, 1.103), (fp8.E5M2, 6.25, 1.28)])
def test_all_3bit_tile_size(fk, bits, ratio):
    """Sign + fraction (4 or 3 bits) + 3-bit code + 0.25 bits of mode per value when every group
    is 3-bit; the slot (planes + 64 escape bytes) and the raw tile are 15 / 13 and 16 granules
    of 128 bytes, which the tags give the pool as 12 + (number of 0xFF tag bytes)."""
    one = 0x38 if fk == fp8.E4M3 else 0x3C
    page = np.full((16, 128), one, dtype=np.uint8)
    e1 = 7 if fk == fp8.E4M3 else 15
    b3 = np.full(128, e1 - 3, np.uint8)
    b4 = np.full(128, 0, np.uint8)
    raw, rec = fp8.encode_tile(page, codec.KIND_V, fk, b3, b4)
    assert not raw
    assert rec.size * 8 / 2048 == bits
    assert round(2048 / rec.size, 3) == ratio
    slot = fp8.slot_bytes(fk)
    assert slot == rec.size + 64
    assert slot == fp8.run_granules(False, fk) * 128
    assert fp8.RAW_TILE_BYTES == fp8.run_granules(True, fk) * 128 == 2048
    assert fp8.run_granules(False, fk) == (15 if fk == fp8.E4M3 else 13)


def test_mode_boundaries():
    """E5M2, b3 = 12, b4 = 8: exponents 12..19 are 3-bit, 8..23 4-bit, others raw."""
    b3, b4 = np.full(8, 12), np.full(8, 8)
    e = np.full(8, 15)
    assert fp8.group_mode(e, b3, b4) == fp8.MODE_3BIT
    for v, mode in [(19, fp8.MODE_3BIT), (20, fp8.MODE_4BIT), (12, fp8.MODE_3BIT),
                    (11, fp8.MODE_4BIT), (8, fp8.MODE_4BIT), (23, fp8.MODE_4BIT),
                    (24, fp8.MODE_RAW), (7, fp8.MODE_RAW), (0, fp8.MODE_RAW), (31, fp8.MODE_RAW)]:
        e2 = e.copy()
        e2[6] = v
        assert fp8.group_mode(e2, b3, b4) == mode, v
    assert list(fp8.group_codes(np.array([31] * 8), fp8.MODE_RAW, b3, b4)) == [31] * 8


def test_calibration_hand_worked():
    """E5M2 exponents {3 x3, 4, 13 x4, 14 x4, 15 x4} of one dim: the best 8-wide window holds 12
    (13..15), smallest base 8; the 16-wide window [0, 15] holds all 16.  Windows stay inside
    the exponent field; in E4M3 the only 16-wide window is [0, 15]."""
    e = [3] * 3 + [4] + [13] * 4 + [14] * 4 + [15] * 4
    assert fp8.best_window(e, 8, fp8.E5M2) == 8
    assert fp8.best_window(e, 16, fp8.E5M2) == 0
    assert fp8.best_window([31] * 5, 8, fp8.E5M2) == 24
    assert fp8.best_window([31] * 5, 16, fp8.E5M2) == 16
    assert fp8.best_window([15] * 5, 8, fp8.E4M3) == 8
    assert fp8.best_window([15, 0], 16, fp8.E4M3) == 0


def test_e4m3_calibrates_b4_zero_and_never_needs_raw():
    rng = np.random.default_rng(3)
    page = rng.integers(0, 256, size=(4, 16, 128)).astype(np.uint8)
    b3, b4 = fp8.calibrate(page, fp8.E4M3)
    assert not b4.any()
    _, e, _ = fp8.fields(page[0], fp8.E4M3)
    for d in range(0, 128, 9):
        assert fp8.group_mode(e[:8, d], b3[d], b4[d]) != fp8.MODE_RAW


def _tile_with_modes(fk, n4, nraw, kind=codec.KIND_K):
    """n4 groups in 4-bit mode and nraw raw (E5M2 only), one out-of-window value in the first
    groups of lanes 0, 1, 2, ... (b3 = 12, b4 = 8 for E5M2; b3 = 4, b4 = 0 for E4M3)."""
    if fk == fp8.E5M2:
        one, wide, far = _byte(0, 15, 0, fk), _byte(0, 20, 1, fk), _byte(1, 2, 3, fk)
        b3, b4 = 12, 8
    else:
        one, wide, far = _byte(0, 7, 0, fk), _byte(0, 12, 5, fk), None
        b3, b4 = 4, 0
    page = np.full((16, 128), one, dtype=np.uint8)
    g = 0
    for val, count in ((wide, n4), (far, nraw)):
        for _ in range(count):
            j, c = g % 4, g // 4
            token, dim = codec.storage_coords(kind, j)
            page[token[8 * c], dim[8 * c]] = val
            g += 1
    return page, np.full(128, b3, np.uint8), np.full(128, b4, np.uint8)


@pytest.mark.parametrize("fk,n4,nraw,compressed", [
    (fp8.E5M2, 0, 0, True), (fp8.E5M2, 64, 0, True), (fp8.E5M2, 65, 0, False),
    (fp8.E5M2, 2, 31, True), (fp8.E5M2, 3, 31, False), (fp8.E5M2, 0, 32, True),
    (fp8.E5M2, 0, 33, False), (fp8.E4M3, 64, 0, True), (fp8.E4M3, 65, 0, False),
    (fp8.E4M3, 256, 0, False)])
def test_escape_slot_capacity(fk, n4, nraw, compressed):
    """Escape bytes = (4-bit groups) + (EW - 3) x (raw groups); a tile is compressed iff they
    fit the 64-byte slot; otherwise it is stored uncompressed in the FP8 chunk layout."""
    page, b3, b4 = _tile_with_modes(fk, n4, nraw)
    raw, rec = fp8.encode_tile(page, codec.KIND_K, fk, b3, b4)
    assert raw == (not compressed)
    if compressed:
        assert rec.size == fp8.esc_off(fk) + n4 + fp8.raw_escape_bytes(fk) * nraw
    else:
        assert rec.size == 2048
        np.testing.assert_array_equal(rec, fp8.raw_tile(page, codec.KIND_K))
    np.testing.assert_array_equal(fp8.decode_tile(rec, raw, codec.KIND_K, fk, b3, b4), page)


def test_raw_tile_layout_partitions_the_tile():
    seen = np.zeros(2048, dtype=np.int64)
    for j in range(4):
        for c in range(64):
            seen[fp8.chunk_offset(j, c):fp8.chunk_offset(j, c) + 8] += 1
    assert np.all(seen == 1)
    # lane c: blocks 0 and 1 in the 16 bytes at 16c, blocks 2 and 3 at 1024 + 16c
    assert fp8.chunk_offset(1, 5) == 88 and fp8.chunk_offset(3, 5) == 1024 + 88


@pytest.mark.parametrize("fk", KINDS)
@pytest.mark.parametrize("kind", [codec.KIND_K, codec.KIND_V])
def test_round_trip_all_fp8_patterns(fk, kind):
    """Every byte pattern (signed zeros, subnormals, NaN, Inf), eight times per tile in a random
    order, with calibrated and with random bases."""
    rng = np.random.default_rng(11 + 2 * fk + kind)
    for _ in range(3):
        page = rng.permutation(np.tile(np.arange(256, dtype=np.uint8), 8)).reshape(16, 128)
        for b3, b4 in (fp8.calibrate(page[None], fk),
                       (rng.integers(0, (1 << fp8.EXP_BITS[fk]) - 7, 128).astype(np.uint8),
                        rng.integers(0, (1 << fp8.EXP_BITS[fk]) - 15, 128).astype(np.uint8))):
            raw, rec = fp8.encode_tile(page, kind, fk, b3, b4)
            np.testing.assert_array_equal(fp8.decode_tile(rec, raw, kind, fk, b3, b4), page)
            raw2, rec2 = fp8.encode_tile(page, kind, fk, b3, b4, force_raw=True)
            assert raw2
            np.testing.assert_array_equal(fp8.decode_tile(rec2, True, kind, fk, b3, b4), page)


@pytest.mark.parametrize("fk", KINDS)
@pytest.mark.parametrize("kind", [codec.KIND_K, codec.KIND_V])
def test_round_trip_narrow_random_tiles(fk, kind):
    """Per-dim exponent spread like scaled KV: every tile compresses and comes back."""
    rng = np.random.default_rng(21 + 2 * fk + kind)
    emax = (1 << fp8.EXP_BITS[fk]) - 1
    for _ in range(4):
        centre = rng.integers(4, emax - 4, size=128)
        e = np.clip(centre[None, :] + rng.integers(-3, 3, size=(16, 128)), 1, emax - 1)
        page = ((rng.integers(0, 2, (16, 128)) << 7) | (e << fp8.FRAC_BITS[fk])
                | rng.integers(0, 1 << fp8.FRAC_BITS[fk], (16, 128))).astype(np.uint8)
        b3, b4 = fp8.calibrate(page[None], fk)
        raw, rec = fp8.encode_tile(page, kind, fk, b3, b4)
        assert not raw
        np.testing.assert_array_equal(fp8.decode_tile(rec, raw, kind, fk, b3, b4), page)


def _rotr32(x, k):
    return ((x >> k) | (x << (32 - k))) & 0xFFFFFFFF


@pytest.mark.parametrize("fk", KINDS)
def test_register_restore_of_the_sign_fraction_plane(fk):
    """The bytes written here give each group's sign+fraction bytes (s << 7 | m) with a mask
    and a rotate per word - the 'mask on one branch, unpack on the other' restore - and an FP8
    byte is then that byte plus (exponent << fraction bits), with no carry between bytes."""
    rng = np.random.default_rng(5 + fk)
    emax = (1 << fp8.EXP_BITS[fk]) - 1
    centre = rng.integers(4, emax - 4, size=128)
    e = np.clip(centre[None, :] + rng.integers(-3, 3, size=(16, 128)), 0, emax)
    page = ((rng.integers(0, 2, (16, 128)) << 7) | (e << fp8.FRAC_BITS[fk])
            | rng.integers(0, 1 << fp8.FRAC_BITS[fk], (16, 128))).astype(np.uint8)
    b3, b4 = fp8.calibrate(page[None], fk)
    raw, rec = fp8.encode_tile(page, codec.KIND_K, fk, b3, b4)
    assert not raw
    vals, _ = fp8.tile_groups(page, codec.KIND_K)
    lane_bytes = fp8.SM_LANE_BYTES[fk]
    mw = fp8.FRAC_BITS[fk]
    for c in range(64):
        w = [int.from_bytes(bytes(rec[lane_bytes * c + 4 * t:lane_bytes * c + 4 * t + 4]), "little")
             for t in range(lane_bytes // 4)]
        xy = []
        if fk == fp8.E4M3:
            for j in range(4):
                xy.append((w[j] & 0x87878787, _rotr32(w[j], 4) & 0x87878787))
        else:
            for t in range(3):
                xy.append((w[t] & 0x83838383, _rotr32(w[t], 3) & 0x83838383))
            xy.append((((w[0] >> 5) & 0x03030303) | ((w[2] << 2) & 0x80808080),
                       ((w[1] >> 5) & 0x03030303) | ((w[2] << 1) & 0x80808080)))
        for j in range(4):
            ex = [(int(vals[j, c, i]) >> mw) & emax for i in range(8)]
            for half in range(2):
                e_word = sum(ex[4 * half + k] << (8 * k + mw) for k in range(4))
                got = xy[j][half] + e_word
                want = sum(int(vals[j, c, 4 * half + k]) << (8 * k) for k in range(4))
                assert got == want, (c, j, half)


def test_planted_mistake_in_decode_is_caught():
    """A decoder that forgets the base (a dropped term) fails the round trip."""
    page, b3, b4 = _tile_with_modes(fp8.E5M2, 3, 2)
    raw, rec = fp8.encode_tile(page, codec.KIND_K, fp8.E5M2, b3, b4)
    wrong = fp8.decode_tile(rec, raw, codec.KIND_K, fp8.E5M2, np.zeros(128, np.uint8), b4)
    assert not np.array_equal(wrong, page)


def test_attention_matches_pure_python_brute_force():
    """Tiny FP8 attention with K/V values from torch's float8 conversion, in plain loops."""
    rng = np.random.default_rng(9)
    for fk in KINDS:
        hq, hkv, t = 4, 2, 5
        q_bits = (torch.randn(hq, 128).to(torch.bfloat16).view(torch.int16).numpy()
                  .astype(np.uint16))
        k8 = rng.integers(0, 256, (t, hkv, 128)).astype(np.uint8)
        v8 = rng.integers(0, 256, (t, hkv, 128)).astype(np.uint8)
        e_ok = lambda x: fp8.fields(x, fk)[1] < (1 << fp8.EXP_BITS[fk]) - 1   # finite only
        k8 = np.where(e_ok(k8), k8, 0).astype(np.uint8)
        v8 = np.where(e_ok(v8), v8, 0).astype(np.uint8)
        kv = torch.from_numpy(k8.copy()).view(TORCH_DTYPE[fk]).double().numpy() * 0.5
        vv = torch.from_numpy(v8.copy()).view(TORCH_DTYPE[fk]).double().numpy() * 2.0
        qv = codec.bf16_bits_to_f64(q_bits)
        got = fp8.attention_fp64(q_bits, k8, v8, fk, 0.01, 0.5, 2.0)
        for h in range(hq):
            g = h // (hq // hkv)
            s = [0.01 * sum(qv[h, d] * kv[tt, g, d] for d in range(128)) for tt in range(t)]
            mx = max(s)
            p = [np.exp(x - mx) for x in s]
            for d in range(0, 128, 17):
                want = sum(p[tt] * vv[tt, g, d] for tt in range(t)) / sum(p)
                assert abs(got[h, d] - want) <= 1e-9 * (1 + abs(want))


def test_paged_fp8_cache_equals_dense_attention():
    """Attention through the arena, block table, metadata and an FP8 tail equals attention on the
    plain FP8 tiles, for compressed, raw and mixed tiles."""
    rng = np.random.default_rng(12)
    fk, hq, hkv, n_pages, n_tail = fp8.E5M2, 8, 2, 3, 5
    pages = np.zeros((n_pages, 2, hkv, 16, 128), dtype=np.uint8)
    for p in range(n_pages):
        centre = rng.integers(6, 20, size=128)
        for kv in range(2):
            for g in range(hkv):
                e = np.clip(centre[None, :] + rng.integers(-3, 3, (16, 128)), 1, 30)
                pages[p, kv, g] = ((rng.integers(0, 2, (16, 128)) << 7) | (e << 2)
                                   | rng.integers(0, 4, (16, 128))).astype(np.uint8)
    pages[1, 0, 1] = rng.integers(0, 0x7B, (16, 128))          # wide: stays raw
    tail = rng.integers(0, 0x70, (2, hkv, 16, 128)).astype(np.uint8)
    bases = [[fp8.calibrate(pages[:, kv, g], fk) for kv in range(2)] for g in range(hkv)]
    oc = cache.Fp8OracleCache(64 * 2048 + 128, fk)
    meta = [[[None, None] for _ in range(hkv)] for _ in range(n_pages)]
    for p in range(n_pages):
        for g in range(hkv):
            for kv in range(2):
                (m,) = oc.encode(pages[p, kv, g][None], [kv], [bases[g][kv]])
                meta[p][g][kv] = m
    assert any(m[1] == fp8.TAGS_RAW for row in meta for pair in row for m in pair)
    q_bits = (torch.randn(1, hq, 128).to(torch.bfloat16).view(torch.int16).numpy()
              .astype(np.uint16))
    bt = np.array([[2, 0, 1]])
    got = fp8.decode_attention(q_bits, oc.arena, meta, bases, bt, [16 * n_pages + n_tail],
                               [n_pages], tail[None], fk, 0.125, 0.75, 1.5)
    k = np.concatenate([np.transpose(pages[bt[0, p], 0], (1, 0, 2)) for p in range(n_pages)]
                       + [np.transpose(tail[0, :, :n_tail], (1, 0, 2))])
    v = np.concatenate([np.transpose(pages[bt[0, p], 1], (1, 0, 2)) for p in range(n_pages)]
                       + [np.transpose(tail[1, :, :n_tail], (1, 0, 2))])
    want = attention.attention_values_fp64(codec.bf16_bits_to_f64(q_bits[0]),
                                           fp8.to_f64(k, fk) * 0.75, fp8.to_f64(v, fk) * 1.5,
                                           0.125)
    np.testing.assert_allclose(got[0], want, rtol=0, atol=0)
