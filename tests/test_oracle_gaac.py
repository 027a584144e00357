"""Pins of the group-adaptive additive code oracle (oracle/gaac.py) to facts outside itself.

"GAAC: Lossless KV Compression for Bandwidth-Efficient LLM Inference on Personal Devices",
sections "Lossless KV Compression" and "Block-Wise Compression Scheduling", appendix "Storage"
(Table 9)."""
import json
import os

import numpy as np
import pytest

from oracle import codec, gaac

HERE = os.path.dirname(os.path.abspath(__file__))
ONE = 0x3F80


def _tile(default=ONE):
    return np.full((16, 128), default, dtype=np.uint16)


def _bases(b3=124, b4=120):
    return np.full(128, b3, dtype=np.uint8), np.full(128, b4, dtype=np.uint8)


def test_hand_worked_bytes():
    with open(os.path.join(HERE, "golden", "gaac_worked_example.json")) as f:
        case = json.load(f)
    page = _tile(int(case["default"], 16))
    for t, d, w in case["set"]:
        page[t, d] = int(w, 16)
    b3, b4 = _bases(case["b3"], case["b4"])
    raw, rec = gaac.encode_tile(page, codec.KIND_K, b3, b4)
    assert not raw
    assert rec.size == case["record_bytes"]
    for at, byte in case["expect"]:
        assert rec[at] == int(byte, 16), f"byte {at}"
    np.testing.assert_array_equal(gaac.decode_tile(rec, False, codec.KIND_K, b3, b4), page)


def test_all_3bit_tile_is_11_25_bits_per_element():
    """8 + 3 + 0.25 bits per element when every group uses the 3-bit mode; 16 / 11.25 = 1.422x."""
    b3, b4 = _bases()
    raw, rec = gaac.encode_tile(_tile(), codec.KIND_V, b3, b4)
    assert not raw and rec.size == 2880
    assert rec.size * 8 / 2048 == 11.25
    assert round(4096 / rec.size, 3) == 1.422
    assert gaac.SLOT_BYTES == 2048 + 768 + 64 + 128 == 3008


def test_mode_boundaries():
    """The narrowest window that holds all eight: e = b3+7 stays 3-bit, b3+8 needs the 16-wide
    window, below b3 but inside the b4 window is 4-bit, outside both is raw (b_8 = 0)."""
    b3, b4 = np.full(8, 124), np.full(8, 120)
    e = np.full(8, 127)
    assert gaac.group_mode(e, b3, b4) == gaac.MODE_3BIT
    for v, mode in [(131, gaac.MODE_3BIT), (132, gaac.MODE_4BIT), (124, gaac.MODE_3BIT),
                    (123, gaac.MODE_4BIT), (120, gaac.MODE_4BIT), (135, gaac.MODE_4BIT),
                    (136, gaac.MODE_RAW), (119, gaac.MODE_RAW), (0, gaac.MODE_RAW),
                    (255, gaac.MODE_RAW)]:
        e2 = e.copy()
        e2[3] = v
        assert gaac.group_mode(e2, b3, b4) == mode, v
    # per-element bases: each value is judged against its own dim's windows
    b3d = np.array([0, 10, 20, 30, 40, 50, 60, 70])
    b4d = b3d - 4
    assert gaac.group_mode(b3d + 7, b3d, b4d) == gaac.MODE_3BIT
    assert gaac.group_mode(b3d - 4, b3d, b4d) == gaac.MODE_4BIT
    assert list(gaac.group_codes(b3d - 4, gaac.MODE_4BIT, b3d, b4d)) == [0] * 8
    assert list(gaac.group_codes(b3d + 7, gaac.MODE_RAW, b3d, b4d)) == list(b3d + 7)


def _tile_with_modes(n4, nraw, kind=codec.KIND_K):
    """A tile with n4 groups in 4-bit mode and nraw in raw mode (bases 124 / 120), made by
    placing one out-of-window value in the first groups of lanes 0, 1, 2, ..."""
    page = _tile()
    b3, b4 = _bases()
    g = 0
    for mode, count in ((gaac.MODE_4BIT, n4), (gaac.MODE_RAW, nraw)):
        for _ in range(count):
            j, c = g % 4, g // 4
            token, dim = codec.storage_coords(kind, j)
            t, d = token[8 * c], dim[8 * c]
            page[t, d] = 0x4280 if mode == gaac.MODE_4BIT else 0x0000   # e = 133 / e = 0
            g += 1
    return page, b3, b4


@pytest.mark.parametrize("n4,nraw,compressed", [(0, 0, True), (128, 0, True), (129, 0, False),
                                                (3, 25, True), (4, 25, False), (0, 26, False),
                                                (256, 0, False)])
def test_escape_slot_capacity(n4, nraw, compressed):
    """Escape bytes = (4-bit groups) + 5 x (raw groups); a tile fits its slot iff they are at most
    128 (the slot of Table 9: 32 used on average + 96 unused); otherwise it stays BF16."""
    page, b3, b4 = _tile_with_modes(n4, nraw)
    raw, rec = gaac.encode_tile(page, codec.KIND_K, b3, b4)
    assert raw == (not compressed)
    if compressed:
        assert rec.size == 2880 + n4 + 5 * nraw
    else:
        assert rec.size == 4096
        # the raw tile is the other format's all-raw group record, byte for byte
        tags, want = codec.encode_group(page, codec.KIND_K, force_raw=True)
        np.testing.assert_array_equal(rec, want)
    np.testing.assert_array_equal(gaac.decode_tile(rec, raw, codec.KIND_K, b3, b4), page)


def test_calibration_hand_worked():
    """One dim with exponents {100 x3, 101, 110 x4, 111 x4, 112 x4}: the best 8-wide window holds
    12 (110..112); its smallest base is 105.  The 16-wide window [97, 112] holds all 16 and
    97 is the smallest such base ([96, 111] misses the 112s)."""
    e = [100] * 3 + [101] + [110] * 4 + [111] * 4 + [112] * 4
    assert gaac.best_window(e, 8) == 105
    assert gaac.best_window(e, 16) == 97
    assert gaac.best_window([255] * 5, 8) == 248          # windows stay inside [0, 255]
    assert gaac.best_window([0] * 5, 16) == 0
    assert gaac.best_window([7, 8, 9], 8) == 2            # 2..9 holds all three; 1..8 holds two


def test_calibrate_per_dim_and_kind_independent():
    """Bases are per dim: dim d of every calibration page carries exponent 100 + (d % 7)."""
    pages = np.zeros((3, 16, 128), dtype=np.uint16)
    for d in range(128):
        pages[:, :, d] = (100 + d % 7) << 7
    b3, b4 = gaac.calibrate(pages, codec.KIND_K)
    for d in range(128):
        e = 100 + d % 7
        assert b3[d] == e - 7 and b4[d] == e - 15      # smallest base whose window holds e


def _round_trip(page, kind, b3, b4):
    raw, rec = gaac.encode_tile(page, kind, b3, b4)
    back = gaac.decode_tile(rec, raw, kind, b3, b4)
    np.testing.assert_array_equal(back, page)
    return raw, rec


@pytest.mark.parametrize("kind", [codec.KIND_K, codec.KIND_V])
def test_round_trip_random_tiles_and_bases(kind):
    rng = np.random.default_rng(7 + kind)
    for _ in range(6):
        sigma = rng.integers(118, 134, size=128)
        e = np.clip(sigma[None, :] + rng.integers(-6, 4, size=(16, 128)), 1, 254)
        words = (rng.integers(0, 2, size=(16, 128)) << 15) | (e << 7) | rng.integers(0, 128, size=(16, 128))
        page = words.astype(np.uint16)
        b3, b4 = gaac.calibrate(page[None], kind)
        raw, _ = _round_trip(page, kind, b3, b4)
        b3r = rng.integers(0, 249, size=128).astype(np.uint8)
        b4r = rng.integers(0, 241, size=128).astype(np.uint8)
        _round_trip(page, kind, b3r, b4r)


def test_round_trip_all_bf16_patterns():
    """All 65,536 BF16 words (signed zeros, subnormals, Inf, NaN payloads) in 32 tiles."""
    words = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(32, 16, 128)
    for t in range(32):
        for kind in (codec.KIND_K, codec.KIND_V):
            b3, b4 = gaac.calibrate(words[t][None], kind)
            _round_trip(words[t], kind, b3, b4)


def test_planted_mistake_in_decode_is_caught():
    """A decoder that forgets the base (a dropped term) fails the hand-worked round trip."""
    page = _tile()
    b3, b4 = _bases()
    raw, rec = gaac.encode_tile(page, codec.KIND_K, b3, b4)
    wrong = gaac.decode_tile(rec, raw, codec.KIND_K, np.zeros(128, np.uint8), b4)
    assert not np.array_equal(wrong, page)
