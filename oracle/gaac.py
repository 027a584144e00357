"""CPU oracle for the group-adaptive additive exponent code (a second lossless page format).

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__ and the CPU-baseline
leg of bench.py may import this module.  The HIP library and its Python binding never do, and
this module imports nothing from them.

What it follows: "GAAC: Lossless KV Compression for Bandwidth-Efficient LLM Inference on Personal
Devices":
  * section "Lossless KV Compression", paragraph on contiguous exponent concentration - sign and
    7 fraction bits of a value stay unchanged in one byte; only the exponent is coded; for every
    head-channel pair, calibration picks the contiguous exponent windows of length 8 and 16 that
    cover the most values, separately for K and V of each layer (bases b3, b4);
  * same section, paragraph on group-adaptive additive coding - groups of eight elements in
    attention-access order share a 2-bit mode: 3-bit offsets, 4-bit offsets, or raw 8-bit
    exponents; d = e - b_w, the group takes the narrowest width that holds all eight, b_8 = 0,
    and reconstruction is e = code + b_w; the low three code bits of every mode go to one
    common packed stream, a 4-bit group adds one byte (its eight high bits), a raw group five
    bytes (the remaining five bits of each exponent); 8 + 3 + 0.25 = 11.25 bits per element in
    the all-3-bit case;
  * section "Block-Wise Compression Scheduling" - fixed-capacity slots; a block whose encoding
    does not fit its slot stays BF16; two storage classes;
  * appendix "Storage", Table 9 - per 16-token tile: 2048 bytes of sign+fraction, 768 of 3-bit
    codes, 64 of mode tags, and an escape slot whose capacity is 128 bytes (32 used on average,
    96 unused).

Readings taken where the pages leave a step open (each is also stated in include/kvz.h):
  * a tile is one page's K (or V) for one KV head: 16 tokens x 128 dims;
  * the groups of eight in attention-access order are the chunks of the other format
    (codec.storage_coords): group g = 64*j + c is chunk c of the 32-dim block j;
  * mode tag values 0 = 3-bit, 1 = 4-bit, 2 = raw;
  * calibration ties go to the smallest base; windows lie inside [0, 255];
  * record layout (compressed): sign+fraction plane (value i of group (j, c) at 512j + 8c + i),
    then the code plane (lane c's 12 bytes at 2048 + 12c: the 24 low-code bits of its group in
    block j at bytes 3j..3j+2, value i at bits 3i..3i+2), then the mode plane (byte c: block j's
    mode at bits 2j..2j+1), then the escape bytes (lanes in order, each lane's groups in block
    order; a 4-bit group's byte has bit i = code bit 3 of value i; a raw group's five bytes hold
    value i's exponent bits 3..7 at bits 5i..5i+4 of a 40-bit little-endian integer);
  * a compressed tile occupies a 3072-byte run (12 granules: 3008 bytes of slot, rounded up to
    the 256-byte granule), a raw tile 4096 bytes in the raw chunk layout of the other format;
    the 8-byte metadata is the other format's, with tags 00 00 00 00 (compressed) or
    FF FF FF FF (raw), so that the same slot pool serves both formats.

Pins (tests/test_oracle_gaac.py): hand-worked bytes in tests/golden/, the 11.25-bit and
1.422x figures of the pages, escape-slot boundaries (and the raw tile equal to the other
format's all-raw record), mode boundaries and calibration cases worked by hand, and round
trips over all 65,536 BF16 patterns and random tiles and bases.
"""
from __future__ import annotations

import numpy as np

from . import codec

TILE_TOKENS = 16
HEAD_DIM = 128
GROUPS = 256                      # 2048 values / 8
LANES = 64
SM_BYTES = 2048                   # sign + fraction, one byte per value
CODE_BYTES = 768                  # 3 bits per value
MODE_BYTES = 64                   # 2 bits per group
ESCAPE_SLOT = 128                 # escape capacity of a compressed tile (Table 9)
CODE_OFF = SM_BYTES
MODE_OFF = SM_BYTES + CODE_BYTES
ESC_OFF = SM_BYTES + CODE_BYTES + MODE_BYTES          # 2880
SLOT_BYTES = ESC_OFF + ESCAPE_SLOT                    # 3008
RAW_TILE_BYTES = 4096
COMPRESSED_RUN_GRANULES = 12                          # 3008 bytes rounded up to 256
RAW_RUN_GRANULES = 16
MODE_3BIT, MODE_4BIT, MODE_RAW = 0, 1, 2
ESCAPE_BYTES = {MODE_3BIT: 0, MODE_4BIT: 1, MODE_RAW: 5}
TAGS_COMPRESSED = [0x00, 0x00, 0x00, 0x00]
TAGS_RAW = [0xFF, 0xFF, 0xFF, 0xFF]


# --------------------------------------------------------------------------------------------
# Calibration ("Lossless KV Compression", contiguous exponent concentration)
# --------------------------------------------------------------------------------------------
def best_window(exponents, width: int) -> int:
    """Base b of the window [b, b + width - 1] inside [0, 255] that holds the most of the given
    exponents (smallest b on ties)."""
    hist = np.bincount(np.asarray(exponents, dtype=np.int64).ravel(), minlength=256)
    best_b, best_n = 0, -1
    for b in range(0, 256 - width + 1):
        n = int(hist[b:b + width].sum())
        if n > best_n:
            best_b, best_n = b, n
    return best_b


def calibrate(pages, kind: int):
    """Bases (b3, b4), each uint8 [128] (one per dim), from calibration pages [..., 16, 128]
    (uint16 BF16 words) of one (layer, K or V, KV head)."""
    pages = np.asarray(pages, dtype=np.uint16).reshape(-1, TILE_TOKENS, HEAD_DIM)
    _, e, _ = codec.fields(pages)
    b3 = np.array([best_window(e[:, :, d], 8) for d in range(HEAD_DIM)], dtype=np.uint8)
    b4 = np.array([best_window(e[:, :, d], 16) for d in range(HEAD_DIM)], dtype=np.uint8)
    return b3, b4


# --------------------------------------------------------------------------------------------
# Groups of eight in attention-access order
# --------------------------------------------------------------------------------------------
def tile_groups(page, kind: int):
    """Natural tile [16, 128] -> (words [4, 64, 8], dims [4, 64, 8]): group (j, c) = chunk c of
    block j, value i, and the head dim each value belongs to."""
    page = np.asarray(page, dtype=np.uint16).reshape(TILE_TOKENS, HEAD_DIM)
    words = np.zeros((4, LANES, 8), dtype=np.uint16)
    dims = np.zeros((4, LANES, 8), dtype=np.int64)
    for j in range(4):
        token, dim = codec.storage_coords(kind, j)
        words[j] = page[token, dim].reshape(LANES, 8)
        dims[j] = dim.reshape(LANES, 8)
    return words, dims


def group_mode(e, b3, b4) -> int:
    """Narrowest width whose offsets d = e - b_w hold all eight exponents of the group."""
    e = np.asarray(e, dtype=np.int64)
    d3 = e - np.asarray(b3, dtype=np.int64)
    if np.all((d3 >= 0) & (d3 <= 7)):
        return MODE_3BIT
    d4 = e - np.asarray(b4, dtype=np.int64)
    if np.all((d4 >= 0) & (d4 <= 15)):
        return MODE_4BIT
    return MODE_RAW


def group_codes(e, mode: int, b3, b4):
    """Codes of the eight exponents: e - b3, e - b4, or e itself (b_8 = 0)."""
    e = np.asarray(e, dtype=np.int64)
    if mode == MODE_3BIT:
        return e - np.asarray(b3, dtype=np.int64)
    if mode == MODE_4BIT:
        return e - np.asarray(b4, dtype=np.int64)
    return e


# --------------------------------------------------------------------------------------------
# Tile encode / decode
# --------------------------------------------------------------------------------------------
def encode_tile(page, kind: int, b3, b4, force_raw: bool = False):
    """One K or V tile [16, 128] (uint16) -> (raw: bool, record uint8[...]).

    Compressed record: 2880 + E bytes (E = escape bytes <= 128).  A tile whose escape bytes
    do not fit the 128-byte slot is stored raw: 4096 bytes in the raw chunk layout."""
    page = np.asarray(page, dtype=np.uint16).reshape(TILE_TOKENS, HEAD_DIM)
    b3 = np.asarray(b3, dtype=np.int64)
    b4 = np.asarray(b4, dtype=np.int64)
    words, dims = tile_groups(page, kind)
    s, e, lo = codec.fields(words)
    sm = (s.astype(np.uint32) << 7) | (lo.astype(np.uint32) & 0x7F)     # sign + 7 fraction bits

    modes = np.zeros((4, LANES), dtype=np.int64)
    codes = np.zeros((4, LANES, 8), dtype=np.int64)
    for j in range(4):
        for c in range(LANES):
            dm = dims[j, c]
            m = group_mode(e[j, c], b3[dm], b4[dm])
            modes[j, c] = m
            codes[j, c] = group_codes(e[j, c], m, b3[dm], b4[dm])
    esc_total = sum(ESCAPE_BYTES[int(m)] for m in modes.ravel())
    if force_raw or esc_total > ESCAPE_SLOT:
        raw = np.concatenate([codec.page_to_storage(page, kind, j) for j in range(4)])
        return True, raw.astype("<u2").view(np.uint8).copy()

    rec = np.zeros(ESC_OFF + esc_total, dtype=np.uint8)
    for j in range(4):
        for c in range(LANES):
            for i in range(8):
                rec[512 * j + 8 * c + i] = sm[j, c, i]
            low24 = 0
            for i in range(8):
                low24 |= (int(codes[j, c, i]) & 0x7) << (3 * i)
            for k in range(3):
                rec[CODE_OFF + 12 * c + 3 * j + k] = (low24 >> (8 * k)) & 0xFF
    for c in range(LANES):
        byte = 0
        for j in range(4):
            byte |= int(modes[j, c]) << (2 * j)
        rec[MODE_OFF + c] = byte
    at = ESC_OFF
    for c in range(LANES):
        for j in range(4):
            m = int(modes[j, c])
            if m == MODE_4BIT:
                byte = 0
                for i in range(8):
                    byte |= ((int(codes[j, c, i]) >> 3) & 1) << i
                rec[at] = byte
                at += 1
            elif m == MODE_RAW:
                bits = 0
                for i in range(8):
                    bits |= ((int(codes[j, c, i]) >> 3) & 0x1F) << (5 * i)
                for k in range(5):
                    rec[at + k] = (bits >> (8 * k)) & 0xFF
                at += 5
    assert at == rec.size
    return False, rec


def decode_tile(record, raw: bool, kind: int, b3, b4) -> np.ndarray:
    """Record -> natural tile [16, 128] (uint16): e = code + b_w, with b_8 = 0."""
    record = np.asarray(record, dtype=np.uint8)
    page = np.zeros((TILE_TOKENS, HEAD_DIM), dtype=np.uint16)
    if raw:
        words = record[:RAW_TILE_BYTES].copy().view("<u2").astype(np.uint16)
        for j in range(4):
            codec.storage_to_page(words[512 * j:512 * (j + 1)], kind, j, page)
        return page
    b3 = np.asarray(b3, dtype=np.int64)
    b4 = np.asarray(b4, dtype=np.int64)
    _, dims = tile_groups(page, kind)
    at = ESC_OFF
    out = np.zeros((4, LANES, 8), dtype=np.uint16)
    for c in range(LANES):
        mode_byte = int(record[MODE_OFF + c])
        for j in range(4):
            m = (mode_byte >> (2 * j)) & 3
            low24 = 0
            for k in range(3):
                low24 |= int(record[CODE_OFF + 12 * c + 3 * j + k]) << (8 * k)
            hi = [0] * 8
            if m == MODE_4BIT:
                byte = int(record[at])
                at += 1
                hi = [(byte >> i) & 1 for i in range(8)]
            elif m == MODE_RAW:
                bits = 0
                for k in range(5):
                    bits |= int(record[at + k]) << (8 * k)
                at += 5
                hi = [(bits >> (5 * i)) & 0x1F for i in range(8)]
            elif m != MODE_3BIT:
                raise ValueError("mode tag 3 is unused")
            for i in range(8):
                code = ((low24 >> (3 * i)) & 0x7) | (hi[i] << 3)
                dim = dims[j, c, i]
                base = b3[dim] if m == MODE_3BIT else (b4[dim] if m == MODE_4BIT else 0)
                e = code + int(base)
                sm = int(record[512 * j + 8 * c + i])
                out[j, c, i] = ((sm >> 7) << 15) | (e << 7) | (sm & 0x7F)
    for j in range(4):
        codec.storage_to_page(out[j].reshape(512), kind, j, page)
    return page


def run_granules(raw: bool) -> int:
    return RAW_RUN_GRANULES if raw else COMPRESSED_RUN_GRANULES


def tags_of(raw: bool):
    return list(TAGS_RAW if raw else TAGS_COMPRESSED)
