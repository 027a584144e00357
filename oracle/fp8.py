"""CPU oracle for exponent-coded FP8 KV tiles (a third lossless page format), and decode
attention over FP8 KV.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__ and the CPU-baseline
leg of bench.py may import this module.  The HIP library and its Python binding never do, and
this module imports nothing from them.

What it follows: "GAAC: Lossless KV Compression for Bandwidth-Efficient LLM Inference on Personal
Devices":
  * appendix "Relation to FP8 KV", Table 7 - the same lossless exponent coding applied to KV
    states that were converted to FP8 (E4M3 and E5M2) compresses them further without adding any
    error beyond the FP8 conversion itself;
  * section "Lossless KV Compression" - sign and fraction bits are kept unchanged; only the
    exponent is coded; per head-channel pair, calibrated contiguous windows of 8 and 16
    exponents (bases b3, b4) separately for K and V; groups of eight in attention-access order
    share a 2-bit mode (3-bit offsets, 4-bit offsets, raw exponents); the group takes the
    narrowest width that holds all eight, reconstruction is e = code + b_w with b_raw = 0; the
    low three code bits of every mode go to one common stream, a 4-bit group adds one byte of
    high bits and a raw group the exponent bits above the low three;
  * section "Block-Wise Compression Scheduling" - fixed-capacity slots; a tile whose encoding
    does not fit its slot keeps its uncompressed form; two storage classes.
FP8 fields follow the OCP 8-bit floating point formats, which the same appendix names:
E4M3 ("e4m3fn": 1 sign, 4 exponent bits with bias 7, 3 fraction bits; exponent 15 with fraction 7
is NaN; no infinities) and E5M2 (1 sign, 5 exponent bits with bias 15, 2 fraction bits; exponent
31 is infinity with fraction 0, NaN otherwise).  Exponent field 0 holds zeros and subnormals.

Readings taken where the pages leave a step open (each is also stated in include/kvz.h):
  * the code is GAAC's, unchanged, applied to the FP8 exponent field (4 or 5 bits): the kept
    part is sign + fraction (4 bits in E4M3, 3 in E5M2); a raw group stores the 1 (E4M3) or 2
    (E5M2) exponent bits above the low three; so the all-3-bit case is 4 + 3 + 0.25 = 7.25 and
    3 + 3 + 0.25 = 6.25 bits per value (1.103x and 1.28x);
  * windows lie inside the exponent field, [0, 15] or [0, 31], ties to the smallest base (so the
    16-wide window of E4M3 is always [0, 15] and its groups never need the raw mode);
  * tile = one page's K or V for one KV head (16 x 128 values), groups = the MFMA operand chunks
    of the BF16 formats (codec.storage_coords): group (j, c) = chunk c of 32-dim block j;
  * uncompressed FP8 tile ("FP8 chunk layout", 2048 bytes): chunk c of block j at byte
    1024*(j//2) + 16*c + 8*(j%2), its eight values in order - lane c finds blocks 0,1 in one
    16-byte piece and blocks 2,3 in another;
  * compressed record: sign+fraction plane (lane c's bytes at SM*c, see _sm_words), code plane
    (768 bytes: lane c's 12 bytes at SM_BYTES + 12c, block j's 24 low code bits at +3j, value i
    at bits 3i..3i+2, little-endian), mode plane (64 bytes: byte c holds block j's mode at bits
    2j..2j+1; 0 = 3-bit, 1 = 4-bit, 2 = raw), then the escape bytes (lanes in order, each lane's
    groups in block order; 4-bit group: one byte, bit i = code bit 3 of value i; raw group: the
    exponent bits 3.. of value i at bits (EW-3)*i.. of a little-endian integer of EW-3 bytes);
  * sign+fraction packing, per lane c and group j, with X = the bytes (s << 7 | fraction) of
    values 0..3 and Y the same of values 4..7 (one byte each, little-endian in a 32-bit word):
      E4M3: word j (bytes SM*c + 4j..) = X | rotl32(Y, 4);
      E5M2: words t = 0, 1, 2 (bytes 12c + 4t..) = X_t | rotl32(Y_t, 3) for groups 0..2, and
            group 3 fills the bits 5 and 6 left free in every byte: word 0 bits 8k+5..8k+6 =
            fraction of value k, word 1 the same of value k+4, word 2 bit 8k+5 = sign of value k,
            bit 8k+6 = sign of value k+4;
  * escape slot 64 bytes; a compressed record takes SLOT_BYTES = 1920 (E4M3) / 1664 (E5M2)
    bytes, 15 / 13 granules of 128 bytes, the raw tile 2048 bytes = 16 granules; so a pool whose
    granule is 128 bytes serves FP8 tiles with its run classes of 12 + k granules: the tags of a
    compressed tile carry k = 3 (E4M3: FF FF FF 00) or k = 1 (E5M2: FF 00 00 00) bytes 0xFF,
    a raw tile FF FF FF FF.

Attention over FP8 KV is the plain definition of oracle/attention.py on the FP8 values decoded
exactly (times a per-layer dequantization scale for K and for V).

Pins (tests/test_oracle_fp8.py): torch's own float8 conversions for every one of the 256 byte
patterns of both kinds, round trips over all patterns and random tiles and bases, hand-worked
bytes in tests/golden/, the 7.25 / 6.25-bit figures, mode, calibration and escape-slot
boundaries worked by hand, the register-restore formulas applied to the bytes written here, and
brute-force attention.
"""
from __future__ import annotations

import numpy as np

from . import attention, codec

E4M3, E5M2 = 0, 1
KIND_NAMES = {E4M3: "e4m3", E5M2: "e5m2"}
EXP_BITS = {E4M3: 4, E5M2: 5}
FRAC_BITS = {E4M3: 3, E5M2: 2}
BIAS = {E4M3: 7, E5M2: 15}

TILE_TOKENS = 16
HEAD_DIM = 128
LANES = 64
SM_BYTES = {E4M3: 1024, E5M2: 768}          # sign + fraction: 4 / 3 bits per value
SM_LANE_BYTES = {E4M3: 16, E5M2: 12}
CODE_BYTES = 768                            # 3 bits per value
MODE_BYTES = 64                             # 2 bits per group
ESCAPE_SLOT = 64
RAW_TILE_BYTES = 2048
GRANULE_BYTES = 128
MODE_3BIT, MODE_4BIT, MODE_RAW = 0, 1, 2
TAGS_RAW = [0xFF, 0xFF, 0xFF, 0xFF]
TAGS_COMPRESSED = {E4M3: [0xFF, 0xFF, 0xFF, 0x00], E5M2: [0xFF, 0x00, 0x00, 0x00]}


def code_off(fk: int) -> int:
    return SM_BYTES[fk]


def mode_off(fk: int) -> int:
    return SM_BYTES[fk] + CODE_BYTES


def esc_off(fk: int) -> int:
    return SM_BYTES[fk] + CODE_BYTES + MODE_BYTES


def slot_bytes(fk: int) -> int:
    return esc_off(fk) + ESCAPE_SLOT


def raw_escape_bytes(fk: int) -> int:
    """Escape bytes of a raw group: the exponent bits above the low three, for eight values."""
    return EXP_BITS[fk] - 3


def escape_bytes(fk: int, mode: int) -> int:
    return {MODE_3BIT: 0, MODE_4BIT: 1, MODE_RAW: raw_escape_bytes(fk)}[mode]


# --------------------------------------------------------------------------------------------
# FP8 fields and values (OCP E4M3 "fn" and E5M2)
# --------------------------------------------------------------------------------------------
def fields(x, fk: int):
    """FP8 bytes -> (sign, exponent field, fraction field)."""
    x = np.asarray(x, dtype=np.uint8).astype(np.int64)
    mw, ew = FRAC_BITS[fk], EXP_BITS[fk]
    return x >> 7, (x >> mw) & ((1 << ew) - 1), x & ((1 << mw) - 1)


def to_f64(x, fk: int) -> np.ndarray:
    """FP8 bytes -> exact float64 values."""
    s, e, m = fields(x, fk)
    mw, bias, emax = FRAC_BITS[fk], BIAS[fk], (1 << EXP_BITS[fk]) - 1
    sign = np.where(s == 1, -1.0, 1.0)
    frac = m.astype(np.float64) / (1 << mw)
    val = np.where(e == 0, frac * 2.0 ** (1 - bias),
                   (1.0 + frac) * np.exp2((e - bias).astype(np.float64)))
    val = sign * val
    if fk == E4M3:
        val = np.where((e == emax) & (m == (1 << mw) - 1), np.nan, val)
    else:
        val = np.where((e == emax) & (m == 0), sign * np.inf, val)
        val = np.where((e == emax) & (m != 0), np.nan, val)
    return val


# --------------------------------------------------------------------------------------------
# Uncompressed tile in the FP8 chunk layout
# --------------------------------------------------------------------------------------------
def chunk_offset(j: int, c: int) -> int:
    return 1024 * (j // 2) + 16 * c + 8 * (j % 2)


def tile_groups(page, kind: int):
    """Natural FP8 tile [16, 128] -> (bytes [4, 64, 8], dims [4, 64, 8]): group (j, c) is
    chunk c of block j in the operand order of codec.storage_coords."""
    page = np.asarray(page, dtype=np.uint8).reshape(TILE_TOKENS, HEAD_DIM)
    vals = np.zeros((4, LANES, 8), dtype=np.uint8)
    dims = np.zeros((4, LANES, 8), dtype=np.int64)
    for j in range(4):
        token, dim = codec.storage_coords(kind, j)
        vals[j] = page[token, dim].reshape(LANES, 8)
        dims[j] = dim.reshape(LANES, 8)
    return vals, dims


def raw_tile(page, kind: int) -> np.ndarray:
    vals, _ = tile_groups(page, kind)
    out = np.zeros(RAW_TILE_BYTES, dtype=np.uint8)
    for j in range(4):
        for c in range(LANES):
            at = chunk_offset(j, c)
            out[at:at + 8] = vals[j, c]
    return out


def _groups_to_page(vals, kind: int) -> np.ndarray:
    page = np.zeros((TILE_TOKENS, HEAD_DIM), dtype=np.uint8)
    for j in range(4):
        token, dim = codec.storage_coords(kind, j)
        page[token, dim] = vals[j].reshape(-1)
    return page


def raw_tile_to_page(rec, kind: int) -> np.ndarray:
    rec = np.asarray(rec, dtype=np.uint8)
    vals = np.zeros((4, LANES, 8), dtype=np.uint8)
    for j in range(4):
        for c in range(LANES):
            at = chunk_offset(j, c)
            vals[j, c] = rec[at:at + 8]
    return _groups_to_page(vals, kind)


# --------------------------------------------------------------------------------------------
# Calibration (GAAC "Lossless KV Compression", contiguous exponent concentration)
# --------------------------------------------------------------------------------------------
def best_window(exponents, width: int, fk: int) -> int:
    """Base b of the window [b, b + width - 1] inside the exponent field that holds the most of
    the given exponents (smallest b on ties)."""
    n_e = 1 << EXP_BITS[fk]
    hist = np.bincount(np.asarray(exponents, dtype=np.int64).ravel(), minlength=n_e)
    best_b, best_n = 0, -1
    for b in range(0, n_e - width + 1):
        n = int(hist[b:b + width].sum())
        if n > best_n:
            best_b, best_n = b, n
    return best_b


def calibrate(pages, fk: int):
    """Bases (b3, b4), uint8 [128] each, from calibration tiles [..., 16, 128] of FP8 bytes of
    one (layer, K or V, KV head)."""
    pages = np.asarray(pages, dtype=np.uint8).reshape(-1, TILE_TOKENS, HEAD_DIM)
    _, e, _ = fields(pages, fk)
    b3 = np.array([best_window(e[:, :, d], 8, fk) for d in range(HEAD_DIM)], dtype=np.uint8)
    b4 = np.array([best_window(e[:, :, d], 16, fk) for d in range(HEAD_DIM)], dtype=np.uint8)
    return b3, b4


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
    e = np.asarray(e, dtype=np.int64)
    if mode == MODE_3BIT:
        return e - np.asarray(b3, dtype=np.int64)
    if mode == MODE_4BIT:
        return e - np.asarray(b4, dtype=np.int64)
    return e


# --------------------------------------------------------------------------------------------
# Sign + fraction plane
# --------------------------------------------------------------------------------------------
def _rotl32(x: int, k: int) -> int:
    return ((x << k) | (x >> (32 - k))) & 0xFFFFFFFF


def _sm_words(s, m, fk: int):
    """Sign and fraction of one lane's four groups (s, m: [4, 8]) -> the lane's 32-bit words."""
    mw = FRAC_BITS[fk]

    def xy(j):
        x = sum(((int(s[j, k]) << 7) | int(m[j, k])) << (8 * k) for k in range(4))
        y = sum(((int(s[j, k + 4]) << 7) | int(m[j, k + 4])) << (8 * k) for k in range(4))
        return x, y

    if fk == E4M3:
        return [xy(j)[0] | _rotl32(xy(j)[1], 4) for j in range(4)]
    words = [xy(t)[0] | _rotl32(xy(t)[1], 3) for t in range(3)]
    for k in range(4):
        words[0] |= int(m[3, k]) << (8 * k + 5)
        words[1] |= int(m[3, k + 4]) << (8 * k + 5)
        words[2] |= (int(s[3, k]) << (8 * k + 5)) | (int(s[3, k + 4]) << (8 * k + 6))
    assert mw == 2
    return words


def _sm_unpack(words, fk: int):
    """Inverse of _sm_words, read field by field: -> (s, m) [4, 8]."""
    s = np.zeros((4, 8), dtype=np.int64)
    m = np.zeros((4, 8), dtype=np.int64)
    if fk == E4M3:
        for j in range(4):
            w = words[j]
            for k in range(4):
                s[j, k] = (w >> (8 * k + 7)) & 1
                m[j, k] = (w >> (8 * k)) & 7
                m[j, k + 4] = (w >> (8 * k + 4)) & 7
                s[j, k + 4] = (w >> (8 * ((k + 1) % 4) + 3)) & 1
        return s, m
    for t in range(3):
        w = words[t]
        for k in range(4):
            s[t, k] = (w >> (8 * k + 7)) & 1
            m[t, k] = (w >> (8 * k)) & 3
            m[t, k + 4] = (w >> (8 * k + 3)) & 3
            s[t, k + 4] = (w >> (8 * ((k + 1) % 4) + 2)) & 1
    for k in range(4):
        m[3, k] = (words[0] >> (8 * k + 5)) & 3
        m[3, k + 4] = (words[1] >> (8 * k + 5)) & 3
        s[3, k] = (words[2] >> (8 * k + 5)) & 1
        s[3, k + 4] = (words[2] >> (8 * k + 6)) & 1
    return s, m


# --------------------------------------------------------------------------------------------
# Tile encode / decode
# --------------------------------------------------------------------------------------------
def encode_tile(page, kind: int, fk: int, b3, b4, force_raw: bool = False):
    """One FP8 K or V tile [16, 128] (uint8) -> (raw: bool, record uint8[...]).

    Compressed record: esc_off + E bytes (E = escape bytes <= 64).  A tile whose escape bytes
    do not fit the slot is stored raw: 2048 bytes in the FP8 chunk layout."""
    page = np.asarray(page, dtype=np.uint8).reshape(TILE_TOKENS, HEAD_DIM)
    b3 = np.asarray(b3, dtype=np.int64)
    b4 = np.asarray(b4, dtype=np.int64)
    vals, dims = tile_groups(page, kind)
    s, e, m = fields(vals, fk)
    modes = np.zeros((4, LANES), dtype=np.int64)
    codes = np.zeros((4, LANES, 8), dtype=np.int64)
    for j in range(4):
        for c in range(LANES):
            dm = dims[j, c]
            modes[j, c] = group_mode(e[j, c], b3[dm], b4[dm])
            codes[j, c] = group_codes(e[j, c], int(modes[j, c]), b3[dm], b4[dm])
    esc_total = sum(escape_bytes(fk, int(md)) for md in modes.ravel())
    if force_raw or esc_total > ESCAPE_SLOT:
        return True, raw_tile(page, kind)

    rec = np.zeros(esc_off(fk) + esc_total, dtype=np.uint8)
    lane_sm = SM_LANE_BYTES[fk]
    for c in range(LANES):
        words = _sm_words(s[:, c, :], m[:, c, :], fk)
        for t, w in enumerate(words):
            for k in range(4):
                rec[lane_sm * c + 4 * t + k] = (w >> (8 * k)) & 0xFF
        for j in range(4):
            low24 = 0
            for i in range(8):
                low24 |= (int(codes[j, c, i]) & 7) << (3 * i)
            for k in range(3):
                rec[code_off(fk) + 12 * c + 3 * j + k] = (low24 >> (8 * k)) & 0xFF
        byte = 0
        for j in range(4):
            byte |= int(modes[j, c]) << (2 * j)
        rec[mode_off(fk) + c] = byte
    at = esc_off(fk)
    hi_bits = EXP_BITS[fk] - 3
    for c in range(LANES):
        for j in range(4):
            md = int(modes[j, c])
            if md == MODE_4BIT:
                byte = 0
                for i in range(8):
                    byte |= ((int(codes[j, c, i]) >> 3) & 1) << i
                rec[at] = byte
                at += 1
            elif md == MODE_RAW:
                bits = 0
                for i in range(8):
                    bits |= ((int(codes[j, c, i]) >> 3) & ((1 << hi_bits) - 1)) << (hi_bits * i)
                for k in range(hi_bits):
                    rec[at + k] = (bits >> (8 * k)) & 0xFF
                at += hi_bits
    assert at == rec.size
    return False, rec


def decode_tile(record, raw: bool, kind: int, fk: int, b3, b4) -> np.ndarray:
    """Record -> natural FP8 tile [16, 128] (uint8): e = code + b_w, with b_raw = 0."""
    record = np.asarray(record, dtype=np.uint8)
    if raw:
        return raw_tile_to_page(record[:RAW_TILE_BYTES], kind)
    b3 = np.asarray(b3, dtype=np.int64)
    b4 = np.asarray(b4, dtype=np.int64)
    _, dims = tile_groups(np.zeros((TILE_TOKENS, HEAD_DIM), np.uint8), kind)
    mw, hi_bits = FRAC_BITS[fk], EXP_BITS[fk] - 3
    lane_sm = SM_LANE_BYTES[fk]
    vals = np.zeros((4, LANES, 8), dtype=np.uint8)
    at = esc_off(fk)
    for c in range(LANES):
        words = [sum(int(record[lane_sm * c + 4 * t + k]) << (8 * k) for k in range(4))
                 for t in range(lane_sm // 4)]
        s, m = _sm_unpack(words, fk)
        mode_byte = int(record[mode_off(fk) + c])
        for j in range(4):
            md = (mode_byte >> (2 * j)) & 3
            low24 = sum(int(record[code_off(fk) + 12 * c + 3 * j + k]) << (8 * k) for k in range(3))
            hi = [0] * 8
            if md == MODE_4BIT:
                byte = int(record[at])
                at += 1
                hi = [(byte >> i) & 1 for i in range(8)]
            elif md == MODE_RAW:
                bits = sum(int(record[at + k]) << (8 * k) for k in range(hi_bits))
                at += hi_bits
                hi = [(bits >> (hi_bits * i)) & ((1 << hi_bits) - 1) for i in range(8)]
            elif md != MODE_3BIT:
                raise ValueError("mode tag 3 is unused")
            for i in range(8):
                code = ((low24 >> (3 * i)) & 7) | (hi[i] << 3)
                dim = dims[j, c, i]
                base = b3[dim] if md == MODE_3BIT else (b4[dim] if md == MODE_4BIT else 0)
                ex = code + int(base)
                vals[j, c, i] = (int(s[j, i]) << 7) | (ex << mw) | int(m[j, i])
    return _groups_to_page(vals, kind)


def tags_of(raw: bool, fk: int):
    return list(TAGS_RAW if raw else TAGS_COMPRESSED[fk])


def run_granules(raw: bool, fk: int) -> int:
    """128-byte granules of a record: 12 + (number of 0xFF tag bytes)."""
    return 12 + sum(1 for t in tags_of(raw, fk) if t == 0xFF)


# --------------------------------------------------------------------------------------------
# Attention over FP8 KV
# --------------------------------------------------------------------------------------------
def attention_fp64(q_bits, k_fp8, v_fp8, fk: int, sm_scale: float, k_scale: float,
                   v_scale: float) -> np.ndarray:
    """One sequence.  q_bits [Hq, D] BF16 words; k_fp8 / v_fp8 [T, Hkv, D] FP8 bytes, whose values
    are to_f64(.) * k_scale / v_scale.  Returns float64 [Hq, D]."""
    q = codec.bf16_bits_to_f64(q_bits)
    k = to_f64(k_fp8, fk) * float(k_scale)
    v = to_f64(v_fp8, fk) * float(v_scale)
    return attention.attention_values_fp64(q, k, v, sm_scale)


def gather_sequence(arena, meta_table, bases, block_table_row, n_comp: int, tail_b, n_tail: int,
                    fk: int):
    """K and V FP8 bytes of one sequence in token order, [T, Hkv, 128].

    meta_table[phys][g][kind] = (off, tags) in 128-byte granules; bases[g][kind] = (b3, b4);
    tail_b: uint8 [2, Hkv, 16, 128] or None."""
    hkv = len(bases)
    t_total = TILE_TOKENS * n_comp + n_tail
    k = np.zeros((t_total, hkv, HEAD_DIM), dtype=np.uint8)
    v = np.zeros_like(k)
    for p in range(n_comp):
        phys = int(block_table_row[p])
        rows = slice(TILE_TOKENS * p, TILE_TOKENS * (p + 1))
        for g in range(hkv):
            for kind, dst in ((codec.KIND_K, k), (codec.KIND_V, v)):
                off, tags = meta_table[phys][g][kind]
                raw = list(tags) == TAGS_RAW
                at = off * GRANULE_BYTES
                rec = arena[at:at + (RAW_TILE_BYTES if raw else slot_bytes(fk))]
                dst[rows, g, :] = decode_tile(rec, raw, kind, fk, *bases[g][kind])
    if n_tail:
        base = TILE_TOKENS * n_comp
        k[base:] = np.transpose(tail_b[0, :, :n_tail, :], (1, 0, 2))
        v[base:] = np.transpose(tail_b[1, :, :n_tail, :], (1, 0, 2))
    return k, v


def decode_attention(q_bits, arena, meta_table, bases, block_table, seq_lens, n_comp_pages,
                     tail, fk: int, sm_scale: float, k_scale: float, v_scale: float,
                     batch_indices=None) -> np.ndarray:
    """Batched decode attention over FP8 tiles plus an FP8 tail ([B, 2, Hkv, 16, 128] or None).
    Returns float64 [B, Hq, 128]; rows of batch entries not in batch_indices stay zero."""
    q_bits = np.asarray(q_bits, dtype=np.uint16)
    out = np.zeros(q_bits.shape, dtype=np.float64)
    for b in (range(q_bits.shape[0]) if batch_indices is None else batch_indices):
        n_comp = int(n_comp_pages[b])
        n_tail = int(seq_lens[b]) - TILE_TOKENS * n_comp
        if not 0 <= n_tail <= TILE_TOKENS:
            raise ValueError("seq_len - 16*n_comp_pages must lie in [0, 16]")
        kb, vb = gather_sequence(arena, meta_table, bases, block_table[b], n_comp,
                                 None if tail is None else tail[b], n_tail, fk)
        out[b] = attention_fp64(q_bits[b], kb, vb, fk, sm_scale, k_scale, v_scale)
    return out
