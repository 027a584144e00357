"""CPU oracle for the 12-bit exponent-coded BF16 KV page format.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__ and the CPU-baseline
leg of bench.py may import this module.  The HIP library and its Python binding never do, and
this module imports nothing from them.

What it follows: "ZipFusion: Fusing Lossless KV Decompression with Attention for Efficient LLM
Decoding", section "How it works":
  * step 1 - a page's K (or V), per layer and KV head, is four independent 512-value blocks;
  * step 2 - base b = minimum exponent rounded down to even; compress only if every exponent
    lies in [b, b+15], else keep the block raw;
  * step 3 - keep each value's low byte (7 fraction bits + exponent LSB) and add a 4-bit code,
    the sign plus d = floor((e-b)/2): 768 B instead of 1024 B per block;
  * step 4 - restore e = b + 2d + r, r taken from the kept low byte, integer work only;
  * the paragraph on layouts - K and V get separate layouts so that each thread's eight operand
    elements sit together; code bytes pair values (x0,x4),(x1,x5),(x2,x6),(x3,x7);
  * the paragraph on metadata - 8 bytes per 4-block K or V group: the first block's offset and
    a raw flag or b/2 per block; later blocks are found by summing the sizes before them.
BF16 fields follow the BF16 word description of the same page and the field split printed in
"ExANS: Exponent Aligned Asymmetric Numeral Systems", section "Encoding Pipeline".

Readings taken where the page leaves a step open (each is also stated in include/kvz.h):
  * block j of a group is tokens 0..15 x dims [32j, 32j+32);
  * element order inside a block (storage order) is the MFMA operand order, see storage_coords();
  * a block is 64 chunks of 8 values; a compressed chunk is 12 bytes (8 low bytes, then a
    32-bit code word), a raw chunk is 16 bytes (8 little-endian BF16 words);
  * the code word of a chunk is X | rotl32(Y, 4), where X holds (s<<7 | d) of elements 0..3 in
    its four bytes and Y holds the same for elements 4..7;
  * raw marker tag 0xFF, offsets in 256-byte granules, meta bytes 0-3 = offset (LE),
    bytes 4-7 = tag of blocks 0..3.

Pins (tests/test_oracle_codec.py): hand-worked examples in tests/golden/, the ExANS field
split, a brute-force search over even exponent windows, all 65,536 BF16 patterns, the exact
768/1024-byte sizes, and the page's register restore (mask on one branch, unpack on the other,
one add of b/2 replicated per byte) applied to the bytes this module writes.
"""
from __future__ import annotations

import numpy as np

PAGE_TOKENS = 16
HEAD_DIM = 128
BLOCK_DIMS = 32
BLOCKS_PER_GROUP = 4
BLOCK_VALUES = PAGE_TOKENS * BLOCK_DIMS          # 512
CHUNKS = 64
CHUNK_VALUES = 8
COMPRESSED_CHUNK_BYTES = 12
RAW_CHUNK_BYTES = 16
COMPRESSED_BLOCK_BYTES = CHUNKS * COMPRESSED_CHUNK_BYTES   # 768
RAW_BLOCK_BYTES = CHUNKS * RAW_CHUNK_BYTES                 # 1024
RAW_TAG = 0xFF
GRANULE_BYTES = 256
OFF_NONE = 0xFFFFFFFF
KIND_K = 0
KIND_V = 1


# --------------------------------------------------------------------------------------------
# BF16 fields (ZipFusion "How it works": 1 sign, 8 exponent, 7 fraction bits)
# --------------------------------------------------------------------------------------------
def fields(w):
    """Split BF16 bit patterns (uint16 array) into sign, exponent and the kept low byte.

    The low byte is the 7 fraction bits plus the exponent's least significant bit (step 3).
    """
    w = np.asarray(w, dtype=np.uint16).astype(np.uint32)
    s = w >> 15
    e = (w >> 7) & 0xFF
    lo = w & 0xFF
    return s, e, lo


def bf16_bits_to_f64(w):
    """BF16 bit patterns -> float64 values (a BF16 word is the top half of an fp32 word)."""
    w32 = np.asarray(w, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return w32.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------------------------
# Block membership and storage order (step 1 + the layout paragraph)
# --------------------------------------------------------------------------------------------
def storage_coords(kind: int, j: int):
    """(token, dim) of storage index n = 8*c + i of block j, for c in 0..63 and i in 0..7.

    K: chunk c holds token c % 16 and dims 32j + 8*(c // 16) + i  (eight consecutive dims).
    V: chunk c holds dim 32j + c % 32 and tokens 8*(c // 32) + i  (eight consecutive tokens).
    Each chunk is what one lane feeds to a bf16 MFMA: K as the token-row operand of a
    16x16x32 product (reduction over dims), V as the dim-column operand of a 32x32x16 product
    (reduction over tokens).
    """
    n = np.arange(BLOCK_VALUES)
    c, i = n // CHUNK_VALUES, n % CHUNK_VALUES
    if kind == KIND_K:
        token = c % 16
        dim = BLOCK_DIMS * j + 8 * (c // 16) + i
    elif kind == KIND_V:
        dim = BLOCK_DIMS * j + c % 32
        token = 8 * (c // 32) + i
    else:
        raise ValueError("kind must be 0 (K) or 1 (V)")
    return token, dim


def page_to_storage(page, kind: int, j: int):
    """Natural page [..., 16 tokens, 128 dims] (uint16) -> block j in storage order [..., 512]."""
    token, dim = storage_coords(kind, j)
    page = np.asarray(page, dtype=np.uint16)
    return page[..., token, dim]


def storage_to_page(words, kind: int, j: int, page):
    """Scatter block j given in storage order [..., 512] back into page [..., 16, 128] in place."""
    token, dim = storage_coords(kind, j)
    page[..., token, dim] = words


# --------------------------------------------------------------------------------------------
# Base and eligibility (step 2)
# --------------------------------------------------------------------------------------------
def base_and_eligible(e):
    """Per block (last axis = the block's 512 exponents): b = min e rounded down to even;
    eligible iff every exponent lies in [b, b+15] (the lower bound holds by construction)."""
    e = np.asarray(e, dtype=np.int64)
    m = e.min(axis=-1)
    b = m - (m % 2)
    eligible = e.max(axis=-1) <= b + 15
    return b, eligible


# --------------------------------------------------------------------------------------------
# Block encode / decode (steps 3 and 4)
# --------------------------------------------------------------------------------------------
def _rotl32(x, k):
    x = np.asarray(x, dtype=np.uint64) & 0xFFFFFFFF
    return ((x << k) | (x >> (32 - k))) & 0xFFFFFFFF


def _rotr32(x, k):
    return _rotl32(x, 32 - k)


def encode_blocks(words, force_raw: bool = False):
    """Encode blocks given in storage order.

    words: uint16 [N, 512].  Returns (tags uint8 [N], records: list of N uint8 arrays of
    768 or 1024 bytes).  tag = b/2 for a compressed block, 0xFF for a raw one.
    """
    words = np.asarray(words, dtype=np.uint16).reshape(-1, BLOCK_VALUES)
    nblk = words.shape[0]
    s, e, lo = fields(words)
    b, eligible = base_and_eligible(e)
    if force_raw:
        eligible = np.zeros_like(eligible)
    tags = np.where(eligible, b // 2, RAW_TAG).astype(np.uint8)

    # the 4-bit code of every value: sign plus d = floor((e - b) / 2)   (step 3)
    d = (e.astype(np.int64) - b[:, None]) // 2
    code = (s.astype(np.int64) << 7) | np.where(eligible[:, None], d, 0)   # bits 7 and 0..2
    code = code.reshape(nblk, CHUNKS, CHUNK_VALUES)
    # pairs (x_k, y_k) = (element k, element k+4) of the chunk share one code byte position:
    # X carries x_k in byte k at bits {7, 2:0}; Y carries y_k the same way and is rotated
    # left by 4 bits into bits {3, 6:4} of the next-up byte positions.
    X = np.zeros((nblk, CHUNKS), dtype=np.uint64)
    Y = np.zeros((nblk, CHUNKS), dtype=np.uint64)
    for k in range(4):
        X |= code[:, :, k].astype(np.uint64) << (8 * k)
        Y |= code[:, :, k + 4].astype(np.uint64) << (8 * k)
    C = X | _rotl32(Y, 4)

    lo_bytes = lo.reshape(nblk, CHUNKS, CHUNK_VALUES).astype(np.uint8)
    C_bytes = np.stack([(C >> (8 * k)) & 0xFF for k in range(4)], axis=-1).astype(np.uint8)
    comp = np.concatenate([lo_bytes, C_bytes], axis=-1).reshape(nblk, COMPRESSED_BLOCK_BYTES)
    raw = words.astype("<u2").view(np.uint8).reshape(nblk, RAW_BLOCK_BYTES)

    records = [comp[n].copy() if eligible[n] else raw[n].copy() for n in range(nblk)]
    return tags, records


def decode_block(tag: int, record) -> np.ndarray:
    """Decode one block record back to its 512 BF16 words in storage order (step 4)."""
    record = np.asarray(record, dtype=np.uint8)
    if tag == RAW_TAG:
        assert record.size >= RAW_BLOCK_BYTES
        return record[:RAW_BLOCK_BYTES].copy().view("<u2").astype(np.uint16)
    assert 0 <= tag <= 127 and record.size >= COMPRESSED_BLOCK_BYTES
    b = 2 * int(tag)
    ch = record[:COMPRESSED_BLOCK_BYTES].reshape(CHUNKS, COMPRESSED_CHUNK_BYTES)
    lo = ch[:, :8].astype(np.uint32)
    C = np.zeros(CHUNKS, dtype=np.uint64)
    for k in range(4):
        C |= ch[:, 8 + k].astype(np.uint64) << (8 * k)
    X = C & 0x87878787
    Y = _rotr32(C, 4) & 0x87878787
    out = np.zeros((CHUNKS, CHUNK_VALUES), dtype=np.uint32)
    for i in range(CHUNK_VALUES):
        src = X if i < 4 else Y
        byte = (src >> (8 * (i % 4))) & 0xFF
        s = (byte >> 7).astype(np.uint32)
        d = (byte & 0x7).astype(np.uint32)
        r = lo[:, i] >> 7                       # the exponent LSB kept in the low byte
        e = b + 2 * d + r                       # step 4
        out[:, i] = (s << 15) | (e << 7) | (lo[:, i] & 0x7F)
    return out.reshape(BLOCK_VALUES).astype(np.uint16)


def block_bytes(tag: int) -> int:
    return RAW_BLOCK_BYTES if tag == RAW_TAG else COMPRESSED_BLOCK_BYTES


# --------------------------------------------------------------------------------------------
# 4-block groups and their 8-byte metadata (metadata paragraph)
# --------------------------------------------------------------------------------------------
def encode_group(page, kind: int, force_raw: bool = False):
    """One K or V page [16, 128] (uint16) -> (tags uint8[4], record uint8[3072 + 256*n_raw])."""
    page = np.asarray(page, dtype=np.uint16).reshape(PAGE_TOKENS, HEAD_DIM)
    blocks = np.stack([page_to_storage(page, kind, j) for j in range(BLOCKS_PER_GROUP)])
    tags, recs = encode_blocks(blocks, force_raw=force_raw)
    return tags, np.concatenate(recs)


def group_bytes(tags) -> int:
    return sum(block_bytes(int(t)) for t in tags)


def group_granules(tags) -> int:
    return group_bytes(tags) // GRANULE_BYTES


def n_raw(tags) -> int:
    return sum(1 for t in tags if int(t) == RAW_TAG)


def block_offset_bytes(off_granules: int, tags, j: int) -> int:
    """Byte offset of block j: first block's offset plus the sizes of blocks 0..j-1."""
    return off_granules * GRANULE_BYTES + sum(block_bytes(int(tags[k])) for k in range(j))


def decode_group(arena, off_granules: int, tags, kind: int) -> np.ndarray:
    """Rebuild the natural page [16, 128] of one group stored in arena at off_granules."""
    arena = np.asarray(arena, dtype=np.uint8)
    page = np.zeros((PAGE_TOKENS, HEAD_DIM), dtype=np.uint16)
    for j in range(BLOCKS_PER_GROUP):
        at = block_offset_bytes(off_granules, tags, j)
        size = block_bytes(int(tags[j]))
        words = decode_block(int(tags[j]), arena[at:at + size])
        storage_to_page(words, kind, j, page)
    return page


def meta_bytes(off_granules: int, tags) -> bytes:
    """8-byte group metadata: offset (u32 LE) then the four block tags."""
    return int(off_granules).to_bytes(4, "little") + bytes(int(t) for t in tags)


def parse_meta(m) -> tuple[int, list[int]]:
    m = bytes(np.asarray(m, dtype=np.uint8).tobytes())
    return int.from_bytes(m[:4], "little"), [m[4], m[5], m[6], m[7]]
