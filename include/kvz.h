/*
 * kvz.h - lossless exponent-coded KV pages (12-bit BF16 pages; group-adaptive BF16 and FP8
 *         tiles) and fused paged decode attention for AMD Instinct MI355X (gfx950).
 *
 * The operations follow two pages:
 *   [ZF]   "ZipFusion: Fusing Lossless KV Decompression with Attention for Efficient LLM
 *          Decoding" - section "How it works" (block format, steps 1-4; K/V layouts and the
 *          register restore; 8-byte group metadata; the memory manager).
 *   [GAAC] "GAAC: Lossless KV Compression for Bandwidth-Efficient LLM Inference on Personal
 *          Devices" - sections "Attention with On-the-Fly Decompression" (compressed blocks and
 *          the BF16 tail share one softmax; no decompressed copy in device memory),
 *          "Block-Wise Compression Scheduling" (fill-then-finalize; fixed-capacity slots in two
 *          storage classes; a block that does not fit keeps its BF16 form), "Lossless KV
 *          Compression" (the group-adaptive code of the second and third formats) and
 *          appendix "Relation to FP8 KV" (the code on FP8 KV).
 *
 * Format (readings where the pages are silent are marked *):
 *   - A page holds 16 tokens.  Per (layer, KV head) its K and its V are each one GROUP of four
 *     BLOCKS; block j = tokens 0..15 x dims [32j, 32j+32)*, 512 BF16 values ([ZF] step 1).
 *   - Block base b = minimum exponent rounded down to even; the block is compressed only if
 *     every exponent lies in [b, b+15], otherwise it stays raw ([ZF] step 2).
 *   - A block is 64 chunks of 8 values, in MFMA operand order*:
 *       K chunk c: token c%16, dims 32j + 8*(c/16) + 0..7;
 *       V chunk c: dim 32j + c%32, tokens 8*(c/32) + 0..7.
 *     Compressed chunk (12 B)*: 8 low bytes (7 fraction bits + exponent LSB) of values 0..7,
 *     then the code word C = X | rotl32(Y, 4) (LE), where byte k of X is s<<7 | d of value k
 *     and byte k of Y the same for value k+4, d = (e - b) >> 1 ([ZF] step 3).  Restore:
 *     high bytes of values 0..3 = (C & 0x87878787) + (b/2)*0x01010101, of values 4..7 =
 *     (rotr32(C,4) & 0x87878787) + (b/2)*0x01010101 (no carry; [ZF] step 4 and the restore
 *     paragraph).  Raw chunk (16 B)*: the 8 BF16 words, little-endian.
 *     Compressed block = 768 B, raw block = 1024 B.
 *   - Group metadata, 8 B ([ZF] metadata paragraph): bytes 0-3 the first block's offset in
 *     256-byte granules from the arena base* (LE), bytes 4-7 the tag of blocks 0..3: b/2 for a
 *     compressed block, 0xFF* for a raw one.  Blocks of a group are contiguous; block j starts
 *     at off*256 + (sizes of blocks 0..j-1).
 *   - Slots: 768-B and 1024-B slots ([GAAC] two storage classes); a group occupies one
 *     contiguous run of 12 + n_raw granules.  See kvz_slot_alloc for the allocation rule.
 *
 * Conventions for every call:
 *   - Pointers named d_* or documented as "device" point to device memory owned by the caller
 *     (e.g. torch tensors).  The library never allocates or frees device memory; it owns only
 *     the small host-side pool handle and, for kvz_decode_attention_noalloc, a static
 *     device-resident scratch array (part of the loaded library, not a run-time allocation).
 *   - Calls that take a hipStream_t enqueue work on that stream and return without waiting,
 *     except kvz_pool_stats, which synchronizes the stream.
 *   - Return value: KVZ_OK or a negative KVZ_E* code; kvz_last_error() gives text (per thread).
 *     Nothing throws or aborts across this interface.  Conditions that only the device can see
 *     (no room in the pool) are counted in the pool state and reported by kvz_pool_stats.
 *   - A pool handle is not thread-safe; calls on one pool must be ordered on one stream.
 */
#ifndef KVZ_H
#define KVZ_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVZ_VERSION 1

enum {
  KVZ_OK = 0,
  KVZ_EINVAL = -1,       /* bad argument (null pointer, size out of range, misalignment)       */
  KVZ_EUNSUPPORTED = -2, /* device is not gfx950, or head_dim != 128, page != 16, group > 16   */
  KVZ_EHIP = -4,         /* a HIP runtime call or kernel launch failed                          */
  KVZ_ESTATE = -5        /* the pool state does not carry the expected magic/version            */
};

#define KVZ_PAGE_TOKENS 16
#define KVZ_HEAD_DIM 128
#define KVZ_GRANULE_BYTES 256
#define KVZ_RAW_TAG 0xFFu
#define KVZ_OFF_NONE 0xFFFFFFFFu
#define KVZ_KIND_K 0u
#define KVZ_KIND_V 1u
#define KVZ_ENC_FORCE_RAW 1u    /* kvz_encode_pages flag: store every block raw */
#define KVZ_ENC_SIMULATE_GIVE_UP 2u  /* kvz_encode_pages / kvz_complete_pages flag, for tests of the
                                        failure path: a call that takes the one-pass launch acts
                                        as if one of its waits had given up (see
                                        kvz_encode_pages); ignored by calls above 16384 items */
#define KVZ_PART_ALL 0           /* kvz_*_decode_attention_part: the whole call                */
#define KVZ_PART_LOAD 1          /* only the page loads of the attention kernel                */
#define KVZ_PART_LOAD_RESTORE 2  /* the page loads and the in-register restore                 */
#define KVZ_WS_BAD_COUNTER 1u   /* kvz_attn_workspace_status flag: a merge counter was found at or
                                   above its pair's number of pieces (workspace not zero-filled,
                                   or reused beyond the fixed counter area); the merge of that
                                   (sequence, KV head) in that call is unreliable */

/* 8-byte metadata of one 4-block K or V group ([ZF] metadata paragraph). */
typedef struct {
  uint32_t off;     /* first block, in 256-B granules from the arena base; KVZ_OFF_NONE = not stored */
  uint8_t tag[4];   /* per block: b/2 in 0..127, or KVZ_RAW_TAG                                     */
} kvz_group_meta;

/* One completed page of one (layer, KV head, K|V) to encode. */
typedef struct {
  const uint16_t* src;   /* device: 16 rows of 128 BF16 values, natural order [token][dim]      */
  kvz_group_meta* dst;   /* device: where the group's metadata is written                        */
  uint32_t src_stride;   /* elements between consecutive tokens of src, >= 128, multiple of 8   */
  uint32_t kind;         /* KVZ_KIND_K or KVZ_KIND_V (selects the chunk order)                  */
} kvz_encode_item;

/* One completed page of one (layer, KV head, K|V) to encode in the group-adaptive format
 * (kvz_gaac_encode_pages): the fields of kvz_encode_item plus the tile's calibrated bases. */
typedef struct {
  const uint16_t* src;   /* device: 16 rows of 128 BF16 values, natural order [token][dim]      */
  kvz_group_meta* dst;   /* device: where the tile's metadata is written                         */
  uint32_t src_stride;   /* elements between consecutive tokens of src, >= 128, multiple of 8   */
  uint32_t kind;         /* KVZ_KIND_K or KVZ_KIND_V                                             */
  const uint8_t* bases;  /* device [2][128]: b3 then b4 of this (layer, K|V, KV head), per dim   */
} kvz_gaac_item;

/* One block to decode: block `block` (0..3) of the group described by *meta. */
typedef struct {
  const kvz_group_meta* meta;  /* device */
  uint32_t block;
  uint32_t kind;
} kvz_block_ref;

typedef struct kvz_pool kvz_pool;   /* opaque host handle */

typedef struct {
  uint64_t capacity_granules;  /* usable granules: arena_bytes/256 - 1 (one guard granule)    */
  uint64_t frontier_granules;  /* granules handed out from the frontier so far                 */
  uint64_t free_runs[5];       /* free runs kept per n_raw bin (run = 12 + n_raw granules)     */
  uint64_t live_runs;          /* groups currently stored                                      */
  uint64_t live_granules;
  uint64_t live_raw_blocks;
  uint64_t enospc;             /* groups that found no room (cumulative)                        */
  uint64_t bad_frees;          /* frees dropped because a bin was full (double free)            */
  uint64_t encoder_halted;     /* 1 once a one-pass encode launch gave up a wait (see
                                  kvz_encode_pages); 0 after kvz_pool_init                      */
} kvz_pool_stats_t;

/* Decode-attention arguments, fused compressed path.
 * For every sequence b: tokens 0 .. 16*n_comp_pages[b]-1 are read from compressed groups
 * through block_table and meta; tokens 16*n_comp_pages[b] .. seq_lens[b]-1 (0..16 of them)
 * from the BF16 tail.  All tokens share one softmax ([GAAC] "Attention with On-the-Fly
 * Decompression").  Query head h uses KV head h / (num_q_heads/num_kv_heads).
 * out[b][h][:] = sum_t softmax_t(sm_scale * q[b][h].K[t]) V[t]; a sequence of length 0 gives
 * zeros.  Values of seq_lens/n_comp_pages outside their documented ranges are clamped, and a
 * page whose block-table entry is outside [0, n_phys_pages) or whose groups are not stored or
 * do not lie inside the arena is skipped (the output for such a sequence is then unspecified,
 * but no memory outside the buffers is read).  The kernel may read up to 16 bytes past the end
 * of a group; a pool arena never holds a group in its last 256-byte granule. */
typedef struct {
  const uint16_t* q;            /* device [B][Hq][128] BF16                                      */
  float* out;                   /* device [B][Hq][128] fp32                                      */
  const uint8_t* arena;         /* device: pool arena base                                       */
  uint64_t arena_bytes;
  const kvz_group_meta* meta;   /* device [n_phys_pages][Hkv][2] (K then V) for this layer       */
  int32_t n_phys_pages;
  const int32_t* block_table;   /* device [B][max_pages]: physical page of logical page p        */
  const int32_t* seq_lens;      /* device [B]                                                    */
  const int32_t* n_comp_pages;  /* device [B]: compressed pages, 0 <= n <= max_pages             */
  const uint16_t* tail;         /* device [B][2][Hkv][16][128] BF16, or NULL if no sequence has
                                   tokens past its compressed pages                             */
  int32_t batch, num_q_heads, num_kv_heads, head_dim, page_size, max_pages;
  int32_t splits;               /* split-K: pieces per sequence on average, 0..4096; 0 =
                                   automatic (one piece per CU).  A piece is one workgroup whose
                                   four waves each take a quarter of its pages and merge in LDS.
                                   With S > 1 a piece holds at most ceil(W / (B*S)) pages (W =
                                   the batch's pages), so longer sequences are cut into more
                                   pieces; equal lengths give exactly S pieces each              */
  float sm_scale;
  void* workspace;              /* device, >= kvz_attn_workspace_bytes(...), 256-B aligned; calls
                                   that share a workspace must be ordered on one stream         */
  uint64_t workspace_bytes;
} kvz_attn_args;

/* Uncompressed baseline.  pages: device [n_phys][2][Hkv][4][64 chunks][16 B]: every block in
 * the raw chunk layout above (what kvz_bf16_pack_pages writes).  Other fields as above, with
 * n_comp_pages counting full BF16 pages. */
typedef struct {
  const uint16_t* q;
  float* out;
  const uint8_t* pages;
  int32_t n_phys_pages;         /* pages holds n_phys_pages pages; other block-table entries are
                                   skipped                                                       */
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* n_comp_pages;
  const uint16_t* tail;
  int32_t batch, num_q_heads, num_kv_heads, head_dim, page_size, max_pages;
  int32_t splits;
  float sm_scale;
  void* workspace;
  uint64_t workspace_bytes;
} kvz_bf16_attn_args;

int kvz_version(void);
const char* kvz_last_error(void);

/* KVZ_OK if `device` is a gfx950 GPU, KVZ_EUNSUPPORTED otherwise. */
int kvz_device_check(int device);

/* Bytes of device state a pool over an arena of arena_bytes needs. */
int kvz_pool_state_bytes(uint64_t arena_bytes, uint64_t* state_bytes);

/* Create a pool over d_arena (>= 2 granules, 256-B aligned) with its state in d_state
 * (>= kvz_pool_state_bytes, 256-B aligned).  Resets the state on stream s: every granule
 * free, frontier 0, bins empty, counters 0.  *out receives the host handle. */
int kvz_pool_init(kvz_pool** out, void* d_arena, uint64_t arena_bytes, void* d_state,
                  uint64_t state_bytes, hipStream_t s);

/* Frees the host handle only; the caller frees arena and state. */
int kvz_pool_destroy(kvz_pool* p);

/* Allocate one run per item, in item order ([GAAC] fixed-capacity slots; [ZF] contiguous
 * group blocks).  d_tags: device [n][4] block tags; d_off: device [n] receives the run offset in
 * granules or KVZ_OFF_NONE.  Rule: an item with k raw blocks pops the most recently freed run
 * of its bin k if there is one; otherwise it asks the frontier, and the frontier requests of one
 * call are served as a prefix: a request succeeds iff frontier + (sizes of this call's frontier
 * requests up to and including it) <= capacity.  Deterministic: the same calls give the same
 * offsets. */
int kvz_slot_alloc(kvz_pool* p, const uint8_t* d_tags, uint32_t* d_off, int32_t n, hipStream_t s);

/* Return the runs of n groups to their bins, in item order, and reset each *d_metas[i] to
 * {KVZ_OFF_NONE, {0,0,0,0}} ([ZF] memory manager: space freed by one layer is reused by
 * another).  d_metas: device array of n device pointers.  Groups with off == KVZ_OFF_NONE are
 * skipped. */
int kvz_slot_free(kvz_pool* p, kvz_group_meta* const* d_metas, int32_t n, hipStream_t s);

/* Page-completion encoder ([GAAC] fill-then-finalize; [ZF] steps 1-3): for each item, tag its
 * four blocks, allocate a run (same rule and order as kvz_slot_alloc), write the blocks into
 * the arena and the 8-byte metadata to item.dst.  If the pool has no room, dst->off is
 * KVZ_OFF_NONE and nothing is written: the caller keeps that page in BF16.  flags:
 * KVZ_ENC_FORCE_RAW stores every block raw; KVZ_ENC_SIMULATE_GIVE_UP (tests only, see below).
 * d_items: device [n].
 * A call of up to 16384 items is one launch whose workgroups wait, each for a bounded time
 * (about a second), for counts published by lower-numbered workgroups of the same launch; such
 * waits only run out if a workgroup cannot start while the rest of the launch runs (e.g. the
 * device is preempted).  A launch whose wait runs out stores nothing (every item KVZ_OFF_NONE,
 * counted in enospc; the bins are emptied, their runs lost) and halts the pool's one-pass
 * encoder: from then on every call of up to 16384 items stores nothing, counted in enospc (a
 * kvz_complete_pages call whose frees share the launch does not free them either), until
 * kvz_pool_init; kvz_pool_stats reports encoder_halted.  Larger calls, kvz_slot_alloc and
 * kvz_slot_free are not affected. */
int kvz_encode_pages(kvz_pool* p, const kvz_encode_item* d_items, int32_t n, uint32_t flags,
                     hipStream_t s);

/* A decode step's page work in one launch: exactly kvz_slot_free(p, d_free, n_free) followed by
 * kvz_encode_pages(p, d_items, n, flags) - the same offsets, records, bins and counters - for a
 * step where finished sequences release their groups and completed pages are encoded ([ZF]
 * "How it works", memory-manager paragraph: space freed by one sequence is reused by the next
 * page; [GAAC] "Block-Wise Compression Scheduling": encode once, at completion).  A group may be
 * both freed and re-encoded (its record is read by the free before the encode writes it).
 * d_free: device array of n_free device pointers (may be null when n_free is 0); d_items:
 * device [n].  Errors as for the two calls; nothing is launched on an argument error. */
int kvz_complete_pages(kvz_pool* p, kvz_group_meta* const* d_free, int32_t n_free,
                       const kvz_encode_item* d_items, int32_t n, uint32_t flags, hipStream_t s);

/* Rebuild n blocks to natural order: d_out device [n][16 tokens][32 dims] BF16 ([ZF] step 4).
 * A block of a group that is not stored, or that does not lie inside the arena_bytes of
 * d_arena, decodes to zeros. */
int kvz_decode_block(const void* d_arena, uint64_t arena_bytes, const kvz_block_ref* d_refs,
                     int32_t n, uint16_t* d_out, hipStream_t s);

/* Decompress-first: rebuild every group of n_pages physical pages (d_meta: device
 * [n_pages][Hkv][2] (K then V), as for kvz_decode_attention) into the baseline's page layout,
 * d_dst device [n_pages][2][Hkv][4][64][16 B] (byte-identical to kvz_bf16_pack_pages of the
 * natural pages), for kvz_bf16_decode_attention.  The decompress-then-attend pipeline that
 * fused attention replaces ([GAAC] section "Attention Time Breakdown", Table 5; [ZF] "What it
 * claims").  A group that is not stored, or does not lie inside arena_bytes, becomes zeros.
 * d_meta 8-byte and d_dst 16-byte aligned (KVZ_EINVAL otherwise). */
int kvz_decompress_pages(const void* d_arena, uint64_t arena_bytes, const kvz_group_meta* d_meta,
                         int64_t n_pages, int32_t num_kv_heads, uint8_t* d_dst, hipStream_t s);

/* ---------------------------------------------------------------------------------------------
 * Second format: the group-adaptive additive exponent code ([GAAC] "GAAC: Lossless KV
 * Compression for Bandwidth-Efficient LLM Inference on Personal Devices", section "Lossless KV
 * Compression"; appendix "Storage", Table 9).  A TILE is one page's K or V for one KV head
 * (2048 values); its groups of eight are the chunks above.  Per dim, calibrated bases b3 and b4
 * open windows of 8 and 16 exponents; a group takes the narrowest of: 3-bit offsets e - b3,
 * 4-bit offsets e - b4, raw 8-bit exponents; sign and 7 fraction bits stay as one byte.
 * Compressed record* (<= 3008 B, in a run of 12 granules): sign+fraction plane 2048 B (value i
 * of group (block j, chunk c) at 512j+8c+i), code plane 768 B (lane c's 12 bytes at 2048+12c:
 * block j's 24 low-code bits at +3j, value i at bits 3i..3i+2), mode plane 64 B (byte c: block
 * j's mode at bits 2j..2j+1; 0 = 3-bit, 1 = 4-bit, 2 = raw), then the escape bytes, at most 128
 * (lanes in order, blocks in order; 4-bit group: one byte, bit i = code bit 3 of value i; raw
 * group: five bytes, value i's exponent bits 3..7 at bits 5i..5i+4, little-endian).  A tile
 * whose escapes exceed 128 bytes is stored raw: 4096 B in the raw chunk layout (16 granules).
 * Metadata: kvz_group_meta with tags 00 00 00 00 (compressed) or FF FF FF FF (raw), so the
 * slot pool and the meta tables are shared with the first format.
 * ------------------------------------------------------------------------------------------- */

/* Calibrate one base set ([GAAC] "Lossless KV Compression": per head-channel pair, the
 * contiguous exponent windows of length 8 and 16 that hold the most values; ties go to the
 * smallest base*).  All n items are pages of the same (layer, K|V, KV head); only src and
 * src_stride are read.  d_hist: device [128][256] uint32 scratch (overwritten).  d_bases:
 * device [2][128] uint8 out (b3 then b4). */
int kvz_gaac_calibrate(const kvz_encode_item* d_items, int32_t n, uint32_t* d_hist,
                       uint8_t* d_bases, hipStream_t s);

/* Encode completed pages in the group-adaptive format: classify the groups of each tile, fall
 * back to raw when the escapes exceed 128 bytes (or with KVZ_ENC_FORCE_RAW), allocate a run of
 * 12 or 16 granules (same pool, same rule and order as kvz_slot_alloc), write the record and
 * the metadata.  Each item's dst must be distinct. */
int kvz_gaac_encode_pages(kvz_pool* p, const kvz_gaac_item* d_items, int32_t n, uint32_t flags,
                          hipStream_t s);

/* Decompress-first for the group-adaptive format: like kvz_decompress_pages, with d_bases device
 * [Hkv][2 (K,V)][2 (b3,b4)][128] uint8 for this layer. */
int kvz_gaac_decompress_pages(const void* d_arena, uint64_t arena_bytes,
                              const kvz_group_meta* d_meta, const uint8_t* d_bases,
                              int64_t n_pages, int32_t num_kv_heads, uint8_t* d_dst,
                              hipStream_t s);

/* Fused decode attention over pages in the group-adaptive format: the arguments of
 * kvz_decode_attention (meta: tile metadata written by kvz_gaac_encode_pages), plus d_bases:
 * device [Hkv][2 (K,V)][2 (b3,b4)][128] uint8, 8-byte aligned, the layer's calibrated bases.
 * Tiles are rebuilt bit-exactly in registers (e = code + b_w) and used at once ([GAAC]
 * "Attention with On-the-Fly Decompression").  A page whose tiles carry tags other than
 * 00x4 / FFx4 is skipped.  Same output contract as kvz_decode_attention. */
int kvz_gaac_decode_attention(const kvz_attn_args* a, const uint8_t* d_bases, hipStream_t s);

/* ---------------------------------------------------------------------------------------------
 * Third format: the same exponent code on FP8 KV ([GAAC] appendix "Relation to FP8 KV", Table 7:
 * KV converted to FP8 - E4M3 or E5M2 - compresses further, losslessly, with the code of section
 * "Lossless KV Compression").  FP8 values follow the OCP formats: E4M3 "fn" (bias 7, no
 * infinities, S.1111.111 is NaN) and E5M2 (bias 15, IEEE-style Inf/NaN).  Reading*: sign and
 * fraction are kept (4 bits in E4M3, 3 in E5M2); the exponent field (4 or 5 bits) takes the group
 * modes of the second format - 3-bit offsets from b3, 4-bit offsets from b4, raw - with windows
 * calibrated inside the field; a raw group's escape holds the exponent bits above the low three
 * (1 byte in E4M3, 2 in E5M2: value i's bits at 2i..2i+1).  All-3-bit tiles are 7.25 / 6.25
 * bits per value.
 * Uncompressed FP8 tile* (2048 B, "FP8 chunk layout"): chunk c of block j (the MFMA operand
 * chunks above, 8 values) at byte 1024*(j/2) + 16c + 8*(j%2).
 * Compressed record*: sign+fraction plane (E4M3: 1024 B, lane c's 16 bytes at 16c, word j =
 * X | rotl32(Y, 4); E5M2: 768 B, lane c's 12 bytes at 12c, words t = 0..2 = X | rotl32(Y, 3)
 * of block t and block 3 in bits 5..6 of every byte: word 0 = fraction of values 0..3, word 1
 * of values 4..7, word 2 bit 5 / bit 6 = sign of value k / k+4; X / Y = the bytes s<<7 | fraction
 * of values 0..3 / 4..7), code plane (768 B as in the second format), mode plane (64 B), then
 * at most 64 escape bytes.  A compressed record takes 1920 B (E4M3) / 1664 B (E5M2), i.e. 15 /
 * 13 granules of 128 bytes; a tile whose escapes exceed 64 bytes is stored uncompressed (2048 B,
 * 16 granules).  FP8 tiles live in a pool made by kvz_fp8_pool_init, whose granule is 128 bytes;
 * the tile's tags give the pool its run class as in the first format (12 + number of 0xFF tag
 * bytes granules): FF FF FF 00 (compressed E4M3), FF 00 00 00 (compressed E5M2), FF FF FF FF
 * (uncompressed).  Metadata offsets count 128-byte granules.
 * ------------------------------------------------------------------------------------------- */
#define KVZ_FP8_E4M3 0u
#define KVZ_FP8_E5M2 1u
#define KVZ_FP8_GRANULE_BYTES 128

/* One completed FP8 page of one (layer, KV head, K|V). */
typedef struct {
  const uint8_t* src;    /* device: 16 rows of 128 FP8 values, natural order [token][dim]       */
  kvz_group_meta* dst;   /* device: where the tile's metadata is written                          */
  uint32_t src_stride;   /* bytes between consecutive tokens of src, >= 128, multiple of 8       */
  uint32_t kind;         /* KVZ_KIND_K or KVZ_KIND_V                                              */
  const uint8_t* bases;  /* device [2][128]: b3 then b4 of this (layer, K|V, KV head), per dim    */
} kvz_fp8_item;

/* Attention over FP8 KV.  Scores use the K values times k_scale, the output the V values times
 * v_scale (a per-layer dequantization scale each).  Fused path (kvz_fp8_decode_attention):
 * arena/arena_bytes/meta/bases as for the second format (meta offsets in 128-byte granules;
 * bases device [Hkv][2 (K,V)][2 (b3,b4)][128], 8-byte aligned); uncompressed path
 * (kvz_fp8_raw_decode_attention): pages device [n_phys][2][Hkv][2048] in the FP8 chunk layout
 * (kvz_fp8_pack_pages).  tail: device [B][2][Hkv][16][128] FP8 or NULL.  Other fields and the
 * output contract as for kvz_decode_attention. */
typedef struct {
  const uint16_t* q;            /* device [B][Hq][128] BF16                                      */
  float* out;                   /* device [B][Hq][128] fp32                                      */
  const uint8_t* arena;         /* fused: FP8 pool arena                                         */
  uint64_t arena_bytes;
  const kvz_group_meta* meta;   /* fused: [n_phys_pages][Hkv][2]                                 */
  const uint8_t* bases;         /* fused: [Hkv][2][2][128]                                       */
  const uint8_t* pages;         /* uncompressed: [n_phys_pages][2][Hkv][2048]                    */
  int32_t n_phys_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* n_comp_pages;
  const uint8_t* tail;
  int32_t batch, num_q_heads, num_kv_heads, head_dim, page_size, max_pages, splits;
  uint32_t format;              /* KVZ_FP8_E4M3 or KVZ_FP8_E5M2                                  */
  float sm_scale, k_scale, v_scale;
  void* workspace;              /* >= kvz_attn_workspace_bytes(...), 256-B aligned               */
  uint64_t workspace_bytes;
} kvz_fp8_attn_args;

/* Bytes of device state, and pool creation, for a pool of FP8 tiles: kvz_pool_state_bytes /
 * kvz_pool_init with 128-byte granules (capacity arena_bytes/128 - 1 granules, one guard
 * granule).  kvz_slot_alloc/free, kvz_pool_stats and kvz_pool_capacity work on it unchanged
 * (in its granules); only kvz_fp8_encode_pages writes tiles into it. */
int kvz_fp8_pool_state_bytes(uint64_t arena_bytes, uint64_t* state_bytes);
int kvz_fp8_pool_init(kvz_pool** out, void* d_arena, uint64_t arena_bytes, void* d_state,
                      uint64_t state_bytes, hipStream_t s);

/* Calibrate one base set of FP8 pages ([GAAC] "Lossless KV Compression": per dim, the windows
 * of 8 and 16 exponents holding the most values, inside [0, 15] (E4M3) or [0, 31] (E5M2); ties
 * to the smallest base).  Only src and src_stride of the n items are read.  d_hist: device
 * [128][32] uint32 scratch (overwritten).  d_bases: device [2][128] uint8 out (b3 then b4). */
int kvz_fp8_calibrate(const kvz_fp8_item* d_items, int32_t n, uint32_t format, uint32_t* d_hist,
                      uint8_t* d_bases, hipStream_t s);

/* Encode completed FP8 pages: classify the groups of each tile, keep it uncompressed when its
 * escapes exceed 64 bytes (or with KVZ_ENC_FORCE_RAW), allocate its run from an FP8 pool (same
 * rule and order as kvz_slot_alloc), write the record and the metadata.  KVZ_EINVAL if the pool
 * was not made by kvz_fp8_pool_init.  Each item's dst must be distinct. */
int kvz_fp8_encode_pages(kvz_pool* p, const kvz_fp8_item* d_items, int32_t n, uint32_t format,
                         uint32_t flags, hipStream_t s);

/* Decompress-first for FP8 tiles: rebuild every tile of n_pages physical pages (d_meta device
 * [n_pages][Hkv][2]) into the uncompressed FP8 pages d_dst [n_pages][2][Hkv][2048] (the FP8
 * chunk layout; byte-identical to kvz_fp8_pack_pages of the natural pages).  A tile that is not
 * stored, carries other tags or does not lie inside arena_bytes becomes zeros. */
int kvz_fp8_decompress_pages(const void* d_arena, uint64_t arena_bytes,
                             const kvz_group_meta* d_meta, const uint8_t* d_bases,
                             int64_t n_pages, int32_t num_kv_heads, uint32_t format,
                             uint8_t* d_dst, hipStream_t s);

/* Lay out natural FP8 pages (device [n_pages][2][Hkv][16][128]) in the FP8 chunk layout
 * (device [n_pages][2][Hkv][2048]): the uncompressed FP8 cache of kvz_fp8_raw_decode_attention. */
int kvz_fp8_pack_pages(const uint8_t* d_src, uint8_t* d_dst, int64_t n_pages,
                       int32_t num_kv_heads, hipStream_t s);

/* Fused decode attention over FP8 tiles: records are rebuilt bit-exactly in registers and the
 * FP8 values converted exactly to BF16 for the MFMA products ([GAAC] "Attention with On-the-Fly
 * Decompression").  A page whose tiles carry other tags is skipped. */
int kvz_fp8_decode_attention(const kvz_fp8_attn_args* a, hipStream_t s);

/* The same attention over uncompressed FP8 pages (the FP8 baseline). */
int kvz_fp8_raw_decode_attention(const kvz_fp8_attn_args* a, hipStream_t s);

/* Workspace bytes the attention calls (kvz_decode_attention, kvz_bf16_decode_attention,
 * kvz_gaac_decode_attention, kvz_fp8_decode_attention, kvz_fp8_raw_decode_attention) need for
 * these sizes.  splits = 0: enough for the automatic split count of every one of them (the
 * coded tiles - group-adaptive and FP8 - use twice as many splits).
 * The workspace must be zero-filled once, before its first call.  Layout: a 256-byte status
 * area (word 0: sticky KVZ_WS_* flags, see kvz_attn_workspace_status), then the per-(sequence,
 * KV head) counters of the merge inside the attention kernel in an area of
 * max(64 KiB, align256(4 * batch * num_kv_heads)) bytes, then the partial results.  Every
 * completed call leaves the counters at zero.  Up to batch * num_kv_heads = 16384 the counter
 * area is the same for every size, so one workspace can be reused across sizes without a new
 * fill; beyond that, zero-fill it again before reusing it for a larger batch * num_kv_heads (its
 * counters would reach into bytes that held partial results - a call that finds such a count
 * sets KVZ_WS_BAD_COUNTER). */
int kvz_attn_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t max_pages, int32_t splits, uint64_t* bytes);

/* Fused paged split-K GQA decode attention over compressed pages plus the BF16 tail: blocks
 * are restored bit-exactly in registers, never written back.  A sequence's only piece writes
 * out directly; with up to 4 splits the last piece of each (sequence, KV head) to finish merges
 * the pieces' partial softmax states inside the attention kernel; with more, a second small
 * kernel merges them. */
int kvz_decode_attention(const kvz_attn_args* a, hipStream_t s);

/* Measurement entry points for the attention time breakdown ([GAAC] "Attention Time
 * Breakdown", Table 5: KV loading, exponent decoding and computation timed apart): the same
 * arguments and launch as kvz_decode_attention / kvz_bf16_decode_attention, but part selects a
 * compile-time variant of the attention kernel.  KVZ_PART_ALL is the full call (identical to
 * the plain entry point).  KVZ_PART_LOAD issues exactly the page loads and waits of the full
 * kernel and nothing else (no restore, no products, no softmax, no tail page, no merge);
 * KVZ_PART_LOAD_RESTORE adds the in-register restore of every K and V block (the BF16 kernel
 * has no restore, so it takes KVZ_PART_ALL and KVZ_PART_LOAD only).  The variants compute
 * nothing useful: out and the workspace are left as they are.  They exist for groups of up to 4
 * query heads per KV head (KVZ_EUNSUPPORTED beyond); KVZ_EINVAL for another part. */
int kvz_decode_attention_part(const kvz_attn_args* a, int32_t part, hipStream_t s);
int kvz_bf16_decode_attention_part(const kvz_bf16_attn_args* a, int32_t part, hipStream_t s);

/* Allocation-free variant of kvz_decode_attention, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and result, with the split-K partial results and merge counters in a
 * device-resident scratch array of the library (16 MiB per GPU, held while the library is
 * loaded) instead of a workspace.  a->workspace and a->workspace_bytes are ignored; every other
 * argument is as for kvz_decode_attention.  The first call on a device looks up the array's
 * device address (hipGetSymbolAddress) and zero-fills its status and counter areas on stream
 * s; nothing is allocated, by this or any later call.  Limits (KVZ_EINVAL beyond them, nothing
 * launched): batch * num_kv_heads <= 16384, and batch * num_kv_heads * splits * (num_q_heads /
 * num_kv_heads) * 520 bytes of partial results (rounded up to 256-byte parts) <= 16 MiB - 64 KiB
 * - 256 B, with splits the automatic count when 0.  All calls on one GPU share its array: calls that
 * overlap in time on one GPU (other streams, other threads) race and give undefined results;
 * order them on one stream.  Each completed call leaves the counters at zero. */
int kvz_decode_attention_noalloc(const kvz_attn_args* a, hipStream_t s);

/* The sticky status flags (KVZ_WS_*) of an attention workspace (device, 256-B aligned), or with
 * d_workspace NULL of kvz_decode_attention_noalloc's scratch on the current device: synchronizes
 * stream s, then copies the status word into *flags (0 when every call so far found its merge
 * counters consistent).  The flags stay set until the caller zero-fills the workspace again
 * (the scratch of the allocation-free call is never refilled: a set flag there means a call
 * was abandoned or overlapped another).  KVZ_EINVAL for a null flags pointer. */
int kvz_attn_workspace_status(const void* d_workspace, uint32_t* flags, hipStream_t s);

/* Lay out n_pages natural BF16 pages (device [n_pages][2][Hkv][16][128]) as the baseline's
 * pages (device [n_pages][2][Hkv][4][64][16 B], the raw chunk layout). */
int kvz_bf16_pack_pages(const uint16_t* d_src, uint8_t* d_dst, int64_t n_pages,
                        int32_t num_kv_heads, hipStream_t s);

/* Uncompressed baseline: the same attention over BF16 pages laid out by kvz_bf16_pack_pages -
 * the uncompressed paged decode attention that both pages measure the fused kernel against
 * ([GAAC] "Long-Context Attention Acceleration" and appendix "Attention Baseline Selection":
 * paged attention over uncompressed BF16 KV in the same process; [ZF] "Evidence"). */
int kvz_bf16_decode_attention(const kvz_bf16_attn_args* a, hipStream_t s);

/* Copy the pool counters (capacity, frontier, free runs per size bin, live groups, granules and
 * raw blocks, failed allocations and dropped frees) to *host_out; synchronizes stream s.  The memory-usage report of the slot pool
 * ([ZF] "How it works", memory-manager paragraph: compressed and raw pages in one managed
 * pool; [GAAC] "Block-Wise Compression Scheduling": two storage classes whose occupancy the
 * serving layer tracks). */
int kvz_pool_stats(kvz_pool* p, kvz_pool_stats_t* host_out, hipStream_t s);

/* Capacity left for KV writes, for a scheduler's admission decision ([ZF] "How it works": the
 * memory manager tracks the space left as pages compress and reports it to the scheduler,
 * which admits requests while reserving room for running generation).  Host arithmetic on a
 * kvz_pool_stats result; no device call.  A page here is one 16-token page of every layer:
 * 2 * num_kv_heads * num_layers groups.
 *   guaranteed_*: what fits whatever the blocks' classes: a group never takes more than 16
 *     granules from the frontier, and only a free run of its own n_raw can be reused, so
 *     floor(unused frontier / 16) + min over bins of the free runs groups always fit.
 *   expected_*: an estimate - all free granules divided by the mean run size of the live
 *     groups (12 + 4 * live raw-block fraction; 16 with nothing live).
 * KVZ_EINVAL for null pointers or num_layers / num_kv_heads <= 0. */
typedef struct {
  uint64_t free_granules;            /* unused frontier + every free run's granules             */
  uint64_t guaranteed_groups;
  uint64_t guaranteed_pages;
  uint64_t guaranteed_tokens;        /* 16 * guaranteed_pages                                    */
  double expected_group_granules;
  uint64_t expected_pages;
  uint64_t expected_tokens;          /* 16 * expected_pages                                      */
} kvz_capacity_t;

int kvz_pool_capacity(const kvz_pool_stats_t* stats, int32_t num_layers, int32_t num_kv_heads,
                      kvz_capacity_t* out);

/* Measurement reference, not part of the path: read `bytes` of device memory d_buf once
 * (16-byte non-temporal loads, the page loads' cache policy) with `workgroups` workgroups of
 * 256 threads (0: four per compute unit).  d_sink: device, 4 bytes, written only when the
 * XOR of everything read equals a fixed key (it exists so the loads cannot be removed).
 * d_buf and bytes must be multiples of 16 (KVZ_EINVAL otherwise). */
int kvz_stream_read(const void* d_buf, uint64_t bytes, uint32_t* d_sink, int32_t workgroups,
                    hipStream_t s);

#ifdef __cplusplus
}
#endif

#endif /* KVZ_H */
