// Page-completion encoder, block decoder and the baseline's BF16 page layout.
//
// Follows "ZipFusion: Fusing Lossless KV Decompression with Attention for Efficient LLM
// Decoding", section "How it works": four 512-value blocks per K or V page (step 1), base b =
// minimum exponent rounded down to even and the [b, b+15] eligibility test (step 2), low byte
// plus a 4-bit sign/offset code (step 3), exact integer restore (step 4), K/V chunk orders that
// put each lane's eight MFMA values together, and 8-byte group metadata.  The encoder runs at
// page completion, once per page ("GAAC: ...", section "Block-Wise Compression Scheduling").
//
// kvz_decompress_pages rebuilds whole pages into the uncompressed layout: the decompress-first
// pipeline that the fused attention is compared against ("GAAC: ...", section "Attention Time
// Breakdown", Table 5, the decompress-first column).
//
// kvz_encode_pages = classify (one wave per item) -> allocate (pool.hip, one workgroup, item
// order) -> pack (one wave per item).  The item's metadata slot carries the tags from classify
// to allocate and the offset from allocate to pack, so the encoder needs no scratch memory.
#include "encode_internal.h"

namespace kvz {

int launch_alloc_for_items(kvz_pool* p, const kvz_encode_item* d_items, int n, hipStream_t s);

namespace {

__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, d, 64));
  return v;
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, d, 64));
  return v;
}

__device__ __forceinline__ uint32_t exp_of(uint32_t w) { return (w >> 7) & 0xFFu; }

__device__ __forceinline__ void chunk_exp_range(uint4 w, uint32_t& lo, uint32_t& hi) {
  const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t e0 = exp_of(d[m] & 0xFFFFu), e1 = exp_of(d[m] >> 16);
    lo = min(lo, min(e0, e1));
    hi = max(hi, max(e0, e1));
  }
}

// Step 2: tags of the four blocks of each item (b/2, or 0xFF when out of window).
template <int kPolicy>
__global__ __launch_bounds__(256) void classify_kernel(const kvz_encode_item* items, int n,
                                                       uint32_t flags) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= n) return;
  const kvz_encode_item it = items[item];
  const bool aligned = item_aligned(it.src, it.src_stride);
  uint32_t tags = 0;
  auto tag_of = [&](uint32_t lo, uint32_t hi) {
    const uint32_t b = lo & 0xFEu;
    return (hi <= b + 15u && !(flags & KVZ_ENC_FORCE_RAW)) ? (b >> 1) : KVZ_RAW_TAG;
  };
  if (aligned) {
    // Only membership matters here, so read the page row by row: load k of lane l is the 16
    // bytes of row l/16 + 4k at dims 8(l%16)..+7, always in block (l%16)/4; each load covers
    // 1 KB of whole rows.  The 16 lanes of a block differ in lane bits 0, 1, 4 and 5.
    const uint32_t row_bytes = uniform_row_bytes(it.src_stride);
    const __amdgpu_buffer_rsrc_t r = page_rsrc(it.src, row_bytes);
    const int voff = (int)((uint32_t)(lane >> 4) * row_bytes + 16u * (uint32_t)(lane & 15));
    uint32_t lo = 255u, hi = 0u;
    i32x4 w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = __builtin_amdgcn_raw_buffer_load_b128(r, voff, (int)(4u * (uint32_t)k * row_bytes),
                                                   kPolicy);
#pragma unroll
    for (int k = 0; k < 4; ++k) chunk_exp_range(__builtin_bit_cast(uint4, w[k]), lo, hi);
#pragma unroll
    for (int d = 1; d <= 32; d <<= 1) {
      if (d == 4 || d == 8) continue;
      lo = min(lo, (uint32_t)__shfl_xor((int)lo, d, 64));
      hi = max(hi, (uint32_t)__shfl_xor((int)hi, d, 64));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)   // block j's range sits in lane 4j (and its partners)
      tags |= tag_of((uint32_t)__builtin_amdgcn_readlane((int)lo, 4 * j),
                     (uint32_t)__builtin_amdgcn_readlane((int)hi, 4 * j)) << (8 * j);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 w = load_chunk(it.src, it.src_stride, KVZ_KIND_K, j, lane, false);
      uint32_t lo = 255u, hi = 0u;
      chunk_exp_range(w, lo, hi);
      tags |= tag_of(wave_min(lo), wave_max(hi)) << (8 * j);
    }
  }
  if (lane == 0) {
    *reinterpret_cast<uint32_t*>(it.dst->tag) = tags;
    it.dst->off = KVZ_OFF_NONE;
  }
}

// Step 3: write the four blocks of each placed item at off*256 + prefix sizes.
template <int kPolicy>
__global__ __launch_bounds__(256) void pack_kernel(const kvz_encode_item* items, int n,
                                                   uint8_t* arena, uint64_t capacity) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= n) return;
  const kvz_encode_item it = items[item];
  // Every load of the item (its metadata, then its source) is issued before the first store:
  // a store into the arena may alias the source as far as the compiler knows, so a load left
  // after one waits for it.
  const uint64_t mt = load_meta_record(it.dst);
  const uint32_t off = (uint32_t)mt;
  const uint32_t tags = (uint32_t)(mt >> 32);
  uint4 w[4];
  load_item_chunks<kPolicy>(it.src, it.src_stride, it.kind, lane, w);
  // an offset only comes from the allocator; the run must still lie inside the pool
  if (off == KVZ_OFF_NONE || (uint64_t)off + run_granules(n_raw_of(tags)) > capacity) return;
  uint8_t* blk = arena + (size_t)off * KVZ_GRANULE_BYTES;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t tag = (tags >> (8 * j)) & 0xFFu;
    if (tag == KVZ_RAW_TAG) {
      *reinterpret_cast<uint4*>(blk + kRawChunkBytes * lane) = w[j];
    } else {
      const uint3 c = compress_chunk(w[j], tag * 0x01010101u);
      uint32_t* d = reinterpret_cast<uint32_t*>(blk + kCompChunkBytes * lane);
      d[0] = c.x;
      d[1] = c.y;
      d[2] = c.z;
    }
    blk += block_bytes(tag);
  }
}

// Step 4: natural-order BF16 [16 tokens][32 dims] of each referenced block.
__global__ __launch_bounds__(256) void decode_block_kernel(const uint8_t* arena,
                                                           uint64_t arena_bytes,
                                                           const kvz_block_ref* refs, int n,
                                                           uint16_t* out) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n) return;
  const kvz_block_ref ref = refs[r];
  const uint32_t off = ref.meta->off;
  const uint32_t tags = *reinterpret_cast<const uint32_t*>(ref.meta->tag);
  uint16_t* o = out + (size_t)r * 512;
  uint64_t start = (uint64_t)off * KVZ_GRANULE_BYTES;
  if (ref.block <= 3)
    for (uint32_t k = 0; k < ref.block; ++k) start += block_bytes((tags >> (8 * k)) & 0xFFu);
  const uint32_t tag = ref.block <= 3 ? (tags >> (8 * ref.block)) & 0xFFu : 0u;
  if (off == KVZ_OFF_NONE || ref.block > 3 || start + block_bytes(tag) > arena_bytes) {
    for (int t = lane; t < 512; t += 64) o[t] = 0;
    return;
  }
  const uint8_t* blk = arena + start;
  uint4 w;
  if (tag == KVZ_RAW_TAG) {
    w = *reinterpret_cast<const uint4*>(blk + kRawChunkBytes * lane);
  } else {
    const uint32_t* s = reinterpret_cast<const uint32_t*>(blk + kCompChunkBytes * lane);
    w = restore_chunk(s[0], s[1], s[2], tag * 0x01010101u);
  }
  const uint32_t d[4] = {w.x, w.y, w.z, w.w};
  if (ref.kind == KVZ_KIND_K) {
    // token lane%16, dims 8*(lane/16)+i: one 16-byte row piece
    *reinterpret_cast<uint4*>(o + (lane & 15) * 32 + 8 * (lane >> 4)) = w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint16_t v = (uint16_t)((d[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
      o[(8 * (lane >> 5) + i) * 32 + (lane & 31)] = v;
    }
  }
}

// Baseline page layout: every block as 64 raw chunks in the same chunk order.
__global__ __launch_bounds__(256) void bf16_pack_kernel(const uint16_t* src, uint8_t* dst,
                                                        int64_t n_groups, int hkv) {
  const int lane = threadIdx.x & 63;
  const int64_t gb = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (group, block)
  if (gb >= n_groups * 4) return;
  const int64_t g = gb >> 2;
  const int j = (int)(gb & 3);
  const uint32_t kind = (uint32_t)((g / hkv) & 1);   // groups are [page][K|V][kv head]
  const uint16_t* s = src + g * 2048;
  const uint4 w = load_chunk(s, 128, kind, j, lane, true);
  *reinterpret_cast<uint4*>(dst + g * 4096 + j * 1024 + kRawChunkBytes * lane) = w;
}

// Decompress-first: every group of a page table rebuilt into the baseline's page layout
// [page][K|V][kv head][4 blocks][64 chunks][16 B].  One wave per group; each lane loads its
// chunk of the four blocks (16 bytes through a buffer resource sized to the group, so the
// 12-byte compressed chunks need no tail handling) and writes 4 x 16 bytes.
__global__ __launch_bounds__(256) void decompress_pages_kernel(const uint8_t* arena,
                                                               uint64_t arena_bytes,
                                                               const kvz_group_meta* meta,
                                                               int64_t n_groups, int hkv,
                                                               uint8_t* dst) {
  const int lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // output group index
  if (g >= n_groups) return;
  const int64_t page = g / (2 * hkv);
  const int rem = (int)(g % (2 * hkv));
  const int kind = rem / hkv, kvh = rem % hkv;
  const kvz_group_meta m = meta[(page * hkv + kvh) * 2 + kind];
  const uint32_t tags = *reinterpret_cast<const uint32_t*>(m.tag);
  uint32_t bytes = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) bytes += block_bytes((tags >> (8 * j)) & 0xFFu);
  const uint64_t start = (uint64_t)m.off * KVZ_GRANULE_BYTES;
  uint4* out = reinterpret_cast<uint4*>(dst + g * 4096 + kRawChunkBytes * lane);
  if (m.off == KVZ_OFF_NONE || start + bytes > arena_bytes) {
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j * 64] = make_uint4(0, 0, 0, 0);
    return;
  }
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(arena + start), 0, (int)bytes, 0x00020000);
  uint4 c[4];
  uint32_t so = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool raw = ((tags >> (8 * j)) & 0xFFu) == KVZ_RAW_TAG;
    c[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                         r, (int)(raw ? kRawChunkBytes * lane : kCompChunkBytes * lane),
                                         (int)so, 2));
    so += raw ? kRawBlockBytes : kCompBlockBytes;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t tag = (tags >> (8 * j)) & 0xFFu;
    out[j * 64] = tag == KVZ_RAW_TAG ? c[j] : restore_chunk(c[j].x, c[j].y, c[j].z, tag * 0x01010101u);
  }
}

}  // namespace
}  // namespace kvz

using namespace kvz;

extern "C" int kvz_encode_pages(kvz_pool* p, const kvz_encode_item* d_items, int32_t n,
                                uint32_t flags, hipStream_t s) {
  if (!p) return set_error(KVZ_EINVAL, "pool handle is null");
  if (p->granule_bytes != KVZ_GRANULE_BYTES)
    return set_error(KVZ_EINVAL, "pool was made for FP8 tiles (kvz_fp8_pool_init)");
  if (n < 0) return set_error(KVZ_EINVAL, "n < 0");
  if (n == 0) return KVZ_OK;
  if (!d_items) return set_error(KVZ_EINVAL, "items pointer is null");
  if (flags & ~KVZ_ENC_FORCE_RAW) return set_error(KVZ_EINVAL, "unknown encode flag");
  const int grid = (n + 3) / 4;
  const bool stream = n > kStreamItems;
  if (stream)
    hipLaunchKernelGGL(classify_kernel<kStreamLoad>, dim3(grid), dim3(256), 0, s, d_items, (int)n, flags);
  else
    hipLaunchKernelGGL(classify_kernel<kCachedLoad>, dim3(grid), dim3(256), 0, s, d_items, (int)n, flags);
  int rc = check_hip(hipGetLastError(), "classify launch");
  if (rc != KVZ_OK) return rc;
  rc = launch_alloc_for_items(p, d_items, n, s);
  if (rc != KVZ_OK) return rc;
  if (stream)
    hipLaunchKernelGGL(pack_kernel<kStreamLoad>, dim3(grid), dim3(256), 0, s, d_items, (int)n,
                       (uint8_t*)p->arena, p->capacity);
  else
    hipLaunchKernelGGL(pack_kernel<kCachedLoad>, dim3(grid), dim3(256), 0, s, d_items, (int)n,
                       (uint8_t*)p->arena, p->capacity);
  return check_hip(hipGetLastError(), "pack launch");
}

extern "C" int kvz_decode_block(const void* d_arena, uint64_t arena_bytes,
                                const kvz_block_ref* d_refs, int32_t n, uint16_t* d_out,
                                hipStream_t s) {
  if (n < 0) return set_error(KVZ_EINVAL, "n < 0");
  if (n == 0) return KVZ_OK;
  if (!d_arena || !d_refs || !d_out) return set_error(KVZ_EINVAL, "null pointer argument");
  if (((uintptr_t)d_out) & 15u) return set_error(KVZ_EINVAL, "out must be 16-byte aligned");
  hipLaunchKernelGGL(decode_block_kernel, dim3((n + 3) / 4), dim3(256), 0, s,
                     (const uint8_t*)d_arena, arena_bytes, d_refs, (int)n, d_out);
  return check_hip(hipGetLastError(), "decode_block launch");
}

extern "C" int kvz_bf16_pack_pages(const uint16_t* d_src, uint8_t* d_dst, int64_t n_pages,
                                   int32_t num_kv_heads, hipStream_t s) {
  if (n_pages < 0 || num_kv_heads <= 0) return set_error(KVZ_EINVAL, "bad sizes");
  if (n_pages == 0) return KVZ_OK;
  if (!d_src || !d_dst) return set_error(KVZ_EINVAL, "null pointer argument");
  if ((((uintptr_t)d_src) | ((uintptr_t)d_dst)) & 15u)
    return set_error(KVZ_EINVAL, "src and dst must be 16-byte aligned");
  const int64_t n_groups = n_pages * 2 * num_kv_heads;
  const int64_t grid = n_groups;   // 4 (group, block) pairs per workgroup
  if (grid > 0x7FFFFFFF) return set_error(KVZ_EINVAL, "too many pages for one call");
  hipLaunchKernelGGL(bf16_pack_kernel, dim3((unsigned)grid), dim3(256), 0, s, d_src, d_dst,
                     n_groups, (int)num_kv_heads);
  return check_hip(hipGetLastError(), "bf16 pack launch");
}

extern "C" int kvz_decompress_pages(const void* d_arena, uint64_t arena_bytes,
                                    const kvz_group_meta* d_meta, int64_t n_pages,
                                    int32_t num_kv_heads, uint8_t* d_dst, hipStream_t s) {
  if (n_pages < 0 || num_kv_heads <= 0) return set_error(KVZ_EINVAL, "bad sizes");
  if (n_pages == 0) return KVZ_OK;
  if (!d_arena || !d_meta || !d_dst) return set_error(KVZ_EINVAL, "null pointer argument");
  if ((((uintptr_t)d_meta) & 7u) || (((uintptr_t)d_dst) & 15u))
    return set_error(KVZ_EINVAL, "meta must be 8-byte and dst 16-byte aligned");
  const int64_t n_groups = n_pages * 2 * num_kv_heads;
  const int64_t grid = (n_groups + 3) / 4;
  if (grid > 0x7FFFFFFF) return set_error(KVZ_EINVAL, "too many pages for one call");
  hipLaunchKernelGGL(decompress_pages_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                     (const uint8_t*)d_arena, arena_bytes, d_meta, n_groups, (int)num_kv_heads, d_dst);
  return check_hip(hipGetLastError(), "decompress launch");
}
