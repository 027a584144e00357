// The page-completion encoders' shared parts (codec.hip, gaac.hip, fp8.hip; the scratch layout
// also for pool.hip): the one-pass encoder's scratch in the pool state, and the source loads,
// one item (one K or V page of one KV head, 16 rows of 128 values) per wave.
#pragma once

#include "kvz_internal.h"

namespace kvz {

// The one-pass page-completion encoder's scratch in the pool state: a 256-byte control area
// (word 0: launches numbered so far, which numbers the next launch's records; word 1: the halt
// flag), then the records of a launch:
//  * one 128-byte slot per free tile: its counts of freed runs per size class in one 64-bit
//    word (a 14-bit form of the epoch, 1..16383, in the top bits, then five 10-bit counts), and
//    status = epoch << 2 | state (3: its bin stores and clears complete, 2: it could not free);
//    slot 0 also holds the bin counts and frontier the launch started from, with their own
//    status word (the epoch once they are out), written by tile 0 whether it frees or encodes.
//    A launch zeroes the count words of the slots it does not use, so a slot's word is always
//    the previous launch's or zero;
//  * one 64-bit word per encode tile: epoch << 32 | its item counts per size class, 6 bits each,
//    stored kRecordCopies times (arrays of kMaxEncodeTiles words, one after the other): every
//    tile polls the records of all others, and workgroup b reading copy b % kRecordCopies
//    spreads those polls over more memory channels (one copy: 13.8 vs 13.0 us per online step).
// A record of another launch has another epoch.
struct EncodeSlot {
  uint64_t aggw;
  uint32_t status;
  uint32_t sstat;
  uint32_t snap[kBins];
  uint32_t f0_lo, f0_hi;
  uint32_t pad[21];
};
static_assert(sizeof(EncodeSlot) == 128, "one record per 128 bytes");
constexpr int kMaxFreeSlots = 256;        // free tiles per launch (one waiting thread each)
constexpr int kMaxEncodeTiles = 4096;     // encode tiles per launch
constexpr int kRecordCopies = 8;
constexpr uint64_t kEncodeCtlBytes = 256;
constexpr uint64_t kEncodeScratchBytes = kEncodeCtlBytes + (uint64_t)kMaxFreeSlots * sizeof(EncodeSlot) +
                                         (uint64_t)kRecordCopies * kMaxEncodeTiles * sizeof(uint64_t);

// Cache policy of the source loads.  A bulk call (prefill: every page of a layer, far more than
// the caches hold) loads non-temporally (bit "nt"): each page is read once by the classify pass
// and once by the pack pass (exponent-coded pages of an 8K layer, 130,816 groups: 286 us vs 333
// us with cached loads).  A decode step's completion (recently written tail pages, often still
// in the last-level cache) keeps cached loads (9,216 groups: 65.3 us vs 69.2 us non-temporal).
// Calls above this many items stream.
constexpr int kStreamItems = 32768;   // 128 MiB of BF16 source
constexpr int kCachedLoad = 0;
constexpr int kStreamLoad = 2;

typedef int i32x4 __attribute__((ext_vector_type(4)));

// The item's source pointer and row stride are wave-uniform.  A buffer resource over its 16
// rows keeps them in SGPRs: the pointer read from the item is generic, and flat loads of it
// were issued a round trip apart (a flat load may alias the arena stores and waits on both
// counters).
__device__ __forceinline__ uint32_t uniform_row_bytes(uint32_t src_stride) {
  return 2u * (uint32_t)__builtin_amdgcn_readfirstlane((int)src_stride);
}
// (value_bytes: 2 for BF16 pages, 1 for FP8 pages; a row holds 128 values)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const void* src, uint32_t row_bytes,
                                                            uint32_t value_bytes = 2) {
  const uint64_t u = (uint64_t)(uintptr_t)src;
  const uint64_t su = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(u >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((uintptr_t)su), 0,
                                           (int)(15u * row_bytes + value_bytes * KVZ_HEAD_DIM),
                                           0x00020000);
}

// The buffer path addresses the 16 rows with 32-bit offsets (the resource size is a signed 32-bit
// count): rows farther apart than this take the element-wise path.
constexpr uint32_t kMaxBufferRowBytes = (0x7FFFFFFFu - 256u) / 15u;

__device__ __forceinline__ bool item_aligned(const uint16_t* src, uint32_t stride) {
  return ((((uintptr_t)src) & 15u) == 0) && ((stride & 7u) == 0) &&
         2ull * stride <= kMaxBufferRowBytes;
}

// The four chunks (blocks 0..3) of the item in lane order, as load_chunk gives them, with every
// load issued before any is used.  K chunk j of lane c: token c%16, dims 32j + 8(c/16)..+7 (16
// contiguous bytes); V: dim 32j + c%32 of tokens 8(c/32)..+7 (one value per row).
template <int kPolicy>
__device__ __forceinline__ void load_item_chunks(const uint16_t* src, uint32_t stride, uint32_t kind,
                                                 int lane, uint4 (&w)[4]) {
  if (item_aligned(src, stride)) {
    const uint32_t row_bytes = uniform_row_bytes(stride);
    const __amdgpu_buffer_rsrc_t r = page_rsrc(src, row_bytes);
    if (__builtin_amdgcn_readfirstlane((int)kind) == KVZ_KIND_K) {
      const int voff = (int)((uint32_t)(lane & 15) * row_bytes + 16u * (uint32_t)(lane >> 4));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 64 * j, kPolicy));
    } else {
      const int voff = (int)(8u * (uint32_t)(lane >> 5) * row_bytes + 2u * (uint32_t)(lane & 31));
      uint32_t v[4][8];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          v[j][i] = __builtin_amdgcn_raw_buffer_load_b16(r, voff, (int)((uint32_t)i * row_bytes) + 64 * j,
                                                         kPolicy);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = make_uint4(v[j][0] | (v[j][1] << 16), v[j][2] | (v[j][3] << 16),
                          v[j][4] | (v[j][5] << 16), v[j][6] | (v[j][7] << 16));
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = load_chunk(src, stride, kind, j, lane, false);
  }
}

// An item's metadata record (device memory) as one global load: off, then tag[0..3].
__device__ __forceinline__ uint64_t load_meta_record(const kvz_group_meta* m) {
  typedef __attribute__((address_space(1))) const uint64_t global_u64;
  return *(global_u64*)(m);
}

}  // namespace kvz
