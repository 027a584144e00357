// Internal declarations shared by the kvz HIP sources (gfx950 only).
//
// Format facts implemented here (see include/kvz.h for the full statement and the passages of
// "ZipFusion: Fusing Lossless KV Decompression with Attention for Efficient LLM Decoding",
// section "How it works", that define them):
//   * chunk = what one lane of a wave holds for one MFMA operand: 8 BF16 values;
//   * compressed chunk = 8 low bytes + code word C = X | rotl32(Y, 4), 12 bytes;
//   * raw chunk = 8 LE BF16 words, 16 bytes;
//   * restore: high bytes of values 0..3 = (C & 0x87878787) + B, of values 4..7 =
//     (rotr32(C, 4) & 0x87878787) + B, with B = (b/2) * 0x01010101 (no carry between bytes).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>

#include "../../include/kvz.h"

namespace kvz {

constexpr uint32_t kPoolMagic = 0x505A564Bu;  // "KVZP"
constexpr uint32_t kPoolVersion = 1;
constexpr int kBins = 5;
constexpr uint32_t kCompBlockBytes = 768;
constexpr uint32_t kRawBlockBytes = 1024;
constexpr uint32_t kCompChunkBytes = 12;
constexpr uint32_t kRawChunkBytes = 16;

// Device-resident pool state header (first 256 bytes of the state buffer); the LIFO bins
// follow it as uint32 granule offsets.
struct PoolHdr {
  uint32_t magic;
  uint32_t version;
  uint64_t capacity;          // usable granules
  uint64_t frontier;          // granules handed out from the frontier
  uint64_t bin_cap[kBins];    // entries each bin can hold
  uint64_t bin_cnt[kBins];    // entries currently held
  uint64_t bin_base[kBins];   // first entry of bin k in the bins array
  uint64_t live_runs;
  uint64_t live_granules;
  uint64_t live_raw_blocks;
  uint64_t enospc;
  uint64_t bad_frees;
};
static_assert(sizeof(PoolHdr) <= 256, "pool header must fit its 256-byte slot");
constexpr uint64_t kPoolHdrBytes = 256;

// Per-thread error text behind kvz_last_error().
int set_error(int code, const std::string& msg);
int check_hip(hipError_t e, const char* what);
// compute units of the current device (cached per device; 256 if the query fails)
int device_cus();

// ---------------------------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t run_granules(uint32_t n_raw) { return 12u + n_raw; }

__device__ __forceinline__ uint32_t n_raw_of(uint32_t tags) {
  uint32_t n = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) n += ((tags >> (8 * k)) & 0xFFu) == KVZ_RAW_TAG;
  return n;
}

__device__ __forceinline__ uint32_t block_bytes(uint32_t tag) {
  return tag == KVZ_RAW_TAG ? kRawBlockBytes : kCompBlockBytes;
}

// The 8 values of chunk c of block j of a natural page (row stride `stride` elements), packed
// as 4 dwords (value 2m in the low half of dword m).  K: token c%16, dims 32j+8(c/16)+0..7;
// V: dim 32j+c%32, tokens 8(c/32)+0..7.
__device__ __forceinline__ uint4 load_chunk(const uint16_t* src, uint32_t stride, uint32_t kind,
                                            int j, int c, bool aligned) {
  uint16_t v[8];
  if (kind == KVZ_KIND_K) {
    const uint16_t* p = src + (size_t)(c & 15) * stride + 32 * j + 8 * (c >> 4);
    if (aligned) {
      return *reinterpret_cast<const uint4*>(p);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = p[i];
  } else {
    const uint16_t* p = src + (size_t)(8 * (c >> 5)) * stride + 32 * j + (c & 31);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = p[(size_t)i * stride];
  }
  uint4 r;
  r.x = (uint32_t)v[0] | ((uint32_t)v[1] << 16);
  r.y = (uint32_t)v[2] | ((uint32_t)v[3] << 16);
  r.z = (uint32_t)v[4] | ((uint32_t)v[5] << 16);
  r.w = (uint32_t)v[6] | ((uint32_t)v[7] << 16);
  return r;
}

// Rebuild 8 BF16 values (4 dwords, value 2m in the low half of dword m) from a compressed chunk:
// lo0/lo1 = low bytes of values 0..3 / 4..7, code = code word, B = (b/2) * 0x01010101.
__device__ __forceinline__ uint4 restore_chunk(uint32_t lo0, uint32_t lo1, uint32_t code,
                                               uint32_t B) {
  const uint32_t hx = (code & 0x87878787u) + B;                                 // mask branch
  const uint32_t hy = (__builtin_amdgcn_alignbit(code, code, 4) & 0x87878787u) + B;  // unpack
  uint4 r;
  r.x = __builtin_amdgcn_perm(hx, lo0, 0x05010400u);   // lo0.b0 hx.b0 lo0.b1 hx.b1
  r.y = __builtin_amdgcn_perm(hx, lo0, 0x07030602u);   // lo0.b2 hx.b2 lo0.b3 hx.b3
  r.z = __builtin_amdgcn_perm(hy, lo1, 0x05010400u);
  r.w = __builtin_amdgcn_perm(hy, lo1, 0x07030602u);
  return r;
}

// Inverse of restore_chunk for an eligible chunk: w = 8 BF16 words as 4 dwords.
// Returns {lo0, lo1, code}.
__device__ __forceinline__ uint3 compress_chunk(uint4 w, uint32_t B) {
  // high bytes of values 0..3 and 4..7, then s<<7 | d = high byte - b/2 per byte (no borrow,
  // since e >> 1 >= b/2 for every value of an eligible block)
  const uint32_t hx = __builtin_amdgcn_perm(w.y, w.x, 0x07050301u);
  const uint32_t hy = __builtin_amdgcn_perm(w.w, w.z, 0x07050301u);
  const uint32_t X = hx - B;
  const uint32_t Y = hy - B;
  uint3 r;
  r.x = __builtin_amdgcn_perm(w.y, w.x, 0x06040200u);
  r.y = __builtin_amdgcn_perm(w.w, w.z, 0x06040200u);
  r.z = X | __builtin_amdgcn_alignbit(Y, Y, 28);       // X | rotl32(Y, 4)
  return r;
}

}  // namespace kvz

struct kvz_pool {
  void* arena;
  uint64_t arena_bytes;
  void* state;
  uint64_t state_bytes;
  uint64_t capacity;
  int device;
  void* scratch;   // device: per-tile counts of the allocation / free passes (in the state buffer)
  uint32_t granule_bytes;   // 256 (BF16 formats) or 128 (FP8 tiles, kvz_fp8_pool_init)
  void* enc_scratch;        // device: the one-pass encoder's records (state buffer)
};

