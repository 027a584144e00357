// Device helpers of the exponent code on FP8 tiles, shared by its encoder / decompressor
// (fp8.hip) and the fused attention (attention.hip).
//
// "GAAC: Lossless KV Compression for Bandwidth-Efficient LLM Inference on Personal Devices",
// appendix "Relation to FP8 KV" (Table 7) with the code of section "Lossless KV Compression":
// sign and fraction stay unchanged, the exponent field (4 bits in E4M3, 5 in E5M2) is coded as
// 3-bit offsets from b3, 4-bit offsets from b4 or raw, per group of eight; e = code + b_w.
// Record layout: include/kvz.h.
#pragma once

#include "gaac_internal.h"

namespace kvz {

constexpr uint32_t kFp8Granule = KVZ_FP8_GRANULE_BYTES;   // 128
constexpr uint32_t kFp8RawTile = 2048;
constexpr uint32_t kFp8EscSlot = 64;
constexpr uint32_t kFp8TagsRaw = 0xFFFFFFFFu;
constexpr uint32_t kFp8Mode3 = 0;
constexpr uint32_t kFp8Mode4 = 1;
constexpr uint32_t kFp8ModeRaw = 2;

// Per-format constants: field widths, plane offsets, slot size, compressed tags (bytes 0xFF
// count the pool's run class: 12 + k granules of 128 bytes).
template <int FK>
struct Fp8Fmt;
template <>
struct Fp8Fmt<KVZ_FP8_E4M3> {
  static constexpr uint32_t kExpBits = 4, kFracBits = 3;
  static constexpr uint32_t kSmLane = 16, kSmBytes = 1024;
  static constexpr uint32_t kCodeOff = 1024, kModeOff = 1792, kEscOff = 1856, kSlot = 1920;
  static constexpr uint32_t kTagsComp = 0x00FFFFFFu;   // FF FF FF 00: 15 granules
  static constexpr uint32_t kRawEsc = 1;               // exponent bit 3 of eight values
};
template <>
struct Fp8Fmt<KVZ_FP8_E5M2> {
  static constexpr uint32_t kExpBits = 5, kFracBits = 2;
  static constexpr uint32_t kSmLane = 12, kSmBytes = 768;
  static constexpr uint32_t kCodeOff = 768, kModeOff = 1536, kEscOff = 1600, kSlot = 1664;
  static constexpr uint32_t kTagsComp = 0x000000FFu;   // FF 00 00 00: 13 granules
  static constexpr uint32_t kRawEsc = 2;               // exponent bits 3..4 of eight values
};

template <int FK>
__device__ __forceinline__ uint32_t fp8_escape_bytes(uint32_t mode) {
  return mode == kFp8Mode4 ? 1u : (mode == kFp8ModeRaw ? Fp8Fmt<FK>::kRawEsc : 0u);
}

// Byte offset of chunk c of block j in an uncompressed FP8 tile: lane c's blocks 0 and 1 are
// the 16 bytes at 16c, blocks 2 and 3 the 16 bytes at 1024 + 16c.
__device__ __forceinline__ uint32_t fp8_chunk_offset(int j, int c) {
  return 1024u * (uint32_t)(j >> 1) + 16u * (uint32_t)c + 8u * (uint32_t)(j & 1);
}

// Sign+fraction bytes (s << 7 | fraction) of values 0..3 (X) and 4..7 (Y) of group j, from
// the lane's words of the sign+fraction plane.  E4M3: word j = X | rotl32(Y, 4).  E5M2:
// words t < 3 = X | rotl32(Y, 3) of group t, group 3 in bits 5 and 6 of every byte.
template <int FK>
__device__ __forceinline__ void fp8_sm_xy(const uint32_t (&w)[4], int j, uint32_t& X, uint32_t& Y) {
  if constexpr (FK == KVZ_FP8_E4M3) {
    X = w[j] & 0x87878787u;
    Y = __builtin_amdgcn_alignbit(w[j], w[j], 4) & 0x87878787u;
  } else {
    if (j < 3) {
      X = w[j] & 0x83838383u;
      Y = __builtin_amdgcn_alignbit(w[j], w[j], 3) & 0x83838383u;
    } else {
      X = ((w[0] >> 5) & 0x03030303u) | ((w[2] << 2) & 0x80808080u);
      Y = ((w[1] >> 5) & 0x03030303u) | ((w[2] << 1) & 0x80808080u);
    }
  }
}

// Eight FP8 values (bytes of f0 = values 0..3, f1 = values 4..7) -> eight BF16 values, value
// 2m in the low half of dword m.  Every E4M3 and E5M2 value is exactly a BF16 value; the
// hardware conversion with a unit scale is exact.
template <int FK>
__device__ __forceinline__ uint4 fp8x8_to_bf16(uint32_t f0, uint32_t f1) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  uint4 r;
  if constexpr (FK == KVZ_FP8_E4M3) {
    r.x = __builtin_bit_cast(uint32_t, (bf16x2_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f0, 1.0f, false));
    r.y = __builtin_bit_cast(uint32_t, (bf16x2_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f0, 1.0f, true));
    r.z = __builtin_bit_cast(uint32_t, (bf16x2_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f1, 1.0f, false));
    r.w = __builtin_bit_cast(uint32_t, (bf16x2_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f1, 1.0f, true));
  } else {
    r.x = __builtin_bit_cast(uint32_t, (bf16x2_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(f0, 1.0f, false));
    r.y = __builtin_bit_cast(uint32_t, (bf16x2_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(f0, 1.0f, true));
    r.z = __builtin_bit_cast(uint32_t, (bf16x2_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(f1, 1.0f, false));
    r.w = __builtin_bit_cast(uint32_t, (bf16x2_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(f1, 1.0f, true));
  }
  return r;
}

// Four 2-bit fields of x (bits 0..7) -> bits 0..1 of one byte each.
__device__ __forceinline__ uint32_t fp8_spread2(uint32_t x) {
  return (x & 3u) | (((x >> 2) & 3u) << 8) | (((x >> 4) & 3u) << 16) | (((x >> 6) & 3u) << 24);
}

// The FP8 bytes of one group (values 0..3 -> .x, 4..7 -> .y) from its sign+fraction bytes X, Y,
// its low 3 code bits spread to bytes (c0: values 0..3, c1: 4..7), its mode and escape bits
// (4-bit: one byte, bit i = code bit 3 of value i; raw: EW-3 bits per value), and the bases
// of its values as bytes.  Codes and bases come already shifted left by the fraction width,
// i.e. in the exponent field of each byte; e <= 2^EW - 1 never carries out of the field, so the
// FP8 byte is one three-way add of code, base and sign+fraction.  E5M2 raw groups only when
// `wave_has_raw` (an E4M3 raw group escapes one bit per value, like a 4-bit group, and is
// always handled).
template <int FK>
__device__ __forceinline__ uint2 fp8_restore_group(uint32_t X, uint32_t Y, uint32_t c0, uint32_t c1,
                                                   uint32_t mode, uint32_t esc, uint32_t b3lo,
                                                   uint32_t b3hi, uint32_t b4lo, uint32_t b4hi,
                                                   bool wave_has_raw) {
  constexpr int kMw = (int)Fp8Fmt<FK>::kFracBits;
  const bool m4 = mode == kFp8Mode4;
  const bool raw = (FK == KVZ_FP8_E4M3 || wave_has_raw) && mode == kFp8ModeRaw;
  const bool one_bit = m4 || (FK == KVZ_FP8_E4M3 && raw);
  gaac_or_bits<3 + kMw>(one_bit ? (esc & 0xFFu) : 0u, c0, c1);
  if constexpr (FK == KVZ_FP8_E5M2) {
    if (raw) {
      c0 |= fp8_spread2(esc & 0xFFu) << (3 + kMw);
      c1 |= fp8_spread2((esc >> 8) & 0xFFu) << (3 + kMw);
    }
  }
  const uint32_t base0 = m4 ? b4lo : (raw ? 0u : b3lo);
  const uint32_t base1 = m4 ? b4hi : (raw ? 0u : b3hi);
  return make_uint2(c0 + base0 + X, c1 + base1 + Y);
}

}  // namespace kvz
