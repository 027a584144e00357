// Device helpers of the group-adaptive additive exponent code, shared by its encoder /
// decompressor (gaac.hip) and the fused attention (attention.hip).
//
// "GAAC: Lossless KV Compression for Bandwidth-Efficient LLM Inference on Personal Devices",
// section "Lossless KV Compression": e = code + b_w (b_8 = 0); sign and 7 fraction bits are
// one unchanged byte.  Record layout: include/kvz.h.
#pragma once

#include "kvz_internal.h"

namespace kvz {

constexpr uint32_t kGaacMode3 = 0;
constexpr uint32_t kGaacMode4 = 1;
constexpr uint32_t kGaacModeRaw = 2;
constexpr uint32_t kGaacCodeOff = 2048;          // after the sign+fraction plane
constexpr uint32_t kGaacModeOff = 2048 + 768;    // after the code plane
constexpr uint32_t kGaacEscOff = 2048 + 768 + 64;
constexpr uint32_t kGaacEscapeSlot = 128;        // escape capacity of a compressed tile
constexpr uint32_t kGaacSlotBytes = kGaacEscOff + kGaacEscapeSlot;   // 3008

__device__ __forceinline__ uint32_t gaac_escape_bytes(uint32_t mode) {
  return mode == kGaacMode4 ? 1u : (mode == kGaacModeRaw ? 5u : 0u);
}

// Exclusive prefix sum over the lanes of the wave (lane order) of v < 32 (a lane's escape
// bytes, at most 4 x 5): bit by bit, the lanes below this one with that bit set are counted
// with a ballot and mbcnt - no cross-lane data movement.
__device__ __forceinline__ uint32_t gaac_exclusive_scan(uint32_t v, int lane) {
  (void)lane;
  uint32_t sum = 0;
#pragma unroll
  for (int bit = 0; bit < 5; ++bit) {
    const uint64_t m = __ballot((v >> bit) & 1u);
    const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    sum += below << bit;
  }
  return sum;
}

// The same scan for v < 8 (at most four one-byte escapes per lane): three bits.
__device__ __forceinline__ uint32_t gaac_exclusive_scan_small(uint32_t v) {
  uint32_t sum = 0;
#pragma unroll
  for (int bit = 0; bit < 3; ++bit) {
    const uint64_t m = __ballot((v >> bit) & 1u);
    const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    sum += below << bit;
  }
  return sum;
}

// Block j's 24 low-code bits from a lane's 12 code bytes (3 dwords, little-endian).
__device__ __forceinline__ uint32_t gaac_low24(const uint32_t (&cw)[3], int j) {
  switch (j) {
    case 0: return cw[0] & 0xFFFFFFu;
    case 1: return __builtin_amdgcn_alignbit(cw[1], cw[0], 24) & 0xFFFFFFu;
    case 2: return __builtin_amdgcn_alignbit(cw[2], cw[1], 16) & 0xFFFFFFu;
    default: return cw[2] >> 8;
  }
}

// Four 3-bit fields of x (bits 0..11) -> one per byte.
__device__ __forceinline__ uint32_t gaac_spread3(uint32_t x) {
  return (x & 7u) | (((x >> 3) & 7u) << 8) | (((x >> 6) & 7u) << 16) | (((x >> 9) & 7u) << 24);
}
// Four 5-bit fields of x (bits 0..19) -> one per byte.
__device__ __forceinline__ uint32_t gaac_spread5(uint32_t x) {
  return (x & 31u) | (((x >> 5) & 31u) << 8) | (((x >> 10) & 31u) << 16) | (((x >> 15) & 31u) << 24);
}
// Bit BIT of the four bytes of c0 / c1 <- bits 0..3 / 4..7 of h (h < 256).  t = h | h<<7 |
// h<<14 | h<<21 holds bit i of h at bit 8i (i < 4) and at bit 8(i-4)+4 (i >= 4), and no other
// bit of h reaches those positions; two shift-ors and two masked merges, no multiply.
template <int BIT>
__device__ __forceinline__ void gaac_or_bits(uint32_t h, uint32_t& c0, uint32_t& c1) {
  static_assert(BIT >= 0 && BIT < 8, "a bit of a byte");
  constexpr uint32_t m = 0x01010101u << BIT;
  uint32_t t = h | (h << 7);
  t |= t << 14;
  c0 |= (t << BIT) & m;
  if constexpr (BIT >= 4) c1 |= (t << (BIT - 4)) & m;
  else c1 |= (t >> (4 - BIT)) & m;
}
__device__ __forceinline__ void gaac_or_bit3(uint32_t h, uint32_t& c0, uint32_t& c1) {
  gaac_or_bits<3>(h, c0, c1);
}

// Rebuild the 8 BF16 values of one group (4 dwords, value 2m in the low half of dword m).
// sm0/sm1: sign+fraction bytes of values 0..3 / 4..7; low24: low 3 code bits; mode; esc /
// esc_hi: the group's escape bits (4-bit: one byte; raw: 40 bits); b3*/b4*: the values' bases
// as bytes.  Exponents are assembled per byte: code + base never carries (e <= 255).
__device__ __forceinline__ uint4 gaac_restore_group(uint32_t sm0, uint32_t sm1, uint32_t low24,
                                                    uint32_t mode, uint32_t esc, uint32_t esc_hi,
                                                    uint32_t b3lo, uint32_t b3hi, uint32_t b4lo,
                                                    uint32_t b4hi) {
  uint32_t c0 = gaac_spread3(low24 & 0xFFFu);
  uint32_t c1 = gaac_spread3(low24 >> 12);
  gaac_or_bit3(mode == kGaacMode4 ? (esc & 0xFFu) : 0u, c0, c1);
  if (mode == kGaacModeRaw) {
    c0 |= gaac_spread5(esc & 0xFFFFFu) << 3;
    c1 |= gaac_spread5((esc >> 20) | (esc_hi << 12)) << 3;
  }
  const uint32_t base0 = mode == kGaacMode3 ? b3lo : (mode == kGaacMode4 ? b4lo : 0u);
  const uint32_t base1 = mode == kGaacMode3 ? b3hi : (mode == kGaacMode4 ? b4hi : 0u);
  const uint32_t e0 = c0 + base0, e1 = c1 + base1;
  // per value: high byte = sign | e >> 1, low byte = (e & 1) << 7 | fraction
  const uint32_t h0 = (sm0 & 0x80808080u) | ((e0 >> 1) & 0x7F7F7F7Fu);
  const uint32_t l0 = (sm0 & 0x7F7F7F7Fu) | ((e0 << 7) & 0x80808080u);
  const uint32_t h1 = (sm1 & 0x80808080u) | ((e1 >> 1) & 0x7F7F7F7Fu);
  const uint32_t l1 = (sm1 & 0x7F7F7F7Fu) | ((e1 << 7) & 0x80808080u);
  uint4 r;
  r.x = __builtin_amdgcn_perm(h0, l0, 0x05010400u);   // l.b0 h.b0 l.b1 h.b1
  r.y = __builtin_amdgcn_perm(h0, l0, 0x07030602u);   // l.b2 h.b2 l.b3 h.b3
  r.z = __builtin_amdgcn_perm(h1, l1, 0x05010400u);
  r.w = __builtin_amdgcn_perm(h1, l1, 0x07030602u);
  return r;
}

// The same rebuild from codes already spread to bytes (c0/c1: the low 3 code bits of values
// 0..3 / 4..7, one per byte).  Raw groups only when `wave_has_raw` (wave-uniform); without it
// every group is 3-bit or 4-bit and the base is a two-way choice.
__device__ __forceinline__ uint4 gaac_restore_group_spread(uint32_t sm0, uint32_t sm1, uint32_t c0,
                                                           uint32_t c1, uint32_t mode, uint32_t esc,
                                                           uint32_t esc_hi, uint32_t b3lo,
                                                           uint32_t b3hi, uint32_t b4lo,
                                                           uint32_t b4hi, bool wave_has_raw) {
  const bool m4 = mode == kGaacMode4;
  const bool raw = wave_has_raw && mode == kGaacModeRaw;
  gaac_or_bit3(m4 ? (esc & 0xFFu) : 0u, c0, c1);
  if (raw) {
    c0 |= gaac_spread5(esc & 0xFFFFFu) << 3;
    c1 |= gaac_spread5((esc >> 20) | (esc_hi << 12)) << 3;
  }
  const uint32_t base0 = m4 ? b4lo : (raw ? 0u : b3lo);
  const uint32_t base1 = m4 ? b4hi : (raw ? 0u : b3hi);
  const uint32_t e0 = c0 + base0, e1 = c1 + base1;
  const uint32_t h0 = (sm0 & 0x80808080u) | ((e0 >> 1) & 0x7F7F7F7Fu);
  const uint32_t l0 = (sm0 & 0x7F7F7F7Fu) | ((e0 << 7) & 0x80808080u);
  const uint32_t h1 = (sm1 & 0x80808080u) | ((e1 >> 1) & 0x7F7F7F7Fu);
  const uint32_t l1 = (sm1 & 0x7F7F7F7Fu) | ((e1 << 7) & 0x80808080u);
  uint4 r;
  r.x = __builtin_amdgcn_perm(h0, l0, 0x05010400u);
  r.y = __builtin_amdgcn_perm(h0, l0, 0x07030602u);
  r.z = __builtin_amdgcn_perm(h1, l1, 0x05010400u);
  r.w = __builtin_amdgcn_perm(h1, l1, 0x07030602u);
  return r;
}

}  // namespace kvz
