// Second page format: the group-adaptive additive exponent code.
//
// Follows "GAAC: Lossless KV Compression for Bandwidth-Efficient LLM Inference on Personal
// Devices": section "Lossless KV Compression" (sign and 7 fraction bits kept as one byte; per
// head-channel pair, calibrated windows of 8 and 16 exponents with bases b3, b4; groups of eight
// in attention-access order share a 2-bit mode - 3-bit offsets, 4-bit offsets, raw 8-bit
// exponents - and reconstruction is e = code + b_w with b_8 = 0; the low three code bits form a
// common stream, a 4-bit group adds one escape byte, a raw group five), section "Block-Wise
// Compression Scheduling" (fixed-capacity slots; a tile that does not fit stays BF16) and
// appendix "Storage", Table 9 (2048 + 768 + 64 bytes per 16-token tile plus a 128-byte escape
// slot).  The record layout is stated in include/kvz.h.
//
// kvz_gaac_calibrate = zero -> histogram (atomics, one wave per page) -> window pick.
// kvz_gaac_encode_pages = classify (one wave per tile: modes, escape total, raw fallback) ->
// allocate (pool.hip, same rule as the first format, runs of 12 or 16 granules) -> pack.
// kvz_gaac_decompress_pages rebuilds whole pages into the raw chunk layout.
#include "gaac_internal.h"
#include "encode_internal.h"

namespace kvz {

int launch_alloc_for_gaac_items(kvz_pool* p, const kvz_gaac_item* d_items, int n, hipStream_t s);

namespace {

constexpr uint32_t kGaacTagsCompressed = 0x00000000u;
constexpr uint32_t kGaacTagsRaw = 0xFFFFFFFFu;

// ---------------------------------------------------------------------------------------------
// Calibration
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gaac_hist_zero_kernel(uint32_t* hist) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < 128 * 256) hist[i] = 0;
}

// One wave per page: lane l counts the exponents of dims 2l and 2l+1 over the 16 tokens.
__global__ __launch_bounds__(256) void gaac_hist_kernel(const kvz_encode_item* items, int n,
                                                        uint32_t* hist) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= n) return;
  const kvz_encode_item it = items[item];
  for (int t = 0; t < KVZ_PAGE_TOKENS; ++t) {
    const uint16_t* row = it.src + (size_t)t * it.src_stride + 2 * lane;
    const uint32_t w0 = row[0], w1 = row[1];
    atomicAdd(&hist[(2 * lane) * 256 + ((w0 >> 7) & 0xFFu)], 1u);
    atomicAdd(&hist[(2 * lane + 1) * 256 + ((w1 >> 7) & 0xFFu)], 1u);
  }
}

// One thread per (dim, width): the base of the window with the most exponents (smallest first).
__global__ __launch_bounds__(256) void gaac_pick_kernel(const uint32_t* hist, uint8_t* bases) {
  const int t = threadIdx.x;
  const int dim = t & 127;
  const int width = t < 128 ? 8 : 16;
  const uint32_t* h = hist + dim * 256;
  uint32_t run = 0;
  for (int e = 0; e < width; ++e) run += h[e];
  uint32_t best = run;
  int best_b = 0;
  for (int b = 1; b + width <= 256; ++b) {
    run += h[b + width - 1];
    run -= h[b - 1];
    if (run > best) {
      best = run;
      best_b = b;
    }
  }
  bases[(t < 128 ? 0 : 128) + dim] = (uint8_t)best_b;
}

// ---------------------------------------------------------------------------------------------
// Encode
// ---------------------------------------------------------------------------------------------
struct GroupCode {
  uint32_t mode;      // 0 = 3-bit, 1 = 4-bit, 2 = raw
  uint32_t low24;     // low 3 code bits of values 0..7
  uint32_t esc;       // 4-bit: bit i = code bit 3 of value i; raw: exponent bits 3..7, low 32 of 40
  uint32_t esc_hi;    // raw: bits 32..39
  uint32_t sm0, sm1;  // sign+fraction bytes of values 0..3 / 4..7
};

// Mode and codes of one group (8 values, value 2m in the low half of dword m of w) with the
// bases of its values (b3 / b4 bytes, values 0..3 then 4..7).
__device__ __forceinline__ GroupCode gaac_code_group(uint4 w, uint32_t b3lo, uint32_t b3hi,
                                                     uint32_t b4lo, uint32_t b4hi) {
  const uint32_t d[4] = {w.x, w.y, w.z, w.w};
  uint32_t e[8], sm[8], b3[8], b4[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t v = (d[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
    e[i] = (v >> 7) & 0xFFu;
    sm[i] = ((v >> 8) & 0x80u) | (v & 0x7Fu);
    b3[i] = ((i < 4 ? b3lo : b3hi) >> (8 * (i & 3))) & 0xFFu;
    b4[i] = ((i < 4 ? b4lo : b4hi) >> (8 * (i & 3))) & 0xFFu;
  }
  bool fit3 = true, fit4 = true;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    fit3 = fit3 && e[i] >= b3[i] && e[i] - b3[i] <= 7u;
    fit4 = fit4 && e[i] >= b4[i] && e[i] - b4[i] <= 15u;
  }
  GroupCode g;
  g.mode = fit3 ? kGaacMode3 : (fit4 ? kGaacMode4 : kGaacModeRaw);
  g.low24 = 0;
  g.esc = 0;
  g.esc_hi = 0;
  uint64_t raw40 = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t code = g.mode == kGaacMode3 ? e[i] - b3[i] : (g.mode == kGaacMode4 ? e[i] - b4[i] : e[i]);
    g.low24 |= (code & 7u) << (3 * i);
    g.esc |= g.mode == kGaacMode4 ? ((code >> 3) & 1u) << i : 0u;
    raw40 |= (uint64_t)((code >> 3) & 0x1Fu) << (5 * i);
  }
  if (g.mode == kGaacModeRaw) {
    g.esc = (uint32_t)raw40;
    g.esc_hi = (uint32_t)(raw40 >> 32);
  }
  g.sm0 = sm[0] | (sm[1] << 8) | (sm[2] << 16) | (sm[3] << 24);
  g.sm1 = sm[4] | (sm[5] << 8) | (sm[6] << 16) | (sm[7] << 24);
  return g;
}

// Bases of the 8 values of lane c's group in block j, as bytes (values 0..3, 4..7).
__device__ __forceinline__ void group_bases(const uint8_t* bases, uint32_t kind, int j, int c,
                                            uint32_t& b3lo, uint32_t& b3hi, uint32_t& b4lo,
                                            uint32_t& b4hi) {
  if (kind == KVZ_KIND_K) {
    const int dim = 32 * j + 8 * (c >> 4);   // eight consecutive dims
    const uint32_t* p3 = reinterpret_cast<const uint32_t*>(bases + dim);
    const uint32_t* p4 = reinterpret_cast<const uint32_t*>(bases + 128 + dim);
    b3lo = p3[0];
    b3hi = p3[1];
    b4lo = p4[0];
    b4hi = p4[1];
  } else {
    const int dim = 32 * j + (c & 31);       // one dim, eight tokens
    b3lo = b3hi = bases[dim] * 0x01010101u;
    b4lo = b4hi = bases[128 + dim] * 0x01010101u;
  }
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += (uint32_t)__shfl_xor((int)v, d, 64);
  return v;
}

// Modes of every group, escape total, raw fallback; tags and "not stored" go to the metadata.
template <int kPolicy>
__global__ __launch_bounds__(256) void gaac_classify_kernel(const kvz_gaac_item* items, int n,
                                                            uint32_t flags) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= n) return;
  const kvz_gaac_item it = items[item];
  uint4 w[4];
  load_item_chunks<kPolicy>(it.src, it.src_stride, it.kind, lane, w);
  uint32_t esc = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t b3lo, b3hi, b4lo, b4hi;
    group_bases(it.bases, it.kind, j, lane, b3lo, b3hi, b4lo, b4hi);
    esc += gaac_escape_bytes(gaac_code_group(w[j], b3lo, b3hi, b4lo, b4hi).mode);
  }
  const uint32_t total = wave_sum(esc);
  const bool raw = (flags & KVZ_ENC_FORCE_RAW) || total > kGaacEscapeSlot;
  if (lane == 0) {
    *reinterpret_cast<uint32_t*>(it.dst->tag) = raw ? kGaacTagsRaw : kGaacTagsCompressed;
    it.dst->off = KVZ_OFF_NONE;
  }
}

// Write each placed tile: raw chunk layout, or the planes and the escape bytes.
template <int kPolicy>
__global__ __launch_bounds__(256) void gaac_pack_kernel(const kvz_gaac_item* items, int n,
                                                        uint8_t* arena, uint64_t capacity) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= n) return;
  const kvz_gaac_item it = items[item];
  // every load of the item (metadata, then source) before the first store into the arena
  const uint64_t mt = load_meta_record(it.dst);
  uint4 w[4];
  load_item_chunks<kPolicy>(it.src, it.src_stride, it.kind, lane, w);
  const uint32_t off = (uint32_t)mt;
  const uint32_t tags = (uint32_t)(mt >> 32);
  const bool raw = tags == kGaacTagsRaw;
  if (off == KVZ_OFF_NONE || (uint64_t)off + (raw ? 16u : 12u) > capacity) return;
  uint8_t* rec = arena + (size_t)off * KVZ_GRANULE_BYTES;
  if (raw) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<uint4*>(rec + j * kRawBlockBytes + kRawChunkBytes * lane) = w[j];
    return;
  }
  GroupCode g[4];
  uint32_t esc_len = 0, modes = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t b3lo, b3hi, b4lo, b4hi;
    group_bases(it.bases, it.kind, j, lane, b3lo, b3hi, b4lo, b4hi);
    g[j] = gaac_code_group(w[j], b3lo, b3hi, b4lo, b4hi);
    esc_len += gaac_escape_bytes(g[j].mode);
    modes |= g[j].mode << (2 * j);
  }
  // sign+fraction plane, code plane, mode plane
  uint8_t code_bytes[12];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    *reinterpret_cast<uint2*>(rec + 512 * j + 8 * lane) = make_uint2(g[j].sm0, g[j].sm1);
#pragma unroll
    for (int k = 0; k < 3; ++k) code_bytes[3 * j + k] = (uint8_t)(g[j].low24 >> (8 * k));
  }
  uint32_t cw[3];
#pragma unroll
  for (int k = 0; k < 3; ++k)
    cw[k] = (uint32_t)code_bytes[4 * k] | ((uint32_t)code_bytes[4 * k + 1] << 8) |
            ((uint32_t)code_bytes[4 * k + 2] << 16) | ((uint32_t)code_bytes[4 * k + 3] << 24);
  uint32_t* cp = reinterpret_cast<uint32_t*>(rec + kGaacCodeOff + 12 * lane);
  cp[0] = cw[0];
  cp[1] = cw[1];
  cp[2] = cw[2];
  rec[kGaacModeOff + lane] = (uint8_t)modes;
  // escape bytes: lanes in order, blocks in order
  uint32_t at = kGaacEscOff + gaac_exclusive_scan(esc_len, lane);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (g[j].mode == kGaacMode4) {
      rec[at++] = (uint8_t)g[j].esc;
    } else if (g[j].mode == kGaacModeRaw) {
#pragma unroll
      for (int k = 0; k < 4; ++k) rec[at + k] = (uint8_t)(g[j].esc >> (8 * k));
      rec[at + 4] = (uint8_t)g[j].esc_hi;
      at += 5;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Decompress-first
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gaac_decompress_kernel(const uint8_t* arena,
                                                              uint64_t arena_bytes,
                                                              const kvz_group_meta* meta,
                                                              const uint8_t* bases,
                                                              int64_t n_groups, int hkv,
                                                              uint8_t* dst) {
  const int lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // output tile index
  if (g >= n_groups) return;
  const int64_t page = g / (2 * hkv);
  const int rem = (int)(g % (2 * hkv));
  const uint32_t kind = (uint32_t)(rem / hkv);
  const int kvh = rem % hkv;
  const kvz_group_meta m = meta[(page * hkv + kvh) * 2 + kind];
  const uint32_t tags = *reinterpret_cast<const uint32_t*>(m.tag);
  const bool raw = tags == kGaacTagsRaw;
  const uint64_t start = (uint64_t)m.off * KVZ_GRANULE_BYTES;
  uint4* out = reinterpret_cast<uint4*>(dst + g * 4096 + kRawChunkBytes * lane);
  const bool known = tags == kGaacTagsRaw || tags == kGaacTagsCompressed;
  if (m.off == KVZ_OFF_NONE || !known || start + (raw ? 4096u : 3072u) > arena_bytes) {
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j * 64] = make_uint4(0, 0, 0, 0);
    return;
  }
  const uint8_t* rec = arena + start;
  if (raw) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      out[j * 64] = *reinterpret_cast<const uint4*>(rec + j * kRawBlockBytes + kRawChunkBytes * lane);
    return;
  }
  const uint8_t* tb = bases + (size_t)(kvh * 2 + kind) * 256;
  const uint32_t* cp = reinterpret_cast<const uint32_t*>(rec + kGaacCodeOff + 12 * lane);
  const uint32_t cw[3] = {cp[0], cp[1], cp[2]};
  const uint32_t modes = rec[kGaacModeOff + lane];
  uint32_t esc_len = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) esc_len += gaac_escape_bytes((modes >> (2 * j)) & 3u);
  uint32_t at = kGaacEscOff + gaac_exclusive_scan(esc_len, lane);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t mode = (modes >> (2 * j)) & 3u;
    const uint32_t nb = gaac_escape_bytes(mode);
    uint64_t e = 0;
    for (uint32_t k = 0; k < nb; ++k)      // never past the slot, whatever the mode plane says
      if (at + k < kGaacSlotBytes) e |= (uint64_t)rec[at + k] << (8 * k);
    at += nb;
    const uint32_t esc = (uint32_t)e, esc_hi = (uint32_t)(e >> 32);
    uint32_t b3lo, b3hi, b4lo, b4hi;
    group_bases(tb, kind, j, lane, b3lo, b3hi, b4lo, b4hi);
    const uint2 sm = *reinterpret_cast<const uint2*>(rec + 512 * j + 8 * lane);
    const uint32_t low24 = gaac_low24(cw, j);
    out[j * 64] = gaac_restore_group(sm.x, sm.y, low24, mode, esc, esc_hi, b3lo, b3hi, b4lo, b4hi);
  }
}

}  // namespace
}  // namespace kvz

using namespace kvz;

extern "C" int kvz_gaac_calibrate(const kvz_encode_item* d_items, int32_t n, uint32_t* d_hist,
                                  uint8_t* d_bases, hipStream_t s) {
  if (n < 0) return set_error(KVZ_EINVAL, "n < 0");
  if (!d_hist || !d_bases || (n > 0 && !d_items)) return set_error(KVZ_EINVAL, "null pointer argument");
  if (((uintptr_t)d_hist) & 3u) return set_error(KVZ_EINVAL, "hist must be 4-byte aligned");
  hipLaunchKernelGGL(gaac_hist_zero_kernel, dim3(128), dim3(256), 0, s, d_hist);
  if (n > 0)
    hipLaunchKernelGGL(gaac_hist_kernel, dim3((n + 3) / 4), dim3(256), 0, s, d_items, (int)n, d_hist);
  hipLaunchKernelGGL(gaac_pick_kernel, dim3(1), dim3(256), 0, s, d_hist, d_bases);
  return check_hip(hipGetLastError(), "gaac calibrate launch");
}

extern "C" int kvz_gaac_encode_pages(kvz_pool* p, const kvz_gaac_item* d_items, int32_t n,
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
    hipLaunchKernelGGL(gaac_classify_kernel<kStreamLoad>, dim3(grid), dim3(256), 0, s, d_items, (int)n, flags);
  else
    hipLaunchKernelGGL(gaac_classify_kernel<kCachedLoad>, dim3(grid), dim3(256), 0, s, d_items, (int)n, flags);
  int rc = check_hip(hipGetLastError(), "gaac classify launch");
  if (rc != KVZ_OK) return rc;
  rc = launch_alloc_for_gaac_items(p, d_items, n, s);
  if (rc != KVZ_OK) return rc;
  if (stream)
    hipLaunchKernelGGL(gaac_pack_kernel<kStreamLoad>, dim3(grid), dim3(256), 0, s, d_items, (int)n,
                       (uint8_t*)p->arena, p->capacity);
  else
    hipLaunchKernelGGL(gaac_pack_kernel<kCachedLoad>, dim3(grid), dim3(256), 0, s, d_items, (int)n,
                       (uint8_t*)p->arena, p->capacity);
  return check_hip(hipGetLastError(), "gaac pack launch");
}

extern "C" int kvz_gaac_decompress_pages(const void* d_arena, uint64_t arena_bytes,
                                         const kvz_group_meta* d_meta, const uint8_t* d_bases,
                                         int64_t n_pages, int32_t num_kv_heads, uint8_t* d_dst,
                                         hipStream_t s) {
  if (n_pages < 0 || num_kv_heads <= 0) return set_error(KVZ_EINVAL, "bad sizes");
  if (n_pages == 0) return KVZ_OK;
  if (!d_arena || !d_meta || !d_bases || !d_dst) return set_error(KVZ_EINVAL, "null pointer argument");
  if ((((uintptr_t)d_meta) & 7u) || (((uintptr_t)d_dst) & 15u) || (((uintptr_t)d_bases) & 3u) ||
      (((uintptr_t)d_arena) & 15u))
    return set_error(KVZ_EINVAL, "misaligned pointer argument");
  const int64_t n_groups = n_pages * 2 * num_kv_heads;
  const int64_t grid = (n_groups + 3) / 4;
  if (grid > 0x7FFFFFFF) return set_error(KVZ_EINVAL, "too many pages for one call");
  hipLaunchKernelGGL(gaac_decompress_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                     (const uint8_t*)d_arena, arena_bytes, d_meta, d_bases, n_groups,
                     (int)num_kv_heads, d_dst);
  return check_hip(hipGetLastError(), "gaac decompress launch");
}
