// Third page format: the exponent code on FP8 KV (E4M3 and E5M2).
//
// Follows "GAAC: Lossless KV Compression for Bandwidth-Efficient LLM Inference on Personal
// Devices": appendix "Relation to FP8 KV" (Table 7: the lossless exponent code applied to KV
// converted to FP8), with the code of section "Lossless KV Compression" (sign and fraction kept;
// per head-channel pair calibrated windows of 8 and 16 exponents; groups of eight share a 2-bit
// mode - 3-bit offsets, 4-bit offsets, raw - and e = code + b_w) and the fixed-capacity slots of
// section "Block-Wise Compression Scheduling" (a tile that does not fit stays uncompressed).
// The record layout is stated in include/kvz.h.
//
// kvz_fp8_calibrate = zero -> histogram (one wave per page) -> window pick.
// kvz_fp8_encode_pages = classify (one wave per tile: modes, escape total, fallback) ->
// allocate (pool.hip, runs of 13/15 or 16 granules of 128 bytes) -> pack.
// kvz_fp8_decompress_pages rebuilds tiles into the FP8 chunk layout; kvz_fp8_pack_pages lays
// natural pages out in it.
#include "fp8_internal.h"
#include "encode_internal.h"

namespace kvz {

int launch_alloc_for_fp8_items(kvz_pool* p, const kvz_fp8_item* d_items, int n, hipStream_t s);

namespace {

// ---------------------------------------------------------------------------------------------
// Calibration
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fp8_hist_zero_kernel(uint32_t* hist) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < 128 * 32) hist[i] = 0;
}

// One wave per page: lane l counts the exponents of dims 2l and 2l+1 over the 16 tokens.
template <int FK>
__global__ __launch_bounds__(256) void fp8_hist_kernel(const kvz_fp8_item* items, int n,
                                                       uint32_t* hist) {
  constexpr uint32_t kMw = Fp8Fmt<FK>::kFracBits, kEmask = (1u << Fp8Fmt<FK>::kExpBits) - 1;
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= n) return;
  const kvz_fp8_item it = items[item];
  for (int t = 0; t < KVZ_PAGE_TOKENS; ++t) {
    const uint8_t* row = it.src + (size_t)t * it.src_stride + 2 * lane;
    const uint32_t x0 = row[0], x1 = row[1];
    atomicAdd(&hist[(2 * lane) * 32 + ((x0 >> kMw) & kEmask)], 1u);
    atomicAdd(&hist[(2 * lane + 1) * 32 + ((x1 >> kMw) & kEmask)], 1u);
  }
}

// One thread per (dim, width): the base of the window with the most exponents (smallest first),
// windows inside [0, 2^EW - 1].
__global__ __launch_bounds__(256) void fp8_pick_kernel(const uint32_t* hist, uint8_t* bases,
                                                       int n_exp) {
  const int t = threadIdx.x;
  const int dim = t & 127;
  const int width = t < 128 ? 8 : 16;
  const uint32_t* h = hist + dim * 32;
  uint32_t run = 0;
  for (int e = 0; e < width; ++e) run += h[e];
  uint32_t best = run;
  int best_b = 0;
  for (int b = 1; b + width <= n_exp; ++b) {
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
// The 8 FP8 values of chunk c of block j of a natural page (row stride in bytes), value i in
// byte i: K: token c%16, dims 32j + 8(c/16) + 0..7; V: dim 32j + c%32, tokens 8(c/32) + 0..7.
__device__ __forceinline__ uint2 fp8_load_chunk(const uint8_t* src, uint32_t stride, uint32_t kind,
                                                int j, int c, bool aligned) {
  uint32_t v[8];
  if (kind == KVZ_KIND_K) {
    const uint8_t* p = src + (size_t)(c & 15) * stride + 32 * j + 8 * (c >> 4);
    if (aligned) return *reinterpret_cast<const uint2*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = p[i];
  } else {
    const uint8_t* p = src + (size_t)(8 * (c >> 5)) * stride + 32 * j + (c & 31);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = p[(size_t)i * stride];
  }
  return make_uint2(v[0] | (v[1] << 8) | (v[2] << 16) | (v[3] << 24),
                    v[4] | (v[5] << 8) | (v[6] << 16) | (v[7] << 24));
}

// The four chunks of an FP8 item as fp8_load_chunk gives them, every load issued before any is
// used, through a buffer resource over the page's rows (source pointer and stride are
// wave-uniform; see encode_internal.h).
template <int kPolicy>
__device__ __forceinline__ void fp8_load_item_chunks(const uint8_t* src, uint32_t stride,
                                                     uint32_t kind, int lane, bool aligned,
                                                     uint2 (&w)[4]) {
  if (aligned) {
    const uint32_t row = (uint32_t)__builtin_amdgcn_readfirstlane((int)stride);
    const __amdgpu_buffer_rsrc_t r = page_rsrc(src, row, 1);
    if (__builtin_amdgcn_readfirstlane((int)kind) == KVZ_KIND_K) {
      const int voff = (int)((uint32_t)(lane & 15) * row + 8u * (uint32_t)(lane >> 4));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, 32 * j, kPolicy));
    } else {
      const int voff = (int)(8u * (uint32_t)(lane >> 5) * row + (uint32_t)(lane & 31));
      uint32_t v[4][8];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          v[j][i] = __builtin_amdgcn_raw_buffer_load_b8(r, voff, (int)((uint32_t)i * row) + 32 * j, kPolicy);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = make_uint2(v[j][0] | (v[j][1] << 8) | (v[j][2] << 16) | (v[j][3] << 24),
                          v[j][4] | (v[j][5] << 8) | (v[j][6] << 16) | (v[j][7] << 24));
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = fp8_load_chunk(src, stride, kind, j, lane, false);
  }
}

struct Fp8GroupCode {
  uint32_t mode;     // 0 = 3-bit, 1 = 4-bit, 2 = raw
  uint32_t low24;    // low 3 code bits of values 0..7
  uint32_t esc;      // escape bits (4-bit: bit i; raw: EW-3 bits per value)
  uint32_t X, Y;     // sign+fraction bytes of values 0..3 / 4..7
};

template <int FK>
__device__ __forceinline__ Fp8GroupCode fp8_code_group(uint2 w, uint32_t b3lo, uint32_t b3hi,
                                                       uint32_t b4lo, uint32_t b4hi) {
  constexpr uint32_t kMw = Fp8Fmt<FK>::kFracBits, kEw = Fp8Fmt<FK>::kExpBits;
  constexpr uint32_t kEmask = (1u << kEw) - 1, kMmask = (1u << kMw) - 1;
  uint32_t e[8], sm[8], b3[8], b4[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t x = ((i < 4 ? w.x : w.y) >> (8 * (i & 3))) & 0xFFu;
    e[i] = (x >> kMw) & kEmask;
    sm[i] = (x & 0x80u) | (x & kMmask);
    b3[i] = ((i < 4 ? b3lo : b3hi) >> (8 * (i & 3))) & 0xFFu;
    b4[i] = ((i < 4 ? b4lo : b4hi) >> (8 * (i & 3))) & 0xFFu;
  }
  bool fit3 = true, fit4 = true;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    fit3 = fit3 && e[i] >= b3[i] && e[i] - b3[i] <= 7u;
    fit4 = fit4 && e[i] >= b4[i] && e[i] - b4[i] <= 15u;
  }
  Fp8GroupCode g;
  g.mode = fit3 ? kFp8Mode3 : (fit4 ? kFp8Mode4 : kFp8ModeRaw);
  g.low24 = 0;
  g.esc = 0;
  constexpr uint32_t kHi = kEw - 3;   // exponent bits above the low three
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t code = g.mode == kFp8Mode3 ? e[i] - b3[i] : (g.mode == kFp8Mode4 ? e[i] - b4[i] : e[i]);
    g.low24 |= (code & 7u) << (3 * i);
    if (g.mode == kFp8Mode4) g.esc |= ((code >> 3) & 1u) << i;
    else if (g.mode == kFp8ModeRaw) g.esc |= ((code >> 3) & ((1u << kHi) - 1)) << (kHi * i);
  }
  g.X = sm[0] | (sm[1] << 8) | (sm[2] << 16) | (sm[3] << 24);
  g.Y = sm[4] | (sm[5] << 8) | (sm[6] << 16) | (sm[7] << 24);
  return g;
}

// Bases of the 8 values of lane c's group in block j, as bytes (values 0..3, 4..7).
__device__ __forceinline__ void fp8_group_bases(const uint8_t* bases, uint32_t kind, int j, int c,
                                                uint32_t& b3lo, uint32_t& b3hi, uint32_t& b4lo,
                                                uint32_t& b4hi) {
  if (kind == KVZ_KIND_K) {
    const int dim = 32 * j + 8 * (c >> 4);
    const uint32_t* p3 = reinterpret_cast<const uint32_t*>(bases + dim);
    const uint32_t* p4 = reinterpret_cast<const uint32_t*>(bases + 128 + dim);
    b3lo = p3[0];
    b3hi = p3[1];
    b4lo = p4[0];
    b4hi = p4[1];
  } else {
    const int dim = 32 * j + (c & 31);
    b3lo = b3hi = bases[dim] * 0x01010101u;
    b4lo = b4hi = bases[128 + dim] * 0x01010101u;
  }
}

__device__ __forceinline__ uint32_t fp8_wave_sum(uint32_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += (uint32_t)__shfl_xor((int)v, d, 64);
  return v;
}

__device__ __forceinline__ bool fp8_src_aligned(const kvz_fp8_item& it) {
  return ((((uintptr_t)it.src) & 7u) == 0) && ((it.src_stride & 7u) == 0) &&
         it.src_stride <= kMaxBufferRowBytes;
}

// Modes of every group, escape total, fallback; tags and "not stored" go to the metadata.
template <int FK, int kPolicy>
__global__ __launch_bounds__(256) void fp8_classify_kernel(const kvz_fp8_item* items, int n,
                                                           uint32_t flags) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= n) return;
  const kvz_fp8_item it = items[item];
  uint2 w[4];
  fp8_load_item_chunks<kPolicy>(it.src, it.src_stride, it.kind, lane, fp8_src_aligned(it), w);
  uint32_t esc = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t b3lo, b3hi, b4lo, b4hi;
    fp8_group_bases(it.bases, it.kind, j, lane, b3lo, b3hi, b4lo, b4hi);
    esc += fp8_escape_bytes<FK>(fp8_code_group<FK>(w[j], b3lo, b3hi, b4lo, b4hi).mode);
  }
  const uint32_t total = fp8_wave_sum(esc);
  const bool raw = (flags & KVZ_ENC_FORCE_RAW) || total > kFp8EscSlot;
  if (lane == 0) {
    *reinterpret_cast<uint32_t*>(it.dst->tag) = raw ? kFp8TagsRaw : Fp8Fmt<FK>::kTagsComp;
    it.dst->off = KVZ_OFF_NONE;
  }
}

// The lane's sign+fraction words from the X/Y bytes of its four groups.
template <int FK>
__device__ __forceinline__ void fp8_sm_pack(const Fp8GroupCode (&g)[4], uint32_t (&w)[4]) {
  if constexpr (FK == KVZ_FP8_E4M3) {
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = g[j].X | __builtin_amdgcn_alignbit(g[j].Y, g[j].Y, 28);
  } else {
#pragma unroll
    for (int t = 0; t < 3; ++t) w[t] = g[t].X | __builtin_amdgcn_alignbit(g[t].Y, g[t].Y, 29);
    w[0] |= (g[3].X & 0x03030303u) << 5;
    w[1] |= (g[3].Y & 0x03030303u) << 5;
    w[2] |= ((g[3].X & 0x80808080u) >> 2) | ((g[3].Y & 0x80808080u) >> 1);
    w[3] = 0;
  }
}

// Write each placed tile: the FP8 chunk layout, or the planes and the escape bytes.
template <int FK, int kPolicy>
__global__ __launch_bounds__(256) void fp8_pack_kernel(const kvz_fp8_item* items, int n,
                                                       uint8_t* arena, uint64_t capacity) {
  using F = Fp8Fmt<FK>;
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= n) return;
  const kvz_fp8_item it = items[item];
  // every load of the item (metadata, then source) before the first store into the arena
  const uint64_t mt = load_meta_record(it.dst);
  uint2 cw8[4];
  fp8_load_item_chunks<kPolicy>(it.src, it.src_stride, it.kind, lane, fp8_src_aligned(it), cw8);
  const uint32_t off = (uint32_t)mt;
  const uint32_t tags = (uint32_t)(mt >> 32);
  const bool raw = tags == kFp8TagsRaw;
  if (off == KVZ_OFF_NONE || (uint64_t)off + run_granules(n_raw_of(tags)) > capacity) return;
  uint8_t* rec = arena + (size_t)off * kFp8Granule;
  if (raw) {
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<uint2*>(rec + fp8_chunk_offset(j, lane)) = cw8[j];
    return;
  }
  Fp8GroupCode g[4];
  uint32_t esc_len = 0, modes = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t b3lo, b3hi, b4lo, b4hi;
    fp8_group_bases(it.bases, it.kind, j, lane, b3lo, b3hi, b4lo, b4hi);
    g[j] = fp8_code_group<FK>(cw8[j], b3lo, b3hi, b4lo, b4hi);
    esc_len += fp8_escape_bytes<FK>(g[j].mode);
    modes |= g[j].mode << (2 * j);
  }
  uint32_t w[4];
  fp8_sm_pack<FK>(g, w);
  uint32_t* sp = reinterpret_cast<uint32_t*>(rec + F::kSmLane * lane);
#pragma unroll
  for (int t = 0; t < (int)(F::kSmLane / 4); ++t) sp[t] = w[t];
  uint8_t code_bytes[12];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int k = 0; k < 3; ++k) code_bytes[3 * j + k] = (uint8_t)(g[j].low24 >> (8 * k));
  uint32_t* cp = reinterpret_cast<uint32_t*>(rec + F::kCodeOff + 12 * lane);
#pragma unroll
  for (int k = 0; k < 3; ++k)
    cp[k] = (uint32_t)code_bytes[4 * k] | ((uint32_t)code_bytes[4 * k + 1] << 8) |
            ((uint32_t)code_bytes[4 * k + 2] << 16) | ((uint32_t)code_bytes[4 * k + 3] << 24);
  rec[F::kModeOff + lane] = (uint8_t)modes;
  // escape bytes: lanes in order, groups in order
  uint32_t at = F::kEscOff + gaac_exclusive_scan(esc_len, lane);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t nb = fp8_escape_bytes<FK>(g[j].mode);
    for (uint32_t k = 0; k < nb; ++k) rec[at + k] = (uint8_t)(g[j].esc >> (8 * k));
    at += nb;
  }
}

// ---------------------------------------------------------------------------------------------
// Decompress-first and the uncompressed layout
// ---------------------------------------------------------------------------------------------
template <int FK>
__global__ __launch_bounds__(256) void fp8_decompress_kernel(const uint8_t* arena,
                                                             uint64_t arena_bytes,
                                                             const kvz_group_meta* meta,
                                                             const uint8_t* bases,
                                                             int64_t n_tiles, int hkv,
                                                             uint8_t* dst) {
  using F = Fp8Fmt<FK>;
  const int lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // output tile index
  if (g >= n_tiles) return;
  const int64_t page = g / (2 * hkv);
  const int rem = (int)(g % (2 * hkv));
  const uint32_t kind = (uint32_t)(rem / hkv);
  const int kvh = rem % hkv;
  const kvz_group_meta m = meta[(page * hkv + kvh) * 2 + kind];
  const uint32_t tags = *reinterpret_cast<const uint32_t*>(m.tag);
  const bool raw = tags == kFp8TagsRaw;
  const uint64_t start = (uint64_t)m.off * kFp8Granule;
  uint8_t* out = dst + g * kFp8RawTile;
  const bool known = raw || tags == F::kTagsComp;
  if (m.off == KVZ_OFF_NONE || !known || start + (raw ? kFp8RawTile : F::kSlot) > arena_bytes) {
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<uint2*>(out + fp8_chunk_offset(j, lane)) = make_uint2(0, 0);
    return;
  }
  const uint8_t* rec = arena + start;
  if (raw) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<uint2*>(out + fp8_chunk_offset(j, lane)) =
          *reinterpret_cast<const uint2*>(rec + fp8_chunk_offset(j, lane));
    return;
  }
  const uint8_t* tb = bases + (size_t)(kvh * 2 + kind) * 256;
  uint32_t w[4] = {0, 0, 0, 0};
  const uint32_t* sp = reinterpret_cast<const uint32_t*>(rec + F::kSmLane * lane);
#pragma unroll
  for (int t = 0; t < (int)(F::kSmLane / 4); ++t) w[t] = sp[t];
  const uint32_t* cp = reinterpret_cast<const uint32_t*>(rec + F::kCodeOff + 12 * lane);
  const uint32_t cw[3] = {cp[0], cp[1], cp[2]};
  const uint32_t modes = rec[F::kModeOff + lane];
  uint32_t esc_len = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) esc_len += fp8_escape_bytes<FK>((modes >> (2 * j)) & 3u);
  uint32_t at = F::kEscOff + gaac_exclusive_scan(esc_len, lane);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t mode = (modes >> (2 * j)) & 3u;
    const uint32_t nb = fp8_escape_bytes<FK>(mode);
    uint32_t esc = 0;
    for (uint32_t k = 0; k < nb; ++k)      // never past the slot, whatever the mode plane says
      if (at + k < F::kSlot) esc |= (uint32_t)rec[at + k] << (8 * k);
    at += nb;
    uint32_t b3lo, b3hi, b4lo, b4hi;
    fp8_group_bases(tb, kind, j, lane, b3lo, b3hi, b4lo, b4hi);
    uint32_t X, Y;
    fp8_sm_xy<FK>(w, j, X, Y);
    const uint32_t low24 = gaac_low24(cw, j);
    constexpr uint32_t kMw = F::kFracBits;   // codes and bases in the exponent field
    *reinterpret_cast<uint2*>(out + fp8_chunk_offset(j, lane)) = fp8_restore_group<FK>(
        X, Y, gaac_spread3(low24 & 0xFFFu) << kMw, gaac_spread3(low24 >> 12) << kMw, mode, esc,
        b3lo << kMw, b3hi << kMw, b4lo << kMw, b4hi << kMw, true);
  }
}

// Natural FP8 pages [n][2][Hkv][16][128] -> [n][2][Hkv][2048] in the FP8 chunk layout.
__global__ __launch_bounds__(256) void fp8_pack_pages_kernel(const uint8_t* src, uint8_t* dst,
                                                             int64_t n_tiles, int hkv) {
  const int lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= n_tiles) return;
  const uint32_t kind = (uint32_t)((g / hkv) % 2);
  const uint8_t* tile = src + g * kFp8RawTile;
  uint8_t* out = dst + g * kFp8RawTile;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<uint2*>(out + fp8_chunk_offset(j, lane)) = fp8_load_chunk(tile, 128, kind, j, lane, true);
}

bool fp8_format_ok(uint32_t format) { return format == KVZ_FP8_E4M3 || format == KVZ_FP8_E5M2; }

}  // namespace
}  // namespace kvz

using namespace kvz;

extern "C" int kvz_fp8_calibrate(const kvz_fp8_item* d_items, int32_t n, uint32_t format,
                                 uint32_t* d_hist, uint8_t* d_bases, hipStream_t s) {
  if (n < 0) return set_error(KVZ_EINVAL, "n < 0");
  if (!fp8_format_ok(format)) return set_error(KVZ_EINVAL, "unknown FP8 format");
  if (!d_hist || !d_bases || (n > 0 && !d_items)) return set_error(KVZ_EINVAL, "null pointer argument");
  if (((uintptr_t)d_hist) & 3u) return set_error(KVZ_EINVAL, "hist must be 4-byte aligned");
  hipLaunchKernelGGL(fp8_hist_zero_kernel, dim3(16), dim3(256), 0, s, d_hist);
  if (n > 0) {
    if (format == KVZ_FP8_E4M3)
      hipLaunchKernelGGL(fp8_hist_kernel<KVZ_FP8_E4M3>, dim3((n + 3) / 4), dim3(256), 0, s, d_items, (int)n, d_hist);
    else
      hipLaunchKernelGGL(fp8_hist_kernel<KVZ_FP8_E5M2>, dim3((n + 3) / 4), dim3(256), 0, s, d_items, (int)n, d_hist);
  }
  hipLaunchKernelGGL(fp8_pick_kernel, dim3(1), dim3(256), 0, s, d_hist, d_bases,
                     format == KVZ_FP8_E4M3 ? 16 : 32);
  return check_hip(hipGetLastError(), "fp8 calibrate launch");
}

extern "C" int kvz_fp8_encode_pages(kvz_pool* p, const kvz_fp8_item* d_items, int32_t n,
                                    uint32_t format, uint32_t flags, hipStream_t s) {
  if (!p) return set_error(KVZ_EINVAL, "pool handle is null");
  if (p->granule_bytes != KVZ_FP8_GRANULE_BYTES)
    return set_error(KVZ_EINVAL, "FP8 tiles need a pool made by kvz_fp8_pool_init");
  if (!fp8_format_ok(format)) return set_error(KVZ_EINVAL, "unknown FP8 format");
  if (n < 0) return set_error(KVZ_EINVAL, "n < 0");
  if (n == 0) return KVZ_OK;
  if (!d_items) return set_error(KVZ_EINVAL, "items pointer is null");
  if (flags & ~KVZ_ENC_FORCE_RAW) return set_error(KVZ_EINVAL, "unknown encode flag");
  const int grid = (n + 3) / 4;
  const bool stream = n > kStreamItems;
#define KVZ_FP8_LAUNCH(kernel, ...)                                                             \
  do {                                                                                          \
    if (format == KVZ_FP8_E4M3) {                                                               \
      if (stream)                                                                               \
        hipLaunchKernelGGL((kernel<KVZ_FP8_E4M3, kStreamLoad>), dim3(grid), dim3(256), 0, s, __VA_ARGS__); \
      else                                                                                      \
        hipLaunchKernelGGL((kernel<KVZ_FP8_E4M3, kCachedLoad>), dim3(grid), dim3(256), 0, s, __VA_ARGS__); \
    } else {                                                                                    \
      if (stream)                                                                               \
        hipLaunchKernelGGL((kernel<KVZ_FP8_E5M2, kStreamLoad>), dim3(grid), dim3(256), 0, s, __VA_ARGS__); \
      else                                                                                      \
        hipLaunchKernelGGL((kernel<KVZ_FP8_E5M2, kCachedLoad>), dim3(grid), dim3(256), 0, s, __VA_ARGS__); \
    }                                                                                           \
  } while (0)
  KVZ_FP8_LAUNCH(fp8_classify_kernel, d_items, (int)n, flags);
  int rc = check_hip(hipGetLastError(), "fp8 classify launch");
  if (rc != KVZ_OK) return rc;
  rc = launch_alloc_for_fp8_items(p, d_items, n, s);
  if (rc != KVZ_OK) return rc;
  KVZ_FP8_LAUNCH(fp8_pack_kernel, d_items, (int)n, (uint8_t*)p->arena, p->capacity);
#undef KVZ_FP8_LAUNCH
  return check_hip(hipGetLastError(), "fp8 pack launch");
}

extern "C" int kvz_fp8_decompress_pages(const void* d_arena, uint64_t arena_bytes,
                                        const kvz_group_meta* d_meta, const uint8_t* d_bases,
                                        int64_t n_pages, int32_t num_kv_heads, uint32_t format,
                                        uint8_t* d_dst, hipStream_t s) {
  if (n_pages < 0 || num_kv_heads <= 0) return set_error(KVZ_EINVAL, "bad sizes");
  if (!fp8_format_ok(format)) return set_error(KVZ_EINVAL, "unknown FP8 format");
  if (n_pages == 0) return KVZ_OK;
  if (!d_arena || !d_meta || !d_bases || !d_dst) return set_error(KVZ_EINVAL, "null pointer argument");
  if ((((uintptr_t)d_meta) & 7u) || (((uintptr_t)d_dst) & 15u) || (((uintptr_t)d_bases) & 3u) ||
      (((uintptr_t)d_arena) & 15u))
    return set_error(KVZ_EINVAL, "misaligned pointer argument");
  const int64_t n_tiles = n_pages * 2 * num_kv_heads;
  const int64_t grid = (n_tiles + 3) / 4;
  if (grid > 0x7FFFFFFF) return set_error(KVZ_EINVAL, "too many pages for one call");
  if (format == KVZ_FP8_E4M3)
    hipLaunchKernelGGL(fp8_decompress_kernel<KVZ_FP8_E4M3>, dim3((unsigned)grid), dim3(256), 0, s,
                       (const uint8_t*)d_arena, arena_bytes, d_meta, d_bases, n_tiles,
                       (int)num_kv_heads, d_dst);
  else
    hipLaunchKernelGGL(fp8_decompress_kernel<KVZ_FP8_E5M2>, dim3((unsigned)grid), dim3(256), 0, s,
                       (const uint8_t*)d_arena, arena_bytes, d_meta, d_bases, n_tiles,
                       (int)num_kv_heads, d_dst);
  return check_hip(hipGetLastError(), "fp8 decompress launch");
}

extern "C" int kvz_fp8_pack_pages(const uint8_t* d_src, uint8_t* d_dst, int64_t n_pages,
                                  int32_t num_kv_heads, hipStream_t s) {
  if (n_pages < 0 || num_kv_heads <= 0) return set_error(KVZ_EINVAL, "bad sizes");
  if (n_pages == 0) return KVZ_OK;
  if (!d_src || !d_dst) return set_error(KVZ_EINVAL, "null pointer argument");
  if ((((uintptr_t)d_src) & 7u) || (((uintptr_t)d_dst) & 7u))
    return set_error(KVZ_EINVAL, "src and dst must be 8-byte aligned");
  const int64_t n_tiles = n_pages * 2 * num_kv_heads;
  const int64_t grid = (n_tiles + 3) / 4;
  if (grid > 0x7FFFFFFF) return set_error(KVZ_EINVAL, "too many pages for one call");
  hipLaunchKernelGGL(fp8_pack_pages_kernel, dim3((unsigned)grid), dim3(256), 0, s, d_src, d_dst,
                     n_tiles, (int)num_kv_heads);
  return check_hip(hipGetLastError(), "fp8 pack pages launch");
}
