// Paged split-K GQA decode attention over losslessly compressed KV pages (three formats, each
// restored bit-exactly in registers), and the same kernel over uncompressed BF16 and FP8 pages
// (the baselines).
//
// Follows "GAAC: Lossless KV Compression for Bandwidth-Efficient LLM Inference on Personal
// Devices", section "Attention with On-the-Fly Decompression": compressed tiles and their
// metadata are read, BF16 is rebuilt only for the working tile and used at once for the scores
// and the weighted sum of values, and compressed pages and the BF16 tail share one softmax.
// The restore and the K/V operand layouts follow "ZipFusion: Fusing Lossless KV Decompression
// with Attention for Efficient LLM Decoding", section "How it works".
//
// Five page formats share the kernel: BF16 (the baseline), the exponent-coded 12-bit pages, the
// group-adaptive additive code ("GAAC: ...", section "Lossless KV Compression"), whose tiles are
// rebuilt with calibrated per-dim bases, and FP8 pages (E4M3 / E5M2) uncompressed or in the same
// group-adaptive code on the FP8 exponent field ("GAAC: ...", appendix "Relation to FP8 KV"),
// converted exactly to BF16 in registers for the MFMA products.
//
// Work decomposition (one workgroup = one unit = (sequence b, KV head, split s)):
//   * a unit covers a contiguous range of its sequence's pages (the tail page counts as the
//     last page); each of its waves (8 for groups of up to 4 query heads, else 4) walks one
//     consecutive part; per page a wave loads the four K and four V blocks of its KV head (16
//     bytes per lane per block: a compressed chunk is 12 bytes and the next 4 are ignored),
//     restores them in registers, and runs
//       S[16 tokens x 16 heads] = K_page(16x128) . Q^T   as 4 x v_mfma_f32_16x16x32_bf16,
//       O[32 rows x 128]       += P(32x16) . V_page    as 4 x v_mfma_f32_32x32x16_bf16,
//     with P split into bf16 hi + lo parts (rows h and 16 + h of P for head h) so that P is
//     carried to ~2^-17 relative;
//   * the query group (G <= 16 heads sharing the KV head) is the MFMA's head dimension;
//   * online softmax in base 2 per head; rows of O are rescaled only when a head's max rises;
//   * the waves' (m, l, O) are merged in LDS; a unit then writes the normalized output (one
//     split per sequence: no further launch) or its partial, merged in the kernel by the last
//     piece to finish (up to 4 splits) or by attn_combine.
#include "fp8_internal.h"

#include <math.h>

#include <algorithm>
#include <mutex>

namespace kvz {

namespace {

constexpr int kFmtBf16 = 0;   // uncompressed pages (baseline)
constexpr int kFmtZf = 1;     // exponent-coded 12-bit pages
constexpr int kFmtGaac = 2;   // group-adaptive additive code
constexpr int kFmtFp8 = 3;    // uncompressed FP8 pages (the FP8 baseline)
constexpr int kFmtFp8c = 4;   // exponent-coded FP8 tiles

// What an attention kernel instance computes: everything, or for the time breakdown only the
// page loads, or the loads and the restore (values of KVZ_PART_* in the public header).
constexpr int kModeFull = 0;
constexpr int kModeLoad = 1;
constexpr int kModeRestore = 2;

struct AttnParams {
  const uint16_t* q;
  const uint8_t* kv;            // pool arena (compressed) or BF16 pages (baseline)
  const uint4* meta;            // [phys][Hkv] : {K off, K tags, V off, V tags}; compressed only
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* n_comp;
  const void* tail;             // BF16 or (FP8 formats) FP8 [B][2][Hkv][16][128]
  const uint8_t* bases;         // GAAC / FP8 tiles: [Hkv][2 (K,V)][2 (b3,b4)][128]
  float* out;                   // [B][Hq][128]
  float* ws_ml;                 // [units][G][2]
  float* ws_o;                  // [units][G][128]
  uint32_t* ws_cnt;             // [Hkv][B] pieces of (sequence, KV head) done; zero between calls
  uint32_t* ws_status;          // sticky flags (KVZ_WS_*): a counter found outside [0, pieces)
  int merge_in_kernel;          // the last piece of a (sequence, KV head) merges (no second launch)
  uint64_t arena_bytes;         // compressed only: groups must end 16 bytes before this
  int B, Hq, Hkv, G, max_pages, S, n_phys;
  float scale_log2;             // sm_scale (* k_scale for FP8) * log2(e)
  float v_scale;                // FP8 formats: the output is multiplied by it
};

struct KV8 {
  uint4 k[4];
  uint4 v[4];
};

// One GAAC tile as loaded: four 16-byte chunks (raw tile: the BF16 chunks; compressed: the
// lane's 8 sign+fraction bytes in the low half), the lane's 12 code bytes, the dword holding
// its mode byte and one dword of the escape area.
struct GaacTileLoad {
  uint4 c[4];
  uint32_t code[3];
  uint32_t mode;
  uint32_t esc;
};
struct GaacPage {
  GaacTileLoad k, v;
};

// One FP8 tile as loaded: a = the lane's sign+fraction words (compressed) or blocks 0,1
// (uncompressed), b = its 12 code bytes (+4 unused) or blocks 2,3, the dword holding its mode
// byte and one dword of the escape area (compressed only).
struct Fp8TileLoad {
  uint4 a, b;
  uint32_t mode;
  uint32_t esc;
};
struct Fp8Page {
  Fp8TileLoad k, v;
};
struct Fp8RawPage {
  uint4 k[2], v[2];
};

template <int FMT>
struct PageBufOf {
  using type = KV8;
};
template <>
struct PageBufOf<kFmtGaac> {
  using type = GaacPage;
};
template <>
struct PageBufOf<kFmtFp8> {
  using type = Fp8RawPage;
};
template <>
struct PageBufOf<kFmtFp8c> {
  using type = Fp8Page;
};

__device__ __forceinline__ float lane_xor(float x, int m) { return __shfl_xor(x, m, 64); }

// XOR of the 32-bit words of a register value (keeps the breakdown variants' loads and restores
// from being removed as unused).
template <typename T>
__device__ __forceinline__ uint32_t fold_words(const T& x) {
  static_assert(sizeof(T) % 4 == 0, "whole words");
  const uint32_t* w = reinterpret_cast<const uint32_t*>(&x);
  uint32_t a = 0;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i) a ^= w[i];
  return a;
}

// max over this lane and lane^16 (v_permlane16_swap: rows 0<->1 and 2<->3 exchange)
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// max over this lane and lane^32 (v_permlane32_swap: lanes 0-31 <-> 32-63)
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// value of lane+16 in rows 0 and 2 (rows 1 and 3 keep their own)
__device__ __forceinline__ uint32_t from_next_row(uint32_t x) {
  return __builtin_amdgcn_permlane16_swap(x, x, false, false)[1];
}

__device__ __forceinline__ uint4 load16(const uint8_t* p) {
  uint4 r;
  __builtin_memcpy(&r, __builtin_assume_aligned(p, 4), 16);
  return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Two wait states, issued as an instruction of their own, between restored operands and the
// matrix instructions that read them.  A VALU write of a VGPR must be at least two wait states
// ahead of an MFMA that reads it.  Where the restored operands reach the products through a
// join of the restore's branches (register copies at the end of each branch), the compiler was
// seen to meet that distance with a copy, an s_waitcnt for the loads of the uncompressed branch
// and one s_nop: counting the s_waitcnt as a wait state.  On the GPU that left the product
// reading a stale operand register for some pages (compressed and uncompressed tiles of equal
// values gave different scores).  With this nop ahead of the waitcnt the distance holds without
// it; a build check keeps such padding out of every kernel.  The operands pass through the asm
// statement, so the products cannot be scheduled above it.
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void operands_settled(uint4 (&ops)[4]) {
  u32x4v a = __builtin_bit_cast(u32x4v, ops[0]), b = __builtin_bit_cast(u32x4v, ops[1]);
  u32x4v c = __builtin_bit_cast(u32x4v, ops[2]), d = __builtin_bit_cast(u32x4v, ops[3]);
  asm volatile("s_nop 1" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
  ops[0] = __builtin_bit_cast(uint4, a);
  ops[1] = __builtin_bit_cast(uint4, b);
  ops[2] = __builtin_bit_cast(uint4, c);
  ops[3] = __builtin_bit_cast(uint4, d);
}

// The same two wait states for one operand (the P operand of the PV products).
__device__ __forceinline__ void operand_settled(uint4& op) {
  u32x4v a = __builtin_bit_cast(u32x4v, op);
  asm volatile("s_nop 1" : "+v"(a));
  op = __builtin_bit_cast(uint4, a);
}

// Ten wait states ahead of the first read of a page's scores, after the V restore.  A VALU read
// of a 16x16x32 product's result must be at least eight wait states after it.  Where an
// uncompressed V block skips the V restore, the products were followed by a branch to the
// block that reads the scores, and the compiler put nothing in between: the first compare then
// read a score register before the last product had written it (the partial sum of the first
// three products), so the choice of the exact score path for a page changed from run to run on
// uncompressed tiles.  The scores pass through the asm statement, so every later read is of its
// output, and the nops lie on every path from the products to those reads.  (Right after the
// products, the statement would also keep the V restore from overlapping their latency.)
__device__ __forceinline__ void scores_settled(f32x4& sacc) {
  asm volatile("s_nop 7\n\ts_nop 1" : "+v"(sacc));
}

// Raw buffer resource over [base, base + bytes); loads beyond `bytes` return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t group_rsrc(const uint8_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, (int)bytes, 0x00020000);
}

// KV pages are read exactly once per call: load them non-temporally (cache-policy bit "nt"),
// which keeps the streaming data from displacing reusable lines and measured ~15% faster.
constexpr int kStreamLoad = 2;

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kStreamLoad));
}

// Bytes of a group with these four tags: 768 per compressed block, 1024 per raw block.
__device__ __forceinline__ uint32_t group_bytes(uint32_t tags) {
  return 4 * kCompBlockBytes + 256u * (uint32_t)__popc(tags & 0x80808080u);
}

__device__ __forceinline__ float readlane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

__device__ __forceinline__ uint4 restore_if_coded(uint4 c, uint32_t tag) {
  if (tag == KVZ_RAW_TAG) return c;
  return restore_chunk(c.x, c.y, c.z, tag * 0x01010101u);
}

// A difference of raw scores in log2 units (a product of its own, never fused with the
// subtraction before it: the largest score of a page then gives exactly exp2(0) = 1).
__device__ __forceinline__ float to_log2(float d, float c) {
#pragma clang fp contract(off)
  return d * c;
}

// Scores are kept in raw units (q.k, before the softmax scale) until the running max is
// subtracted; the scale to log2 units is applied to the difference, so the rounding of a
// large score times the scale never enters the weights.
//
// Pages with very large scores.  The bf16 matrix instruction sums its 32 products with an error
// of a few units in the last place of the largest product (measured up to ~6 ulp on gfx950), so
// a score of magnitude M carries an absolute error of ~6 M 2^-24.  Near 1e4 in log2 units (keys
// holding sigma * 2^12 outliers against unit queries) two nearly tied top scores then get softmax
// weights ~0.5% off.  On such pages (rare: none on data without outliers) the scores are
// recomputed as an exact pair: the K values are split by magnitude into "big" elements (those
// whose product with the largest query value can reach 2^9) and the rest, each half goes
// through the same four products, and the score is carried as big + small.  The big half of a
// row normally holds one product, which the instruction returns exactly; the small half's error
// is a few ulp of 2^9.
constexpr float kPreciseScoreMin = 256.f;   // in log2 units: scores this large take the pair path

typedef short i16x2 __attribute__((ext_vector_type(2)));

// The exponent-field threshold (in bits 7..14 of each bf16 half, replicated to both halves)
// from which a K value counts as big: with q_e the largest biased exponent of the wave's query
// values, |q| < 2^(q_e - 126); a K value of biased exponent e has |k| < 2^(e - 126), so below the
// threshold T = 262 - q_e every product is smaller than 2^(261 - q_e + q_e - 252) = 2^9.
__device__ __forceinline__ uint32_t big_threshold(const uint4 (&qop)[4]) {
  uint32_t e = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w[4] = {qop[j].x, qop[j].y, qop[j].z, qop[j].w};
#pragma unroll
    for (int m = 0; m < 4; ++m) e = max(e, max((w[m] >> 7) & 0xFFu, (w[m] >> 23) & 0xFFu));
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) e = max(e, (uint32_t)__shfl_xor((int)e, d, 64));
  int t = 262 - (int)e;
  t = t < 0 ? 0 : (t > 255 ? 255 : t);
  return ((uint32_t)t << 7) * 0x00010001u;
}

// Split one dword of two bf16 values: small keeps the values whose exponent field is below the
// threshold, big the others (small + big = w, one of each pair zero).
__device__ __forceinline__ void split_big(uint32_t w, uint32_t thr2, uint32_t& small, uint32_t& big) {
  const i16x2 e = __builtin_bit_cast(i16x2, w & 0x7F807F80u);
  const i16x2 below = (e - __builtin_bit_cast(i16x2, thr2)) >> (i16x2){15, 15};   // 0xFFFF where e < thr
  small = w & __builtin_bit_cast(uint32_t, below);
  big = w ^ small;
}

// A page's raw scores as the exact pair big + small (see above).
__device__ __forceinline__ void split_scores(const uint4 (&kops)[4], const uint4 (&qop)[4], uint32_t thr2,
                                             float (&hi)[4], float (&lo)[4]) {
  f32x4 sb = {0.f, 0.f, 0.f, 0.f}, ss = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint4 ks, kb;
    split_big(kops[j].x, thr2, ks.x, kb.x);
    split_big(kops[j].y, thr2, ks.y, kb.y);
    split_big(kops[j].z, thr2, ks.z, kb.z);
    split_big(kops[j].w, thr2, ks.w, kb.w);
    sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kb), as_bf16x8(qop[j]), sb, 0, 0, 0);
    ss = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ks), as_bf16x8(qop[j]), ss, 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    hi[r] = sb[r];
    lo[r] = __builtin_isfinite(sb[r]) ? ss[r] : 0.f;   // non-finite scores as on the plain path
  }
}

// The largest of a page's scores per head (every lane of head lane%16 gets it).
__device__ __forceinline__ float page_max(const float (&sv)[4]) {
  float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
  mx = max_xor16(mx);
  return max_xor32(mx);
}

// Whether a page's raw scores need the pair: some valid score is at least big_min (=
// kPreciseScoreMin in log2 units) in magnitude and no more than near (= 40 in log2 units, 2^-40
// in weight) below its head's running max before this page (a score further below carries no
// weight in fp32; one above it is a new max).  Non-finite scores may take the pair too (their
// low half is zero).  Written without short-circuit operators, so that it compiles to compares
// and one scalar branch.  Wave-uniform.
__device__ __forceinline__ bool needs_precise(const float (&sv)[4], float m_run, float big_min, float near) {
  const float floor = m_run - near;
  uint32_t big = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) big |= (uint32_t)(fabsf(sv[r]) >= big_min) & (uint32_t)(sv[r] >= floor);
  return __ballot(big != 0u) != 0ull;
}

template <int GB>
struct Softmax {
  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x16 o[4];

  __device__ Softmax() {
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = f32x16{};
  }

  // sv: raw scores q.k of this lane (tokens 4*(lane/16)+r, head lane%16), already
  // valid-masked (-inf); sl: what the score is beyond sv (zero, or the small half of a split
  // score: score = sv + sl); mx: page_max of the scores; c: the scale to log2 units
  // (sm_scale * log2(e)).  The running max m_run is in raw units.  vop: the four V chunks of
  // the page in operand order.
  __device__ __forceinline__ void page(const float (&sv)[4], const float (&sl)[4], float mx,
                                       const uint4 (&vop)[4], int lane, float c) {
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(to_log2(m_run - m_use, c));
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = __builtin_amdgcn_exp2f(to_log2((sv[r] - m_use) + sl[r], c));
    l_run = l_run * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    m_run = m_new;
    if (__ballot(alpha != 1.0f)) rescale(alpha, lane);

    // P as the row operand of one 32x32x16 product per V chunk: hi = bf16(p) and lo =
    // bf16(p - hi), both rounded to nearest even, in rows 0-15 (hi) and 16-31 (lo) for heads
    // 0-15, so that O rows h and 16 + h accumulate the two halves (added up by fold()).  Lane l
    // holds row l%32 and tokens 8*(l/32)+0..7; this lane has tokens 4*(l/16)+0..3 of head l%16
    // and lane l^16 the other four of its eight: a lane of rows 0-15 takes that lane's hi, a lane
    // of rows 16-31 its lo, in one exchange per pair of tokens.
    // (each pair converted by one packed instruction, round to nearest even as for one value)
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    uint32_t hi[2], lo[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const f32x2_t pp = {pr[2 * m], pr[2 * m + 1]};
      hi[m] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pp, bf16x2_t));
      const f32x2_t rr = {pp[0] - __uint_as_float(hi[m] << 16), pp[1] - __uint_as_float(hi[m] & 0xFFFF0000u)};
      lo[m] = __builtin_bit_cast(uint32_t, __builtin_convertvector(rr, bf16x2_t));
    }
    const bool lo_rows = (lane & 16) != 0;
    // v_permlane16_swap of a value with itself: result [1] gives rows 0 and 2 of lanes the values
    // of rows 1 and 3, result [0] gives rows 1 and 3 the values of rows 0 and 2
    const auto x0 = __builtin_amdgcn_permlane16_swap(lo_rows ? hi[0] : lo[0], lo_rows ? hi[0] : lo[0], false, false);
    const auto x1 = __builtin_amdgcn_permlane16_swap(lo_rows ? hi[1] : lo[1], lo_rows ? hi[1] : lo[1], false, false);
    const uint32_t got0 = lo_rows ? x0[0] : x0[1];
    const uint32_t got1 = lo_rows ? x1[0] : x1[1];
    uint4 a;
    a.x = lo_rows ? got0 : hi[0];
    a.y = lo_rows ? got1 : hi[1];
    a.z = lo_rows ? lo[0] : got0;
    a.w = lo_rows ? lo[1] : got1;
    operand_settled(a);   // the same VALU -> MFMA distance as for the score operands
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(vop[j]), o[j], 0, 0, 0);
  }

  // O rows 16-31 (the lo halves) added into rows 0-15: register r + 8 holds row 16 + the row
  // of register r.  Once, after the last page.
  __device__ __forceinline__ void fold() {
    constexpr int NR = GB <= 8 ? 4 : 8;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < NR; ++r) o[j][r] += o[j][r + 8];
  }

  // O tile register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4 (a query head of the group).
  __device__ __forceinline__ void rescale(float alpha, int lane) {
    constexpr int NR = GB <= 8 ? 4 : 8;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int row_lo = 8 * (r / 4) + (r % 4);
      const float a_lo = readlane_f(alpha, row_lo);
      float a = a_lo;
      if constexpr (GB > 4) {
        const float a_hi = readlane_f(alpha, row_lo + 4);
        a = lane < 32 ? a_lo : a_hi;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[j][r] *= a;
        o[j][r + 8] *= a;
      }
    }
  }
};

constexpr int kMaxSplits = 4096;
// Merging in the attention kernel: for automatic or given split counts up to this.
constexpr int kInKernelMergeMax = 4;

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// Balanced split-K.  The B*S splits of a KV head are shared by page count: sequence b is cut
// into S_b = ceil(T_b / P) pieces of at most P pages, with P the smallest piece size for which
// the S_b add up to at most B*S (searched between ceil(W / (B*S)) and ceil(W / (B*S - B)),
// which always fits; W = the batch's pages per KV head; beyond 64 sequences the upper bound is
// used).  A long sequence gets more pieces than a short one, so one long sequence no longer
// sets the kernel time.  With equal lengths S_b = S and the pieces are exactly the uniform ones
// (that case skips the search, at any batch size); with S = 1 every sequence keeps one piece.
// Sequence b owns splits [base_b, base_b + S_b); the rest stay unused.  Computed by one whole
// wave (every lane gets the result); the sequence's clamped n_comp and tail tokens come with it.
struct SplitOf {
  int b;       // sequence (-1: unused split)
  int base;    // first split of the sequence
  int sb;      // splits of the sequence
  int total;   // its pages
  int n_comp;  // its compressed pages, clamped to [0, max_pages]
  int n_tail;  // its tail tokens, clamped to [0, 16] (0 without a tail buffer)
};

__device__ __forceinline__ void seq_counts(const int32_t* n_comp_v, const int32_t* seq_lens,
                                           bool has_tail, int max_pages, int b, int& n, int& t) {
  n = n_comp_v[b];
  n = n < 0 ? 0 : (n > max_pages ? max_pages : n);
  t = 0;
  if (has_tail) {
    t = seq_lens[b] - 16 * n;
    t = t < 0 ? 0 : (t > 16 ? 16 : t);
  }
}

__device__ __forceinline__ SplitOf split_of(const int32_t* n_comp_v, const int32_t* seq_lens,
                                            bool has_tail, int max_pages, int B, int S, int k,
                                            int want_b) {
  const int lane = threadIdx.x & 63;
  SplitOf r{-1, 0, 0, 0, 0, 0};
  // pass 1: W, and whether every sequence has the same page count
  int64_t W = 0;
  bool uniform = true;
  int t0 = -1;
  int T_first = 0;                   // this lane's page count in the first 64 sequences
  for (int c0 = 0; c0 < B; c0 += 64) {
    const int b = c0 + lane;
    int n = 0, t = 0;
    if (b < B) seq_counts(n_comp_v, seq_lens, has_tail, max_pages, b, n, t);
    int T = n + (t > 0 ? 1 : 0);
    if (c0 == 0) T_first = T;
    if (t0 < 0) t0 = __builtin_amdgcn_readfirstlane(T);
    uniform = uniform && !__ballot(b < B && T != t0);
    if (B <= 64 && (uniform || S == 1)) {   // S_b = S, base_b = b * S
      const int bb = want_b >= 0 ? want_b : k / S;
      if (bb >= B) return r;
      r.b = bb;
      r.base = bb * S;
      r.sb = S;
      r.total = __builtin_amdgcn_readlane(T, bb);
      r.n_comp = __builtin_amdgcn_readlane(n, bb);
      r.n_tail = __builtin_amdgcn_readlane(t, bb);
      return r;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) T += __shfl_xor(T, d, 64);
    W += T;
  }
  if (uniform || S == 1) {               // more than 64 sequences: the same uniform pieces
    const int bb = want_b >= 0 ? want_b : k / S;
    if (bb >= B) return r;
    int n, t;
    seq_counts(n_comp_v, seq_lens, has_tail, max_pages, bb, n, t);
    r.b = bb;
    r.base = bb * S;
    r.sb = S;
    r.total = n + (t > 0 ? 1 : 0);
    r.n_comp = n;
    r.n_tail = t;
    return r;
  }
  // the piece size: smallest P whose pieces fit the B*S splits
  const int64_t BS = (int64_t)B * S;
  int64_t P = 1;
  if (S > 1 && W > 0) {
    int64_t lo = (W + BS - 1) / BS;
    int64_t hi = (W + (BS - B) - 1) / (BS - B);      // sum of ceil(T/hi) <= W/hi + B <= BS
    if (B <= 64) {
      while (lo < hi) {
        const int64_t mid = (lo + hi) / 2;
        int c = T_first > 0 ? (int)((T_first + mid - 1) / mid) : 1;
        c = c > kMaxSplits ? kMaxSplits : c;
        if (lane >= B) c = 0;
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) c += __shfl_xor(c, d, 64);
        if (c <= BS) hi = mid;
        else lo = mid + 1;
      }
    }
    P = hi;
  }
  // pass 2: prefix sums of S_b, find the owner
  int base = 0;
  for (int c0 = 0; c0 < B; c0 += 64) {
    const int b = c0 + lane;
    int n = 0, t = 0, T = 0, sb = 0;
    if (b < B) {
      seq_counts(n_comp_v, seq_lens, has_tail, max_pages, b, n, t);
      T = n + (t > 0 ? 1 : 0);
      sb = S == 1 ? 1 : (T > 0 ? (int)((T + P - 1) / P) : 1);
      sb = sb > kMaxSplits ? kMaxSplits : sb;
    }
    const int incl = wave_incl_scan(sb) + base;
    const int start = incl - sb;
    const bool mine = b < B && (want_b >= 0 ? b == want_b : (k >= start && k < incl));
    const uint64_t m = __ballot(mine);
    if (m) {
      const int src = __builtin_ctzll(m);
      r.b = __builtin_amdgcn_readlane(b, src);
      r.base = __builtin_amdgcn_readlane(start, src);
      r.sb = __builtin_amdgcn_readlane(sb, src);
      r.total = __builtin_amdgcn_readlane(T, src);
      r.n_comp = __builtin_amdgcn_readlane(n, src);
      r.n_tail = __builtin_amdgcn_readlane(t, src);
      return r;
    }
    base = __builtin_amdgcn_readlane(incl, 63);
  }
  return r;
}

template <int GB, int FMT, int FK = 0, int MODE = kModeFull, int NW = 4>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_split_kernel(AttnParams p) {
  // COMP: pages are found through the pool metadata (exponent-coded, GAAC or FP8 tiles)
  constexpr bool COMP = FMT == kFmtZf || FMT == kFmtGaac || FMT == kFmtFp8c;
  constexpr bool IS_FP8 = FMT == kFmtFp8 || FMT == kFmtFp8c;
  constexpr bool CODED = FMT == kFmtGaac || FMT == kFmtFp8c;   // group-adaptive modes
  using PageBuf = typename PageBufOf<FMT>::type;
  // group-adaptive tiles: a 16 KiB table from four packed 3-bit codes to four bytes, filled by
  // the whole workgroup before any wave leaves (one LDS read replaces the bit-field spreading)
  // (FP8 tiles: entries and bases are kept shifted into the FP8 exponent field)
  constexpr uint32_t kFieldShift = FMT == kFmtFp8c ? Fp8Fmt<FK>::kFracBits : 0u;
  __shared__ uint32_t s_spread3[CODED ? 4096 : 1];
  if constexpr (CODED) {
    for (int x = threadIdx.x; x < 4096; x += 64 * NW) s_spread3[x] = gaac_spread3((uint32_t)x) << kFieldShift;
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // unit = kvh * U + k = the workgroup: split k of KV head kvh, whose page range its four waves
  // divide into four consecutive quarters (merged in LDS at the end)
  const int unit = blockIdx.x;
  const int U = p.B * p.S;                 // splits per KV head
  if (unit >= U * p.Hkv) return;
  const int kvh = unit / U;
  const int k = unit % U;
  const SplitOf so = split_of(p.n_comp, p.seq_lens, p.tail != nullptr, p.max_pages, p.B, p.S, k,
                              -1);
  if (so.b < 0) return;                    // an unused split
  const int b = so.b;
  const int s = k - so.base;
  const int n_comp = so.n_comp;
  const int n_tail = so.n_tail;
  const int total = so.total;
  const int P0 = (int)(((int64_t)s * total) / so.sb);       // the workgroup's pages
  const int P1 = (int)(((int64_t)(s + 1) * total) / so.sb);
  const int p0 = P0 + (int)(((int64_t)wave * (P1 - P0)) / NW);   // this wave's part
  const int p1 = P0 + (int)(((int64_t)(wave + 1) * (P1 - P0)) / NW);

  // Q as the column operand of the 16x16x32 product: head lane%16, dims 32j + 8*(lane/16) + i.
  const int head = lane & 15;
  uint4 qop[4];
  if (head < p.G) {
    const uint16_t* qrow = p.q + ((size_t)b * p.Hq + (size_t)kvh * p.G + head) * KVZ_HEAD_DIM + 8 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) qop[j] = *reinterpret_cast<const uint4*>(qrow + 32 * j);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) qop[j] = make_uint4(0, 0, 0, 0);
  }

  Softmax<GB> sm;
  uint32_t probe = 0;   // breakdown variants: what their loads and restores produced
  // pages with very large scores (see split_scores): the K split threshold, and the magnitude
  // and the distance below the max that make a score count, in raw units
  const uint32_t big_thr = big_threshold(qop);
  const float c_log2 = p.scale_log2;
  const float big_min = c_log2 > 0.f ? kPreciseScoreMin / c_log2 : INFINITY;
  const float near = c_log2 > 0.f ? 40.f / c_log2 : INFINITY;
  // per-lane byte offsets of a chunk inside a compressed / raw block (loop invariant), so that
  // every page load is "uniform block base (SGPRs) + this offset"
  const uint32_t lane12 = kCompChunkBytes * lane;
  const uint32_t lane16 = kRawChunkBytes * lane;

  // GAAC: the calibrated bases of this lane's values, as bytes.  K chunk (block j) = dims
  // 32j + 8*(lane/16) + 0..7: two dwords per base per block.  V chunk = dim 32j + lane%32 for
  // all eight values: one byte per base per block (byte j of vb3 / vb4).
  uint32_t kb3[4][2], kb4[4][2], vb3 = 0, vb4 = 0;
  if constexpr (CODED) {
    const uint8_t* kbase = p.bases + (size_t)(kvh * 2 + 0) * 256;
    const uint8_t* vbase = p.bases + (size_t)(kvh * 2 + 1) * 256;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int dim = 32 * j + 8 * (lane >> 4);
      const uint2 b3 = *reinterpret_cast<const uint2*>(kbase + dim);
      const uint2 b4 = *reinterpret_cast<const uint2*>(kbase + 128 + dim);
      kb3[j][0] = b3.x << kFieldShift;
      kb3[j][1] = b3.y << kFieldShift;
      kb4[j][0] = b4.x << kFieldShift;
      kb4[j][1] = b4.y << kFieldShift;
      vb3 |= ((uint32_t)vbase[32 * j + (lane & 31)] << kFieldShift) << (8 * j);
      vb4 |= ((uint32_t)vbase[128 + 32 * j + (lane & 31)] << kFieldShift) << (8 * j);
    }
  }
  const int pc_end = p1 < n_comp ? p1 : n_comp;
  // With eight waves, waves w and w + 4 share a SIMD, and the older one wins every contended
  // issue: measured at the 8K layer, waves 0-3 ended their pages at ~56 us and waves 4-7 at
  // ~73 us, the workgroup waiting for the last.  In the kernels over coded pages each such pair
  // publishes its pages done, and the wave behind takes the higher issue priority (timing only:
  // the pages and their order per wave stay the same).  Measured: 8K layer 82.8-83.0 vs
  // 83.4 us, the 2K batch 38.0 vs 39.0, the ragged batch 45.1-45.4 vs 46.2-46.5; the BF16
  // kernel got slower with it (87.1 vs 86.0 us at 8K) and keeps the plain order.
  constexpr bool kBalance = NW == 8 && MODE == kModeFull && COMP;
  __shared__ uint32_t s_done[kBalance ? 8 : 1];
  auto balance = [&](int done) {
    if constexpr (kBalance) {
      __hip_atomic_store(&s_done[wave], (uint32_t)done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      const uint32_t other = __hip_atomic_load(&s_done[wave ^ 4], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if ((uint32_t)done > other)
        __builtin_amdgcn_s_setprio(0);
      else
        __builtin_amdgcn_s_setprio(1);
    }
  };
  balance(0);
  for (int cbase = p0; cbase < pc_end; cbase += 64) {
    const int cnt = (pc_end - cbase) < 64 ? (pc_end - cbase) : 64;
    // lane i describes page cbase + i: its physical page, its two metadata records, and
    // whether the page can be read at all (a page that cannot is skipped)
    int phys_l = 0;
    bool ok_l = false;
    if (lane < cnt) {
      phys_l = p.block_table[(size_t)b * p.max_pages + cbase + lane];
      ok_l = phys_l >= 0 && phys_l < p.n_phys;
      if (!ok_l) phys_l = 0;
    }
    uint4 meta_l = make_uint4(0, 0, 0, 0);
    if constexpr (COMP) {
      if (ok_l) {
        meta_l = p.meta[(size_t)phys_l * p.Hkv + kvh];
        uint64_t kend, vend;
        if constexpr (FMT == kFmtFp8c) {
          using F = Fp8Fmt<FK>;
          kend = (uint64_t)meta_l.x * kFp8Granule + (meta_l.y == kFp8TagsRaw ? kFp8RawTile : F::kSlot);
          vend = (uint64_t)meta_l.z * kFp8Granule + (meta_l.w == kFp8TagsRaw ? kFp8RawTile : F::kSlot);
        } else {
          kend = (uint64_t)meta_l.x * KVZ_GRANULE_BYTES + group_bytes(meta_l.y);
          vend = (uint64_t)meta_l.z * KVZ_GRANULE_BYTES + group_bytes(meta_l.w);
        }
        ok_l = meta_l.x != KVZ_OFF_NONE && meta_l.z != KVZ_OFF_NONE && kend <= p.arena_bytes &&
               vend <= p.arena_bytes;
        if (FMT == kFmtGaac)   // a tile is either compressed (tags 0) or raw (tags all 0xFF)
          ok_l = ok_l && (meta_l.y == 0u || meta_l.y == 0xFFFFFFFFu) &&
                 (meta_l.w == 0u || meta_l.w == 0xFFFFFFFFu);
        if (FMT == kFmtFp8c)   // compressed tags of this FP8 format, or raw
          ok_l = ok_l && (meta_l.y == Fp8Fmt<FK>::kTagsComp || meta_l.y == kFp8TagsRaw) &&
                 (meta_l.w == Fp8Fmt<FK>::kTagsComp || meta_l.w == kFp8TagsRaw);
        if (!ok_l) meta_l = make_uint4(0, 0, 0, 0);   // loads then stay at the arena start
      }
    }
    const uint64_t ok_mask = __ballot(ok_l);

    // Page i of the chunk: one buffer resource per group (base = the group's first block,
    // size = the group's bytes, so the 4-byte over-read of a compressed block's last chunk is
    // clipped by the hardware), block j at a uniform soffset, each lane at its chunk offset.
    // A load that only keeps the loop's shape (`real` false) gets a zero-size resource: the
    // hardware returns zeros without touching memory.
    auto load_gaac_tile = [&](uint32_t off, bool raw, bool real, GaacTileLoad& t) {
      // the same seven loads for a raw and a compressed tile (so every wait is exact); a raw
      // tile's code/mode/escape loads get a zero-size resource and touch no memory
      const uint8_t* base = p.kv + (size_t)off * KVZ_GRANULE_BYTES;
      const __amdgpu_buffer_rsrc_t r = group_rsrc(base, real ? (raw ? 4096u : kGaacSlotBytes) : 0u);
      const __amdgpu_buffer_rsrc_t aux = group_rsrc(base, (real && !raw) ? kGaacSlotBytes : 0u);
      const uint32_t voff = raw ? lane16 : 8u * lane;
      const uint32_t step = raw ? kRawBlockBytes : 512u;
#pragma unroll
      for (int j = 0; j < 4; ++j) t.c[j] = bload16(r, voff, step * j);
      typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
      const u32x3 cw = __builtin_amdgcn_raw_buffer_load_b96(aux, (int)(kGaacCodeOff + 12u * lane), 0, kStreamLoad);
      t.code[0] = cw.x;
      t.code[1] = cw.y;
      t.code[2] = cw.z;
      t.mode = __builtin_amdgcn_raw_buffer_load_b32(aux, (int)(kGaacModeOff + 4u * (lane >> 2)), 0, kStreamLoad);
      t.esc = __builtin_amdgcn_raw_buffer_load_b32(aux, (int)(kGaacEscOff + 4u * (lane & 31)), 0, kStreamLoad);
    };
    // FP8 tile: the same four loads whether it is compressed or not - the lane's 16 bytes at
    // 16c (sign+fraction words, E5M2 ignoring the last 4) or blocks 0,1; its 12 code bytes (+4
    // ignored) or blocks 2,3; the dword holding its mode byte; one dword of the escape area.
    // An uncompressed tile's last two loads get a zero-size resource and touch no memory.
    auto load_fp8_tile = [&](uint32_t off, bool raw, bool real, Fp8TileLoad& t) {
      using F = Fp8Fmt<FK>;
      const uint8_t* base = p.kv + (size_t)off * kFp8Granule;
      const __amdgpu_buffer_rsrc_t r = group_rsrc(base, real ? (raw ? kFp8RawTile : F::kSlot) : 0u);
      const __amdgpu_buffer_rsrc_t aux = group_rsrc(base, (real && !raw) ? F::kSlot : 0u);
      t.a = bload16(r, raw ? 16u * lane : F::kSmLane * lane, 0);
      t.b = bload16(r, raw ? 1024u + 16u * lane : F::kCodeOff + 12u * lane, 0);
      t.mode = __builtin_amdgcn_raw_buffer_load_b32(aux, (int)(F::kModeOff + 4u * (lane >> 2)), 0, kStreamLoad);
      t.esc = __builtin_amdgcn_raw_buffer_load_b32(aux, (int)(F::kEscOff + 4u * (lane & 15)), 0, kStreamLoad);
    };
    auto load_page = [&](int i, PageBuf& r, bool real) {
      real = real && ((ok_mask >> i) & 1ull);   // a page that cannot be read is never touched
      if constexpr (FMT == kFmtFp8c) {
        const uint32_t koff = (uint32_t)__builtin_amdgcn_readlane((int)meta_l.x, i);
        const uint32_t voff = (uint32_t)__builtin_amdgcn_readlane((int)meta_l.z, i);
        const uint32_t kt = (uint32_t)__builtin_amdgcn_readlane((int)meta_l.y, i);
        const uint32_t vt = (uint32_t)__builtin_amdgcn_readlane((int)meta_l.w, i);
        load_fp8_tile(koff, kt == kFp8TagsRaw, real, r.k);
        load_fp8_tile(voff, vt == kFp8TagsRaw, real, r.v);
        return;
      } else if constexpr (FMT == kFmtFp8) {
        const int phys = __builtin_amdgcn_readlane(phys_l, i);
        const uint8_t* kb = p.kv + ((size_t)phys * 2 * p.Hkv + kvh) * kFp8RawTile;
        const __amdgpu_buffer_rsrc_t kr = group_rsrc(kb, real ? kFp8RawTile : 0u);
        const __amdgpu_buffer_rsrc_t vr = group_rsrc(kb + (size_t)p.Hkv * kFp8RawTile, real ? kFp8RawTile : 0u);
        r.k[0] = bload16(kr, 16u * lane, 0);
        r.k[1] = bload16(kr, 1024u + 16u * lane, 0);
        r.v[0] = bload16(vr, 16u * lane, 0);
        r.v[1] = bload16(vr, 1024u + 16u * lane, 0);
        return;
      } else if constexpr (FMT == kFmtGaac) {
        const uint32_t koff = (uint32_t)__builtin_amdgcn_readlane((int)meta_l.x, i);
        const uint32_t voff = (uint32_t)__builtin_amdgcn_readlane((int)meta_l.z, i);
        const uint32_t kt = (uint32_t)__builtin_amdgcn_readlane((int)meta_l.y, i);
        const uint32_t vt = (uint32_t)__builtin_amdgcn_readlane((int)meta_l.w, i);
        load_gaac_tile(koff, kt != 0u, real, r.k);
        load_gaac_tile(voff, vt != 0u, real, r.v);
        return;
      } else {
      __amdgpu_buffer_rsrc_t kr, vr;
      uint32_t kt, vt;
      if constexpr (COMP) {
        const uint32_t koff = (uint32_t)__builtin_amdgcn_readlane((int)meta_l.x, i);
        const uint32_t voff = (uint32_t)__builtin_amdgcn_readlane((int)meta_l.z, i);
        kt = (uint32_t)__builtin_amdgcn_readlane((int)meta_l.y, i);
        vt = (uint32_t)__builtin_amdgcn_readlane((int)meta_l.w, i);
        kr = group_rsrc(p.kv + (size_t)koff * KVZ_GRANULE_BYTES, real ? group_bytes(kt) : 0u);
        vr = group_rsrc(p.kv + (size_t)voff * KVZ_GRANULE_BYTES, real ? group_bytes(vt) : 0u);
      } else {
        const int phys = __builtin_amdgcn_readlane(phys_l, i);
        const uint8_t* kb = p.kv + ((size_t)phys * 2 * p.Hkv + kvh) * 4096;
        kr = group_rsrc(kb, real ? 4096u : 0u);
        vr = group_rsrc(kb + (size_t)p.Hkv * 4096, real ? 4096u : 0u);
        kt = vt = 0xFFFFFFFFu;
      }
      uint32_t ks = 0, vs = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool kraw = ((kt >> (8 * j)) & 0xFFu) == KVZ_RAW_TAG;
        r.k[j] = bload16(kr, kraw ? lane16 : lane12, ks);
        ks += kraw ? kRawBlockBytes : kCompBlockBytes;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool vraw = ((vt >> (8 * j)) & 0xFFu) == KVZ_RAW_TAG;
        r.v[j] = bload16(vr, vraw ? lane16 : lane12, vs);
        vs += vraw ? kRawBlockBytes : kCompBlockBytes;
      }
      }
    };
    // The bases of block j of this lane's values, as bytes (group-adaptive and FP8 tiles).
    auto bases_of = [&](bool is_k, int j, uint32_t& b3lo, uint32_t& b3hi, uint32_t& b4lo,
                        uint32_t& b4hi) {
      if (is_k) {
        b3lo = kb3[j][0];
        b3hi = kb3[j][1];
        b4lo = kb4[j][0];
        b4hi = kb4[j][1];
      } else {
        b3lo = b3hi = __builtin_amdgcn_perm(0u, vb3, 0x01010101u * j);   // byte j, four times
        b4lo = b4hi = __builtin_amdgcn_perm(0u, vb4, 0x01010101u * j);
      }
    };
    // The lane's mode byte (four 2-bit group modes) of a coded tile.
    auto mode_byte = [&](uint32_t mode_dword) { return (mode_dword >> (8 * (lane & 3))) & 0xFFu; };
    // GAAC tile with no raw group in the wave (the common case) -> the four operand chunks.
    // Each lane finds its escape bytes by an exclusive scan of the lanes' escape counts; lanes
    // 0..31 hold the 128-byte escape area as dwords.  A lane has at most four one-byte escapes
    // (one per 4-bit group, i.e. per mode with bit 0 set), all in the two dwords at its first
    // escape byte; the four groups are one straight-line block (no branch), so their dependent
    // chains interleave.
    auto gaac_fast = [&](const GaacTileLoad& t, uint32_t m8, bool is_k, uint4 (&ops)[4]) {
      const uint32_t pos = gaac_exclusive_scan_small(__builtin_popcount(m8 & 0x55u));
      const int q = (int)(pos >> 2);
      const uint32_t d0 = (uint32_t)__shfl((int)t.esc, q, 64);
      const uint32_t d1 = (uint32_t)__shfl((int)t.esc, q + 1, 64);
      uint32_t win = __builtin_amdgcn_alignbit(d1, d0, 8u * (pos & 3u));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t mode = (m8 >> (2 * j)) & 3u;
        const uint32_t esc = win & 0xFFu;        // this group's byte if it is a 4-bit group
        win = mode == kGaacMode4 ? win >> 8 : win;
        uint32_t b3lo, b3hi, b4lo, b4hi;
        bases_of(is_k, j, b3lo, b3hi, b4lo, b4hi);
        const uint32_t low24 = gaac_low24(t.code, j);
        ops[j] = gaac_restore_group_spread(t.c[j].x, t.c[j].y, s_spread3[low24 & 0xFFFu],
                                           s_spread3[low24 >> 12], mode, esc, 0u, b3lo, b3hi,
                                           b4lo, b4hi, false);
      }
    };
    // Any GAAC tile -> the four operand chunks.  With a raw group in the wave a lane has up to
    // 20 escape bytes, fetched group by group (a group's five bytes never reach past the area,
    // so the second dword is always one of the 32).
    auto gaac_ops = [&](const GaacTileLoad& t, bool raw, bool is_k, uint4 (&ops)[4]) {
      if (raw) {
#pragma unroll
        for (int j = 0; j < 4; ++j) ops[j] = t.c[j];
        return;
      }
      const uint32_t m8 = mode_byte(t.mode);
      if (!__ballot((m8 & 0xAAu) != 0u)) {
        gaac_fast(t, m8, is_k, ops);
        return;
      }
      uint32_t len = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) len += gaac_escape_bytes((m8 >> (2 * j)) & 3u);
      uint32_t pos = gaac_exclusive_scan(len, lane);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t mode = (m8 >> (2 * j)) & 3u;
        uint32_t esc = 0, esc_hi = 0;
        if (__ballot(mode != kGaacMode3)) {
          const int q = (int)(pos >> 2);
          const uint32_t d0 = (uint32_t)__shfl((int)t.esc, q, 64);
          const uint32_t d1 = (uint32_t)__shfl((int)t.esc, q + 1, 64);
          const uint32_t sh = 8u * (pos & 3u);
          esc = __builtin_amdgcn_alignbit(d1, d0, sh);
          esc_hi = (sh ? (d1 >> sh) : d1) & 0xFFu;
          if (mode == kGaacMode4) esc &= 0xFFu;
          pos += gaac_escape_bytes(mode);
        }
        uint32_t b3lo, b3hi, b4lo, b4hi;
        bases_of(is_k, j, b3lo, b3hi, b4lo, b4hi);
        const uint32_t low24 = gaac_low24(t.code, j);
        ops[j] = gaac_restore_group_spread(t.c[j].x, t.c[j].y, s_spread3[low24 & 0xFFFu],
                                           s_spread3[low24 >> 12], mode, esc, esc_hi, b3lo, b3hi,
                                           b4lo, b4hi, true);
      }
    };
    // One group of a compressed FP8 tile -> its operand chunk (BF16): sign+fraction bytes from
    // the lane's words, codes from the spread table, exponents rebuilt per byte in the exponent
    // field, then the exact conversion.
    auto fp8_group = [&](const Fp8TileLoad& t, bool is_k, int j, uint32_t mode, uint32_t esc,
                         bool wave_has_raw) {
      uint32_t b3lo, b3hi, b4lo, b4hi;
      bases_of(is_k, j, b3lo, b3hi, b4lo, b4hi);
      const uint32_t w[4] = {t.a.x, t.a.y, t.a.z, t.a.w};
      const uint32_t cw[3] = {t.b.x, t.b.y, t.b.z};
      uint32_t X, Y;
      fp8_sm_xy<FK>(w, j, X, Y);
      const uint32_t low24 = gaac_low24(cw, j);
      const uint2 f = fp8_restore_group<FK>(X, Y, s_spread3[low24 & 0xFFFu], s_spread3[low24 >> 12],
                                            mode, esc, b3lo, b3hi, b4lo, b4hi, wave_has_raw);
      return fp8x8_to_bf16<FK>(f.x, f.y);
    };
    // Compressed FP8 tile with at most one escape byte per group (every E4M3 tile; E5M2 without
    // a raw group in the wave): at most four per lane (E4M3: modes 1 and 2, the two bits of the
    // mode differ; E5M2: mode 1), in the two dwords at its first escape byte (lanes 0..15 hold
    // the 64-byte escape area); the four groups are one straight-line block.
    auto fp8_fast = [&](const Fp8TileLoad& t, uint32_t m8, bool is_k, uint4 (&ops)[4]) {
      const uint32_t ones = FK == KVZ_FP8_E4M3 ? (m8 ^ (m8 >> 1)) & 0x55u : m8 & 0x55u;
      const uint32_t pos = gaac_exclusive_scan_small(__builtin_popcount(ones));
      const int q = (int)(pos >> 2);
      const uint32_t d0 = (uint32_t)__shfl((int)t.esc, q, 64);
      const uint32_t d1 = (uint32_t)__shfl((int)t.esc, q + 1, 64);
      uint32_t win = __builtin_amdgcn_alignbit(d1, d0, 8u * (pos & 3u));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t mode = (m8 >> (2 * j)) & 3u;
        const uint32_t esc = win & 0xFFu;
        win = fp8_escape_bytes<FK>(mode) ? win >> 8 : win;
        ops[j] = fp8_group(t, is_k, j, mode, esc, false);
      }
    };
    // Any FP8 tile -> the four operand chunks.  Uncompressed: each block's 8 bytes are
    // converted.  A raw E5M2 group in the wave: up to 8 escape bytes per lane; three lane
    // shuffles give every lane a 64-bit window from its first escape byte, consumed group by
    // group.
    auto fp8_ops = [&](const Fp8TileLoad& t, bool raw, bool is_k, uint4 (&ops)[4]) {
      if (raw) {
        ops[0] = fp8x8_to_bf16<FK>(t.a.x, t.a.y);
        ops[1] = fp8x8_to_bf16<FK>(t.a.z, t.a.w);
        ops[2] = fp8x8_to_bf16<FK>(t.b.x, t.b.y);
        ops[3] = fp8x8_to_bf16<FK>(t.b.z, t.b.w);
        return;
      }
      const uint32_t m8 = mode_byte(t.mode);
      // E5M2 raw groups escape two bytes; E4M3 groups never more than one
      if (FK == KVZ_FP8_E4M3 || !__ballot((m8 & 0xAAu) != 0u)) {
        fp8_fast(t, m8, is_k, ops);
        return;
      }
      uint32_t len = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) len += fp8_escape_bytes<FK>((m8 >> (2 * j)) & 3u);
      const uint32_t pos = gaac_exclusive_scan(len, lane);
      const int q = (int)(pos >> 2);
      const uint32_t d0 = (uint32_t)__shfl((int)t.esc, q, 64);
      const uint32_t d1 = (uint32_t)__shfl((int)t.esc, q + 1, 64);
      const uint32_t d2 = (uint32_t)__shfl((int)t.esc, q + 2, 64);
      const uint32_t sh = 8u * (pos & 3u);
      uint32_t lo = __builtin_amdgcn_alignbit(d1, d0, sh);
      uint32_t hi = __builtin_amdgcn_alignbit(d2, d1, sh);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t mode = (m8 >> (2 * j)) & 3u;
        const uint32_t esc = lo;
        const uint32_t nb8 = 8u * fp8_escape_bytes<FK>(mode);
        lo = __builtin_amdgcn_alignbit(hi, lo, nb8);
        hi = nb8 ? hi >> nb8 : hi;
        ops[j] = fp8_group(t, is_k, j, mode, esc, true);
      }
    };
    auto process = [&](const PageBuf& buf, int i) {
      if (!((ok_mask >> i) & 1ull)) return;
      if constexpr (MODE == kModeLoad) {
        probe ^= fold_words(buf);
        return;
      }
      uint32_t kt = 0xFFFFFFFFu, vt = 0xFFFFFFFFu;
      if constexpr (COMP) {
        kt = (uint32_t)__builtin_amdgcn_readlane((int)meta_l.y, i);
        vt = (uint32_t)__builtin_amdgcn_readlane((int)meta_l.w, i);
      }
      uint4 kops[4], vop[4];
      if constexpr (FMT == kFmtGaac) {
        gaac_ops(buf.k, kt != 0u, true, kops);
      } else if constexpr (FMT == kFmtFp8c) {
        fp8_ops(buf.k, kt == kFp8TagsRaw, true, kops);
      } else if constexpr (FMT == kFmtFp8) {
        kops[0] = fp8x8_to_bf16<FK>(buf.k[0].x, buf.k[0].y);
        kops[1] = fp8x8_to_bf16<FK>(buf.k[0].z, buf.k[0].w);
        kops[2] = fp8x8_to_bf16<FK>(buf.k[1].x, buf.k[1].y);
        kops[3] = fp8x8_to_bf16<FK>(buf.k[1].z, buf.k[1].w);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) kops[j] = restore_if_coded(buf.k[j], (kt >> (8 * j)) & 0xFFu);
      }
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (MODE == kModeFull) {
        operands_settled(kops);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kops[j]), as_bf16x8(qop[j]), sacc, 0, 0, 0);
      }
      if constexpr (FMT == kFmtGaac) {
        gaac_ops(buf.v, vt != 0u, false, vop);
      } else if constexpr (FMT == kFmtFp8c) {
        fp8_ops(buf.v, vt == kFp8TagsRaw, false, vop);
      } else if constexpr (FMT == kFmtFp8) {
        vop[0] = fp8x8_to_bf16<FK>(buf.v[0].x, buf.v[0].y);
        vop[1] = fp8x8_to_bf16<FK>(buf.v[0].z, buf.v[0].w);
        vop[2] = fp8x8_to_bf16<FK>(buf.v[1].x, buf.v[1].y);
        vop[3] = fp8x8_to_bf16<FK>(buf.v[1].z, buf.v[1].w);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) vop[j] = restore_if_coded(buf.v[j], (vt >> (8 * j)) & 0xFFu);
      }
      if constexpr (MODE == kModeRestore) {
        probe ^= fold_words(kops) ^ fold_words(vop);
        return;
      }
      // the V restore above overlaps the score products; the rare split (a separate block) and
      // the softmax follow
      scores_settled(sacc);
      float sv[4], sl[4] = {0.f, 0.f, 0.f, 0.f}, t[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[r] = t[r] = sacc[r];
      if (needs_precise(sv, sm.m_run, big_min, near)) {
        split_scores(kops, qop, big_thr, sv, sl);
#pragma unroll
        for (int r = 0; r < 4; ++r) t[r] = sv[r] + sl[r];
      }
      sm.page(sv, sl, page_max(t), vop, lane, c_log2);
    };

    // Two one-page buffers in a ring: the loads of page i+1 are in flight while page i is
    // computed.  The loop runs whole rounds of two (a load past the chunk's end is issued with
    // a zero-size resource and never computed), so the wait before each compute covers exactly
    // that page's eight loads.
    const int last = cnt - 1;
    PageBuf buf[2];
    load_page(0, buf[0], true);
    const int rounds = (cnt + 1) / 2;
    for (int r = 0; r < rounds; ++r) {
      balance(cbase - p0 + 2 * r);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int i = 2 * r + k;
        load_page(i + 1 < last ? i + 1 : last, buf[k ^ 1], i + 1 <= last);
        if (i <= last) process(buf[k], i);
      }
    }
  }

  // The tail page (natural layout [16][128], BF16 - or FP8 for the FP8 formats), masked to its
  // n_tail tokens; masked V values are zeros, so they add nothing even where p is 0.
  if (MODE == kModeFull && n_tail > 0 && p0 <= n_comp && n_comp < p1) {
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
    uint4 kops[4], vop[4];
    if constexpr (IS_FP8) {
      const uint8_t* kt = static_cast<const uint8_t*>(p.tail) + (((size_t)b * 2 + 0) * p.Hkv + kvh) * 2048;
      const uint8_t* vt = static_cast<const uint8_t*>(p.tail) + (((size_t)b * 2 + 1) * p.Hkv + kvh) * 2048;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint2 k8 = *reinterpret_cast<const uint2*>(kt + (lane & 15) * 128 + 32 * j + 8 * (lane >> 4));
        kops[j] = fp8x8_to_bf16<FK>(k8.x, k8.y);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kops[j]), as_bf16x8(qop[j]), sacc, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t f[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int t0 = 8 * (lane >> 5) + i;
          const uint32_t x = t0 < n_tail ? vt[t0 * 128 + 32 * j + (lane & 31)] : 0u;
          f[i >> 2] |= x << (8 * (i & 3));
        }
        vop[j] = fp8x8_to_bf16<FK>(f[0], f[1]);
      }
    } else {
      const uint16_t* kt = static_cast<const uint16_t*>(p.tail) + (((size_t)b * 2 + 0) * p.Hkv + kvh) * 2048;
      const uint16_t* vt = static_cast<const uint16_t*>(p.tail) + (((size_t)b * 2 + 1) * p.Hkv + kvh) * 2048;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kops[j] = *reinterpret_cast<const uint4*>(kt + (lane & 15) * 128 + 32 * j + 8 * (lane >> 4));
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kops[j]), as_bf16x8(qop[j]), sacc, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t w[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int t0 = 8 * (lane >> 5) + 2 * m;
          const uint32_t a = t0 < n_tail ? vt[t0 * 128 + 32 * j + (lane & 31)] : 0u;
          const uint32_t c = t0 + 1 < n_tail ? vt[(t0 + 1) * 128 + 32 * j + (lane & 31)] : 0u;
          w[m] = a | (c << 16);
        }
        vop[j] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    float sv[4], sl[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = 4 * (lane >> 4) + r;
      sv[r] = tok < n_tail ? sacc[r] : -INFINITY;
    }
    float t[4] = {sv[0], sv[1], sv[2], sv[3]};
    if (needs_precise(sv, sm.m_run, big_min, near)) {
      split_scores(kops, qop, big_thr, sv, sl);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (4 * (lane >> 4) + r >= n_tail) {
          sv[r] = -INFINITY;
          sl[r] = 0.f;
        }
        t[r] = sv[r] + sl[r];
      }
    }
    sm.page(sv, sl, page_max(t), vop, lane, c_log2);
  }

  if constexpr (MODE != kModeFull) {
    // breakdown variants: nothing is merged or written (a store that never happens keeps the
    // loads and restores alive)
    if (probe == 0x7FC00001u && lane == 0) p.out[(size_t)b * p.Hq * KVZ_HEAD_DIM] = 1.f;
    return;
  }
  sm.fold();
  if constexpr (IS_FP8) {   // the V dequantization scale, applied once to O
#pragma unroll
    for (int j = 0; j < 4; ++j) sm.o[j] *= p.v_scale;
  }

  float l_tot = sm.l_run + lane_xor(sm.l_run, 16);
  l_tot += lane_xor(l_tot, 32);          // lane h (h < 16) now holds l of head h
  constexpr int NR = GB <= 8 ? 4 : 8;

  // The four waves' (m, l) per head and unnormalized O rows meet in LDS; one merge per
  // (head, dim): M = max m_w, L = sum l_w 2^((m_w - M) c), O = sum O_w 2^((m_w - M) c), in wave
  // order (m: raw scores; c: the scale to log2 units).
  __shared__ float s_m[NW][16], s_l[NW][16];
  __shared__ float s_o[NW][GB * KVZ_HEAD_DIM];
  if (lane < 16) {
    s_m[wave][lane] = sm.m_run;
    s_l[wave][lane] = l_tot;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int row = 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
      if (row < p.G) s_o[wave][row * KVZ_HEAD_DIM + 32 * j + (lane & 31)] = sm.o[j][r];
    }
  }
  __syncthreads();
  const bool empty_seq = p.seq_lens[b] <= 0;
  // the only piece of its sequence normalizes in place
  const bool direct = p.merge_in_kernel ? so.sb == 1 : p.S == 1;
  const bool fused_merge = p.merge_in_kernel && !direct;
  for (int idx = threadIdx.x; idx < p.G * KVZ_HEAD_DIM; idx += 64 * NW) {
    const int h = idx / KVZ_HEAD_DIM, d = idx % KVZ_HEAD_DIM;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = s_m[w][h];
      const float c = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(to_log2(mw - M, c_log2));
      L += c * s_l[w][h];
      O += c * s_o[w][idx];
    }
    float* po = p.ws_o + ((size_t)unit * p.G + h) * KVZ_HEAD_DIM + d;
    float* pml = p.ws_ml + ((size_t)unit * p.G + h) * 2;
    if (direct) {
      p.out[((size_t)b * p.Hq + (size_t)kvh * p.G + h) * KVZ_HEAD_DIM + d] = empty_seq ? 0.f : O / L;
    } else if (fused_merge) {
      // written through to memory (device-scope stores), read back by the merging piece
      __hip_atomic_store(po, O, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (d == 0) {
        __hip_atomic_store(pml, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(pml + 1, L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      *po = O;
      if (d == 0) {
        pml[0] = M;
        pml[1] = L;
      }
    }
  }
  if (!fused_merge) return;
  // Merge in the kernel (split counts up to kInKernelMergeMax): each piece counts itself in at
  // its (sequence, KV head) with one atomic add; the piece that arrives last merges every piece
  // in piece order (the same sums whichever piece is last) and returns the counter to zero for
  // the next call.  Only the partials and the counter pass between workgroups, and all of them
  // with device-scope accesses: the partial stores above are written through past this
  // chiplet's L2 (scope bit sc1), each wave waits for them to complete before the barrier that
  // precedes the atomic, the atomic is device-coherent, and the merging piece reads the
  // partials with device-scope loads issued after the atomic's result.  A release/acquire pair
  // would instead write back and invalidate the whole L2 of the chiplet, once per workgroup:
  // that measured slower than the separate merge launch, this is faster than it.
  __shared__ uint32_t s_last;
  __builtin_amdgcn_s_waitcnt(0);   // this wave's partial stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t* cnt = p.ws_cnt + (size_t)kvh * p.B + b;
    const uint32_t before = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t last = before + 1u == (uint32_t)so.sb ? 1u : 0u;
    if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // a count at or above the number of pieces cannot come from a zeroed workspace (one that
    // was not zero-filled, or reused for a larger batch * KV heads beyond the fixed counter
    // area): this call's merge of the pair is then unreliable; the flag stays for the host
    if (before >= (uint32_t)so.sb)
      __hip_atomic_fetch_or(p.ws_status, KVZ_WS_BAD_COUNTER, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  const size_t u0 = (size_t)kvh * U + so.base;
  for (int idx = threadIdx.x; idx < p.G * KVZ_HEAD_DIM; idx += 64 * NW) {
    const int h = idx / KVZ_HEAD_DIM, d = idx % KVZ_HEAD_DIM;
    const float* ml = p.ws_ml + (u0 * p.G + h) * 2;
    const float* o = p.ws_o + u0 * p.G * KVZ_HEAD_DIM + (size_t)h * KVZ_HEAD_DIM + d;
    auto ld = [](const float* q) { return __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
    const size_t mls = (size_t)p.G * 2, os = (size_t)p.G * KVZ_HEAD_DIM;
    // Up to four pieces (the split counts that merge here): every load in one round trip.  A
    // ragged batch can give a longer sequence more pieces: they are taken four at a time, each
    // group's loads issued together, the maximum first, then the sums - in piece order either
    // way, so the result does not depend on which piece merges.
    float M = -INFINITY, L = 0.f, O = 0.f;
    if (so.sb <= kInKernelMergeMax) {
      float mv[kInKernelMergeMax], lv[kInKernelMergeMax], ov[kInKernelMergeMax];
#pragma unroll
      for (int i = 0; i < kInKernelMergeMax; ++i) {
        if (i < so.sb) {
          mv[i] = ld(ml + i * mls);
          lv[i] = ld(ml + i * mls + 1);
          ov[i] = ld(o + i * os);
        }
      }
#pragma unroll
      for (int i = 0; i < kInKernelMergeMax; ++i)
        if (i < so.sb) M = fmaxf(M, mv[i]);
#pragma unroll
      for (int i = 0; i < kInKernelMergeMax; ++i) {
        if (i < so.sb) {
          const float c = mv[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(to_log2(mv[i] - M, c_log2));
          L += c * lv[i];
          O += c * ov[i];
        }
      }
    } else {
      for (int i0 = 0; i0 < so.sb; i0 += kInKernelMergeMax) {
        float mv[kInKernelMergeMax];
#pragma unroll
        for (int i = 0; i < kInKernelMergeMax; ++i) mv[i] = i0 + i < so.sb ? ld(ml + (i0 + i) * mls) : -INFINITY;
#pragma unroll
        for (int i = 0; i < kInKernelMergeMax; ++i) M = fmaxf(M, mv[i]);
      }
      for (int i0 = 0; i0 < so.sb; i0 += kInKernelMergeMax) {
        float mv[kInKernelMergeMax], lv[kInKernelMergeMax], ov[kInKernelMergeMax];
#pragma unroll
        for (int i = 0; i < kInKernelMergeMax; ++i) {
          if (i0 + i < so.sb) {
            mv[i] = ld(ml + (i0 + i) * mls);
            lv[i] = ld(ml + (i0 + i) * mls + 1);
            ov[i] = ld(o + (i0 + i) * os);
          }
        }
#pragma unroll
        for (int i = 0; i < kInKernelMergeMax; ++i) {
          if (i0 + i < so.sb) {
            const float c = mv[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(to_log2(mv[i] - M, c_log2));
            L += c * lv[i];
            O += c * ov[i];
          }
        }
      }
    }
    p.out[((size_t)b * p.Hq + (size_t)kvh * p.G + h) * KVZ_HEAD_DIM + d] = empty_seq ? 0.f : O / L;
  }
}

// Merge the splits of every (sequence, query head): M = max m_s, L = sum l_s 2^((m_s - M) c),
// out = sum O_s 2^((m_s - M) c) / L, over the sequence's S_b splits (split_of); the maxima are
// raw scores and c the scale to log2 units.  A sequence of
// length 0 gives zeros.  A separate launch, for split counts above kInKernelMergeMax (one long
// sequence over many CUs: its pieces are merged in parallel here rather than serially by the
// last piece).  One workgroup of 256 threads per (sequence, query head), parallel over the
// splits.
constexpr int kCombineThreads = 256;

__device__ __forceinline__ float block_reduce(float v, float* s_red, bool is_max) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const float o = __shfl_xor(v, d, 64);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = s_red[0];
#pragma unroll
  for (int w = 1; w < kCombineThreads / 64; ++w) r = is_max ? fmaxf(r, s_red[w]) : r + s_red[w];
  __syncthreads();
  return r;
}

// Splits merged from registers when the batch's split map is the uniform one (sequence b owns
// splits b*S .. b*S+S-1): every partial of (b, head) is loaded in the same round trip as the
// lengths that confirm the map.  Larger S, or a ragged map, takes the general path.
constexpr int kSpecSplits = 32;

__global__ __launch_bounds__(kCombineThreads) void attn_combine_kernel(
    const float* ws_ml, const float* ws_o, float* out, const int32_t* seq_lens,
    const int32_t* n_comp_v, bool has_tail, int max_pages, int B, int Hq, int G, int S_avg,
    float c_log2) {
  __shared__ float s_w[kMaxSplits];
  __shared__ float s_red[kCombineThreads / 64];
  __shared__ float s_part[kCombineThreads];
  __shared__ float s_ml[2][kSpecSplits];
  const int bh = blockIdx.x;
  const int b = bh / Hq, h = bh % Hq;
  const int kvh = h / G, g = h % G;
  const int t = threadIdx.x;
  const int d = t & (KVZ_HEAD_DIM - 1);
  const int half = t >> 7;                                 // 256 threads: two per dim
  const int32_t slen = seq_lens[b];
  // speculative loads of the uniform map's partials (issued before the map is known)
  const bool spec = S_avg <= kSpecSplits;
  const size_t ubase = (size_t)kvh * B * S_avg;
  float m_sp = -INFINITY, l_sp = 0.f;
  float o_sp[kSpecSplits / 2];
  if (spec) {
    const size_t u0 = ubase + (size_t)b * S_avg;
    if (t < S_avg) {
      m_sp = ws_ml[((u0 + t) * G + g) * 2];
      l_sp = ws_ml[((u0 + t) * G + g) * 2 + 1];
    }
#pragma unroll
    for (int i = 0; i < kSpecSplits / 2; ++i) {
      const int sp = half + 2 * i;
      o_sp[i] = sp < S_avg ? ws_o[((u0 + sp) * G + g) * KVZ_HEAD_DIM + d] : 0.f;
    }
  }
  const SplitOf so = split_of(n_comp_v, seq_lens, has_tail, max_pages, B, S_avg, 0, b);
  const int S = so.sb;
  if (spec && so.base == b * S_avg && S == S_avg) {
    if (t < S) {
      s_ml[0][t] = m_sp;
      s_ml[1][t] = l_sp;
    }
    __syncthreads();
    float M = -INFINITY;
    for (int sp = 0; sp < S; ++sp) M = fmaxf(M, s_ml[0][sp]);
    float L = 0.f, acc = 0.f;
    for (int sp = 0; sp < S; ++sp) {
      const float m = s_ml[0][sp];
      L += ((m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(to_log2(m - M, c_log2))) * s_ml[1][sp];
    }
#pragma unroll
    for (int i = 0; i < kSpecSplits / 2; ++i) {
      const int sp = half + 2 * i;
      if (sp < S) {
        const float m = s_ml[0][sp];
        acc += ((m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(to_log2(m - M, c_log2))) * o_sp[i];
      }
    }
    s_part[t] = acc;
    __syncthreads();
    if (t < KVZ_HEAD_DIM) {
      const float o = (s_part[t] + s_part[t + KVZ_HEAD_DIM]) / L;
      out[(size_t)bh * KVZ_HEAD_DIM + d] = slen <= 0 ? 0.f : o;
    }
    return;
  }
  // general path: any split map, any S
  auto unit_of = [&](int sp) { return ubase + so.base + sp; };
  float m_loc = -INFINITY;
  for (int sp = t; sp < S; sp += kCombineThreads) m_loc = fmaxf(m_loc, ws_ml[(unit_of(sp) * G + g) * 2]);
  const float M = block_reduce(m_loc, s_red, true);
  float l_loc = 0.f;
  for (int sp = t; sp < S; sp += kCombineThreads) {
    const size_t ug = unit_of(sp) * G + g;
    const float m = ws_ml[ug * 2];
    const float w = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(to_log2(m - M, c_log2));
    s_w[sp] = w;
    l_loc += w * ws_ml[ug * 2 + 1];
  }
  const float L = block_reduce(l_loc, s_red, false);   // its barrier also publishes s_w
  float acc = 0.f;
#pragma unroll 4
  for (int sp = half; sp < S; sp += kCombineThreads / KVZ_HEAD_DIM)
    acc += s_w[sp] * ws_o[(unit_of(sp) * G + g) * KVZ_HEAD_DIM + d];
  s_part[t] = acc;
  __syncthreads();
  if (t < KVZ_HEAD_DIM) {
    const float o = (s_part[t] + s_part[t + KVZ_HEAD_DIM]) / L;
    out[(size_t)bh * KVZ_HEAD_DIM + d] = slen <= 0 ? 0.f : o;
  }
}

// Split count: one workgroup (one split) per CU, with at least 4 pages per wave.  A group of up
// to 4 query heads per KV head (every workload shape here) runs 8 waves per workgroup, two per
// SIMD: one wave's softmax and products overlap the other's loads, and the 8 partial results
// meet in LDS rather than in more splits (measured against 4 waves per workgroup on one box:
// the 2K batch 40.0 / 39.3 vs 41.5 / 40.0 us per layer, one 131K sequence 93.7 / 93.9 vs
// 96.5 / 98.2, the ragged batch 46.6 vs 49.2, the 8K layer 86.4 vs 86.9).  Larger groups run 4
// waves per workgroup; their coded tiles two workgroups per CU (two waves per SIMD).  Workgroup
// counts that are not a multiple of the CU count leave some CUs one workgroup more than others
// (measured 10-20% slower).
constexpr int kSmallGroupWaves = 8;
constexpr int kCodedWgsPerCu = 2;
int wgs_per_cu(bool coded, int G) { return (coded && G > 4) ? kCodedWgsPerCu : 1; }

int choose_splits(int B, int Hkv, int max_pages, int n_cu, int wgs_per_cu = 1) {
  const int64_t units = (int64_t)(B * Hkv > 0 ? B * Hkv : 1);
  const int64_t pages = (int64_t)max_pages + 1;
  int64_t S = ((int64_t)wgs_per_cu * n_cu + units - 1) / units;
  const int64_t by_pages = (pages + 15) / 16;
  if (S > by_pages) S = by_pages;
  if (S > kMaxSplits) S = kMaxSplits;
  return (int)(S < 1 ? 1 : S);
}

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

// workspace = [status: 256 B, word 0 = sticky flags][counters: B*Hkv u32, in an area of at least
// 64 KiB][m, l: units*G*2 f32][O: units*G*128 f32], 256-B aligned parts.  The status word and the
// counters are zero between calls (zero-filled once by the caller).  Up to 16384 (sequence, KV
// head) pairs the counter area has the same place and size for every call, so reusing one
// workspace across sizes never puts counters over bytes that held partial results.
constexpr uint64_t kWsStatusBytes = 256;
constexpr uint64_t kWsMinCounterBytes = 64ull << 10;
struct WsLayout {
  uint64_t cnt_off, ml_off, o_off, total;
};
WsLayout workspace_layout(int B, int Hq, int Hkv, int S) {
  const uint64_t units = (uint64_t)B * Hkv * S;
  const uint64_t G = Hkv > 0 ? (uint64_t)(Hq / Hkv) : 0;
  const uint64_t cnt = std::max(kWsMinCounterBytes, align256((uint64_t)B * Hkv * sizeof(uint32_t)));
  WsLayout w;
  w.cnt_off = kWsStatusBytes;
  w.ml_off = w.cnt_off + cnt;
  w.o_off = w.ml_off + align256(units * G * 2 * sizeof(float));
  w.total = w.o_off + align256(units * G * KVZ_HEAD_DIM * sizeof(float));
  return w;
}

struct CommonArgs {
  const uint16_t* q;
  float* out;
  uint64_t arena_bytes;
  int32_t n_phys_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* n_comp_pages;
  const void* tail;
  int32_t batch, num_q_heads, num_kv_heads, head_dim, page_size, max_pages, splits;
  float sm_scale;
  void* workspace;
  uint64_t workspace_bytes;
  float k_scale = 1.f, v_scale = 1.f;   // FP8 formats only
};

template <int FMT, int FK = 0, int MODE = kModeFull>
int launch_attention(const CommonArgs& a, const uint8_t* kv, const kvz_group_meta* meta,
                     const uint8_t* bases, hipStream_t s) {
  constexpr bool COMP = FMT == kFmtZf || FMT == kFmtGaac || FMT == kFmtFp8c;
  constexpr bool CODED = FMT == kFmtGaac || FMT == kFmtFp8c;
  if (a.head_dim != KVZ_HEAD_DIM || a.page_size != KVZ_PAGE_TOKENS)
    return set_error(KVZ_EUNSUPPORTED, "only head_dim 128 and 16-token pages are supported");
  if (a.batch < 0 || a.num_q_heads <= 0 || a.num_kv_heads <= 0 || a.max_pages < 0)
    return set_error(KVZ_EINVAL, "bad sizes");
  if (a.num_q_heads % a.num_kv_heads != 0)
    return set_error(KVZ_EINVAL, "num_q_heads must be a multiple of num_kv_heads");
  const int G = a.num_q_heads / a.num_kv_heads;
  if (G > 16) return set_error(KVZ_EUNSUPPORTED, "query group larger than 16");
  if (a.batch == 0) return KVZ_OK;
  if (!a.q || !a.out || !a.seq_lens || !a.n_comp_pages || !a.workspace)
    return set_error(KVZ_EINVAL, "null pointer argument");
  if (a.max_pages > 0 && (!kv || !a.block_table || (COMP && !meta)))
    return set_error(KVZ_EINVAL, "null page pointer argument");
  if (a.n_phys_pages < 0) return set_error(KVZ_EINVAL, "n_phys_pages < 0");
  if (COMP && a.max_pages > 0 && a.arena_bytes < (FMT == kFmtFp8c ? 2048u : 4096u))
    return set_error(KVZ_EINVAL, "arena smaller than one record");
  if ((((uintptr_t)a.q) | ((uintptr_t)a.tail)) & 15u)
    return set_error(KVZ_EINVAL, "q and tail must be 16-byte aligned");
  if (FMT == kFmtFp8 && (((uintptr_t)kv) & 15u))
    return set_error(KVZ_EINVAL, "pages must be 16-byte aligned");
  if (COMP && (((uintptr_t)meta) & 15u)) return set_error(KVZ_EINVAL, "meta must be 16-byte aligned");
  if (CODED && (!bases || (((uintptr_t)bases) & 7u)))
    return set_error(KVZ_EINVAL, "bases must be a non-null 8-byte aligned pointer");
  if (((uintptr_t)a.workspace) & 255u) return set_error(KVZ_EINVAL, "workspace must be 256-byte aligned");
  if (a.splits < 0 || a.splits > kMaxSplits) return set_error(KVZ_EINVAL, "splits out of range");
  const int S = a.splits ? a.splits
                         : choose_splits(a.batch, a.num_kv_heads, a.max_pages, device_cus(),
                                         wgs_per_cu(CODED, G));
  const WsLayout wl = workspace_layout(a.batch, a.num_q_heads, a.num_kv_heads, S);
  if (a.workspace_bytes < wl.total) return set_error(KVZ_EINVAL, "workspace too small");
  const uint64_t units = (uint64_t)a.batch * a.num_kv_heads * S;
  if (units > 0x7FFFFFFFull) return set_error(KVZ_EINVAL, "too many units");

  AttnParams p;
  p.q = a.q;
  p.kv = kv;
  p.meta = reinterpret_cast<const uint4*>(meta);
  p.block_table = a.block_table;
  p.seq_lens = a.seq_lens;
  p.n_comp = a.n_comp_pages;
  p.tail = a.tail;
  p.bases = bases;
  p.out = a.out;
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  p.ws_status = reinterpret_cast<uint32_t*>(ws);
  p.ws_cnt = reinterpret_cast<uint32_t*>(ws + wl.cnt_off);
  p.ws_ml = reinterpret_cast<float*>(ws + wl.ml_off);
  p.ws_o = reinterpret_cast<float*>(ws + wl.o_off);
  // (a ragged batch can still give one sequence more pieces: the merge loops over them)
  p.merge_in_kernel = S <= kInKernelMergeMax;
  p.arena_bytes = a.arena_bytes;
  p.n_phys = a.n_phys_pages;
  p.B = a.batch;
  p.Hq = a.num_q_heads;
  p.Hkv = a.num_kv_heads;
  p.G = G;
  p.max_pages = a.max_pages;
  p.S = S;
  p.scale_log2 = a.sm_scale * a.k_scale * 1.4426950408889634f;
  p.v_scale = a.v_scale;

  const dim3 grid((unsigned)units);
  if constexpr (MODE != kModeFull) {   // breakdown variants: groups of up to 4 query heads
    if (G > 4) return set_error(KVZ_EUNSUPPORTED, "the breakdown variants take up to 4 query heads per KV head");
    hipLaunchKernelGGL((attn_split_kernel<4, FMT, FK, MODE, kSmallGroupWaves>), grid,
                       dim3(64 * kSmallGroupWaves), 0, s, p);
    return check_hip(hipGetLastError(), "attention launch");
  }
  if (G <= 4)
    hipLaunchKernelGGL((attn_split_kernel<4, FMT, FK, kModeFull, kSmallGroupWaves>), grid,
                       dim3(64 * kSmallGroupWaves), 0, s, p);
  else if (G <= 8)
    hipLaunchKernelGGL((attn_split_kernel<8, FMT, FK>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((attn_split_kernel<16, FMT, FK>), grid, dim3(256), 0, s, p);
  int rc = check_hip(hipGetLastError(), "attention launch");
  if (rc != KVZ_OK || S == 1 || p.merge_in_kernel) return rc;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(a.batch * a.num_q_heads)),
                     dim3(kCombineThreads), 0, s,
                     p.ws_ml, p.ws_o, a.out, a.seq_lens, a.n_comp_pages, a.tail != nullptr,
                     p.max_pages, p.B, p.Hq, G, S, p.scale_log2);
  return check_hip(hipGetLastError(), "combine launch");
}

// Device-resident scratch of the allocation-free attention call (kvz_decode_attention_noalloc):
// a workspace of 16 MiB in the layout above (status word and the fixed 64 KiB counter area,
// which every call leaves zero, then the partial softmax states).  One copy per GPU, held while
// the library is loaded.
constexpr uint64_t kScratchBytes = 16ull << 20;
constexpr uint64_t kScratchZeroBytes = kWsStatusBytes + kWsMinCounterBytes;
constexpr int kMaxDevices = 64;

__global__ void zero_words_kernel(uint32_t* p, uint32_t n) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

}  // namespace
}  // namespace kvz

using namespace kvz;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices];   // the device address of `scratch`, per device

// The current device's scratch address, looked up (and its counter area zero-filled on stream
// s) at the first call on that device.  The array's host-side name is not a device address:
// every kernel argument and fill below uses the looked-up pointer.
int scratch_of_current_device(hipStream_t s, uint8_t** out) {
  int dev = 0;
  int rc = check_hip(hipGetDevice(&dev), "hipGetDevice");
  if (rc != KVZ_OK) return rc;
  if (dev < 0 || dev >= kMaxDevices) return set_error(KVZ_EUNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    rc = check_hip(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (rc != KVZ_OK) return rc;
    if (!ptr || (reinterpret_cast<uintptr_t>(ptr) & 255u))
      return set_error(KVZ_EHIP, "scratch symbol has no 256-byte aligned device address");
    hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, s, static_cast<uint32_t*>(ptr),
                       (uint32_t)(kScratchZeroBytes / 4));
    rc = check_hip(hipGetLastError(), "scratch counter fill");
    if (rc != KVZ_OK) return rc;
    g_scratch_ptr[dev] = static_cast<uint8_t*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return KVZ_OK;
}
}  // namespace

extern "C" int kvz_attn_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t max_pages, int32_t splits, uint64_t* bytes) {
  if (!bytes) return set_error(KVZ_EINVAL, "bytes is null");
  if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_pages < 0 || splits < 0)
    return set_error(KVZ_EINVAL, "bad sizes");
  if (splits > kMaxSplits) return set_error(KVZ_EINVAL, "splits out of range");
  // sized for the format with the most splits, so one workspace serves every format
  const int S = splits ? splits
                       : choose_splits(batch, num_kv_heads, max_pages, device_cus(), kCodedWgsPerCu);
  *bytes = workspace_layout(batch, num_q_heads, num_kv_heads, S).total;
  return KVZ_OK;
}

extern "C" int kvz_decode_attention(const kvz_attn_args* a, hipStream_t s) {
  if (!a) return set_error(KVZ_EINVAL, "args is null");
  CommonArgs c{a->q, a->out, a->arena_bytes, a->n_phys_pages, a->block_table, a->seq_lens,
               a->n_comp_pages, a->tail, a->batch, a->num_q_heads, a->num_kv_heads, a->head_dim,
               a->page_size, a->max_pages, a->splits, a->sm_scale, a->workspace,
               a->workspace_bytes};
  return launch_attention<kFmtZf>(c, a->arena, a->meta, nullptr, s);
}

extern "C" int kvz_decode_attention_noalloc(const kvz_attn_args* a, hipStream_t s) {
  if (!a) return set_error(KVZ_EINVAL, "args is null");
  if (a->batch < 0 || a->num_q_heads <= 0 || a->num_kv_heads <= 0 || a->max_pages < 0 ||
      a->splits < 0 || a->splits > kMaxSplits)
    return set_error(KVZ_EINVAL, "bad sizes");
  if (a->batch == 0) return KVZ_OK;
  if (a->num_q_heads % a->num_kv_heads != 0)
    return set_error(KVZ_EINVAL, "num_q_heads must be a multiple of num_kv_heads");
  // the same split count and workspace layout as kvz_decode_attention
  const int S = a->splits ? a->splits : choose_splits(a->batch, a->num_kv_heads, a->max_pages, device_cus());
  if ((int64_t)a->batch * a->num_kv_heads > (int64_t)(kWsMinCounterBytes / 4))
    return set_error(KVZ_EINVAL, "batch * num_kv_heads above 16384: too large for the allocation-free call");
  const WsLayout wl = workspace_layout(a->batch, a->num_q_heads, a->num_kv_heads, S);
  if (wl.total > kScratchBytes)
    return set_error(KVZ_EINVAL, "the partial results of these sizes need " + std::to_string(wl.total - wl.ml_off) +
                                     " bytes, above the allocation-free call's " +
                                     std::to_string(kScratchBytes - wl.ml_off));
  uint8_t* base = nullptr;
  const int rc = scratch_of_current_device(s, &base);
  if (rc != KVZ_OK) return rc;
  // the counter area is the fixed 64 KiB one for every size accepted here, so counters of calls
  // with other sizes (all zero between calls) never overlap partial results
  kvz_attn_args b = *a;
  b.workspace = base;
  b.workspace_bytes = kScratchBytes;
  b.splits = S;
  return kvz_decode_attention(&b, s);
}

extern "C" int kvz_attn_workspace_status(const void* d_workspace, uint32_t* flags, hipStream_t s) {
  if (!flags) return set_error(KVZ_EINVAL, "flags is null");
  const uint8_t* ws = static_cast<const uint8_t*>(d_workspace);
  if (!ws) {
    uint8_t* base = nullptr;
    const int rc = scratch_of_current_device(s, &base);
    if (rc != KVZ_OK) return rc;
    ws = base;
  } else if (((uintptr_t)ws) & 255u) {
    return set_error(KVZ_EINVAL, "workspace must be 256-byte aligned");
  }
  uint32_t v = 0;
  int rc = check_hip(hipMemcpyAsync(&v, ws, sizeof(v), hipMemcpyDeviceToHost, s), "status copy");
  if (rc != KVZ_OK) return rc;
  rc = check_hip(hipStreamSynchronize(s), "hipStreamSynchronize");
  if (rc != KVZ_OK) return rc;
  *flags = v;
  return KVZ_OK;
}

extern "C" int kvz_gaac_decode_attention(const kvz_attn_args* a, const uint8_t* d_bases,
                                         hipStream_t s) {
  if (!a) return set_error(KVZ_EINVAL, "args is null");
  CommonArgs c{a->q, a->out, a->arena_bytes, a->n_phys_pages, a->block_table, a->seq_lens,
               a->n_comp_pages, a->tail, a->batch, a->num_q_heads, a->num_kv_heads, a->head_dim,
               a->page_size, a->max_pages, a->splits, a->sm_scale, a->workspace,
               a->workspace_bytes};
  return launch_attention<kFmtGaac>(c, a->arena, a->meta, d_bases, s);
}

extern "C" int kvz_bf16_decode_attention(const kvz_bf16_attn_args* a, hipStream_t s) {
  if (!a) return set_error(KVZ_EINVAL, "args is null");
  CommonArgs c{a->q, a->out, 0, a->n_phys_pages, a->block_table, a->seq_lens,
               a->n_comp_pages, a->tail, a->batch, a->num_q_heads, a->num_kv_heads, a->head_dim,
               a->page_size, a->max_pages, a->splits, a->sm_scale, a->workspace,
               a->workspace_bytes};
  return launch_attention<kFmtBf16>(c, a->pages, nullptr, nullptr, s);
}

extern "C" int kvz_decode_attention_part(const kvz_attn_args* a, int32_t part, hipStream_t s) {
  if (!a) return set_error(KVZ_EINVAL, "args is null");
  CommonArgs c{a->q, a->out, a->arena_bytes, a->n_phys_pages, a->block_table, a->seq_lens,
               a->n_comp_pages, a->tail, a->batch, a->num_q_heads, a->num_kv_heads, a->head_dim,
               a->page_size, a->max_pages, a->splits, a->sm_scale, a->workspace,
               a->workspace_bytes};
  switch (part) {
    case KVZ_PART_ALL: return launch_attention<kFmtZf>(c, a->arena, a->meta, nullptr, s);
    case KVZ_PART_LOAD: return launch_attention<kFmtZf, 0, kModeLoad>(c, a->arena, a->meta, nullptr, s);
    case KVZ_PART_LOAD_RESTORE:
      return launch_attention<kFmtZf, 0, kModeRestore>(c, a->arena, a->meta, nullptr, s);
    default: return set_error(KVZ_EINVAL, "part must be KVZ_PART_ALL, KVZ_PART_LOAD or KVZ_PART_LOAD_RESTORE");
  }
}

extern "C" int kvz_bf16_decode_attention_part(const kvz_bf16_attn_args* a, int32_t part, hipStream_t s) {
  if (!a) return set_error(KVZ_EINVAL, "args is null");
  CommonArgs c{a->q, a->out, 0, a->n_phys_pages, a->block_table, a->seq_lens,
               a->n_comp_pages, a->tail, a->batch, a->num_q_heads, a->num_kv_heads, a->head_dim,
               a->page_size, a->max_pages, a->splits, a->sm_scale, a->workspace,
               a->workspace_bytes};
  switch (part) {
    case KVZ_PART_ALL: return launch_attention<kFmtBf16>(c, a->pages, nullptr, nullptr, s);
    case KVZ_PART_LOAD: return launch_attention<kFmtBf16, 0, kModeLoad>(c, a->pages, nullptr, nullptr, s);
    default: return set_error(KVZ_EINVAL, "part must be KVZ_PART_ALL or KVZ_PART_LOAD");
  }
}

extern "C" int kvz_fp8_decode_attention(const kvz_fp8_attn_args* a, hipStream_t s) {
  if (!a) return set_error(KVZ_EINVAL, "args is null");
  CommonArgs c{a->q, a->out, a->arena_bytes, a->n_phys_pages, a->block_table, a->seq_lens,
               a->n_comp_pages, a->tail, a->batch, a->num_q_heads, a->num_kv_heads, a->head_dim,
               a->page_size, a->max_pages, a->splits, a->sm_scale, a->workspace,
               a->workspace_bytes, a->k_scale, a->v_scale};
  if (a->format == KVZ_FP8_E4M3)
    return launch_attention<kFmtFp8c, KVZ_FP8_E4M3>(c, a->arena, a->meta, a->bases, s);
  if (a->format == KVZ_FP8_E5M2)
    return launch_attention<kFmtFp8c, KVZ_FP8_E5M2>(c, a->arena, a->meta, a->bases, s);
  return set_error(KVZ_EINVAL, "unknown FP8 format");
}

extern "C" int kvz_fp8_raw_decode_attention(const kvz_fp8_attn_args* a, hipStream_t s) {
  if (!a) return set_error(KVZ_EINVAL, "args is null");
  CommonArgs c{a->q, a->out, 0, a->n_phys_pages, a->block_table, a->seq_lens,
               a->n_comp_pages, a->tail, a->batch, a->num_q_heads, a->num_kv_heads, a->head_dim,
               a->page_size, a->max_pages, a->splits, a->sm_scale, a->workspace,
               a->workspace_bytes, a->k_scale, a->v_scale};
  if (a->format == KVZ_FP8_E4M3)
    return launch_attention<kFmtFp8, KVZ_FP8_E4M3>(c, a->pages, nullptr, nullptr, s);
  if (a->format == KVZ_FP8_E5M2)
    return launch_attention<kFmtFp8, KVZ_FP8_E5M2>(c, a->pages, nullptr, nullptr, s);
  return set_error(KVZ_EINVAL, "unknown FP8 format");
}
