// Two-size-class slot pool: deterministic allocation and free of contiguous group runs.
//
// Follows "GAAC: Lossless KV Compression for Bandwidth-Efficient LLM Inference on Personal
// Devices", section "Block-Wise Compression Scheduling" (fixed-capacity slots, two storage
// classes, a block that does not fit keeps its BF16 form) and "ZipFusion: Fusing Lossless KV
// Decompression with Attention for Efficient LLM Decoding", "How it works" (blocks of a group
// found from the first offset plus summed sizes, so a group is one contiguous run; space freed
// in one layer is reused by another).  A group with n_raw raw blocks takes 12 + n_raw granules
// of 256 B (768-B and 1024-B slots).
//
// Allocation and free follow item order exactly (the i-th item of class k pops bin k from the
// top, or pushes onto it; frontier requests get prefix-summed offsets), computed in parallel as
// a three-pass scan over tiles of 1024 items: count the classes per tile, scan the tiles in one
// workgroup, then assign (or push) per tile.  Calls of more than kMaxTiles tiles run as
// consecutive chunks.  The per-tile counts and bases live in a fixed scratch area of the pool
// state, so the pool needs no memory beyond the state the caller allocated.
#include "encode_internal.h"

#include <algorithm>

namespace kvz {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;

constexpr int kIpt = 2;   // items per thread (tiles of 1024 items: small calls still spread over several
                          // workgroups; measured 89 -> 69 us for a 9,216-group completion + free)
constexpr int kTile = kThreads * kIpt;
constexpr int kMaxTiles = 2 * kThreads;   // tiles per chunk: the scan pass takes 2 per thread
constexpr int kChunkItems = kTile * kMaxTiles;

// Scratch of the three passes (after the bins in the state buffer).
struct PoolScratch {
  uint32_t tile_cnt[kMaxTiles][kBins];    // items of each class in the tile
  uint32_t tile_base[kMaxTiles][kBins];   // rank of the tile's first item of each class
  uint64_t tile_fbase[kMaxTiles];         // frontier granules requested by earlier tiles
  uint64_t snap_cnt[kBins];               // bin counts when the chunk started
  uint64_t pend;                          // frontier + all requests of the call so far
  uint64_t f_chunk;                       // `pend` when this chunk started
};

__device__ __forceinline__ uint64_t lanemask_lt() {
  const uint32_t lane = threadIdx.x & 63u;
  return lane == 0 ? 0ull : (~0ull >> (64u - lane));
}

// Block-wide exclusive scan of C columns in thread order (thread t's values come after those
// of threads < t); excl[c] = sum over earlier threads, tot[c] = block total.
template <int C>
__device__ void block_scan_cols(const uint32_t (&v)[C], uint32_t (&excl)[C], uint32_t (&tot)[C],
                                uint32_t (*s_wave)[8], uint32_t (*s_pre)[8], uint32_t* s_tot) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t incl[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    incl[c] = v[c];
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t o = __shfl_up(incl[c], d, 64);
      if (lane >= d) incl[c] += o;
    }
    if (lane == 63) s_wave[wave][c] = incl[c];
  }
  __syncthreads();
  if ((int)threadIdx.x < C) {
    uint32_t acc = 0;
    for (int w = 0; w < kWaves; ++w) {
      s_pre[w][threadIdx.x] = acc;
      acc += s_wave[w][threadIdx.x];
    }
    s_tot[threadIdx.x] = acc;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < C; ++c) {
    excl[c] = s_pre[wave][c] + incl[c] - v[c];
    tot[c] = s_tot[c];
  }
  __syncthreads();
}

struct ScanShared {
  uint32_t wave[kWaves][8];
  uint32_t pre[kWaves][8];
  uint32_t tot[8];
};

// Sum of v over the block (result valid in every thread).
__device__ uint64_t block_sum(uint64_t v, uint64_t* s_red) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint64_t t = 0;
  for (int w = 0; w < kWaves; ++w) t += s_red[w];
  return t;
}

// Item accessors: tags in / offset out, either from plain arrays or from encode items' metadata.
struct TagArrayAccess {
  const uint8_t* tags;
  uint32_t* off;
  __device__ uint32_t get_tags(int i) const {
    const uint8_t* t = tags + 4 * (size_t)i;
    return (uint32_t)t[0] | ((uint32_t)t[1] << 8) | ((uint32_t)t[2] << 16) | ((uint32_t)t[3] << 24);
  }
  __device__ void set_off(int i, uint32_t o) const { off[i] = o; }
};

template <class Item>
struct ItemMetaAccess {
  const Item* items;
  __device__ uint32_t get_tags(int i) const {
    const kvz_group_meta* m = items[i].dst;
    return *reinterpret_cast<const uint32_t*>(m->tag);
  }
  __device__ void set_off(int i, uint32_t o) const { items[i].dst->off = o; }
};

// Free requests: a pointer to a group's metadata; a null pointer or an unstored group is no
// request (class -1), but its metadata is still cleared.
struct FreeAccess {
  kvz_group_meta* const* metas;
  __device__ int cls(int i) const {
    const kvz_group_meta* m = metas[i];
    if (!m) return -1;
    const uint2 rec = *reinterpret_cast<const uint2*>(m);
    return rec.x == KVZ_OFF_NONE ? -1 : (int)n_raw_of(rec.y);
  }
};

template <class Access>
__device__ __forceinline__ int alloc_cls(const Access& acc, int i) {
  return (int)n_raw_of(acc.get_tags(i));
}
template <>
__device__ __forceinline__ int alloc_cls<FreeAccess>(const FreeAccess& acc, int i) {
  return acc.cls(i);
}

// Items of one tile (kTile consecutive items; thread t owns 8t..8t+7) by class, with each
// item's rank among the same-class items of its thread.
struct TileItems {
  int key[kIpt];
  uint32_t lrank[kIpt];
  uint32_t lcnt[kBins];
};

template <class Access>
__device__ __forceinline__ void tile_classes(const Access& acc, int i0, int n_end, TileItems& t) {
#pragma unroll
  for (int k = 0; k < kBins; ++k) t.lcnt[k] = 0;
#pragma unroll
  for (int sub = 0; sub < kIpt; ++sub) t.key[sub] = i0 + sub < n_end ? alloc_cls(acc, i0 + sub) : -1;
#pragma unroll
  for (int sub = 0; sub < kIpt; ++sub) {
    t.lrank[sub] = 0;
#pragma unroll
    for (int k = 0; k < kBins; ++k) {
      if (t.key[sub] == k) {
        t.lrank[sub] = t.lcnt[k];
        t.lcnt[k] += 1;
      }
    }
  }
}

__device__ __forceinline__ uint32_t pick(const uint32_t (&v)[kBins], int k) {
  uint32_t r = v[0];
#pragma unroll
  for (int j = 1; j < kBins; ++j) r = (k == j) ? v[j] : r;
  return r;
}

// Pass 1 (one workgroup per tile): items of each class in the tile.
template <class Access>
__global__ __launch_bounds__(kThreads) void pool_count_kernel(const PoolHdr* hdr, PoolScratch* sc,
                                                              Access acc, int first, int n_end) {
  __shared__ ScanShared sh;
  if (hdr->magic != kPoolMagic) return;   // host checked; never write through a bad state
  const int tile = blockIdx.x;
  TileItems t;
  tile_classes(acc, first + tile * kTile + (int)threadIdx.x * kIpt, n_end, t);
  uint32_t ex[kBins], tot[kBins];
  block_scan_cols<kBins>(t.lcnt, ex, tot, sh.wave, sh.pre, sh.tot);
  if (threadIdx.x < kBins) sc->tile_cnt[tile][threadIdx.x] = pick(tot, (int)threadIdx.x);
}

// Pass 2 (one workgroup): scan over the tiles (2 per thread).  Gives each tile the rank of its
// first item of every class; for allocation, also the granules that earlier tiles request
// from the frontier (an item of class k asks the frontier iff its rank >= the bin's count).
// Updates the bin counts for the whole chunk and keeps the counts it started from.
template <bool ALLOC>
__global__ __launch_bounds__(kThreads) void pool_scan_kernel(PoolHdr* hdr, PoolScratch* sc,
                                                             int n_tiles, int first_chunk) {
  __shared__ ScanShared sh;
  if (hdr->magic != kPoolMagic) return;
  const int t0 = 2 * (int)threadIdx.x, t1 = t0 + 1;
  uint64_t cnt[kBins];
#pragma unroll
  for (int k = 0; k < kBins; ++k) cnt[k] = hdr->bin_cnt[k];
  const uint64_t pend = ALLOC ? (first_chunk ? hdr->frontier : sc->pend) : 0;
  uint32_t c0[kBins], c1[kBins], v[kBins];
#pragma unroll
  for (int k = 0; k < kBins; ++k) {
    c0[k] = t0 < n_tiles ? sc->tile_cnt[t0][k] : 0u;
    c1[k] = t1 < n_tiles ? sc->tile_cnt[t1][k] : 0u;
    v[k] = c0[k] + c1[k];
  }
  uint32_t b0[kBins], tot[kBins];
  block_scan_cols<kBins>(v, b0, tot, sh.wave, sh.pre, sh.tot);   // its barriers order the reads above
  uint32_t b1[kBins];
#pragma unroll
  for (int k = 0; k < kBins; ++k) b1[k] = b0[k] + c0[k];
  if (t0 < n_tiles) {
#pragma unroll
    for (int k = 0; k < kBins; ++k) sc->tile_base[t0][k] = b0[k];
  }
  if (t1 < n_tiles) {
#pragma unroll
    for (int k = 0; k < kBins; ++k) sc->tile_base[t1][k] = b1[k];
  }
  if constexpr (ALLOC) {
    auto frontier_granules = [&](const uint32_t (&base)[kBins], const uint32_t (&c)[kBins]) {
      uint32_t g = 0;
#pragma unroll
      for (int k = 0; k < kBins; ++k) {
        const uint64_t lo = base[k] > cnt[k] ? base[k] : cnt[k];
        const uint64_t hi = (uint64_t)base[k] + c[k];
        if (hi > lo) g += (uint32_t)(hi - lo) * run_granules((uint32_t)k);
      }
      return g;
    };
    const uint32_t f0 = t0 < n_tiles ? frontier_granules(b0, c0) : 0u;
    const uint32_t f1 = t1 < n_tiles ? frontier_granules(b1, c1) : 0u;
    uint32_t fv[1] = {f0 + f1}, fex[1], ftot[1];
    block_scan_cols<1>(fv, fex, ftot, sh.wave, sh.pre, sh.tot);
    if (t0 < n_tiles) sc->tile_fbase[t0] = fex[0];
    if (t1 < n_tiles) sc->tile_fbase[t1] = (uint64_t)fex[0] + f0;
    if (threadIdx.x == 0) {
      sc->f_chunk = pend;
      sc->pend = pend + ftot[0];
    }
  }
  if (threadIdx.x < kBins) {
    const int k = (int)threadIdx.x;
    const uint64_t tk = pick(tot, k);
    sc->snap_cnt[k] = cnt[k];
    if (ALLOC) {
      hdr->bin_cnt[k] = cnt[k] - (tk < cnt[k] ? tk : cnt[k]);
    } else {
      const uint64_t c = cnt[k] + tk;
      hdr->bin_cnt[k] = c < hdr->bin_cap[k] ? c : hdr->bin_cap[k];
    }
  }
}

__device__ __forceinline__ void add_u64(uint64_t* p, uint64_t v) {
  if (v) atomicAdd(reinterpret_cast<unsigned long long*>(p), (unsigned long long)v);
}

// Pass 3 of allocation (one workgroup per tile): rank r of an item among its class: r < the
// bin's count pops the bin from the top; otherwise the frontier request starts after every
// earlier request of the call (granted or not) and is granted iff it ends within capacity.
template <class Access>
__global__ __launch_bounds__(kThreads) void pool_alloc_assign_kernel(PoolHdr* hdr,
                                                                     const uint32_t* bins,
                                                                     const PoolScratch* sc,
                                                                     Access acc, int first,
                                                                     int n_end) {
  __shared__ ScanShared sh;
  __shared__ uint64_t s_red[kWaves];
  if (hdr->magic != kPoolMagic) return;
  const int tile = blockIdx.x;
  const int i0 = first + tile * kTile + (int)threadIdx.x * kIpt;
  TileItems t;
  tile_classes(acc, i0, n_end, t);
  uint32_t kbase[kBins], ktot[kBins];
  block_scan_cols<kBins>(t.lcnt, kbase, ktot, sh.wave, sh.pre, sh.tot);
  const uint64_t cap = hdr->capacity;
  uint64_t off[kIpt];
  bool from_bin[kIpt];
  uint32_t zoff[kIpt];
  uint32_t lz[1] = {0};
#pragma unroll
  for (int sub = 0; sub < kIpt; ++sub) {
    const int k = t.key[sub];
    from_bin[sub] = false;
    off[sub] = KVZ_OFF_NONE;
    zoff[sub] = lz[0];
    if (k >= 0) {
      const uint64_t rank = (uint64_t)sc->tile_base[tile][k] + pick(kbase, k) + t.lrank[sub];
      const uint64_t ck = sc->snap_cnt[k];
      if (rank < ck) {
        from_bin[sub] = true;
        off[sub] = hdr->bin_base[k] + ck - 1 - rank;   // bin slot, read below
      } else {
        lz[0] += run_granules((uint32_t)k);
      }
    }
  }
  uint32_t zbase[1], ztot[1];
  block_scan_cols<1>(lz, zbase, ztot, sh.wave, sh.pre, sh.tot);
  const uint64_t fstart = sc->f_chunk + sc->tile_fbase[tile] + zbase[0];
  uint64_t my_granted = 0, my_runs = 0, my_gran = 0, my_raw = 0, my_fail = 0;
#pragma unroll
  for (int sub = 0; sub < kIpt; ++sub) {
    const int k = t.key[sub];
    if (k < 0) continue;
    const uint32_t z = run_granules((uint32_t)k);
    if (!from_bin[sub]) {
      const uint64_t start = fstart + zoff[sub];
      if (start + z <= cap) {
        off[sub] = start;
        my_granted += z;
      }
    }
    if (from_bin[sub] || off[sub] != KVZ_OFF_NONE) {
      my_runs += 1;
      my_gran += z;
      my_raw += (uint32_t)k;
    } else {
      my_fail += 1;
    }
  }
#pragma unroll
  for (int sub = 0; sub < kIpt; ++sub)
    if (from_bin[sub]) off[sub] = bins[off[sub]];
#pragma unroll
  for (int sub = 0; sub < kIpt; ++sub)
    if (t.key[sub] >= 0) acc.set_off(i0 + sub, (uint32_t)off[sub]);
  const uint64_t granted = block_sum(my_granted, s_red);
  const uint64_t runs = block_sum(my_runs, s_red);
  const uint64_t gran = block_sum(my_gran, s_red);
  const uint64_t raw = block_sum(my_raw, s_red);
  const uint64_t fail = block_sum(my_fail, s_red);
  if (threadIdx.x == 0) {
    add_u64(&hdr->frontier, granted);
    add_u64(&hdr->live_runs, runs);
    add_u64(&hdr->live_granules, gran);
    add_u64(&hdr->live_raw_blocks, raw);
    add_u64(&hdr->enospc, fail);
  }
}

// Pass 3 of free (one workgroup per tile): the i-th freed run of class k in item order goes to
// bin slot count + i (dropped and counted as a bad free if the bin is full).
__global__ __launch_bounds__(kThreads) void pool_free_apply_kernel(PoolHdr* hdr, uint32_t* bins,
                                                                   const PoolScratch* sc,
                                                                   kvz_group_meta* const* metas,
                                                                   int first, int n_end) {
  __shared__ ScanShared sh;
  __shared__ uint64_t s_red[kWaves];
  if (hdr->magic != kPoolMagic) return;
  const int tile = blockIdx.x;
  const int i0 = first + tile * kTile + (int)threadIdx.x * kIpt;
  kvz_group_meta* m[kIpt];
  uint2 rec[kIpt];
#pragma unroll
  for (int sub = 0; sub < kIpt; ++sub) m[sub] = i0 + sub < n_end ? metas[i0 + sub] : nullptr;
#pragma unroll
  for (int sub = 0; sub < kIpt; ++sub)
    rec[sub] = m[sub] ? *reinterpret_cast<const uint2*>(m[sub]) : make_uint2(KVZ_OFF_NONE, 0u);
  TileItems t;
#pragma unroll
  for (int k = 0; k < kBins; ++k) t.lcnt[k] = 0;
#pragma unroll
  for (int sub = 0; sub < kIpt; ++sub) {
    t.key[sub] = rec[sub].x != KVZ_OFF_NONE ? (int)n_raw_of(rec[sub].y) : -1;
    t.lrank[sub] = 0;
#pragma unroll
    for (int k = 0; k < kBins; ++k) {
      if (t.key[sub] == k) {
        t.lrank[sub] = t.lcnt[k];
        t.lcnt[k] += 1;
      }
    }
  }
  uint32_t kbase[kBins], ktot[kBins];
  block_scan_cols<kBins>(t.lcnt, kbase, ktot, sh.wave, sh.pre, sh.tot);
  uint64_t my_runs = 0, my_gran = 0, my_raw = 0, my_bad = 0;
#pragma unroll
  for (int sub = 0; sub < kIpt; ++sub) {
    const int k = t.key[sub];
    if (k >= 0) {
      const uint64_t slot = sc->snap_cnt[k] + sc->tile_base[tile][k] + pick(kbase, k) + t.lrank[sub];
      if (slot < hdr->bin_cap[k]) {
        bins[hdr->bin_base[k] + slot] = rec[sub].x;
        my_runs += 1;
        my_gran += run_granules((uint32_t)k);
        my_raw += (uint32_t)k;
      } else {
        my_bad += 1;
      }
    }
  }
  const uint64_t runs = block_sum(my_runs, s_red);
  const uint64_t gran = block_sum(my_gran, s_red);
  const uint64_t raw = block_sum(my_raw, s_red);
  const uint64_t bad = block_sum(my_bad, s_red);
  if (threadIdx.x == 0) {
    add_u64(&hdr->live_runs, 0ull - runs);
    add_u64(&hdr->live_granules, 0ull - gran);
    add_u64(&hdr->live_raw_blocks, 0ull - raw);
    add_u64(&hdr->bad_frees, bad);
  }
}

// Pass 4 of free: clear every listed metadata record (after pass 3 has read them all, so a
// record listed twice is seen the same way by every pass).
__global__ __launch_bounds__(kThreads) void pool_clear_meta_kernel(kvz_group_meta* const* metas,
                                                                   int first, int n_end) {
  const int tile_first = first + (int)blockIdx.x * kTile;
  const int tile_end = n_end - tile_first < kTile ? n_end : tile_first + kTile;
  for (int k = tile_first + (int)threadIdx.x; k < tile_end; k += kThreads) {
    kvz_group_meta* m = metas[k];
    if (m) *reinterpret_cast<uint2*>(m) = make_uint2(KVZ_OFF_NONE, 0u);
  }
}

// Calls of up to 4,096 items run in one workgroup, in one launch instead of three (allocation)
// or four (free): each thread takes a contiguous run of up to PER items and the ranks come from
// two block scans (class counts, then frontier granules).  Both the allocation and the free rule
// depend on item order only - an item's rank among the items of its class, and the granules all
// earlier frontier requests asked for - so this gives the same offsets, bins and counters as
// the tiled passes above.  Measured encode + free (graph replays): 576 items 41.6 -> 22.2 us
// (PER 2), 1,152 items 43.4 -> 25.9 us, 4,032 items 48.9 -> 43.7 us (PER 8); larger calls stay
// tiled (one workgroup took 37 us instead of 21 us for 9,216 items).
constexpr int kSmallPerLo = 2;                          // up to 1,024 items
constexpr int kSmallPerHi = 8;                          // up to 4,096 items
constexpr int kSmallItems = kThreads * kSmallPerHi;

template <int kSmallPer, class Access>
__global__ __launch_bounds__(kThreads) void pool_alloc_small_kernel(PoolHdr* hdr,
                                                                    const uint32_t* bins,
                                                                    Access acc, int n) {
  __shared__ ScanShared sh;
  __shared__ uint64_t s_red[kWaves];
  if (hdr->magic != kPoolMagic) return;
  const int per = (n + kThreads - 1) / kThreads;
  const int i0 = (int)threadIdx.x * per;
  int key[kSmallPer];
#pragma unroll
  for (int u = 0; u < kSmallPer; ++u) key[u] = (u < per && i0 + u < n) ? alloc_cls(acc, i0 + u) : -1;
  uint64_t cnt[kBins];
#pragma unroll
  for (int k = 0; k < kBins; ++k) cnt[k] = hdr->bin_cnt[k];
  const uint64_t f0 = hdr->frontier;
  const uint64_t cap = hdr->capacity;
  uint32_t lcnt[kBins];
#pragma unroll
  for (int k = 0; k < kBins; ++k) lcnt[k] = 0;
#pragma unroll
  for (int u = 0; u < kSmallPer; ++u)
#pragma unroll
    for (int k = 0; k < kBins; ++k) lcnt[k] += key[u] == k ? 1u : 0u;
  uint32_t kbase[kBins], ktot[kBins];
  block_scan_cols<kBins>(lcnt, kbase, ktot, sh.wave, sh.pre, sh.tot);
  // rank of each item among its class: below the bin's count it pops the bin from the top,
  // otherwise it asks the frontier for its run (prefix of every earlier request of the call)
  uint32_t pos[kSmallPer];     // bin slot, or granules requested before it by this thread
  uint32_t z = 0;
#pragma unroll
  for (int u = 0; u < kSmallPer; ++u) {
    const int k = key[u];
    pos[u] = 0;
    if (k < 0) continue;
    const uint64_t rank = pick(kbase, k);
#pragma unroll
    for (int j = 0; j < kBins; ++j) kbase[j] += j == k ? 1u : 0u;
    const uint64_t ck = cnt[k];
    if (rank < ck) {
      pos[u] = (uint32_t)(hdr->bin_base[k] + ck - 1 - rank);
    } else {
      pos[u] = z;
      key[u] = k + kBins;      // marks a frontier request
      z += run_granules((uint32_t)k);
    }
  }
  uint32_t zv[1] = {z}, zex[1], ztot[1];
  block_scan_cols<1>(zv, zex, ztot, sh.wave, sh.pre, sh.tot);
  uint64_t my_granted = 0, my_runs = 0, my_gran = 0, my_raw = 0, my_fail = 0;
  uint32_t off[kSmallPer];
#pragma unroll
  for (int u = 0; u < kSmallPer; ++u) {
    off[u] = KVZ_OFF_NONE;
    const int kk = key[u];
    if (kk < 0) continue;
    const bool frontier = kk >= kBins;
    const int k = frontier ? kk - kBins : kk;
    const uint32_t g = run_granules((uint32_t)k);
    if (frontier) {
      const uint64_t start = f0 + zex[0] + pos[u];
      if (start + g <= cap) {
        off[u] = (uint32_t)start;
        my_granted += g;
      }
    } else {
      off[u] = bins[pos[u]];
    }
    if (off[u] != KVZ_OFF_NONE || !frontier) {
      my_runs += 1;
      my_gran += g;
      my_raw += (uint32_t)k;
    } else {
      my_fail += 1;
    }
  }
#pragma unroll
  for (int u = 0; u < kSmallPer; ++u)
    if (key[u] >= 0) acc.set_off(i0 + u, off[u]);
  const uint64_t granted = block_sum(my_granted, s_red);
  const uint64_t runs = block_sum(my_runs, s_red);
  const uint64_t gran = block_sum(my_gran, s_red);
  const uint64_t raw = block_sum(my_raw, s_red);
  const uint64_t fail = block_sum(my_fail, s_red);
  // every thread read the header before the scans' barriers; one workgroup writes it back
  if (threadIdx.x < kBins) {
    const int k = (int)threadIdx.x;
    const uint64_t tk = pick(ktot, k);
    hdr->bin_cnt[k] = cnt[k] - (tk < cnt[k] ? tk : cnt[k]);
  }
  if (threadIdx.x == 0) {
    hdr->frontier = f0 + granted;
    hdr->live_runs += runs;
    hdr->live_granules += gran;
    hdr->live_raw_blocks += raw;
    hdr->enospc += fail;
  }
}

// The free of up to kSmallItems records in one workgroup: the i-th freed run of class k in item
// order goes to bin slot count + i (dropped and counted as a bad free if the bin is full); every
// listed record is cleared after all of them have been read.
template <int kSmallPer>
__global__ __launch_bounds__(kThreads) void pool_free_small_kernel(PoolHdr* hdr, uint32_t* bins,
                                                                   kvz_group_meta* const* metas,
                                                                   int n) {
  __shared__ ScanShared sh;
  __shared__ uint64_t s_red[kWaves];
  if (hdr->magic != kPoolMagic) return;
  const int per = (n + kThreads - 1) / kThreads;
  const int i0 = (int)threadIdx.x * per;
  kvz_group_meta* m[kSmallPer];
  uint2 rec[kSmallPer];
#pragma unroll
  for (int u = 0; u < kSmallPer; ++u) m[u] = (u < per && i0 + u < n) ? metas[i0 + u] : nullptr;
  typedef __attribute__((address_space(1))) uint64_t global_u64;   // global, not flat, accesses
#pragma unroll
  for (int u = 0; u < kSmallPer; ++u) {
    const uint64_t v = m[u] ? *(const global_u64*)(m[u]) : (uint64_t)KVZ_OFF_NONE;
    rec[u] = make_uint2((uint32_t)v, (uint32_t)(v >> 32));
  }
  // the header's per-class fields in LDS before any store (the bins share the state buffer with
  // the header, so a field read after a bin store would be a new round trip per item; a
  // register array indexed by class would live in scratch memory); the scan's barriers order
  // these writes before every read
  __shared__ uint64_t s_cnt[kBins], s_cap[kBins], s_base[kBins];
  if (threadIdx.x < kBins) {
    s_cnt[threadIdx.x] = hdr->bin_cnt[threadIdx.x];
    s_cap[threadIdx.x] = hdr->bin_cap[threadIdx.x];
    s_base[threadIdx.x] = hdr->bin_base[threadIdx.x];
  }
  uint32_t lcnt[kBins];
#pragma unroll
  for (int k = 0; k < kBins; ++k) lcnt[k] = 0;
  int key[kSmallPer];
#pragma unroll
  for (int u = 0; u < kSmallPer; ++u) {
    key[u] = rec[u].x != KVZ_OFF_NONE ? (int)n_raw_of(rec[u].y) : -1;
#pragma unroll
    for (int k = 0; k < kBins; ++k) lcnt[k] += key[u] == k ? 1u : 0u;
  }
  uint32_t kbase[kBins], ktot[kBins];
  block_scan_cols<kBins>(lcnt, kbase, ktot, sh.wave, sh.pre, sh.tot);   // orders all reads above
  uint64_t my_runs = 0, my_gran = 0, my_raw = 0, my_bad = 0;
#pragma unroll
  for (int u = 0; u < kSmallPer; ++u) {
    const int k = key[u];
    if (k < 0) continue;
    const uint64_t slot = s_cnt[k] + pick(kbase, k);
#pragma unroll
    for (int j = 0; j < kBins; ++j) kbase[j] += j == k ? 1u : 0u;
    if (slot < s_cap[k]) {
      bins[s_base[k] + slot] = rec[u].x;
      my_runs += 1;
      my_gran += run_granules((uint32_t)k);
      my_raw += (uint32_t)k;
    } else {
      my_bad += 1;
    }
  }
#pragma unroll
  for (int u = 0; u < kSmallPer; ++u)
    if (m[u]) *(global_u64*)(m[u]) = (uint64_t)KVZ_OFF_NONE;
  const uint64_t runs = block_sum(my_runs, s_red);
  const uint64_t gran = block_sum(my_gran, s_red);
  const uint64_t raw = block_sum(my_raw, s_red);
  const uint64_t bad = block_sum(my_bad, s_red);
  if (threadIdx.x < kBins) {
    const int k = (int)threadIdx.x;
    const uint64_t c = s_cnt[k] + pick(ktot, k);
    hdr->bin_cnt[k] = c < s_cap[k] ? c : s_cap[k];
  }
  if (threadIdx.x == 0) {
    hdr->live_runs -= runs;
    hdr->live_granules -= gran;
    hdr->live_raw_blocks -= raw;
    hdr->bad_frees += bad;
  }
}

__global__ void zero_words_kernel(uint32_t* p, uint32_t n) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

__global__ void pool_init_kernel(PoolHdr* hdr, uint64_t capacity, PoolHdr tmpl) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    *hdr = tmpl;
    hdr->capacity = capacity;
  }
}

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

void bin_layout(uint64_t capacity, uint64_t* cap, uint64_t* base, uint64_t* entries) {
  uint64_t at = 0;
  for (int k = 0; k < kBins; ++k) {
    cap[k] = capacity / (12 + k) + 1;
    base[k] = at;
    at += cap[k];
  }
  *entries = at;
}

template <class Access>
int run_alloc(kvz_pool* p, Access acc, int n, hipStream_t s) {
  PoolHdr* hdr = (PoolHdr*)p->state;
  const uint32_t* bins = (const uint32_t*)((uint8_t*)p->state + kPoolHdrBytes);
  PoolScratch* sc = (PoolScratch*)p->scratch;
  if (n <= kSmallItems) {
    if (n <= kThreads * kSmallPerLo)
      hipLaunchKernelGGL((pool_alloc_small_kernel<kSmallPerLo, Access>), dim3(1), dim3(kThreads), 0,
                         s, hdr, bins, acc, n);
    else
      hipLaunchKernelGGL((pool_alloc_small_kernel<kSmallPerHi, Access>), dim3(1), dim3(kThreads), 0,
                         s, hdr, bins, acc, n);
    return check_hip(hipGetLastError(), "slot alloc launch");
  }
  for (int first = 0; first < n; first += kChunkItems) {
    const int n_end = n - first < kChunkItems ? n : first + kChunkItems;
    const int tiles = (n_end - first + kTile - 1) / kTile;
    hipLaunchKernelGGL(pool_count_kernel<Access>, dim3(tiles), dim3(kThreads), 0, s, hdr, sc, acc,
                       first, n_end);
    hipLaunchKernelGGL(pool_scan_kernel<true>, dim3(1), dim3(kThreads), 0, s, hdr, sc, tiles,
                       first == 0 ? 1 : 0);
    hipLaunchKernelGGL(pool_alloc_assign_kernel<Access>, dim3(tiles), dim3(kThreads), 0, s, hdr,
                       bins, sc, acc, first, n_end);
    const int rc = check_hip(hipGetLastError(), "slot alloc launch");
    if (rc != KVZ_OK) return rc;
  }
  return KVZ_OK;
}

int check_pool(const kvz_pool* p) {
  if (!p) return set_error(KVZ_EINVAL, "pool handle is null");
  return KVZ_OK;
}

}  // namespace

}  // namespace kvz

using namespace kvz;

namespace kvz {
namespace {

// A pool over `granule`-byte granules: capacity = whole granules minus one kept as a guard.
int pool_state_bytes_g(uint64_t arena_bytes, uint64_t granule, uint64_t* state_bytes) {
  if (!state_bytes) return set_error(KVZ_EINVAL, "state_bytes is null");
  if (arena_bytes < 2 * granule) return set_error(KVZ_EINVAL, "arena smaller than 2 granules");
  const uint64_t capacity = arena_bytes / granule - 1;
  if (capacity >= KVZ_OFF_NONE) return set_error(KVZ_EINVAL, "arena too large for 32-bit granule offsets");
  uint64_t cap[kBins], base[kBins], entries;
  bin_layout(capacity, cap, base, &entries);
  *state_bytes = align256(kPoolHdrBytes + 4 * entries) + align256(sizeof(PoolScratch)) +
                 align256(kEncodeScratchBytes);
  return KVZ_OK;
}

int pool_init_g(kvz_pool** out, void* d_arena, uint64_t arena_bytes, void* d_state,
                uint64_t state_bytes, uint32_t granule, hipStream_t s) {
  if (!out || !d_arena || !d_state) return set_error(KVZ_EINVAL, "null pointer argument");
  if (((uintptr_t)d_arena | (uintptr_t)d_state) & 255u)
    return set_error(KVZ_EINVAL, "arena and state must be 256-byte aligned");
  uint64_t need = 0;
  int rc = pool_state_bytes_g(arena_bytes, granule, &need);
  if (rc != KVZ_OK) return rc;
  if (state_bytes < need) return set_error(KVZ_EINVAL, "state buffer too small");
  int dev = 0;
  rc = check_hip(hipGetDevice(&dev), "hipGetDevice");
  if (rc != KVZ_OK) return rc;
  const uint64_t capacity = arena_bytes / granule - 1;
  PoolHdr t = {};
  t.magic = kPoolMagic;
  t.version = kPoolVersion;
  t.capacity = capacity;
  uint64_t entries;
  bin_layout(capacity, t.bin_cap, t.bin_base, &entries);
  hipLaunchKernelGGL(pool_init_kernel, dim3(1), dim3(64), 0, s, (PoolHdr*)d_state, capacity, t);
  rc = check_hip(hipGetLastError(), "pool init launch");
  if (rc != KVZ_OK) return rc;
  // the one-pass encoder's records and ticket start cleared (no record carries an epoch yet)
  uint8_t* enc = (uint8_t*)d_state + align256(kPoolHdrBytes + 4 * entries) + align256(sizeof(PoolScratch));
  hipLaunchKernelGGL(zero_words_kernel, dim3(256), dim3(256), 0, s, (uint32_t*)enc,
                     (uint32_t)(kEncodeScratchBytes / 4));
  rc = check_hip(hipGetLastError(), "pool init launch");
  if (rc != KVZ_OK) return rc;
  kvz_pool* p = new (std::nothrow) kvz_pool;
  if (!p) return set_error(KVZ_EINVAL, "out of host memory");
  p->arena = d_arena;
  p->arena_bytes = arena_bytes;
  p->state = d_state;
  p->state_bytes = state_bytes;
  p->capacity = capacity;
  p->device = dev;
  p->scratch = (uint8_t*)d_state + align256(kPoolHdrBytes + 4 * entries);
  p->granule_bytes = granule;
  p->enc_scratch = enc;
  *out = p;
  return KVZ_OK;
}

}  // namespace
}  // namespace kvz

extern "C" int kvz_pool_state_bytes(uint64_t arena_bytes, uint64_t* state_bytes) {
  return pool_state_bytes_g(arena_bytes, KVZ_GRANULE_BYTES, state_bytes);
}

extern "C" int kvz_pool_init(kvz_pool** out, void* d_arena, uint64_t arena_bytes, void* d_state,
                             uint64_t state_bytes, hipStream_t s) {
  return pool_init_g(out, d_arena, arena_bytes, d_state, state_bytes, KVZ_GRANULE_BYTES, s);
}

extern "C" int kvz_fp8_pool_state_bytes(uint64_t arena_bytes, uint64_t* state_bytes) {
  return pool_state_bytes_g(arena_bytes, KVZ_FP8_GRANULE_BYTES, state_bytes);
}

extern "C" int kvz_fp8_pool_init(kvz_pool** out, void* d_arena, uint64_t arena_bytes, void* d_state,
                                 uint64_t state_bytes, hipStream_t s) {
  return pool_init_g(out, d_arena, arena_bytes, d_state, state_bytes, KVZ_FP8_GRANULE_BYTES, s);
}

extern "C" int kvz_pool_destroy(kvz_pool* p) {
  delete p;
  return KVZ_OK;
}

extern "C" int kvz_slot_alloc(kvz_pool* p, const uint8_t* d_tags, uint32_t* d_off, int32_t n,
                              hipStream_t s) {
  int rc = check_pool(p);
  if (rc != KVZ_OK) return rc;
  if (n < 0) return set_error(KVZ_EINVAL, "n < 0");
  if (n == 0) return KVZ_OK;
  if (!d_tags || !d_off) return set_error(KVZ_EINVAL, "null pointer argument");
  return run_alloc(p, TagArrayAccess{d_tags, d_off}, (int)n, s);
}

extern "C" int kvz_slot_free(kvz_pool* p, kvz_group_meta* const* d_metas, int32_t n, hipStream_t s) {
  int rc = check_pool(p);
  if (rc != KVZ_OK) return rc;
  if (n < 0) return set_error(KVZ_EINVAL, "n < 0");
  if (n == 0) return KVZ_OK;
  if (!d_metas) return set_error(KVZ_EINVAL, "null pointer argument");
  PoolHdr* hdr = (PoolHdr*)p->state;
  uint32_t* bins = (uint32_t*)((uint8_t*)p->state + kPoolHdrBytes);
  PoolScratch* sc = (PoolScratch*)p->scratch;
  const FreeAccess acc{d_metas};
  if (n <= kSmallItems) {
    if (n <= kThreads * kSmallPerLo)
      hipLaunchKernelGGL(pool_free_small_kernel<kSmallPerLo>, dim3(1), dim3(kThreads), 0, s, hdr,
                         bins, d_metas, n);
    else
      hipLaunchKernelGGL(pool_free_small_kernel<kSmallPerHi>, dim3(1), dim3(kThreads), 0, s, hdr,
                         bins, d_metas, n);
    return check_hip(hipGetLastError(), "slot free launch");
  }
  for (int first = 0; first < n; first += kChunkItems) {
    const int n_end = n - first < kChunkItems ? n : first + kChunkItems;
    const int tiles = (n_end - first + kTile - 1) / kTile;
    hipLaunchKernelGGL(pool_count_kernel<FreeAccess>, dim3(tiles), dim3(kThreads), 0, s, hdr, sc,
                       acc, first, n_end);
    hipLaunchKernelGGL(pool_scan_kernel<false>, dim3(1), dim3(kThreads), 0, s, hdr, sc, tiles,
                       first == 0 ? 1 : 0);
    hipLaunchKernelGGL(pool_free_apply_kernel, dim3(tiles), dim3(kThreads), 0, s, hdr, bins, sc,
                       d_metas, first, n_end);
    hipLaunchKernelGGL(pool_clear_meta_kernel, dim3(tiles), dim3(kThreads), 0, s, d_metas, first,
                       n_end);
    rc = check_hip(hipGetLastError(), "slot free launch");
    if (rc != KVZ_OK) return rc;
  }
  return KVZ_OK;
}

namespace kvz {
// Used by the encoders: the allocation step of kvz_encode_pages, kvz_gaac_encode_pages and
// kvz_fp8_encode_pages.
int launch_alloc_for_items(kvz_pool* p, const kvz_encode_item* d_items, int n, hipStream_t s) {
  return run_alloc(p, ItemMetaAccess<kvz_encode_item>{d_items}, n, s);
}
int launch_alloc_for_gaac_items(kvz_pool* p, const kvz_gaac_item* d_items, int n, hipStream_t s) {
  return run_alloc(p, ItemMetaAccess<kvz_gaac_item>{d_items}, n, s);
}
int launch_alloc_for_fp8_items(kvz_pool* p, const kvz_fp8_item* d_items, int n, hipStream_t s) {
  return run_alloc(p, ItemMetaAccess<kvz_fp8_item>{d_items}, n, s);
}
}  // namespace kvz

extern "C" int kvz_pool_stats(kvz_pool* p, kvz_pool_stats_t* host_out, hipStream_t s) {
  int rc = check_pool(p);
  if (rc != KVZ_OK) return rc;
  if (!host_out) return set_error(KVZ_EINVAL, "host_out is null");
  PoolHdr h;
  uint32_t ctl[2] = {0u, 0u};   // the one-pass encoder's launch number and halt flag
  rc = check_hip(hipMemcpyAsync(&h, p->state, sizeof(h), hipMemcpyDeviceToHost, s), "stats copy");
  if (rc != KVZ_OK) return rc;
  rc = check_hip(hipMemcpyAsync(ctl, p->enc_scratch, sizeof(ctl), hipMemcpyDeviceToHost, s), "stats copy");
  if (rc != KVZ_OK) return rc;
  rc = check_hip(hipStreamSynchronize(s), "stats sync");
  if (rc != KVZ_OK) return rc;
  if (h.magic != kPoolMagic || h.version != kPoolVersion)
    return set_error(KVZ_ESTATE, "pool state has a bad magic or version");
  host_out->capacity_granules = h.capacity;
  host_out->frontier_granules = h.frontier;
  for (int k = 0; k < kBins; ++k) host_out->free_runs[k] = h.bin_cnt[k];
  host_out->live_runs = h.live_runs;
  host_out->live_granules = h.live_granules;
  host_out->live_raw_blocks = h.live_raw_blocks;
  host_out->enospc = h.enospc;
  host_out->bad_frees = h.bad_frees;
  host_out->encoder_halted = ctl[1] ? 1u : 0u;
  return KVZ_OK;
}

extern "C" int kvz_pool_capacity(const kvz_pool_stats_t* st, int32_t num_layers,
                                 int32_t num_kv_heads, kvz_capacity_t* out) {
  if (!st || !out) return set_error(KVZ_EINVAL, "null pointer argument");
  if (num_layers <= 0 || num_kv_heads <= 0) return set_error(KVZ_EINVAL, "bad sizes");
  const uint64_t frontier_free =
      st->capacity_granules > st->frontier_granules ? st->capacity_granules - st->frontier_granules : 0;
  uint64_t binned = 0, min_bin = st->free_runs[0];
  for (int k = 0; k < kBins; ++k) {
    binned += st->free_runs[k] * (12u + (uint64_t)k);
    min_bin = st->free_runs[k] < min_bin ? st->free_runs[k] : min_bin;
  }
  const uint64_t groups_per_page = 2ull * (uint64_t)num_kv_heads * (uint64_t)num_layers;
  out->free_granules = frontier_free + binned;
  out->guaranteed_groups = frontier_free / 16u + min_bin;
  out->guaranteed_pages = out->guaranteed_groups / groups_per_page;
  out->guaranteed_tokens = 16u * out->guaranteed_pages;
  out->expected_group_granules =
      st->live_runs ? 12.0 + 4.0 * (double)st->live_raw_blocks / (4.0 * (double)st->live_runs) : 16.0;
  out->expected_pages = (uint64_t)((double)out->free_granules /
                                   (out->expected_group_granules * (double)groups_per_page));
  out->expected_tokens = 16u * out->expected_pages;
  return KVZ_OK;
}
