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
// kvz_encode_pages (and kvz_complete_pages, which also frees a list of groups first): a decode
// step's completion (up to kOnePassMaxItems items) is one launch of the one-pass encoder below
// (classify, allocate from published per-tile counts, pack from registers; each source read
// once); a bulk call is classify (one wave per item) -> allocate (pool.hip, multi-pass scan,
// item order) -> pack (one wave per item), the item's metadata slot carrying the tags from
// classify to allocate and the offset from allocate to pack.  Both give the same offsets.
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

// One-pass page completion: classify, allocate and pack in one launch, each source read once;
// optionally the free of a list of groups first, in the same launch.
//
// The launch is persistent: G = gridDim.x workgroups, no more than fit on the device at once,
// workgroup b taking tiles b, b + G, b + 2G, ... in order, so a tile only ever waits for lower
// tiles, which are resident or done.  Tiles [0, Tf) free up to kFreeTileItems listed groups
// each (only when every free tile is in the first round), tiles [Tf, T) encode kEncWaves * IPW
// items each.
//
// Every tile publishes its counts per size class as soon as it has classified its items.  An
// encode tile's exclusive prefix of those counts is its workgroup's previous encode tile's
// inclusive prefix (exactly G tiles back, kept in registers) plus the counts of the G - 1 tiles
// in between - published records, summed by the 256 threads at once.  No tile waits for
// another tile's prefix, so the tiles of a round only wait for each other's loads.  With those
// counts every item gets exactly the result of the item-order rule:
//  * the i-th freed run of class k goes to bin slot (count at launch start) + i, or is dropped
//    and counted as a bad free when the bin is full;
//  * after the free, the i-th encoded item of class k pops its bin from the top while the bin
//    lasts; later ones take prefix-summed frontier runs.
// A free tile clears its listed metadata records only after every free tile has read its
// records (as a separate free does), and marks itself done after its bin stores; encode tiles
// wait for every free tile to be done before popping a bin or writing a record.  Tile 0 also
// publishes the pool counters the launch starts from; the last tile writes the bins' new counts
// and adds the launch's totals as if every request were granted; a tile whose frontier requests
// do not fit subtracts them again and counts them as failed.
//
// Records, bin entries written in the launch and cleared metadata pass between workgroups with
// agent-scope (sc1) stores and loads: a record's fields are stored, the thread waits for those
// stores to complete (s_waitcnt vmcnt(0)), then its status is stored; a reader loads the status
// and only then the fields.  An encode tile's record, and a free tile's counts, are one 64-bit
// word each (tag and counts), stored and read with no status.  The tag is the epoch (the
// launch's number), read from the pool state at the start of the launch and advanced by the
// last tile's workgroup once every workgroup has read it (see the kernel), so every execution -
// a replay of a captured graph too - tags its records anew.
constexpr int kEncWaves = 4;
constexpr int kEncThreads = kEncWaves * 64;
constexpr int kFreePer = 2;                                  // listed groups per thread of a free tile
constexpr int kFreeTileItems = kEncThreads * kFreePer;
constexpr int kMaxFreeTiles = kMaxFreeSlots;
static_assert(kMaxFreeTiles <= kEncThreads, "one waiting thread per free tile");
constexpr uint32_t kMaxSpins = 1u << 20;   // a wait that never ends marks its tile's items unstored
constexpr uint32_t kStBad = 2, kStDone = 3;                  // free-slot states (low two status bits)
constexpr int kAggBits = 10;                                 // per class in a free tile's count word
static_assert(kFreePer * kEncThreads < (1 << kAggBits), "a free tile's counts fit their fields");
constexpr int kCountBits = 6;                                // per class in an encode record
constexpr int kPollBatch = 4;                                // record loads in flight per thread
// the control area's first two words, read and written as one 64-bit word: launches completed,
// and the halt flag (set by a launch that gave up a wait; see the kernel)
constexpr int kCtlLaunches = 0, kCtlHalted = 1;

__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_agent64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void add_agent(uint64_t* p, uint64_t v) {
  if (v) atomicAdd(reinterpret_cast<unsigned long long*>(p), (unsigned long long)v);
}

// The state of a free slot of this launch once it is at least `min_state` (0 if the wait gave up).
__device__ __forceinline__ uint32_t wait_state(const EncodeSlot* s, uint32_t epoch, uint32_t min_state) {
  for (uint32_t spins = 0;; ++spins) {
    const uint32_t st = ld_agent(&s->status);
    if ((st >> 2) == epoch && (st & 3u) >= min_state) return st & 3u;
    if (spins > kMaxSpins) return 0u;
    __builtin_amdgcn_s_sleep(1);
  }
}
// An encode tile's record of this launch (counts in the low 32 bits), or ~0 if the wait gave up.
__device__ __forceinline__ uint64_t wait_record(const uint64_t* r, uint32_t epoch) {
  for (uint32_t spins = 0;; ++spins) {
    const uint64_t v = ld_agent64(r);
    if ((uint32_t)(v >> 32) == epoch) return v;
    if (spins > kMaxSpins) return ~0ull;
    __builtin_amdgcn_s_sleep(1);
  }
}

// The 14-bit form of an epoch in a free tile's count word (never 0: a zeroed word matches none).
__device__ __forceinline__ uint32_t epoch14(uint32_t epoch) { return epoch % 16383u + 1u; }
// A free tile's count word of this launch, or ~0 if the wait gave up.
__device__ __forceinline__ uint64_t wait_agg(const uint64_t* w, uint32_t epoch) {
  const uint64_t want = epoch14(epoch);
  for (uint32_t spins = 0;; ++spins) {
    const uint64_t v = ld_agent64(w);
    if ((v >> (kBins * kAggBits)) == want) return v;
    if (spins > kMaxSpins) return ~0ull;
    __builtin_amdgcn_s_sleep(1);
  }
}
__device__ __forceinline__ uint32_t agg_count(uint64_t w, int k) {
  return (uint32_t)(w >> (kAggBits * k)) & ((1u << kAggBits) - 1u);
}

struct OnePassShared {
  uint32_t part[kEncWaves][kBins];
  uint32_t bad;
  uint32_t snap[kBins];      // bin counts the launch started from
  uint32_t f0_lo, f0_hi;     // frontier the launch started from
};

// Block sum of five counters; the result in every thread.
__device__ __forceinline__ void block_sum5(uint32_t (&v)[kBins], OnePassShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < kBins; ++k) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v[k] += (uint32_t)__shfl_xor((int)v[k], d, 64);
  }
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < kBins; ++k) sh.part[wave][k] = v[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kBins; ++k) {
    uint32_t s = 0;
#pragma unroll
    for (int w = 0; w < kEncWaves; ++w) s += sh.part[w][k];
    v[k] = s;
  }
  __syncthreads();
}

// The launch's starting counters (tile 0's slot), by one thread; false if the wait gave up.
__device__ __forceinline__ bool read_start(const EncodeSlot* slots, uint32_t epoch, OnePassShared& sh) {
  for (uint32_t spins = 0; ld_agent(&slots[0].sstat) != epoch; ++spins) {
    if (spins > kMaxSpins) return false;
    __builtin_amdgcn_s_sleep(1);
  }
#pragma unroll
  for (int k = 0; k < kBins; ++k) sh.snap[k] = ld_agent(&slots[0].snap[k]);
  sh.f0_lo = ld_agent(&slots[0].f0_lo);
  sh.f0_hi = ld_agent(&slots[0].f0_hi);
  return true;
}

template <int kPolicy, int IPW>
__global__ __launch_bounds__(kEncThreads, 4) void encode_onepass_kernel(
    const kvz_encode_item* items, int n, kvz_group_meta* const* frees, int n_free, uint32_t flags,
    PoolHdr* hdr, uint32_t* bins, uint8_t* arena, uint32_t* ctl, EncodeSlot* slots, uint64_t* erec,
    int n_free_tiles, int n_tiles) {
  constexpr int kTileItems = kEncWaves * IPW;
  static_assert(kTileItems < (1 << kCountBits), "a tile's counts fit their record fields");
  typedef __attribute__((address_space(1))) uint64_t global_u64;
  __shared__ OnePassShared sh;
  __shared__ uint32_t s_cls[kTileItems];      // size class (raw blocks) of each item; 0xFF: none
  __shared__ uint32_t s_rank[kTileItems];     // rank of each item among the launch's items of its class
  __shared__ uint64_t s_start[kTileItems];    // frontier start of each item if it asks the frontier
  __shared__ uint32_t s_avail[kBins];         // bin counts after this launch's free
  __shared__ uint32_t s_ok;
  __shared__ uint64_t s_fail[kEncWaves][4];   // failed requests: count, granules, raw blocks
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if (hdr->magic != kPoolMagic) return;   // host checked; never write through a bad state
  const uint64_t cap = hdr->capacity;
  // per-class pool constants (never written by a launch), read before any store; in LDS, as
  // the bin of an item is a per-lane index (the first barrier of a tile orders these writes)
  __shared__ uint32_t s_bcap[kBins];
  __shared__ uint64_t s_bbase[kBins];
  if (threadIdx.x < kBins) {
    s_bcap[threadIdx.x] = (uint32_t)hdr->bin_cap[threadIdx.x];
    s_bbase[threadIdx.x] = hdr->bin_base[threadIdx.x];
  }
  const int Tf = n_free_tiles;
  const int G = gridDim.x;
  // The launch's number tags its records: read from the device at the start (so a replayed
  // graph gets a new one each time), and taken - put in LDS for the tile's first barrier - once
  // the workgroup's first loads are out, so that waiting for it costs nothing.  Every workgroup
  // publishes a record or a slot status with it before the last tile's waits end; so the
  // workgroup of the last tile, once those waits have all succeeded, has seen every read of the
  // number, and it advances the number at its end.  If one of its waits gave up instead, a
  // workgroup may not have started yet; started later, it would read the advanced number and
  // could leave records that the next launch took for its own.  That launch therefore sets the
  // halt flag with the number: a workgroup that reads the flag (a late one, or one of any later
  // launch until the pool is initialised again) stores nothing and publishes nothing.
  __shared__ uint32_t s_epoch;   // 0: halted
  uint32_t launches = 0, halted = 0;
  if (threadIdx.x == 0) {
    sh.bad = 0u;
    const uint64_t c = ld_agent64(reinterpret_cast<const uint64_t*>(ctl));
    launches = (uint32_t)c;
    halted = (uint32_t)(c >> 32);
    // the counters the launch starts from: tile 0 publishes them; a free tile reads the bin
    // counts itself (only the last tile writes them, after every free tile has published)
    if (blockIdx.x == 0 || (int)blockIdx.x < Tf) {
#pragma unroll
      for (int k = 0; k < kBins; ++k) sh.snap[k] = (uint32_t)hdr->bin_cnt[k];
    }
    if (blockIdx.x == 0) {
      const uint64_t f0 = hdr->frontier;
      sh.f0_lo = (uint32_t)f0;
      sh.f0_hi = (uint32_t)(f0 >> 32);
    }
  }
  // (thread 0, before a barrier that the whole workgroup reaches; once per workgroup)
  auto take_number = [&]() {
    if (threadIdx.x != 0) return;
    s_epoch = halted ? 0u : launches % ((1u << 30) - 1u) + 1u;
    if (halted) return;
    if (flags & KVZ_ENC_SIMULATE_GIVE_UP) sh.bad = 1u;   // as if a wait of this workgroup gave up
  };
  // tile 0's start counters, stored once its first loads are out (thread 0; their status
  // follows a wait for its stores: after the free tile's scan, or after the encode tile's
  // record, which every other tile waits for and so goes first)
  auto store_start = [&]() {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
#pragma unroll
    for (int k = 0; k < kBins; ++k) st_agent(&slots[0].snap[k], sh.snap[k]);
    st_agent(&slots[0].f0_lo, sh.f0_lo);
    st_agent(&slots[0].f0_hi, sh.f0_hi);
  };
  uint32_t epoch = 0;   // from s_epoch after the first barrier past take_number
  bool numbered = false, last_tile = false;

  // ---------------- a free tile (at most one per workgroup: every free tile is in the first
  // round): kFreePer listed groups per thread, in item order
  if ((int)blockIdx.x < Tf) {
    const int tile = blockIdx.x;
    EncodeSlot* me = slots + tile;
    const int e0 = tile * kFreeTileItems + (int)threadIdx.x * kFreePer;
    kvz_group_meta* m[kFreePer];
    uint64_t rec[kFreePer];
#pragma unroll
    for (int u = 0; u < kFreePer; ++u) m[u] = e0 + u < n_free ? frees[e0 + u] : nullptr;
    store_start();
#pragma unroll
    for (int u = 0; u < kFreePer; ++u) rec[u] = m[u] ? *(const global_u64*)(m[u]) : (uint64_t)KVZ_OFF_NONE;
    int key[kFreePer];
    uint32_t mine[kBins] = {0u, 0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < kFreePer; ++u) {
      key[u] = (uint32_t)rec[u] != KVZ_OFF_NONE ? (int)n_raw_of((uint32_t)(rec[u] >> 32)) : -1;
#pragma unroll
      for (int k = 0; k < kBins; ++k) mine[k] += key[u] == k ? 1u : 0u;
    }
    // this thread's first rank in the tile per class: an exclusive scan over the threads
    uint32_t incl_t[kBins];
#pragma unroll
    for (int k = 0; k < kBins; ++k) {
      incl_t[k] = mine[k];
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = (uint32_t)__shfl_up((int)incl_t[k], d, 64);
        if (lane >= d) incl_t[k] += o;
      }
      if (lane == 63) sh.part[wave][k] = incl_t[k];
    }
    take_number();
    numbered = true;
    __syncthreads();
    epoch = s_epoch;
    if (epoch != 0u) {   // (halted: this launch frees nothing)
      uint32_t agg[kBins], rank0[kBins];
#pragma unroll
      for (int k = 0; k < kBins; ++k) {
        uint32_t below = 0, tot = 0;
#pragma unroll
        for (int w = 0; w < kEncWaves; ++w) {
          below += w < wave ? sh.part[w][k] : 0u;
          tot += sh.part[w][k];
        }
        rank0[k] = below + incl_t[k] - mine[k];
        agg[k] = tot;
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        if (tile == 0) {   // the start counters (stored with the first loads: complete by now)
          __builtin_amdgcn_s_waitcnt(0);
          st_agent(&slots[0].sstat, epoch);
        }
        uint64_t w = (uint64_t)epoch14(epoch) << (kBins * kAggBits);
#pragma unroll
        for (int k = 0; k < kBins; ++k) w |= (uint64_t)agg[k] << (kAggBits * k);
        st_agent64(&me->aggw, w);   // one word: readers need no status for it
      }
      // every free tile's counts (each published only after its records were read): the runs
      // freed by the tiles below this one, and leave to clear
      uint32_t pre[kBins] = {0u, 0u, 0u, 0u, 0u};
      if ((int)threadIdx.x < Tf && (int)threadIdx.x != tile) {   // (its own records are read)
        const uint64_t w = wait_agg(&slots[threadIdx.x].aggw, epoch);
        if (w == ~0ull) {
          sh.bad = 1u;
        } else if ((int)threadIdx.x < tile) {
#pragma unroll
          for (int k = 0; k < kBins; ++k) pre[k] = agg_count(w, k);
        }
      }
      block_sum5(pre, sh);
      const bool ok = sh.bad == 0u;
      uint64_t my_runs = 0, my_gran = 0, my_raw = 0, my_bad = 0;
#pragma unroll
      for (int u = 0; u < kFreePer; ++u) {
        const int k = key[u];
        if (k < 0) continue;
        uint32_t r = 0;
#pragma unroll
        for (int j = 0; j < kBins; ++j) {
          if (j == k) {
            r = sh.snap[j] + pre[j] + rank0[j];
            rank0[j] += 1;
          }
        }
        if (ok && r < s_bcap[k]) {
          st_agent(bins + s_bbase[k] + r, (uint32_t)rec[u]);
          my_runs += 1;
          my_gran += run_granules((uint32_t)k);
          my_raw += (uint32_t)k;
        } else {
          my_bad += 1;
        }
      }
      if (ok) {
#pragma unroll
        for (int u = 0; u < kFreePer; ++u)
          if (m[u]) st_agent64((uint64_t*)(m[u]), (uint64_t)KVZ_OFF_NONE);
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();   // every thread's bin stores and clears are complete
      if (threadIdx.x == 0) {
        // a free tile that gave up a wait pushed nothing: the launch's encode tiles then store
        // nothing and empty the bins (runs leak; no bin entry is ever stale)
        st_agent(&me->status, (epoch << 2) | (ok ? kStDone : kStBad));
      }
      // the tile's totals (the counters of a free that cannot happen stay as they were)
      uint32_t tot[kBins] = {(uint32_t)my_runs, (uint32_t)my_gran, (uint32_t)my_raw, (uint32_t)my_bad, 0u};
      block_sum5(tot, sh);
      if (threadIdx.x == 0) {
        add_agent(&hdr->live_runs, (uint64_t)0 - tot[0]);
        add_agent(&hdr->live_granules, (uint64_t)0 - tot[1]);
        add_agent(&hdr->live_raw_blocks, (uint64_t)0 - tot[2]);
        add_agent(&hdr->bad_frees, tot[3]);
      }
    }
  }

  // ---------------- encode tiles
  const int t_first = (int)blockIdx.x < Tf ? (int)blockIdx.x + G : (int)blockIdx.x;
  uint32_t freed[kBins] = {0u, 0u, 0u, 0u, 0u};   // runs this launch's free put in each bin
  uint32_t carry[kBins] = {0u, 0u, 0u, 0u, 0u};   // inclusive prefix of this workgroup's last tile

  for (int tile = t_first; tile < n_tiles; tile += G) {
    const int et = tile - Tf;                 // encode tile index
    last_tile = tile == n_tiles - 1;
    // load and classify this wave's items
    uint4 w[IPW][4];
    uint32_t tags[IPW];
    kvz_encode_item it[IPW];
#pragma unroll
    for (int u = 0; u < IPW; ++u) {
      const int item = (et * kEncWaves + wave) * IPW + u;
      tags[u] = 0;
      if (item < n) {
        it[u] = items[item];
        load_item_chunks<kPolicy>(it[u].src, it[u].src_stride, it[u].kind, lane, w[u]);
      }
    }
    if (!numbered && Tf == 0) store_start();
#pragma unroll
    for (int u = 0; u < IPW; ++u) {
      const int item = (et * kEncWaves + wave) * IPW + u;
      if (item >= n) {
        if (lane == 0) s_cls[wave * IPW + u] = 0xFFu;
        continue;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t lo = 255u, hi = 0u;
        chunk_exp_range(w[u][j], lo, hi);
        lo = wave_min(lo);
        hi = wave_max(hi);
        const uint32_t b = lo & 0xFEu;
        const uint32_t tag = (hi <= b + 15u && !(flags & KVZ_ENC_FORCE_RAW)) ? (b >> 1) : KVZ_RAW_TAG;
        tags[u] |= tag << (8 * j);
      }
      if (lane == 0) s_cls[wave * IPW + u] = n_raw_of(tags[u]);
    }
    if (!numbered) take_number();
    __syncthreads();
    if (!numbered) {
      epoch = s_epoch;
      numbered = true;
    }
    if (epoch == 0u) {   // halted: the items are stored nowhere, counted as failed
      uint32_t failed = 0;
#pragma unroll
      for (int u = 0; u < IPW; ++u) {
        const int item = (et * kEncWaves + wave) * IPW + u;
        if (item >= n) continue;
        failed += 1;
        if (lane == 0) *(global_u64*)(it[u].dst) = (uint64_t)KVZ_OFF_NONE | ((uint64_t)tags[u] << 32);
      }
      if (lane == 0) add_agent(&hdr->enospc, failed);
      continue;
    }
    uint32_t agg[kBins];
#pragma unroll
    for (int k = 0; k < kBins; ++k) agg[k] = 0;
    for (int i = 0; i < kTileItems; ++i) {
      const uint32_t c = s_cls[i];
#pragma unroll
      for (int k = 0; k < kBins; ++k) agg[k] += c == (uint32_t)k ? 1u : 0u;
    }
    if (threadIdx.x == 0) {
      uint64_t packed = (uint64_t)epoch << 32;
#pragma unroll
      for (int k = 0; k < kBins; ++k) packed |= (uint64_t)agg[k] << (kCountBits * k);
#pragma unroll
      for (int c = 0; c < kRecordCopies; ++c) st_agent64(erec + c * kMaxEncodeTiles + et, packed);
      if (blockIdx.x == 0 && Tf == 0 && tile == t_first) {   // tile 0 encodes: the start counters
        __builtin_amdgcn_s_waitcnt(0);
        st_agent(&slots[0].sstat, epoch);
      }
    }

    // the counts of the encode tiles between this workgroup's previous tile and this one
    uint32_t pre[kBins] = {0u, 0u, 0u, 0u, 0u};
    // (every kEncThreads-th record below this tile per thread, kPollBatch loads in flight at
    // once; only a record not yet published is polled again)
    const int lo = et - G + 1 > 0 ? et - G + 1 : 0;
    const uint64_t* rec_copy = erec + (blockIdx.x % kRecordCopies) * kMaxEncodeTiles;
    bool gave_up = false;
    for (int i0 = et - 1 - (int)threadIdx.x; i0 >= lo && !gave_up; i0 -= kPollBatch * kEncThreads) {
      uint64_t r[kPollBatch];
#pragma unroll
      for (int u = 0; u < kPollBatch; ++u) {
        const int i = i0 - u * kEncThreads;
        r[u] = i >= lo ? ld_agent64(rec_copy + i) : (uint64_t)epoch << 32;
      }
#pragma unroll
      for (int u = 0; u < kPollBatch; ++u) {
        if ((uint32_t)(r[u] >> 32) != epoch && !gave_up) {
          r[u] = wait_record(rec_copy + (i0 - u * kEncThreads), epoch);
          gave_up = r[u] == ~0ull;
        }
        if ((uint32_t)(r[u] >> 32) != epoch) continue;
#pragma unroll
        for (int k = 0; k < kBins; ++k) pre[k] += (uint32_t)(r[u] >> (kCountBits * k)) & ((1u << kCountBits) - 1u);
      }
    }
    if (gave_up) sh.bad = 1u;
    block_sum5(pre, sh);
#pragma unroll
    for (int k = 0; k < kBins; ++k) {
      pre[k] += carry[k];
      carry[k] = pre[k] + agg[k];
    }
    if (tile == t_first) {
      // once per workgroup, after its first tile's loads and counts: the launch's start counters
      // (tile 0 has them already) and the bins after this launch's free (every free tile done:
      // its bin stores and clears are out)
      if (threadIdx.x == kEncThreads - 1 && blockIdx.x != 0 && !read_start(slots, epoch, sh))
        sh.bad = 1u;
      if ((int)threadIdx.x < Tf) {
        if (wait_state(slots + threadIdx.x, epoch, kStBad) != kStDone) sh.bad = 1u;
        const uint64_t w = ld_agent64(&slots[threadIdx.x].aggw);   // (complete before the status)
#pragma unroll
        for (int k = 0; k < kBins; ++k) freed[k] = agg_count(w, k);
      }
      block_sum5(freed, sh);   // (its barriers also order the shared counters above)
    }
    const bool ok = sh.bad == 0u;

    if (threadIdx.x == 0) {
      uint32_t snap[kBins];
      uint64_t f0 = ((uint64_t)sh.f0_hi << 32) | sh.f0_lo;
#pragma unroll
      for (int k = 0; k < kBins; ++k) {
        const uint32_t c = sh.snap[k] + freed[k];   // bins after the free (full bins drop runs)
        snap[k] = c < s_bcap[k] ? c : s_bcap[k];
      }
      if (!ok) {   // never happens while every lower tile is resident or done
#pragma unroll
        for (int k = 0; k < kBins; ++k) snap[k] = 0;
        f0 = cap;
      }
      // each item's rank in its class and, for a frontier request, where its run starts: the
      // frontier requests of earlier tiles are the items of class k beyond the bin's count
      uint64_t fnext = f0;
#pragma unroll
      for (int k = 0; k < kBins; ++k) {
        s_avail[k] = snap[k];
        if (pre[k] > snap[k]) fnext += (uint64_t)(pre[k] - snap[k]) * run_granules((uint32_t)k);
      }
      uint32_t run_k[kBins];
#pragma unroll
      for (int k = 0; k < kBins; ++k) run_k[k] = pre[k];
      for (int i = 0; i < kTileItems; ++i) {
        const uint32_t c = s_cls[i];
        if (c == 0xFFu) continue;
        uint32_t r = 0, sc = 0;
#pragma unroll
        for (int k = 0; k < kBins; ++k) {
          if (c == (uint32_t)k) {
            r = run_k[k];
            run_k[k] += 1;
            sc = snap[k];
          }
        }
        s_rank[i] = r;
        s_start[i] = fnext;
        if (r >= sc) fnext += run_granules(c);
      }
      s_ok = ok ? 1u : 0u;
      // the last tile knows every item of the launch: the bins' new counts, and the launch's
      // totals as if every request were granted (tiles with failed requests correct them)
      if (tile == n_tiles - 1) {
        uint64_t runs = 0, gran = 0, raw = 0;
#pragma unroll
        for (int k = 0; k < kBins; ++k) {
          const uint32_t tot = carry[k];
          hdr->bin_cnt[k] = snap[k] - (tot < snap[k] ? tot : snap[k]);
          runs += tot;
          gran += (uint64_t)tot * run_granules((uint32_t)k);
          raw += (uint64_t)tot * (uint32_t)k;
        }
        add_agent(&hdr->frontier, fnext - f0);
        add_agent(&hdr->live_runs, runs);
        add_agent(&hdr->live_granules, gran);
        add_agent(&hdr->live_raw_blocks, raw);
      }
    }
    __syncthreads();

    // allocate this wave's items in item order, then pack them from registers
    uint64_t fail = 0, fail_gran = 0, fail_raw = 0, fail_front = 0;
#pragma unroll
    for (int u = 0; u < IPW; ++u) {
      const int idx = wave * IPW + u;
      const int item = et * kTileItems + idx;
      if (item >= n) continue;
      const uint32_t k = s_cls[idx];
      const uint32_t rank = s_rank[idx];
      const uint32_t z = run_granules(k);
      const uint32_t avail = s_avail[k];
      uint32_t off = KVZ_OFF_NONE;
      const bool from_bin = rank < avail;
      if (from_bin) {
        off = ld_agent(bins + s_bbase[k] + avail - 1u - rank);   // may have been pushed by this launch
      } else if (s_start[idx] + z <= cap) {
        off = (uint32_t)s_start[idx];
      }
      if (!s_ok) off = KVZ_OFF_NONE;
      if (off == KVZ_OFF_NONE) {
        fail += 1;
        fail_gran += z;
        fail_raw += k;
        if (!from_bin) fail_front += z;
      }
      if (lane == 0) *(global_u64*)(it[u].dst) = (uint64_t)off | ((uint64_t)tags[u] << 32);
      if (off == KVZ_OFF_NONE) continue;
      // non-temporal stores: the records stream to memory instead of staying dirty in the L2
      // until the end of the launch
      uint8_t* blk = arena + (size_t)off * KVZ_GRANULE_BYTES;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t tag = (tags[u] >> (8 * j)) & 0xFFu;
        if (tag == KVZ_RAW_TAG) {
          typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
          __builtin_nontemporal_store(__builtin_bit_cast(u32x4, w[u][j]),
                                      reinterpret_cast<u32x4*>(blk + kRawChunkBytes * lane));
        } else {
          const uint3 c = compress_chunk(w[u][j], tag * 0x01010101u);
          uint32_t* d = reinterpret_cast<uint32_t*>(blk + kCompChunkBytes * lane);
          __builtin_nontemporal_store(c.x, d);
          __builtin_nontemporal_store(c.y, d + 1);
          __builtin_nontemporal_store(c.z, d + 2);
        }
        blk += block_bytes(tag);
      }
    }
    // failed requests (a full pool): taken back out of the totals, counted as failed
    if (lane == 0) {
      s_fail[wave][0] = fail;
      s_fail[wave][1] = fail_gran;
      s_fail[wave][2] = fail_raw;
      s_fail[wave][3] = fail_front;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      uint64_t f[4] = {0, 0, 0, 0};
      for (int q = 0; q < kEncWaves; ++q)
#pragma unroll
        for (int c = 0; c < 4; ++c) f[c] += s_fail[q][c];
      if (f[0]) {
        add_agent(&hdr->enospc, f[0]);
        add_agent(&hdr->live_runs, (uint64_t)0 - f[0]);
        add_agent(&hdr->live_granules, (uint64_t)0 - f[1]);
        add_agent(&hdr->live_raw_blocks, (uint64_t)0 - f[2]);
        add_agent(&hdr->frontier, (uint64_t)0 - f[3]);
      }
    }
  }
  // the last tile's workgroup: the count words of the slots this launch did not use zeroed, the
  // next number, and the halt flag if one of its waits gave up (every sh.bad write is ordered
  // before this by the tile's last barrier)
  if (last_tile && epoch != 0u) {
    for (int i = Tf + (int)threadIdx.x; i < kMaxFreeSlots; i += kEncThreads) st_agent64(&slots[i].aggw, 0ull);
  }
  if (threadIdx.x == 0 && last_tile && epoch != 0u)
    st_agent64(reinterpret_cast<uint64_t*>(ctl),
               ((uint64_t)(sh.bad != 0u ? 1u : 0u) << 32) | (uint64_t)(launches + 1u));
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

namespace kvz {
namespace {

// Calls of up to this many items take the one-pass kernel (at most two rounds of tiles).
// Larger (bulk, prefill) calls take classify -> the multi-pass allocation -> pack, each a fully
// parallel stream: measured on an 8K layer (130,816 groups) 284 us of kernels against 380 us
// for the one-pass kernel, whose tiles of a round all wait for each other's counts (250 us
// with that wait taken out, 232 us with the stores also taken out).
constexpr int kOnePassMaxItems = 16384;
static_assert(kOnePassMaxItems <= kMaxEncodeTiles * kEncWaves * 2 && 4096 <= kMaxEncodeTiles * kEncWaves,
              "every one-pass tile has a record");

// One one-pass launch for n items, also freeing the n_free listed groups first when all of its
// free tiles fit in the first round; otherwise the free runs first as its own call.
int encode_onepass(kvz_pool* p, const kvz_encode_item* d_items, int n,
                   kvz_group_meta* const* d_free, int n_free, uint32_t flags, hipStream_t s) {
  PoolHdr* hdr = (PoolHdr*)p->state;
  uint32_t* bins = (uint32_t*)((uint8_t*)p->state + kPoolHdrBytes);
  uint32_t* ctl = (uint32_t*)p->enc_scratch;
  EncodeSlot* slots = (EncodeSlot*)((uint8_t*)p->enc_scratch + kEncodeCtlBytes);
  uint64_t* erec = (uint64_t*)(slots + kMaxFreeSlots);
  const int ipw = n <= 4096 ? 1 : 2;
  const void* fn = ipw == 1 ? (const void*)encode_onepass_kernel<kCachedLoad, 1>
                            : (const void*)encode_onepass_kernel<kCachedLoad, 2>;
  int per_cu = 0;
  int rc = check_hip(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kEncThreads, 0),
                     "occupancy query");
  if (rc != KVZ_OK) return rc;
  const int resident = (per_cu > 0 ? per_cu : 1) * device_cus();
  int tf = n_free > 0 ? (n_free + kFreeTileItems - 1) / kFreeTileItems : 0;
  if (tf > resident || tf > kMaxFreeTiles) {
    rc = kvz_slot_free(p, d_free, n_free, s);
    if (rc != KVZ_OK) return rc;
    tf = 0;
  }
  const int per_tile = kEncWaves * ipw;
  const int tiles = tf + (n + per_tile - 1) / per_tile;
  const int grid = tiles < resident ? tiles : resident;
  if (ipw == 1)
    hipLaunchKernelGGL((encode_onepass_kernel<kCachedLoad, 1>), dim3(grid), dim3(kEncThreads), 0, s,
                       d_items, n, d_free, tf ? n_free : 0, flags, hdr, bins, (uint8_t*)p->arena,
                       ctl, slots, erec, tf, tiles);
  else
    hipLaunchKernelGGL((encode_onepass_kernel<kCachedLoad, 2>), dim3(grid), dim3(kEncThreads), 0, s,
                       d_items, n, d_free, tf ? n_free : 0, flags, hdr, bins, (uint8_t*)p->arena,
                       ctl, slots, erec, tf, tiles);
  return check_hip(hipGetLastError(), "encode launch");
}

// The bulk path: classify (tags into each item's metadata), allocate (pool.hip, item order),
// pack (offset from the metadata) - each source read twice.
int encode_bulk(kvz_pool* p, const kvz_encode_item* d_items, int n, uint32_t flags, hipStream_t s) {
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

int check_encode_args(kvz_pool* p, const kvz_encode_item* d_items, int32_t n, uint32_t flags) {
  if (!p) return set_error(KVZ_EINVAL, "pool handle is null");
  if (p->granule_bytes != KVZ_GRANULE_BYTES)
    return set_error(KVZ_EINVAL, "pool was made for FP8 tiles (kvz_fp8_pool_init)");
  if (n < 0) return set_error(KVZ_EINVAL, "n < 0");
  if (n > 0 && !d_items) return set_error(KVZ_EINVAL, "items pointer is null");
  if (flags & ~(KVZ_ENC_FORCE_RAW | KVZ_ENC_SIMULATE_GIVE_UP))
    return set_error(KVZ_EINVAL, "unknown encode flag");
  return KVZ_OK;
}

}  // namespace
}  // namespace kvz

extern "C" int kvz_encode_pages(kvz_pool* p, const kvz_encode_item* d_items, int32_t n,
                                uint32_t flags, hipStream_t s) {
  const int rc = check_encode_args(p, d_items, n, flags);
  if (rc != KVZ_OK) return rc;
  if (n == 0) return KVZ_OK;
  if (n > kOnePassMaxItems) return encode_bulk(p, d_items, n, flags, s);
  return encode_onepass(p, d_items, n, nullptr, 0, flags, s);
}

extern "C" int kvz_complete_pages(kvz_pool* p, kvz_group_meta* const* d_free, int32_t n_free,
                                  const kvz_encode_item* d_items, int32_t n, uint32_t flags,
                                  hipStream_t s) {
  const int rc = check_encode_args(p, d_items, n, flags);
  if (rc != KVZ_OK) return rc;
  if (n_free < 0) return set_error(KVZ_EINVAL, "n_free < 0");
  if (n_free > 0 && !d_free) return set_error(KVZ_EINVAL, "free list pointer is null");
  if (n == 0) return n_free ? kvz_slot_free(p, d_free, n_free, s) : KVZ_OK;
  if (n > kOnePassMaxItems) {
    if (n_free) {
      const int rc2 = kvz_slot_free(p, d_free, n_free, s);
      if (rc2 != KVZ_OK) return rc2;
    }
    return encode_bulk(p, d_items, n, flags, s);
  }
  return encode_onepass(p, d_items, n, d_free, n_free, flags, s);
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
