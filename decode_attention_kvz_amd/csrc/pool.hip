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
// Both kernels run as ONE workgroup of 512 threads that walks the items in passes of 4096 (8
// consecutive items per thread), so the result depends only on item order: the i-th item of
// bin k pops the bin from the top, frontier requests get prefix-summed offsets.
#include "kvz_internal.h"

#include <algorithm>

namespace kvz {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;

constexpr int kIpt = 8;   // items per thread per pass: the loads of 4096 items are in flight together

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

struct EncodeItemAccess {
  const kvz_encode_item* items;
  __device__ uint32_t get_tags(int i) const {
    const kvz_group_meta* m = items[i].dst;
    return *reinterpret_cast<const uint32_t*>(m->tag);
  }
  __device__ void set_off(int i, uint32_t o) const { items[i].dst->off = o; }
};

// Allocation in item order.  A pass covers 4096 items; thread t owns items 8t..8t+7 of it, so
// "earlier in item order" = earlier thread, or the same thread and a smaller index.
template <class Access>
__global__ __launch_bounds__(kThreads) void pool_alloc_kernel(PoolHdr* hdr, uint32_t* bins,
                                                              Access acc, int n) {
  __shared__ ScanShared sh;
  __shared__ uint64_t s_red[kWaves];
  __shared__ uint64_t s_cnt[kBins], s_base[kBins];   // bin state, uniform over the block
  __shared__ uint32_t s_ktot[kBins];
  if (hdr->magic != kPoolMagic) return;   // host checked; never write through a bad state

  const uint64_t cap = hdr->capacity;
  const uint64_t f0 = hdr->frontier;
  if (threadIdx.x < kBins) {
    s_cnt[threadIdx.x] = hdr->bin_cnt[threadIdx.x];
    s_base[threadIdx.x] = hdr->bin_base[threadIdx.x];
  }
  __syncthreads();
  uint64_t pending = 0;   // sizes of this call's frontier requests so far (granted or not)
  uint64_t my_granted = 0, my_runs = 0, my_gran = 0, my_raw = 0, my_fail = 0;

  for (int pass = 0; pass < n; pass += kThreads * kIpt) {
    const int first = pass + (int)threadIdx.x * kIpt;
    uint32_t tags[kIpt];
#pragma unroll
    for (int sub = 0; sub < kIpt; ++sub) tags[sub] = first + sub < n ? acc.get_tags(first + sub) : 0u;
    // ranks among same-size items: local prefix, then across threads
    int key[kIpt];
    uint32_t lrank[kIpt];
    uint32_t lcnt[kBins] = {0, 0, 0, 0, 0};
#pragma unroll
    for (int sub = 0; sub < kIpt; ++sub) {
      key[sub] = first + sub < n ? (int)n_raw_of(tags[sub]) : -1;
      lrank[sub] = 0;
#pragma unroll
      for (int k = 0; k < kBins; ++k) {
        if (key[sub] == k) {
          lrank[sub] = lcnt[k];
          lcnt[k] += 1;
        }
      }
    }
    uint32_t kbase[kBins], ktot[kBins];
    block_scan_cols<kBins>(lcnt, kbase, ktot, sh.wave, sh.pre, sh.tot);
    if (threadIdx.x == 0) {
#pragma unroll
      for (int k = 0; k < kBins; ++k) s_ktot[k] = ktot[k];
    }
    // pop the bin while it lasts, else ask the frontier
    uint64_t off[kIpt];
    bool from_bin[kIpt];
    uint32_t zoff[kIpt];
    uint32_t lz[1] = {0};
#pragma unroll
    for (int sub = 0; sub < kIpt; ++sub) {
      const int k = key[sub];
      from_bin[sub] = false;
      off[sub] = KVZ_OFF_NONE;
      zoff[sub] = lz[0];
      if (k >= 0) {
        uint32_t kb = kbase[0];
#pragma unroll
        for (int j = 1; j < kBins; ++j) kb = (k == j) ? kbase[j] : kb;
        const uint64_t rank = (uint64_t)kb + lrank[sub];
        const uint64_t ck = s_cnt[k];
        if (rank < ck) {
          from_bin[sub] = true;
          off[sub] = s_base[k] + ck - 1 - rank;   // bin slot, read below
        } else {
          lz[0] += run_granules((uint32_t)k);
        }
      }
    }
    uint32_t zbase[1], ztot[1];
    block_scan_cols<1>(lz, zbase, ztot, sh.wave, sh.pre, sh.tot);
#pragma unroll
    for (int sub = 0; sub < kIpt; ++sub) {
      const int k = key[sub];
      if (k < 0) continue;
      if (!from_bin[sub]) {
        const uint32_t z = run_granules((uint32_t)k);
        const uint64_t start = f0 + pending + zbase[0] + zoff[sub];
        if (start + z <= cap) {
          off[sub] = start;
          my_granted += z;
        }
      }
      if (from_bin[sub] || off[sub] != KVZ_OFF_NONE) {
        my_runs += 1;
        my_gran += run_granules((uint32_t)k);
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
      if (key[sub] >= 0) acc.set_off(first + sub, (uint32_t)off[sub]);
    pending += ztot[0];
    __syncthreads();
    if (threadIdx.x < kBins) {
      const uint64_t c = s_cnt[threadIdx.x], t = s_ktot[threadIdx.x];
      s_cnt[threadIdx.x] = c - (t < c ? t : c);
    }
    __syncthreads();
  }
  const uint64_t granted = block_sum(my_granted, s_red);
  const uint64_t runs = block_sum(my_runs, s_red);
  const uint64_t gran = block_sum(my_gran, s_red);
  const uint64_t raw = block_sum(my_raw, s_red);
  const uint64_t fail = block_sum(my_fail, s_red);
  if (threadIdx.x < kBins) hdr->bin_cnt[threadIdx.x] = s_cnt[threadIdx.x];
  if (threadIdx.x == 0) {
    hdr->frontier = f0 + granted;
    hdr->live_runs += runs;
    hdr->live_granules += gran;
    hdr->live_raw_blocks += raw;
    hdr->enospc += fail;
  }
}

// Free in item order: item i pushes its run onto bin[n_raw] at position count + rank.
__global__ __launch_bounds__(kThreads) void pool_free_kernel(PoolHdr* hdr, uint32_t* bins,
                                                             kvz_group_meta* const* metas, int n) {
  __shared__ ScanShared sh;
  __shared__ uint64_t s_red[kWaves];
  __shared__ uint64_t s_cnt[kBins], s_base[kBins], s_bcap[kBins];
  __shared__ uint32_t s_ktot[kBins];
  if (hdr->magic != kPoolMagic) return;
  if (threadIdx.x < kBins) {
    s_cnt[threadIdx.x] = hdr->bin_cnt[threadIdx.x];
    s_base[threadIdx.x] = hdr->bin_base[threadIdx.x];
    s_bcap[threadIdx.x] = hdr->bin_cap[threadIdx.x];
  }
  __syncthreads();
  uint64_t my_runs = 0, my_gran = 0, my_raw = 0, my_bad = 0;
  for (int pass = 0; pass < n; pass += kThreads * kIpt) {
    const int first = pass + (int)threadIdx.x * kIpt;
    kvz_group_meta* m[kIpt];
#pragma unroll
    for (int sub = 0; sub < kIpt; ++sub) m[sub] = first + sub < n ? metas[first + sub] : nullptr;
    uint2 rec[kIpt];
#pragma unroll
    for (int sub = 0; sub < kIpt; ++sub)
      rec[sub] = m[sub] ? *reinterpret_cast<const uint2*>(m[sub]) : make_uint2(KVZ_OFF_NONE, 0u);
    int key[kIpt];
    uint32_t lrank[kIpt];
    uint32_t lcnt[kBins] = {0, 0, 0, 0, 0};
#pragma unroll
    for (int sub = 0; sub < kIpt; ++sub) {
      key[sub] = (m[sub] && rec[sub].x != KVZ_OFF_NONE) ? (int)n_raw_of(rec[sub].y) : -1;
      lrank[sub] = 0;
#pragma unroll
      for (int k = 0; k < kBins; ++k) {
        if (key[sub] == k) {
          lrank[sub] = lcnt[k];
          lcnt[k] += 1;
        }
      }
    }
    uint32_t kbase[kBins], ktot[kBins];
    block_scan_cols<kBins>(lcnt, kbase, ktot, sh.wave, sh.pre, sh.tot);
    if (threadIdx.x == 0) {
#pragma unroll
      for (int k = 0; k < kBins; ++k) s_ktot[k] = ktot[k];
    }
#pragma unroll
    for (int sub = 0; sub < kIpt; ++sub) {
      const int k = key[sub];
      if (k >= 0) {
        uint32_t kb = kbase[0];
#pragma unroll
        for (int j = 1; j < kBins; ++j) kb = (k == j) ? kbase[j] : kb;
        const uint64_t slot = s_cnt[k] + kb + lrank[sub];
        if (slot < s_bcap[k]) {
          bins[s_base[k] + slot] = rec[sub].x;
          my_runs += 1;
          my_gran += run_granules((uint32_t)k);
          my_raw += (uint32_t)k;
        } else {
          my_bad += 1;
        }
      }
      if (m[sub]) *reinterpret_cast<uint2*>(m[sub]) = make_uint2(KVZ_OFF_NONE, 0u);
    }
    __syncthreads();
    if (threadIdx.x < kBins) {
      const uint64_t c = s_cnt[threadIdx.x] + s_ktot[threadIdx.x];
      s_cnt[threadIdx.x] = c < s_bcap[threadIdx.x] ? c : s_bcap[threadIdx.x];
    }
    __syncthreads();
  }
  const uint64_t runs = block_sum(my_runs, s_red);
  const uint64_t gran = block_sum(my_gran, s_red);
  const uint64_t raw = block_sum(my_raw, s_red);
  const uint64_t bad = block_sum(my_bad, s_red);
  if (threadIdx.x < kBins) hdr->bin_cnt[threadIdx.x] = s_cnt[threadIdx.x];
  if (threadIdx.x == 0) {
    hdr->live_runs -= runs;
    hdr->live_granules -= gran;
    hdr->live_raw_blocks -= raw;
    hdr->bad_frees += bad;
  }
}

__global__ void pool_init_kernel(PoolHdr* hdr, uint64_t capacity, PoolHdr tmpl) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    *hdr = tmpl;
    hdr->capacity = capacity;
  }
}

void bin_layout(uint64_t capacity, uint64_t* cap, uint64_t* base, uint64_t* entries) {
  uint64_t at = 0;
  for (int k = 0; k < kBins; ++k) {
    cap[k] = capacity / (12 + k) + 1;
    base[k] = at;
    at += cap[k];
  }
  *entries = at;
}

int check_pool(const kvz_pool* p) {
  if (!p) return set_error(KVZ_EINVAL, "pool handle is null");
  return KVZ_OK;
}

}  // namespace

}  // namespace kvz

using namespace kvz;

extern "C" int kvz_pool_state_bytes(uint64_t arena_bytes, uint64_t* state_bytes) {
  if (!state_bytes) return set_error(KVZ_EINVAL, "state_bytes is null");
  if (arena_bytes < 2 * KVZ_GRANULE_BYTES) return set_error(KVZ_EINVAL, "arena smaller than 2 granules");
  const uint64_t capacity = arena_bytes / KVZ_GRANULE_BYTES - 1;
  if (capacity >= KVZ_OFF_NONE) return set_error(KVZ_EINVAL, "arena too large for 32-bit granule offsets");
  uint64_t cap[kBins], base[kBins], entries;
  bin_layout(capacity, cap, base, &entries);
  *state_bytes = kPoolHdrBytes + 4 * entries;
  return KVZ_OK;
}

extern "C" int kvz_pool_init(kvz_pool** out, void* d_arena, uint64_t arena_bytes, void* d_state,
                             uint64_t state_bytes, hipStream_t s) {
  if (!out || !d_arena || !d_state) return set_error(KVZ_EINVAL, "null pointer argument");
  if (((uintptr_t)d_arena | (uintptr_t)d_state) & 255u)
    return set_error(KVZ_EINVAL, "arena and state must be 256-byte aligned");
  uint64_t need = 0;
  int rc = kvz_pool_state_bytes(arena_bytes, &need);
  if (rc != KVZ_OK) return rc;
  if (state_bytes < need) return set_error(KVZ_EINVAL, "state buffer too small");
  int dev = 0;
  rc = check_hip(hipGetDevice(&dev), "hipGetDevice");
  if (rc != KVZ_OK) return rc;
  const uint64_t capacity = arena_bytes / KVZ_GRANULE_BYTES - 1;
  PoolHdr t = {};
  t.magic = kPoolMagic;
  t.version = kPoolVersion;
  t.capacity = capacity;
  uint64_t entries;
  bin_layout(capacity, t.bin_cap, t.bin_base, &entries);
  hipLaunchKernelGGL(pool_init_kernel, dim3(1), dim3(64), 0, s, (PoolHdr*)d_state, capacity, t);
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
  *out = p;
  return KVZ_OK;
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
  PoolHdr* hdr = (PoolHdr*)p->state;
  uint32_t* bins = (uint32_t*)((uint8_t*)p->state + kPoolHdrBytes);
  hipLaunchKernelGGL(pool_alloc_kernel<TagArrayAccess>, dim3(1), dim3(kThreads), 0, s, hdr, bins,
                     TagArrayAccess{d_tags, d_off}, (int)n);
  return check_hip(hipGetLastError(), "slot alloc launch");
}

extern "C" int kvz_slot_free(kvz_pool* p, kvz_group_meta* const* d_metas, int32_t n, hipStream_t s) {
  int rc = check_pool(p);
  if (rc != KVZ_OK) return rc;
  if (n < 0) return set_error(KVZ_EINVAL, "n < 0");
  if (n == 0) return KVZ_OK;
  if (!d_metas) return set_error(KVZ_EINVAL, "null pointer argument");
  PoolHdr* hdr = (PoolHdr*)p->state;
  uint32_t* bins = (uint32_t*)((uint8_t*)p->state + kPoolHdrBytes);
  hipLaunchKernelGGL(pool_free_kernel, dim3(1), dim3(kThreads), 0, s, hdr, bins, d_metas, (int)n);
  return check_hip(hipGetLastError(), "slot free launch");
}

namespace kvz {
// Used by the encoder: the allocation step of kvz_encode_pages.
int launch_alloc_for_items(kvz_pool* p, const kvz_encode_item* d_items, int n, hipStream_t s) {
  PoolHdr* hdr = (PoolHdr*)p->state;
  uint32_t* bins = (uint32_t*)((uint8_t*)p->state + kPoolHdrBytes);
  hipLaunchKernelGGL(pool_alloc_kernel<EncodeItemAccess>, dim3(1), dim3(kThreads), 0, s, hdr, bins,
                     EncodeItemAccess{d_items}, n);
  return check_hip(hipGetLastError(), "encode alloc launch");
}
}  // namespace kvz

extern "C" int kvz_pool_stats(kvz_pool* p, kvz_pool_stats_t* host_out, hipStream_t s) {
  int rc = check_pool(p);
  if (rc != KVZ_OK) return rc;
  if (!host_out) return set_error(KVZ_EINVAL, "host_out is null");
  PoolHdr h;
  rc = check_hip(hipMemcpyAsync(&h, p->state, sizeof(h), hipMemcpyDeviceToHost, s), "stats copy");
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
  return KVZ_OK;
}
