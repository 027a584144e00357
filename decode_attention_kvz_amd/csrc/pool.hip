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
// Both kernels run as ONE workgroup of 1024 threads that walks the items in chunks of 1024,
// so the result depends only on item order: the i-th item of bin k pops the bin from the top,
// frontier requests get prefix-summed offsets.
#include "kvz_internal.h"

#include <algorithm>

namespace kvz {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ uint64_t lanemask_lt() {
  const uint32_t lane = threadIdx.x & 63u;
  return lane == 0 ? 0ull : (~0ull >> (64u - lane));
}

// Exclusive prefix sum over the 1024 threads of the block; returns the block total in *total.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_tmp, uint32_t* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) s_tmp[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    uint32_t w = lane < kWaves ? s_tmp[lane] : 0u;
    uint32_t wi = w;
#pragma unroll
    for (int d = 1; d < kWaves; d <<= 1) {
      const uint32_t o = __shfl_up(wi, d, 64);
      if (lane >= d) wi += o;
    }
    if (lane < kWaves) s_tmp[kWaves + lane] = wi - w;   // exclusive wave offsets
    if (lane == kWaves - 1) s_tmp[2 * kWaves] = wi;
  }
  __syncthreads();
  const uint32_t r = s_tmp[kWaves + wave] + incl - v;
  *total = s_tmp[2 * kWaves];
  __syncthreads();
  return r;
}

// Rank of this thread among the threads of the block whose key equals its key (key in
// 0..kBins-1, or -1 for none), in thread order; counts[k] receives the block count of key k.
__device__ uint32_t block_rank_by_key(int key, uint32_t (*s_cnt)[kBins], uint32_t* counts) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t rank = 0;
#pragma unroll
  for (int k = 0; k < kBins; ++k) {
    const uint64_t m = __ballot(key == k);
    if (key == k) rank = __popcll(m & lanemask_lt());
    if (lane == 0) s_cnt[wave][k] = __popcll(m);
  }
  __syncthreads();
  uint32_t before = 0;
  for (int w = 0; w < kWaves; ++w) {
#pragma unroll
    for (int k = 0; k < kBins; ++k) {
      const uint32_t c = s_cnt[w][k];
      if (w < wave && key == k) before += c;
    }
  }
#pragma unroll
  for (int k = 0; k < kBins; ++k) {
    uint32_t c = 0;
    for (int w = 0; w < kWaves; ++w) c += s_cnt[w][k];
    counts[k] = c;
  }
  __syncthreads();
  return before + rank;
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

template <class Access>
__global__ __launch_bounds__(kThreads) void pool_alloc_kernel(PoolHdr* hdr, uint32_t* bins,
                                                              Access acc, int n) {
  __shared__ uint32_t s_cnt[kWaves][kBins];
  __shared__ uint32_t s_tmp[2 * kWaves + 1];
  __shared__ uint32_t s_stat[4];   // successes, granules, raw blocks, failures of the chunk
  if (hdr->magic != kPoolMagic) return;   // host checked; never write through a bad state

  const uint64_t cap = hdr->capacity;
  const uint64_t f0 = hdr->frontier;
  uint64_t cnt[kBins], base[kBins];
#pragma unroll
  for (int k = 0; k < kBins; ++k) {
    cnt[k] = hdr->bin_cnt[k];
    base[k] = hdr->bin_base[k];
  }
  uint64_t pending = 0;   // sizes of this call's frontier requests so far (granted or not)
  uint64_t granted = 0;
  uint64_t st_runs = 0, st_gran = 0, st_raw = 0, st_fail = 0;

  for (int chunk = 0; chunk < n; chunk += kThreads) {
    const int i = chunk + (int)threadIdx.x;
    const bool valid = i < n;
    uint32_t tags = valid ? acc.get_tags(i) : 0u;
    const int k = valid ? (int)n_raw_of(tags) : -1;
    uint32_t counts[kBins];
    const uint32_t rank = block_rank_by_key(k, s_cnt, counts);

    bool from_bin = false;
    uint64_t off = KVZ_OFF_NONE;
    if (valid && rank < cnt[k]) {
      from_bin = true;
      off = bins[base[k] + cnt[k] - 1 - rank];
    }
    const uint32_t z = (valid && !from_bin) ? run_granules((uint32_t)k) : 0u;
    uint32_t ztot;
    const uint32_t zpre = block_exclusive_scan(z, s_tmp, &ztot);
    if (valid && !from_bin) {
      const uint64_t start = f0 + pending + zpre;
      off = (start + z <= cap) ? start : (uint64_t)KVZ_OFF_NONE;
    }
    if (threadIdx.x < 4) s_stat[threadIdx.x] = 0;
    __syncthreads();
    if (valid) {
      acc.set_off(i, (uint32_t)off);
      if (off != KVZ_OFF_NONE) {
        atomicAdd(&s_stat[0], 1u);
        atomicAdd(&s_stat[1], run_granules((uint32_t)k));
        atomicAdd(&s_stat[2], (uint32_t)k);
      } else {
        atomicAdd(&s_stat[3], 1u);
      }
    }
    __syncthreads();
    // frontier granules granted in this chunk = granules of successful frontier requests
    uint32_t gz = (valid && !from_bin && off != KVZ_OFF_NONE) ? z : 0u;
    uint32_t gtot;
    (void)block_exclusive_scan(gz, s_tmp, &gtot);
    granted += gtot;
    pending += ztot;
#pragma unroll
    for (int kk = 0; kk < kBins; ++kk) cnt[kk] -= (counts[kk] < cnt[kk] ? counts[kk] : cnt[kk]);
    st_runs += s_stat[0];
    st_gran += s_stat[1];
    st_raw += s_stat[2];
    st_fail += s_stat[3];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    hdr->frontier = f0 + granted;
#pragma unroll
    for (int k = 0; k < kBins; ++k) hdr->bin_cnt[k] = cnt[k];
    hdr->live_runs += st_runs;
    hdr->live_granules += st_gran;
    hdr->live_raw_blocks += st_raw;
    hdr->enospc += st_fail;
  }
}

__global__ __launch_bounds__(kThreads) void pool_free_kernel(PoolHdr* hdr, uint32_t* bins,
                                                             kvz_group_meta* const* metas, int n) {
  __shared__ uint32_t s_cnt[kWaves][kBins];
  __shared__ uint32_t s_stat[4];   // freed runs, granules, raw blocks, dropped
  if (hdr->magic != kPoolMagic) return;
  uint64_t cnt[kBins], base[kBins], bcap[kBins];
#pragma unroll
  for (int k = 0; k < kBins; ++k) {
    cnt[k] = hdr->bin_cnt[k];
    base[k] = hdr->bin_base[k];
    bcap[k] = hdr->bin_cap[k];
  }
  uint64_t st_runs = 0, st_gran = 0, st_raw = 0, st_bad = 0;
  for (int chunk = 0; chunk < n; chunk += kThreads) {
    const int i = chunk + (int)threadIdx.x;
    kvz_group_meta* m = i < n ? metas[i] : nullptr;
    uint32_t off = KVZ_OFF_NONE, tags = 0;
    if (m) {
      off = m->off;
      tags = *reinterpret_cast<const uint32_t*>(m->tag);
    }
    const bool valid = m && off != KVZ_OFF_NONE;
    const int k = valid ? (int)n_raw_of(tags) : -1;
    uint32_t counts[kBins];
    const uint32_t rank = block_rank_by_key(k, s_cnt, counts);
    if (threadIdx.x < 4) s_stat[threadIdx.x] = 0;
    __syncthreads();
    if (valid) {
      const uint64_t slot = cnt[k] + rank;
      if (slot < bcap[k]) {
        bins[base[k] + slot] = off;
        atomicAdd(&s_stat[0], 1u);
        atomicAdd(&s_stat[1], run_granules((uint32_t)k));
        atomicAdd(&s_stat[2], (uint32_t)k);
      } else {
        atomicAdd(&s_stat[3], 1u);
      }
    }
    if (m) {
      m->off = KVZ_OFF_NONE;
      *reinterpret_cast<uint32_t*>(m->tag) = 0u;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kBins; ++kk) {
      const uint64_t c = cnt[kk] + counts[kk];
      cnt[kk] = c < bcap[kk] ? c : bcap[kk];
    }
    st_runs += s_stat[0];
    st_gran += s_stat[1];
    st_raw += s_stat[2];
    st_bad += s_stat[3];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
#pragma unroll
    for (int k = 0; k < kBins; ++k) hdr->bin_cnt[k] = cnt[k];
    hdr->live_runs -= st_runs;
    hdr->live_granules -= st_gran;
    hdr->live_raw_blocks -= st_raw;
    hdr->bad_frees += st_bad;
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
