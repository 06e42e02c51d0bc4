// Refinement slot cache: device slots + unit->slot table per pool, host-side
// replacement policy, fills from a host refinement store by one hipMemcpyAsync per
// pool on a side stream.
//
// Method: rag-lover.com StrataFlux summary, explainer dialogue (解説) -- fetched
// precision is cached on the GPU and reused across decode steps, and delivery is
// overlapped with computation; limitations section -- a miss keeps resident
// precision.  Paper abstract (arXiv 2611.08363): generation need not wait for
// every transfer.
//
// Consistency: the unit->slot table is only changed by small kernels on the
// compute stream (stream-ordered with every lookup), never while a reader can
// use the entry.  A fill first unmaps its victims on the compute stream, then the
// side stream (after that point of the compute stream) copies the new units into
// the freed slots, and only after that copy has completed is a map kernel enqueued
// on the compute stream.  Deterministic mode enqueues the map right away behind a
// stream wait; async mode enqueues it at the next fill call.
#include <algorithm>
#include <cstring>
#include <map>
#include <mutex>

#include "sf_internal.h"

namespace {

struct FillHeader {  // device staging header of one fill
  int32_t n_unmap, n_map, pad0, pad1;
};

struct HostPool {
  sf_pool_desc d{};
  bool resident = false;
  // device
  int32_t* d_unit2slot = nullptr;
  uint8_t* d_slots = nullptr;  // owned unless resident
  int32_t* d_log_units = nullptr;
  int32_t* d_log_slots = nullptr;
  uint32_t* d_log_count = nullptr;
  int32_t log_cap = 0;
  uint8_t* d_stage = nullptr;  // [header | unmap ids | map (unit, slot) | unit bytes]
  // host
  uint8_t* h_stage = nullptr;  // pinned, same layout
  size_t stage_bytes = 0;
  int64_t stage_units = 0;
  std::vector<int64_t> slot_unit;  // -1 free
  std::vector<int64_t> slot_last;
  std::vector<int32_t> unit_slot;  // host view (includes units whose copy is in flight)
  std::vector<int32_t> free_slots; // kept sorted descending: back() is the lowest
  std::map<int64_t, std::vector<int64_t>> buckets;  // last-use step -> units (lazy)
  std::map<int64_t, size_t> bucket_pos;             // consumed prefix of a sorted bucket
  std::vector<int64_t> pending;
  std::vector<uint8_t> pending_flag;  // per unit
  std::vector<int32_t> log_u, log_s;
  hipEvent_t copy_done = nullptr;
  bool in_flight = false;  // a copy whose map has not been enqueued
  int32_t flight_maps = 0;
  // stats
  int64_t n_lookups = 0, n_hits = 0, n_installed = 0, h2d_bytes = 0;
};

}  // namespace

struct sf_refine_cache {
  std::vector<HostPool> pools;
  int mode = SF_CACHE_DETERMINISTIC;
  int64_t max_fill = 0;
  int64_t step = 0;
  int device = 0;
  hipEvent_t ev_compute = nullptr;
  uint32_t* h_counts = nullptr;  // pinned [n_pools]
};

namespace {

__global__ void iota_kernel(int32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = (int32_t)i;
}

__global__ void fill_kernel(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void zero_u32_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

__global__ void unmap_kernel(int32_t* unit2slot, const uint8_t* stage) {
  const FillHeader* h = (const FillHeader*)stage;
  const int32_t* ids = (const int32_t*)(stage + 16);
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < h->n_unmap; i += gridDim.x * blockDim.x)
    unit2slot[ids[i]] = -1;
}

__global__ void map_kernel(int32_t* unit2slot, const uint8_t* stage, int64_t map_off) {
  const FillHeader* h = (const FillHeader*)stage;
  const int32_t* pairs = (const int32_t*)(stage + map_off);
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < h->n_map; i += gridDim.x * blockDim.x)
    unit2slot[pairs[2 * i]] = pairs[2 * i + 1];
}

// Copies unit bytes from the device staging into their slots (4-byte words).
__global__ void scatter_kernel(uint8_t* slots, const uint8_t* stage, int64_t map_off,
                               int64_t data_off, int64_t unit_bytes) {
  const FillHeader* h = (const FillHeader*)stage;
  const int32_t* pairs = (const int32_t*)(stage + map_off);
  const int64_t wpu = unit_bytes / 4;
  const int64_t total = (int64_t)h->n_map * wpu;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / wpu, w = i - m * wpu;
    const int32_t slot = pairs[2 * m + 1];
    ((uint32_t*)(slots + (int64_t)slot * unit_bytes))[w] =
        ((const uint32_t*)(stage + data_off + m * unit_bytes))[w];
  }
}

// Lookup by one workgroup so that log entries keep the order of unit_ids.
__global__ __launch_bounds__(1024) void lookup_kernel(PoolDev p, int64_t n_units,
                                                      const int32_t* ids, int32_t n,
                                                      int32_t* slot_out) {
  __shared__ int base;
  if (threadIdx.x == 0) {
    base = -1;
    if (p.log_count) {
      const uint32_t b = atomicAdd(p.log_count, (uint32_t)n);
      base = (b + (uint32_t)n <= (uint32_t)p.log_cap) ? (int)b : -1;
    }
  }
  __syncthreads();
  for (int j = threadIdx.x; j < n; j += blockDim.x) {
    const int32_t u = ids[j];
    const int32_t slot = (p.unit2slot && u >= 0 && u < n_units) ? p.unit2slot[u] : -1;
    if (slot_out) slot_out[j] = slot;
    if (base >= 0) {
      p.log_units[base + j] = u;
      p.log_slots[base + j] = slot;
    }
  }
}

size_t stage_layout(int64_t units, int64_t unit_bytes, int64_t* map_off, int64_t* data_off) {
  *map_off = sf_align256(16 + (size_t)units * 4);
  *data_off = sf_align256((size_t)*map_off + (size_t)units * 8);
  return sf_align256((size_t)*data_off + (size_t)units * unit_bytes);
}

void destroy_pool(HostPool& p) {
  if (p.d_unit2slot) hipFree(p.d_unit2slot);
  if (p.d_slots && !p.resident) hipFree(p.d_slots);
  if (p.d_log_units) hipFree(p.d_log_units);
  if (p.d_log_slots) hipFree(p.d_log_slots);
  if (p.d_log_count) hipFree(p.d_log_count);
  if (p.d_stage) hipFree(p.d_stage);
  if (p.h_stage) hipHostFree(p.h_stage);
  if (p.copy_done) hipEventDestroy(p.copy_done);
  p = HostPool();
}

// Smallest (last use, unit id) resident unit with last use < step, or -1.
int64_t pick_victim(HostPool& p, int64_t step) {
  while (!p.buckets.empty()) {
    auto it = p.buckets.begin();
    if (it->first >= step) return -1;
    std::vector<int64_t>& v = it->second;
    size_t& pos = p.bucket_pos[it->first];
    if (pos == 0) {
      std::sort(v.begin(), v.end());
      v.erase(std::unique(v.begin(), v.end()), v.end());
    }
    while (pos < v.size()) {
      const int64_t u = v[pos++];
      const int32_t s = p.unit_slot[u];
      if (s >= 0 && p.slot_last[s] == it->first) return u;
    }
    p.bucket_pos.erase(it->first);
    p.buckets.erase(it);
  }
  return -1;
}

sf_status publish(sf_refine_cache* c, HostPool& p, hipStream_t compute) {
  if (!p.in_flight) return SF_OK;
  int64_t map_off, data_off;
  stage_layout(p.stage_units, p.d.unit_bytes, &map_off, &data_off);
  SF_HIP(hipStreamWaitEvent(compute, p.copy_done, 0));
  if (p.flight_maps > 0) {
    hipLaunchKernelGGL(map_kernel, dim3((p.flight_maps + 255) / 256), dim3(256), 0, compute,
                       p.d_unit2slot, (const uint8_t*)p.d_stage, map_off);
    SF_LAUNCH_CHECK();
  }
  p.in_flight = false;
  p.flight_maps = 0;
  (void)c;
  return SF_OK;
}

}  // namespace

sf_status sf_cache_pool_view(sf_refine_cache* c, int32_t pool, PoolDev* out) {
  *out = PoolDev{};
  if (!c || pool < 0) return SF_OK;
  SF_REQUIRE(pool < (int32_t)c->pools.size(), SF_EINVAL, "pool index out of range");
  HostPool& p = c->pools[pool];
  out->unit2slot = p.d_unit2slot;
  out->slots = p.d_slots;
  if (!p.resident) {  // a resident pool never misses: nothing to record
    out->log_units = p.d_log_units;
    out->log_slots = p.d_log_slots;
    out->log_count = p.d_log_count;
  }
  out->log_cap = p.log_cap;
  out->resident = p.resident ? 1 : 0;
  out->unit_bytes = (int32_t)p.d.unit_bytes;
  out->n_units = p.d.n_units;
  return SF_OK;
}

extern "C" sf_status sf_refine_cache_create(const sf_pool_desc* pools, int32_t n_pools, int32_t mode,
                                            int32_t max_fill, sf_refine_cache** out) {
  SF_REQUIRE(out && pools && n_pools >= 1, SF_EINVAL, "bad arguments");
  SF_REQUIRE(mode == SF_CACHE_DETERMINISTIC || mode == SF_CACHE_ASYNC, SF_EINVAL, "bad mode");
  SF_REQUIRE(max_fill >= 0, SF_EINVAL, "max_fill must be >= 0");
  *out = nullptr;
  for (int i = 0; i < n_pools; ++i) {
    const sf_pool_desc& d = pools[i];
    SF_REQUIRE(d.unit_bytes > 0 && d.unit_bytes % 4 == 0 && d.unit_bytes < (1 << 24), SF_EINVAL,
               "unit_bytes must be a positive multiple of 4");
    SF_REQUIRE(d.n_units > 0 && d.n_units < (1ll << 31), SF_EINVAL, "bad n_units");
    SF_REQUIRE(d.capacity >= 0 && d.capacity <= d.n_units, SF_EINVAL, "capacity out of range");
    SF_REQUIRE(d.max_lookup >= 0, SF_EINVAL, "bad max_lookup");
    if (d.device_store)
      SF_REQUIRE(d.capacity == d.n_units, SF_EINVAL, "a resident pool needs capacity == n_units");
    else
      SF_REQUIRE(d.host_store || d.capacity == 0, SF_EINVAL, "a pool with slots needs a host store");
  }
  sf_refine_cache* c = new sf_refine_cache();
  c->mode = mode;
  c->max_fill = max_fill;
  hipGetDevice(&c->device);
  c->pools.resize(n_pools);
  auto fail = [&](sf_status st) {
    for (auto& p : c->pools) destroy_pool(p);
    if (c->ev_compute) hipEventDestroy(c->ev_compute);
    if (c->h_counts) hipHostFree(c->h_counts);
    delete c;
    return st;
  };
#define CK(call)                                                                  \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess) {                                                       \
      sf_set_error(std::string("sf_refine_cache_create: " #call ": ") + hipGetErrorString(e_)); \
      return fail(e_ == hipErrorOutOfMemory ? SF_ENOMEM : SF_EHIP);               \
    }                                                                             \
  } while (0)
  CK(hipEventCreateWithFlags(&c->ev_compute, hipEventDisableTiming));
  CK(hipHostMalloc((void**)&c->h_counts, sizeof(uint32_t) * n_pools, hipHostMallocDefault));
  for (int i = 0; i < n_pools; ++i) {
    HostPool& p = c->pools[i];
    p.d = pools[i];
    p.resident = pools[i].device_store != nullptr;
    const int64_t nu = p.d.n_units, cap = p.d.capacity;
    p.log_cap = p.d.max_lookup > 0 ? p.d.max_lookup : 65536;
    CK(hipMalloc((void**)&p.d_unit2slot, sizeof(int32_t) * nu));
    CK(hipMalloc((void**)&p.d_log_units, sizeof(int32_t) * p.log_cap));
    CK(hipMalloc((void**)&p.d_log_slots, sizeof(int32_t) * p.log_cap));
    CK(hipMalloc((void**)&p.d_log_count, 256));
    hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, 0, p.d_log_count, 64);
    p.unit_slot.assign(nu, -1);
    p.pending_flag.assign(nu, 0);
    if (p.resident) {
      p.d_slots = p.d.device_store;
      hipLaunchKernelGGL(iota_kernel, dim3((unsigned)((nu + 255) / 256)), dim3(256), 0, 0, p.d_unit2slot, nu);
      for (int64_t u = 0; u < nu; ++u) p.unit_slot[u] = (int32_t)u;
      p.slot_unit.resize(nu);
      for (int64_t u = 0; u < nu; ++u) p.slot_unit[u] = u;
      p.slot_last.assign(nu, -1);
      std::vector<int64_t>& b = p.buckets[-1];
      b.resize(nu);
      for (int64_t u = 0; u < nu; ++u) b[u] = u;
    } else {
      hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((nu + 255) / 256)), dim3(256), 0, 0, p.d_unit2slot, nu, -1);
      if (cap > 0) CK(hipMalloc((void**)&p.d_slots, (size_t)cap * p.d.unit_bytes));
      p.slot_unit.assign(cap, -1);
      p.slot_last.assign(cap, -1);
      p.free_slots.resize(cap);
      for (int64_t s = 0; s < cap; ++s) p.free_slots[s] = (int32_t)(cap - 1 - s);
      p.stage_units = std::min<int64_t>(cap, max_fill > 0 ? max_fill : cap);
      if (p.stage_units > 0) {
        int64_t mo, dof;
        p.stage_bytes = stage_layout(p.stage_units, p.d.unit_bytes, &mo, &dof);
        CK(hipMalloc((void**)&p.d_stage, p.stage_bytes));
        CK(hipHostMalloc((void**)&p.h_stage, p.stage_bytes, hipHostMallocDefault));
      }
      CK(hipEventCreateWithFlags(&p.copy_done, hipEventDisableTiming));
    }
  }
  CK(hipGetLastError());
  CK(hipDeviceSynchronize());
#undef CK
  *out = c;
  return SF_OK;
}

extern "C" sf_status sf_refine_cache_destroy(sf_refine_cache* c) {
  if (!c) return SF_OK;
  hipDeviceSynchronize();
  for (auto& p : c->pools) destroy_pool(p);
  if (c->ev_compute) hipEventDestroy(c->ev_compute);
  if (c->h_counts) hipHostFree(c->h_counts);
  delete c;
  return SF_OK;
}

extern "C" sf_status sf_refine_cache_lookup(sf_refine_cache* c, int32_t pool, const int32_t* unit_ids,
                                            int32_t n, int32_t* slot_out, sf_stream compute) {
  SF_REQUIRE(c, SF_EINVAL, "null cache");
  SF_REQUIRE(pool >= 0 && pool < (int32_t)c->pools.size(), SF_EINVAL, "pool index out of range");
  SF_REQUIRE(n >= 0 && (n == 0 || unit_ids), SF_EINVAL, "bad ids");
  if (n == 0) return SF_OK;
  PoolDev v;
  sf_status st = sf_cache_pool_view(c, pool, &v);
  if (st != SF_OK) return st;
  hipLaunchKernelGGL(lookup_kernel, dim3(1), dim3(1024), 0, (hipStream_t)compute, v,
                     c->pools[pool].d.n_units, unit_ids, n, slot_out);
  SF_LAUNCH_CHECK();
  return SF_OK;
}

extern "C" sf_status sf_refine_cache_fill(sf_refine_cache* c, sf_stream compute_, sf_stream side_,
                                          int64_t* n_filled) {
  SF_REQUIRE(c, SF_EINVAL, "null cache");
  hipStream_t compute = (hipStream_t)compute_, side = (hipStream_t)side_;
  const int64_t t = c->step;
  bool any = false;
  for (const auto& p : c->pools) any = any || !p.resident;
  if (!any) {  // only resident pools: nothing is ever missing
    c->step = t + 1;
    if (n_filled) *n_filled = 0;
    return SF_OK;
  }
  const int np = (int)c->pools.size();
  int64_t filled = 0;
  bool overflow = false;
  // 1. read the step's lookup logs
  for (int i = 0; i < np; ++i)
    SF_HIP(hipMemcpyAsync(c->h_counts + i, c->pools[i].d_log_count, 4, hipMemcpyDeviceToHost, compute));
  SF_HIP(hipStreamSynchronize(compute));
  for (int i = 0; i < np; ++i) {
    HostPool& p = c->pools[i];
    uint32_t cnt = c->h_counts[i];
    if (cnt > (uint32_t)p.log_cap) {
      overflow = true;
      cnt = (uint32_t)p.log_cap;
    }
    p.log_u.resize(cnt);
    p.log_s.resize(cnt);
    if (cnt) {
      SF_HIP(hipMemcpyAsync(p.log_u.data(), p.d_log_units, 4 * (size_t)cnt, hipMemcpyDeviceToHost, compute));
      SF_HIP(hipMemcpyAsync(p.log_s.data(), p.d_log_slots, 4 * (size_t)cnt, hipMemcpyDeviceToHost, compute));
    }
    hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, compute, p.d_log_count, 1);
    SF_LAUNCH_CHECK();
  }
  SF_HIP(hipStreamSynchronize(compute));
  // 2. async mode: publish the previous fill (its copy must be complete by now)
  for (int i = 0; i < np; ++i) {
    HostPool& p = c->pools[i];
    if (p.in_flight) {
      SF_HIP(hipEventSynchronize(p.copy_done));
      sf_status st = publish(c, p, compute);
      if (st != SF_OK) return st;
    }
  }
  // 3. policy, gather, copy, install
  for (int i = 0; i < np; ++i) {
    HostPool& p = c->pools[i];
    for (size_t e = 0; e < p.log_u.size(); ++e) {
      const int64_t u = p.log_u[e];
      const int32_t s = p.log_s[e];
      ++p.n_lookups;
      if (u < 0 || u >= p.d.n_units) continue;
      if (s >= 0) {
        ++p.n_hits;
        p.slot_last[s] = t;
        p.buckets[t].push_back(u);
      } else if (p.unit_slot[u] < 0 && !p.pending_flag[u]) {
        p.pending_flag[u] = 1;
        p.pending.push_back(u);
      }
    }
    if (p.resident || p.d.capacity == 0) {
      for (int64_t u : p.pending) p.pending_flag[u] = 0;
      p.pending.clear();
      continue;
    }
    int64_t map_off, data_off;
    stage_layout(p.stage_units, p.d.unit_bytes, &map_off, &data_off);
    FillHeader* hdr = (FillHeader*)p.h_stage;
    int32_t* unmap_ids = (int32_t*)(p.h_stage + 16);
    int32_t* pairs = (int32_t*)(p.h_stage + map_off);
    int32_t n_unmap = 0, n_map = 0;
    const int64_t cap_fill = c->max_fill > 0 ? c->max_fill : (int64_t)p.pending.size();
    for (size_t q = 0; q < p.pending.size(); ++q) {
      const int64_t u = p.pending[q];
      p.pending_flag[u] = 0;
      if ((int64_t)q >= cap_fill || n_map >= p.stage_units) continue;
      int32_t slot;
      if (!p.free_slots.empty()) {
        slot = p.free_slots.back();
        p.free_slots.pop_back();
      } else {
        const int64_t victim = pick_victim(p, t);
        if (victim < 0) continue;
        slot = p.unit_slot[victim];
        p.unit_slot[victim] = -1;
        unmap_ids[n_unmap++] = (int32_t)victim;
      }
      p.slot_unit[slot] = u;
      p.unit_slot[u] = slot;
      p.slot_last[slot] = t;
      p.buckets[t].push_back(u);
      pairs[2 * n_map] = (int32_t)u;
      pairs[2 * n_map + 1] = slot;
      std::memcpy(p.h_stage + data_off + (int64_t)n_map * p.d.unit_bytes,
                  p.d.host_store + u * p.d.unit_bytes, (size_t)p.d.unit_bytes);
      ++n_map;
    }
    p.pending.clear();
    if (n_map == 0) continue;
    hdr->n_unmap = n_unmap;
    hdr->n_map = n_map;
    // header + lists first, on the compute stream, then unmap there
    SF_HIP(hipMemcpyAsync(p.d_stage, p.h_stage, (size_t)map_off + (size_t)n_map * 8,
                          hipMemcpyHostToDevice, compute));
    if (n_unmap > 0) {
      hipLaunchKernelGGL(unmap_kernel, dim3((n_unmap + 255) / 256), dim3(256), 0, compute,
                         p.d_unit2slot, (const uint8_t*)p.d_stage);
      SF_LAUNCH_CHECK();
    }
    SF_HIP(hipEventRecord(c->ev_compute, compute));
    SF_HIP(hipStreamWaitEvent(side, c->ev_compute, 0));
    const size_t bytes = (size_t)n_map * p.d.unit_bytes;
    SF_HIP(hipMemcpyAsync(p.d_stage + data_off, p.h_stage + data_off, bytes, hipMemcpyHostToDevice, side));
    const int64_t words = bytes / 4;
    const unsigned blocks = (unsigned)std::min<int64_t>((words + 255) / 256, 4096);
    hipLaunchKernelGGL(scatter_kernel, dim3(blocks), dim3(256), 0, side, p.d_slots,
                       (const uint8_t*)p.d_stage, map_off, data_off, p.d.unit_bytes);
    SF_LAUNCH_CHECK();
    SF_HIP(hipEventRecord(p.copy_done, side));
    p.in_flight = true;
    p.flight_maps = n_map;
    p.n_installed += n_map;
    p.h2d_bytes += (int64_t)bytes;
    filled += n_map;
    if (c->mode == SF_CACHE_DETERMINISTIC) {
      sf_status st = publish(c, p, compute);
      if (st != SF_OK) return st;
    }
  }
  if (c->mode == SF_CACHE_DETERMINISTIC) SF_HIP(hipStreamSynchronize(compute));
  c->step = t + 1;
  if (n_filled) *n_filled = filled;
  if (overflow) {
    sf_set_error("sf_refine_cache_fill: lookup log overflow (raise max_lookup); some lookups were not recorded");
    return SF_ESTATE;
  }
  return SF_OK;
}

extern "C" sf_status sf_refine_cache_stats(sf_refine_cache* c, int32_t pool, int64_t* lookups,
                                           int64_t* hits, int64_t* installed, int64_t* h2d_bytes) {
  SF_REQUIRE(c, SF_EINVAL, "null cache");
  SF_REQUIRE(pool < (int32_t)c->pools.size(), SF_EINVAL, "pool index out of range");
  int64_t a = 0, b = 0, d = 0, e = 0;
  for (int i = 0; i < (int)c->pools.size(); ++i) {
    if (pool >= 0 && i != pool) continue;
    const HostPool& p = c->pools[i];
    a += p.n_lookups;
    b += p.n_hits;
    d += p.n_installed;
    e += p.h2d_bytes;
  }
  if (lookups) *lookups = a;
  if (hits) *hits = b;
  if (installed) *installed = d;
  if (h2d_bytes) *h2d_bytes = e;
  return SF_OK;
}

extern "C" sf_status sf_refine_cache_resident(sf_refine_cache* c, int32_t pool, int64_t* ids, int64_t* n) {
  SF_REQUIRE(c && ids && n, SF_EINVAL, "bad arguments");
  SF_REQUIRE(pool >= 0 && pool < (int32_t)c->pools.size(), SF_EINVAL, "pool index out of range");
  const HostPool& p = c->pools[pool];
  int64_t m = 0;
  for (int64_t u = 0; u < p.d.n_units; ++u)
    if (p.unit_slot[u] >= 0) ids[m++] = u;
  *n = m;
  return SF_OK;
}
