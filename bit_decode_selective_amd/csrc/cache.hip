// Refinement slot cache: device slots + unit->slot table per pool, host-side
// replacement policy, fills from the pools' host refinement stores.
//
// Method: rag-lover.com StrataFlux summary, explainer dialogue (解説) -- fetched
// precision is cached on the GPU and reused across decode steps, and delivery is
// overlapped with computation; limitations section -- a miss keeps resident
// precision.  Paper abstract (arXiv 2611.08363): generation need not wait for
// every transfer.
//
// A decode step touches every pool of the model (a few hundred for an 8B decoder:
// seven weight matrices and one KV cache per layer), so one fill handles all of
// them at once: one kernel copies every pool's lookup log into a pinned host
// mirror, the policy runs on the host and lists the installs of every pool (two
// small entry copies per fill); an unmap kernel (compute stream), a scatter kernel
// (side stream; it reads the units straight from the pinned host stores over PCIe
// into their slots) and a map kernel (compute stream, behind the scatter) apply
// them.  No host-side gather of unit bytes and no bulk staging copy.
//
// Consistency: the unit->slot tables are only changed by small kernels on the
// compute stream (stream-ordered with every lookup), never while a reader can
// use the entry.  A fill first unmaps its victims on the compute stream, then the
// side stream (after that point of the compute stream) copies the new units into
// the freed slots, and only after that copy has completed is the map kernel
// enqueued on the compute stream.  Deterministic mode enqueues the map right away
// behind a stream wait; async mode enqueues it at the next fill call.
#include <algorithm>
#include <cstring>
#include <map>
#include <mutex>

#include "sf_internal.h"

namespace {

struct LogTab {  // where a pool's lookup log sits in the log block
  int64_t off;   // byte offset of units[cap]; slots[cap] follow
  int32_t cap;   // 0: the pool keeps no log (resident)
  int32_t pad;
};

struct PoolTab {  // what the fill kernels need of a pool
  int32_t* unit2slot;
  uint8_t* slots;
  const uint8_t* store;  // the pinned host store, device view
  int64_t unit_bytes;
};

struct UnmapEnt {
  int32_t pool, unit;
};

struct MapEnt {
  int32_t pool, unit, slot, pad;
};

struct HostPool {
  sf_pool_desc d{};
  bool resident = false;
  int32_t* d_unit2slot = nullptr;
  uint8_t* d_slots = nullptr;  // owned unless resident
  int64_t log_off = 0;         // in the cache's log block
  int32_t log_cap = 0;
  int64_t stage_units = 0;     // most units one fill installs
  const uint8_t* store_dev = nullptr;  // device view of d.host_store
  std::vector<int64_t> slot_unit;  // -1 free
  std::vector<int64_t> slot_last;
  std::vector<int32_t> unit_slot;  // host view (includes units whose copy is in flight)
  std::vector<int32_t> free_slots; // kept sorted descending: back() is the lowest
  std::map<int64_t, std::vector<int64_t>> buckets;  // last-use step -> units (lazy, may hold stale ids)
  std::map<int64_t, size_t> bucket_pos;             // consumed prefix of a sorted bucket
  int64_t bucket_entries = 0;                       // ids held by all buckets
  std::vector<int64_t> pending;
  std::vector<uint8_t> pending_flag;  // per unit
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
  bool any_cached = false;  // some pool is not resident
  hipEvent_t ev_compute = nullptr;
  hipEvent_t copy_done = nullptr;
  // lookup logs: [u32 count per pool, 256-aligned][per pool: units[cap] | slots[cap]],
  // on the device and mirrored in pinned host memory at the same offsets
  uint8_t* d_logs = nullptr;
  uint8_t* h_logs = nullptr;
  uint8_t* h_logs_dev = nullptr;  // the mirror's device address
  size_t logs_bytes = 0;
  LogTab* d_logtab = nullptr;
  PoolTab* d_pooltab = nullptr;
  // fill entries, device and pinned host: [unmaps | maps]
  uint8_t* d_stage = nullptr;
  uint8_t* h_stage = nullptr;
  size_t stage_bytes = 0;
  int64_t map_off = 0;
  bool in_flight = false;  // a copy whose map has not been enqueued
  int32_t flight_maps = 0;
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
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

// One workgroup per pool: copies the step's count and the logged entries into the
// pinned host mirror and clears the device count for the next step.
__global__ __launch_bounds__(256) void logs_to_host_kernel(uint8_t* d_logs, uint8_t* h_logs, const LogTab* tab) {
  __shared__ uint32_t s_cnt;
  const int i = blockIdx.x;
  uint32_t* dc = (uint32_t*)d_logs;
  if (threadIdx.x == 0) {
    const uint32_t c = dc[i];
    s_cnt = c;
    ((uint32_t*)h_logs)[i] = c;
    dc[i] = 0;
  }
  __syncthreads();
  const LogTab t = tab[i];
  const uint32_t n = min(s_cnt, (uint32_t)t.cap);
  const int32_t* src = (const int32_t*)(d_logs + t.off);
  int32_t* dst = (int32_t*)(h_logs + t.off);
  for (uint32_t j = threadIdx.x; j < n; j += 256) {
    dst[j] = src[j];
    dst[t.cap + j] = src[t.cap + j];
  }
}

__global__ void unmap_kernel(const PoolTab* tab, const UnmapEnt* ents, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const UnmapEnt e = ents[i];
    tab[e.pool].unit2slot[e.unit] = -1;
  }
}

__global__ void map_kernel(const PoolTab* tab, const MapEnt* ents, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const MapEnt e = ents[i];
    tab[e.pool].unit2slot[e.unit] = e.slot;
  }
}

// One workgroup per installed unit (grid-stride): copies its bytes from the pinned
// host store (over PCIe) into its slot, 16 bytes per thread where the unit size
// allows (a pinned store is at least 16-byte aligned).
__global__ __launch_bounds__(256) void scatter_kernel(const PoolTab* tab, const MapEnt* ents, int n) {
  for (int e = blockIdx.x; e < n; e += gridDim.x) {
    const MapEnt m = ents[e];
    const PoolTab p = tab[m.pool];
    const uint8_t* src = p.store + (int64_t)m.unit * p.unit_bytes;
    uint8_t* dst = p.slots + (int64_t)m.slot * p.unit_bytes;
    if ((p.unit_bytes & 15) == 0 && (((uintptr_t)p.store | (uintptr_t)p.slots) & 15) == 0) {
      for (int64_t w = threadIdx.x; w < p.unit_bytes / 16; w += 256) ((uint4*)dst)[w] = ((const uint4*)src)[w];
    } else {
      for (int64_t w = threadIdx.x; w < p.unit_bytes / 4; w += 256)
        ((uint32_t*)dst)[w] = ((const uint32_t*)src)[w];
    }
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

void destroy_cache(sf_refine_cache* c) {
  for (auto& p : c->pools) {
    if (p.d_unit2slot) hipFree(p.d_unit2slot);
    if (p.d_slots && !p.resident) hipFree(p.d_slots);
  }
  if (c->d_logs) hipFree(c->d_logs);
  if (c->h_logs) hipHostFree(c->h_logs);
  if (c->d_logtab) hipFree(c->d_logtab);
  if (c->d_pooltab) hipFree(c->d_pooltab);
  if (c->d_stage) hipFree(c->d_stage);
  if (c->h_stage) hipHostFree(c->h_stage);
  if (c->ev_compute) hipEventDestroy(c->ev_compute);
  if (c->copy_done) hipEventDestroy(c->copy_done);
  delete c;
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
    p.bucket_entries -= (int64_t)v.size();
    p.bucket_pos.erase(it->first);
    p.buckets.erase(it);
  }
  return -1;
}

// Buckets keep one id per use, most of them stale once the unit is used again;
// past a few times the slot count they are rebuilt from the slots (one id each).
// The victim order (last use, unit id) does not change.
void compact_buckets(HostPool& p) {
  if (p.bucket_entries <= 4 * ((int64_t)p.slot_unit.size() + 1024)) return;
  p.buckets.clear();
  p.bucket_pos.clear();
  int64_t n = 0;
  for (size_t s = 0; s < p.slot_unit.size(); ++s)
    if (p.slot_unit[s] >= 0) {
      p.buckets[p.slot_last[s]].push_back(p.slot_unit[s]);
      ++n;
    }
  p.bucket_entries = n;
}

sf_status publish(sf_refine_cache* c, hipStream_t compute) {
  if (!c->in_flight) return SF_OK;
  SF_HIP(hipStreamWaitEvent(compute, c->copy_done, 0));
  if (c->flight_maps > 0) {
    hipLaunchKernelGGL(map_kernel, dim3((c->flight_maps + 255) / 256), dim3(256), 0, compute, c->d_pooltab,
                       (const MapEnt*)(c->d_stage + c->map_off), c->flight_maps);
    SF_LAUNCH_CHECK();
  }
  c->in_flight = false;
  c->flight_maps = 0;
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
    out->log_units = (int32_t*)(c->d_logs + p.log_off);
    out->log_slots = out->log_units + p.log_cap;
    out->log_count = (uint32_t*)c->d_logs + pool;
    out->log_cap = p.log_cap;
  }
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
#define CK(call)                                                                  \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess) {                                                       \
      sf_set_error(std::string("sf_refine_cache_create: " #call ": ") + hipGetErrorString(e_)); \
      destroy_cache(c);                                                           \
      return e_ == hipErrorOutOfMemory ? SF_ENOMEM : SF_EHIP;                     \
    }                                                                             \
  } while (0)
  // layouts of the log block and of the staging
  int64_t log_bytes = (int64_t)sf_align256(4 * (size_t)n_pools);
  int64_t stage_ents = 0;
  for (int i = 0; i < n_pools; ++i) {
    HostPool& p = c->pools[i];
    p.d = pools[i];
    p.resident = pools[i].device_store != nullptr;
    if (p.resident) continue;
    c->any_cached = true;
    p.log_cap = p.d.max_lookup > 0 ? p.d.max_lookup : 65536;
    p.log_off = log_bytes;
    log_bytes += (int64_t)sf_align256(8 * (size_t)p.log_cap);
    p.stage_units = std::min<int64_t>(p.d.capacity, max_fill > 0 ? max_fill : p.d.capacity);
    stage_ents += p.stage_units;
  }
  c->logs_bytes = (size_t)log_bytes;
  c->map_off = (int64_t)sf_align256((size_t)stage_ents * sizeof(UnmapEnt));
  c->stage_bytes = sf_align256((size_t)c->map_off + (size_t)stage_ents * sizeof(MapEnt));
  CK(hipEventCreateWithFlags(&c->ev_compute, hipEventDisableTiming));
  CK(hipEventCreateWithFlags(&c->copy_done, hipEventDisableTiming));
  CK(hipMalloc((void**)&c->d_logs, c->logs_bytes));
  CK(hipHostMalloc((void**)&c->h_logs, c->logs_bytes, hipHostMallocDefault));
  CK(hipHostGetDevicePointer((void**)&c->h_logs_dev, c->h_logs, 0));
  hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(256), 0, 0, (uint32_t*)c->d_logs, n_pools);
  if (stage_ents > 0) {
    CK(hipMalloc((void**)&c->d_stage, c->stage_bytes));
    CK(hipHostMalloc((void**)&c->h_stage, c->stage_bytes, hipHostMallocDefault));
  }
  std::vector<LogTab> logtab(n_pools);
  std::vector<PoolTab> pooltab(n_pools);
  for (int i = 0; i < n_pools; ++i) {
    HostPool& p = c->pools[i];
    const int64_t nu = p.d.n_units, cap = p.d.capacity;
    CK(hipMalloc((void**)&p.d_unit2slot, sizeof(int32_t) * nu));
    p.unit_slot.assign(nu, -1);
    p.pending_flag.assign(nu, 0);
    if (p.resident) {
      p.d_slots = p.d.device_store;
      hipLaunchKernelGGL(iota_kernel, dim3((unsigned)((nu + 255) / 256)), dim3(256), 0, 0, p.d_unit2slot, nu);
      for (int64_t u = 0; u < nu; ++u) p.unit_slot[u] = (int32_t)u;
    } else {
      hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((nu + 255) / 256)), dim3(256), 0, 0, p.d_unit2slot, nu, -1);
      if (cap > 0) {
        CK(hipMalloc((void**)&p.d_slots, (size_t)cap * p.d.unit_bytes));
        // the fill kernels read the store directly: it must be pinned host memory
        hipPointerAttribute_t attr{};
        if (hipPointerGetAttributes(&attr, p.d.host_store) != hipSuccess || attr.type != hipMemoryTypeHost ||
            attr.devicePointer == nullptr) {
          (void)hipGetLastError();
          sf_set_error("sf_refine_cache_create: host_store of pool " + std::to_string(i) +
                       " is not pinned host memory (hipHostMalloc / pin_memory)");
          destroy_cache(c);
          return SF_EINVAL;
        }
        p.store_dev = (const uint8_t*)attr.devicePointer;
      }
      p.slot_unit.assign(cap, -1);
      p.slot_last.assign(cap, -1);
      p.free_slots.resize(cap);
      for (int64_t s = 0; s < cap; ++s) p.free_slots[s] = (int32_t)(cap - 1 - s);
    }
    logtab[i] = LogTab{p.log_off, p.log_cap, 0};
    pooltab[i] = PoolTab{p.d_unit2slot, p.d_slots, p.store_dev, p.d.unit_bytes};
  }
  CK(hipMalloc((void**)&c->d_logtab, sizeof(LogTab) * n_pools));
  CK(hipMalloc((void**)&c->d_pooltab, sizeof(PoolTab) * n_pools));
  CK(hipMemcpy(c->d_logtab, logtab.data(), sizeof(LogTab) * n_pools, hipMemcpyHostToDevice));
  CK(hipMemcpy(c->d_pooltab, pooltab.data(), sizeof(PoolTab) * n_pools, hipMemcpyHostToDevice));
  CK(hipGetLastError());
  CK(hipDeviceSynchronize());
#undef CK
  *out = c;
  return SF_OK;
}

extern "C" sf_status sf_refine_cache_destroy(sf_refine_cache* c) {
  if (!c) return SF_OK;
  hipDeviceSynchronize();
  destroy_cache(c);
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
  if (!c->any_cached) {  // only resident pools: nothing is ever missing
    c->step = t + 1;
    if (n_filled) *n_filled = 0;
    return SF_OK;
  }
  const int np = (int)c->pools.size();
  // 1. every pool's lookup log into the pinned mirror (device counts cleared)
  hipLaunchKernelGGL(logs_to_host_kernel, dim3(np), dim3(256), 0, compute, c->d_logs, c->h_logs_dev,
                     (const LogTab*)c->d_logtab);
  SF_LAUNCH_CHECK();
  SF_HIP(hipStreamSynchronize(compute));
  // 2. async mode: publish the previous fill (its copy must be complete by now,
  //    and the staging is free again after this wait)
  if (c->in_flight) {
    SF_HIP(hipEventSynchronize(c->copy_done));
    sf_status st = publish(c, compute);
    if (st != SF_OK) return st;
  }
  // 3. policy of every pool; installs listed in the pinned entry buffer
  const uint32_t* counts = (const uint32_t*)c->h_logs;
  UnmapEnt* unm = (UnmapEnt*)c->h_stage;
  MapEnt* mp = (MapEnt*)(c->h_stage + c->map_off);
  int32_t n_unmap = 0, n_map = 0;
  bool overflow = false;
  for (int i = 0; i < np; ++i) {
    HostPool& p = c->pools[i];
    if (p.resident) continue;
    uint32_t cnt = counts[i];
    if (cnt > (uint32_t)p.log_cap) {
      overflow = true;
      cnt = (uint32_t)p.log_cap;
    }
    const int32_t* log_u = (const int32_t*)(c->h_logs + p.log_off);
    const int32_t* log_s = log_u + p.log_cap;
    const int64_t cap = p.d.capacity;
    std::vector<int64_t>* now = nullptr;  // bucket of step t
    for (uint32_t e = 0; e < cnt; ++e) {
      const int64_t u = log_u[e];
      const int32_t s = log_s[e];
      ++p.n_lookups;
      if (u < 0 || u >= p.d.n_units) continue;
      if (s >= 0 && s < cap) {
        ++p.n_hits;
        p.slot_last[s] = t;
        if (!now) now = &p.buckets[t];
        now->push_back(u);
        ++p.bucket_entries;
      } else if (p.unit_slot[u] < 0 && !p.pending_flag[u]) {
        p.pending_flag[u] = 1;
        p.pending.push_back(u);
      }
    }
    const int64_t cap_fill = c->max_fill > 0 ? c->max_fill : (int64_t)p.pending.size();
    int64_t n_pool = 0;
    for (size_t q = 0; q < p.pending.size(); ++q) {
      const int64_t u = p.pending[q];
      p.pending_flag[u] = 0;
      if (cap == 0 || (int64_t)q >= cap_fill || n_pool >= p.stage_units) continue;
      int32_t slot;
      if (!p.free_slots.empty()) {
        slot = p.free_slots.back();
        p.free_slots.pop_back();
      } else {
        const int64_t victim = pick_victim(p, t);
        if (victim < 0) continue;
        slot = p.unit_slot[victim];
        p.unit_slot[victim] = -1;
        unm[n_unmap++] = UnmapEnt{i, (int32_t)victim};
      }
      p.slot_unit[slot] = u;
      p.unit_slot[u] = slot;
      p.slot_last[slot] = t;
      if (!now) now = &p.buckets[t];
      now->push_back(u);
      ++p.bucket_entries;
      mp[n_map] = MapEnt{i, (int32_t)u, slot, 0};
      ++n_map;
      ++n_pool;
      ++p.n_installed;
      p.h2d_bytes += p.d.unit_bytes;
    }
    p.pending.clear();
    compact_buckets(p);
  }
  if (n_map > 0) {
    // 4. entries and unmaps on the compute stream; the scatter (units read from the
    //    pinned stores) on the side stream once the unmaps are done there
    if (n_unmap > 0)
      SF_HIP(hipMemcpyAsync(c->d_stage, c->h_stage, sizeof(UnmapEnt) * (size_t)n_unmap, hipMemcpyHostToDevice,
                            compute));
    SF_HIP(hipMemcpyAsync(c->d_stage + c->map_off, c->h_stage + c->map_off, sizeof(MapEnt) * (size_t)n_map,
                          hipMemcpyHostToDevice, compute));
    if (n_unmap > 0) {
      hipLaunchKernelGGL(unmap_kernel, dim3((n_unmap + 255) / 256), dim3(256), 0, compute, c->d_pooltab,
                         (const UnmapEnt*)c->d_stage, n_unmap);
      SF_LAUNCH_CHECK();
    }
    SF_HIP(hipEventRecord(c->ev_compute, compute));
    SF_HIP(hipStreamWaitEvent(side, c->ev_compute, 0));
    hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)std::min(n_map, 4096)), dim3(256), 0, side, c->d_pooltab,
                       (const MapEnt*)(c->d_stage + c->map_off), n_map);
    SF_LAUNCH_CHECK();
    SF_HIP(hipEventRecord(c->copy_done, side));
    c->in_flight = true;
    c->flight_maps = n_map;
    if (c->mode == SF_CACHE_DETERMINISTIC) {
      sf_status st = publish(c, compute);
      if (st != SF_OK) return st;
    }
  }
  c->step = t + 1;
  if (n_filled) *n_filled = n_map;
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
