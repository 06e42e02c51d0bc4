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
//
// A pool whose store is a file (the SSD tier) has pinned staging of its own: the
// fill reads each installed unit from the file into staging with a positioned
// read (direct I/O where possible, up to 8 reads in flight), and the scatter
// kernel copies from staging instead of from a host store.  The staging of one
// fill is reused by the next only after that fill's copy has completed (the fill
// waits for the compute stream, which waited for the copy, or for the copy itself).
#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <cerrno>
#include <chrono>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <thread>

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
  const uint8_t* store;  // the pinned host store (or the file pool's staging), device view
  int64_t unit_bytes;
  int64_t staged;        // 1: the unit of a map entry sits at staging position `pad`
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
  const uint8_t* host_dev = nullptr;   // device view of d.host_store
  const uint8_t* store_dev = nullptr;  // what the scatter reads: host store or file staging (device view)
  std::vector<int64_t> slot_unit;  // -1 free
  std::vector<int64_t> slot_last;
  std::vector<int32_t> unit_slot;  // host view (includes units whose copy is in flight)
  std::vector<int32_t> free_slots; // kept sorted descending: back() is the lowest
  std::map<int64_t, std::vector<int64_t>> buckets;  // last-use step -> units (lazy, may hold stale ids)
  std::map<int64_t, size_t> bucket_pos;             // consumed prefix of a sorted bucket
  int64_t bucket_entries = 0;                       // ids held by all buckets
  std::vector<int64_t> pending;
  std::vector<uint8_t> pending_flag;  // per unit
  // fetch lead: ring slots [capacity, capacity + lead) of d_slots
  int32_t lead = 0;
  int32_t* d_ring = nullptr;  // [lead] unit held by each ring slot, -1 = empty
  int32_t* d_plan = nullptr;  // [2 * lead] (unit, slot) fetched by a prefetch | [1] count
  // store file (SSD tier)
  int fd = -1;
  bool direct = false;
  uint8_t* h_fstage = nullptr;  // pinned staging [stage_units][unit_bytes]
  const uint8_t* fstage_dev = nullptr;
  std::vector<float> lat_us;    // ring of the last read times
  size_t lat_next = 0;
  int64_t io_reads = 0, io_bytes = 0;
  double io_ms = 0.0;
  // stats
  int64_t n_lookups = 0, n_hits = 0, n_installed = 0, h2d_bytes = 0;
};

struct FileRead {
  int32_t pool;
  int32_t stage;
  int64_t unit;
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
  uint8_t* h_logs[2] = {nullptr, nullptr};      // two mirrors (async mode alternates)
  uint8_t* h_logs_dev[2] = {nullptr, nullptr};  // their device addresses
  hipEvent_t ev_logs[2] = {nullptr, nullptr};   // a mirror's copy has landed
  size_t logs_bytes = 0;
  LogTab* d_logtab = nullptr;
  PoolTab* d_pooltab = nullptr;
  // fill entries, device and pinned host: [unmaps | maps]
  uint8_t* d_stage[2] = {nullptr, nullptr};  // async mode alternates between the two
  uint8_t* h_stage[2] = {nullptr, nullptr};
  int flight_buf = 0;                         // the staging of the fill in flight
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
  const uint32_t n = min(s_cnt & 0x7FFFFFFFu, (uint32_t)t.cap);
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
    const uint8_t* src = p.store + (int64_t)(p.staged ? m.pad : m.unit) * p.unit_bytes;
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
      base = sf_log_reserve(p.log_count, (uint32_t)n, (uint32_t)p.log_cap);
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
    if (p.h_fstage) hipHostFree(p.h_fstage);
    if (p.d_ring) hipFree(p.d_ring);
    if (p.d_plan) hipFree(p.d_plan);
    if (p.fd >= 0) close(p.fd);
  }
  if (c->d_logs) hipFree(c->d_logs);
  for (int i = 0; i < 2; ++i) {
    if (c->h_logs[i]) hipHostFree(c->h_logs[i]);
    if (c->d_stage[i]) hipFree(c->d_stage[i]);
    if (c->h_stage[i]) hipHostFree(c->h_stage[i]);
    if (c->ev_logs[i]) hipEventDestroy(c->ev_logs[i]);
  }
  if (c->d_logtab) hipFree(c->d_logtab);
  if (c->d_pooltab) hipFree(c->d_pooltab);
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

// Reads n bytes at offset off of a store file into dst.  Direct I/O reads whole
// 4 KiB blocks into an aligned bounce buffer (at least n + 8 KiB) and copies the
// unit out of it.
bool read_unit(int fd, bool direct, int64_t off, int64_t n, uint8_t* dst, uint8_t* bounce) {
  if (!direct) {
    int64_t done = 0;
    while (done < n) {
      const ssize_t g = pread(fd, dst + done, (size_t)(n - done), (off_t)(off + done));
      if (g <= 0) {
        if (g < 0 && errno == EINTR) continue;
        return false;
      }
      done += g;
    }
    return true;
  }
  const int64_t a0 = off & ~(int64_t)4095, a1 = (off + n + 4095) & ~(int64_t)4095;
  int64_t got = 0;
  while (got < off + n - a0) {
    const ssize_t g = pread(fd, bounce + got, (size_t)(a1 - a0 - got), (off_t)(a0 + got));
    if (g <= 0) {
      if (g < 0 && errno == EINTR) continue;
      return false;
    }
    got += g;
  }
  std::memcpy(dst, bounce + (off - a0), (size_t)n);
  return true;
}

// The file reads of one fill, up to 8 at a time; per-read times go to the pools'
// rings.  False if a read failed.
bool run_file_reads(sf_refine_cache* c, const std::vector<FileRead>& reads) {
  if (reads.empty()) return true;
  const auto t0 = std::chrono::steady_clock::now();
  const int nt = (int)std::min<size_t>(8, reads.size());
  std::vector<float> us(reads.size(), 0.f);
  std::vector<uint8_t> ok(nt, 1);
  int64_t max_unit = 0;
  for (const FileRead& r : reads) max_unit = std::max(max_unit, c->pools[r.pool].d.unit_bytes);
  const size_t bounce_bytes = (size_t)((max_unit + 8192 + 4095) & ~(int64_t)4095);
  auto work = [&](int w) {
    uint8_t* bounce = (uint8_t*)std::aligned_alloc(4096, bounce_bytes);
    if (!bounce) {
      ok[w] = 0;
      return;
    }
    for (size_t i = (size_t)w; i < reads.size(); i += (size_t)nt) {
      const FileRead& r = reads[i];
      HostPool& p = c->pools[r.pool];
      const int64_t ub = p.d.unit_bytes;
      const auto a = std::chrono::steady_clock::now();
      if (!read_unit(p.fd, p.direct, p.d.store_offset + r.unit * ub, ub, p.h_fstage + (int64_t)r.stage * ub,
                     bounce)) {
        ok[w] = 0;
        break;
      }
      us[i] = std::chrono::duration<float, std::micro>(std::chrono::steady_clock::now() - a).count();
    }
    std::free(bounce);
  };
  if (nt == 1) {
    work(0);
  } else {
    std::vector<std::thread> th;
    for (int w = 0; w < nt; ++w) th.emplace_back(work, w);
    for (auto& t : th) t.join();
  }
  const double ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
  for (size_t i = 0; i < reads.size(); ++i) {
    HostPool& p = c->pools[reads[i].pool];
    if (p.lat_us.size() < 65536) {
      p.lat_us.push_back(us[i]);
    } else {
      p.lat_us[p.lat_next] = us[i];
      p.lat_next = (p.lat_next + 1) % p.lat_us.size();
    }
    ++p.io_reads;
    p.io_bytes += p.d.unit_bytes;
  }
  for (const FileRead& r : reads) c->pools[r.pool].io_ms += ms / (double)reads.size();
  return std::all_of(ok.begin(), ok.end(), [](uint8_t v) { return v != 0; });
}

sf_status publish(sf_refine_cache* c, hipStream_t compute) {
  if (!c->in_flight) return SF_OK;
  SF_HIP(hipStreamWaitEvent(compute, c->copy_done, 0));
  if (c->flight_maps > 0) {
    hipLaunchKernelGGL(map_kernel, dim3((c->flight_maps + 255) / 256), dim3(256), 0, compute, c->d_pooltab,
                       (const MapEnt*)(c->d_stage[c->flight_buf] + c->map_off), c->flight_maps);
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
      SF_REQUIRE(d.capacity == d.n_units && !d.store_file, SF_EINVAL,
                 "a resident pool needs capacity == n_units and no store file");
    else
      SF_REQUIRE(d.host_store || d.store_file || d.capacity == 0, SF_EINVAL,
                 "a pool with slots needs a host store or a store file");
    SF_REQUIRE(!(d.store_file && d.host_store), SF_EINVAL, "give a host store or a store file, not both");
    SF_REQUIRE(d.store_offset >= 0, SF_EINVAL, "bad store_offset");
    SF_REQUIRE(d.lead_slots >= 0 && d.lead_slots <= 16384 && d.lead_slots <= d.n_units, SF_EINVAL,
               "lead_slots must be in [0, min(n_units, 16384)]");
    SF_REQUIRE(d.lead_slots == 0 || (d.host_store && !d.device_store), SF_EINVAL,
               "lead slots need a pinned host store");
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
  for (int i = 0; i < 2; ++i) {
    CK(hipHostMalloc((void**)&c->h_logs[i], c->logs_bytes, hipHostMallocDefault));
    CK(hipHostGetDevicePointer((void**)&c->h_logs_dev[i], c->h_logs[i], 0));
    CK(hipEventCreateWithFlags(&c->ev_logs[i], hipEventDisableTiming));
  }
  hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(256), 0, 0, (uint32_t*)c->d_logs, n_pools);
  if (stage_ents > 0) {
    for (int i = 0; i < 2; ++i) {
      CK(hipMalloc((void**)&c->d_stage[i], c->stage_bytes));
      CK(hipHostMalloc((void**)&c->h_stage[i], c->stage_bytes, hipHostMallocDefault));
    }
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
      if (cap > 0 && p.d.store_file) {
        CK(hipMalloc((void**)&p.d_slots, (size_t)cap * p.d.unit_bytes));
        p.fd = open(p.d.store_file, O_RDONLY | O_DIRECT);
        p.direct = p.fd >= 0;
        if (p.fd < 0) p.fd = open(p.d.store_file, O_RDONLY);
        struct stat stt {};
        if (p.fd < 0 || fstat(p.fd, &stt) != 0 ||
            (int64_t)stt.st_size < p.d.store_offset + p.d.n_units * p.d.unit_bytes) {
          sf_set_error("sf_refine_cache_create: store file of pool " + std::to_string(i) +
                       " cannot be opened or is shorter than its units");
          destroy_cache(c);
          return SF_EINVAL;
        }
        CK(hipHostMalloc((void**)&p.h_fstage, (size_t)std::max<int64_t>(1, p.stage_units) * p.d.unit_bytes,
                         hipHostMallocDefault));
        CK(hipHostGetDevicePointer((void**)&p.fstage_dev, p.h_fstage, 0));
        p.store_dev = p.fstage_dev;
      } else if (p.d.host_store) {
        p.lead = p.d.lead_slots;
        if (cap + p.lead > 0) CK(hipMalloc((void**)&p.d_slots, (size_t)(cap + p.lead) * p.d.unit_bytes));
        if (p.lead > 0) {
          CK(hipMalloc((void**)&p.d_ring, sizeof(int32_t) * p.lead));
          CK(hipMalloc((void**)&p.d_plan, sizeof(int32_t) * (2 * (size_t)p.lead + 1)));
          hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((p.lead + 255) / 256)), dim3(256), 0, 0, p.d_ring,
                             (int64_t)p.lead, -1);
        }
        // the fill and lag kernels read the store directly: it must be pinned host memory
        hipPointerAttribute_t attr{};
        const bool pinned = hipPointerGetAttributes(&attr, p.d.host_store) == hipSuccess &&
                            attr.type == hipMemoryTypeHost && attr.devicePointer != nullptr;
        if (!pinned) (void)hipGetLastError();
        if (!pinned && cap == 0 && p.lead == 0) {
          // a pool without slots never fills; only sf_refine_lag_delta would read it
        } else if (!pinned) {
          sf_set_error("sf_refine_cache_create: host_store of pool " + std::to_string(i) +
                       " is not pinned host memory (hipHostMalloc / pin_memory)");
          destroy_cache(c);
          return SF_EINVAL;
        } else {
          p.store_dev = (const uint8_t*)attr.devicePointer;
          p.host_dev = p.store_dev;
        }
      }
      p.slot_unit.assign(cap, -1);
      p.slot_last.assign(cap, -1);
      p.free_slots.resize(cap);
      for (int64_t s = 0; s < cap; ++s) p.free_slots[s] = (int32_t)(cap - 1 - s);
    }
    logtab[i] = LogTab{p.log_off, p.log_cap, 0};
    pooltab[i] = PoolTab{p.d_unit2slot, p.d_slots, p.store_dev, p.d.unit_bytes, p.fd >= 0 ? 1 : 0};
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
  // Async mode lags the policy by one step so that the host never waits for the
  // step in flight: this call copies step t's logs into one mirror and runs the
  // policy on step t-1's logs (copied by the previous call, complete once step t-1
  // has finished); its installs are copied while step t+1 runs and mapped by the
  // next call, so they serve lookups from step t+2.  Deterministic mode runs the
  // policy on step t's logs after one wait for the compute stream.
  const bool lag = c->mode == SF_CACHE_ASYNC;
  const int cur = lag ? (int)(t & 1) : 0;
  // 1. every pool's lookup log into a pinned mirror (device counts cleared)
  hipLaunchKernelGGL(logs_to_host_kernel, dim3(np), dim3(256), 0, compute, c->d_logs, c->h_logs_dev[cur],
                     (const LogTab*)c->d_logtab);
  SF_LAUNCH_CHECK();
  if (lag)
    SF_HIP(hipEventRecord(c->ev_logs[cur], compute));
  else
    SF_HIP(hipStreamSynchronize(compute));
  // 2. async mode: map the previous call's installs behind their copy (a wait of the
  //    compute stream, not of the host)
  if (c->in_flight) {
    sf_status st = publish(c, compute);
    if (st != SF_OK) return st;
  }
  int src = cur;  // the mirror the policy reads
  int64_t tl = t;  // the step whose logs they are
  if (lag) {
    if (t == 0) {  // no earlier step to act on yet
      c->step = 1;
      if (n_filled) *n_filled = 0;
      return SF_OK;
    }
    src = cur ^ 1;
    tl = t - 1;
    // step t-1's logs have landed; so have the entry copies of the call before the
    // previous one, which used the staging this call writes
    SF_HIP(hipEventSynchronize(c->ev_logs[src]));
  }
  const int sb = cur;  // staging of this call's installs
  // 3. policy of every pool; installs listed in the pinned entry buffer
  const uint32_t* counts = (const uint32_t*)c->h_logs[src];
  UnmapEnt* unm = (UnmapEnt*)c->h_stage[sb];
  MapEnt* mp = (MapEnt*)(c->h_stage[sb] + c->map_off);
  int32_t n_unmap = 0, n_map = 0;
  bool overflow = false;
  std::vector<FileRead> file_reads;
  for (int i = 0; i < np; ++i) {
    HostPool& p = c->pools[i];
    if (p.resident) continue;
    // entries below the count are complete; bit 31 marks a lookup that did not fit
    uint32_t cnt = counts[i] & 0x7FFFFFFFu;
    if (counts[i] & 0x80000000u) overflow = true;
    if (cnt > (uint32_t)p.log_cap) cnt = (uint32_t)p.log_cap;
    const int32_t* log_u = (const int32_t*)(c->h_logs[src] + p.log_off);
    const int32_t* log_s = log_u + p.log_cap;
    const int64_t cap = p.d.capacity;
    std::vector<int64_t>* now = nullptr;  // bucket of step tl
    for (uint32_t e = 0; e < cnt; ++e) {
      const int64_t u = log_u[e];
      const int32_t s = log_s[e];
      ++p.n_lookups;
      if (u < 0 || u >= p.d.n_units) continue;
      if (s >= cap) {  // a ring slot (fetch lead): a hit that is not an LRU use
        ++p.n_hits;
      } else if (s >= 0) {
        ++p.n_hits;
        p.slot_last[s] = tl;
        if (!now) now = &p.buckets[tl];
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
        const int64_t victim = pick_victim(p, tl);
        if (victim < 0) continue;
        slot = p.unit_slot[victim];
        p.unit_slot[victim] = -1;
        unm[n_unmap++] = UnmapEnt{i, (int32_t)victim};
      }
      p.slot_unit[slot] = u;
      p.unit_slot[u] = slot;
      p.slot_last[slot] = tl;
      if (!now) now = &p.buckets[tl];
      now->push_back(u);
      ++p.bucket_entries;
      mp[n_map] = MapEnt{i, (int32_t)u, slot, (int32_t)n_pool};
      if (p.fd >= 0) file_reads.push_back(FileRead{i, (int32_t)n_pool, u});
      ++n_map;
      ++n_pool;
      ++p.n_installed;
      p.h2d_bytes += p.d.unit_bytes;
    }
    p.pending.clear();
    compact_buckets(p);
  }
  // the SSD tier's units into the pools' staging (the previous fill's copy out of
  // it has completed: see step 2 and the wait on `compute` in step 1)
  if (!run_file_reads(c, file_reads)) {
    sf_set_error(std::string("sf_refine_cache_fill: a store file read failed: ") + std::strerror(errno));
    return SF_ESTATE;
  }
  if (n_map > 0) {
    // 4. entries and unmaps on the compute stream; the scatter (units read from the
    //    pinned stores) on the side stream once the unmaps are done there
    if (n_unmap > 0)
      SF_HIP(hipMemcpyAsync(c->d_stage[sb], c->h_stage[sb], sizeof(UnmapEnt) * (size_t)n_unmap, hipMemcpyHostToDevice,
                            compute));
    SF_HIP(hipMemcpyAsync(c->d_stage[sb] + c->map_off, c->h_stage[sb] + c->map_off, sizeof(MapEnt) * (size_t)n_map,
                          hipMemcpyHostToDevice, compute));
    if (n_unmap > 0) {
      hipLaunchKernelGGL(unmap_kernel, dim3((n_unmap + 255) / 256), dim3(256), 0, compute, c->d_pooltab,
                         (const UnmapEnt*)c->d_stage[sb], n_unmap);
      SF_LAUNCH_CHECK();
    }
    SF_HIP(hipEventRecord(c->ev_compute, compute));
    SF_HIP(hipStreamWaitEvent(side, c->ev_compute, 0));
    hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)std::min(n_map, 4096)), dim3(256), 0, side, c->d_pooltab,
                       (const MapEnt*)(c->d_stage[sb] + c->map_off), n_map);
    SF_LAUNCH_CHECK();
    SF_HIP(hipEventRecord(c->copy_done, side));
    c->in_flight = true;
    c->flight_maps = n_map;
    c->flight_buf = sb;
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

namespace {

// Exclusive prefix of a per-thread flag over a 1024-thread workgroup (in thread
// order); *total = the number of set flags.  Uses wsum[16]; ends with a barrier.
__device__ __forceinline__ int block_rank(bool f, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t m = __ballot(f);
  const int below = __popcll(m & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
  __syncthreads();
  if (lane == 0) wsum[wave] = __popcll(m);
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < 16; ++w) {
    const int v = wsum[w];
    base += w < wave ? v : 0;
    tot += v;
  }
  *total = tot;
  __syncthreads();
  return base + below;
}

// Fetch lead, planning: one 1024-thread workgroup.  Ring slots whose unit is named
// again are kept; the others are emptied (their unit unmapped if the slot still
// serves it); the named units mapped nowhere take the empty slots in ascending
// order.  The plan lists (unit, slot) pairs; the count follows them.
constexpr int LEAD_T = 1024, LEAD_MAX = 16384;
__global__ __launch_bounds__(LEAD_T) void lead_plan_kernel(int32_t* unit2slot, int64_t n_units, int32_t cap,
                                                           int32_t lead, int32_t* ring, const int32_t* ids, int32_t n,
                                                           int32_t* plan) {
  __shared__ uint8_t keep[LEAD_MAX];
  __shared__ uint16_t free_slot[LEAD_MAX];
  __shared__ int wsum[16];
  const int tid = threadIdx.x;
  for (int j = tid; j < lead; j += LEAD_T) keep[j] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += LEAD_T) {
    const int32_t u = ids[i];
    if (u >= 0 && u < n_units) {
      const int32_t sl = unit2slot[u];
      if (sl >= cap && sl < cap + lead) keep[sl - cap] = 1;
    }
  }
  __syncthreads();
  int n_free = 0;
  for (int j0 = 0; j0 < lead; j0 += LEAD_T) {
    const int j = j0 + tid;
    const bool fr = j < lead && !keep[j];
    int tot;
    const int rk = block_rank(fr, wsum, &tot);
    if (fr) {
      free_slot[n_free + rk] = (uint16_t)j;
      const int32_t o = ring[j];
      if (o >= 0 && unit2slot[o] == cap + j) unit2slot[o] = -1;
      ring[j] = -1;
    }
    n_free += tot;
  }
  // (a named unit is never one emptied here: its ring slot was kept)
  int n_new = 0;
  for (int i0 = 0; i0 < n; i0 += LEAD_T) {
    const int i = i0 + tid;
    int32_t u = -1;
    bool miss = false;
    if (i < n) {
      u = ids[i];
      miss = u >= 0 && u < n_units && unit2slot[u] < 0;
    }
    int tot;
    const int rk = n_new + block_rank(miss, wsum, &tot);
    if (miss && rk < n_free) {
      const int j = free_slot[rk];
      ring[j] = u;
      plan[2 * rk] = u;
      plan[2 * rk + 1] = cap + j;
    }
    n_new += tot;
  }
  if (tid == 0) plan[2 * lead] = min(n_new, n_free);
}

// Copies the planned units from the pinned host store (over PCIe) into their slots.
__global__ __launch_bounds__(256) void lead_copy_kernel(const uint8_t* store, uint8_t* slots, int64_t unit_bytes,
                                                        const int32_t* plan, int32_t lead) {
  const int cnt = plan[2 * lead];
  for (int e = blockIdx.x; e < cnt; e += gridDim.x) {
    const uint8_t* src = store + (int64_t)plan[2 * e] * unit_bytes;
    uint8_t* dst = slots + (int64_t)plan[2 * e + 1] * unit_bytes;
    if ((unit_bytes & 15) == 0 && (((uintptr_t)store | (uintptr_t)slots) & 15) == 0) {
      for (int64_t w = threadIdx.x; w < unit_bytes / 16; w += 256) ((uint4*)dst)[w] = ((const uint4*)src)[w];
    } else {
      for (int64_t w = threadIdx.x; w < unit_bytes / 4; w += 256) ((uint32_t*)dst)[w] = ((const uint32_t*)src)[w];
    }
  }
}

// Maps the planned units once their bytes are in place (a launch after the copy).
__global__ __launch_bounds__(256) void lead_map_kernel(int32_t* unit2slot, const int32_t* plan, int32_t lead) {
  const int cnt = plan[2 * lead];
  for (int e = threadIdx.x; e < cnt; e += 256) unit2slot[plan[2 * e]] = plan[2 * e + 1];
}

}  // namespace

extern "C" sf_status sf_refine_cache_prefetch(sf_refine_cache* c, int32_t pool, const int32_t* unit_ids, int32_t n,
                                              sf_stream stream_) {
  SF_REQUIRE(c, SF_EINVAL, "null cache");
  SF_REQUIRE(pool >= 0 && pool < (int32_t)c->pools.size(), SF_EINVAL, "pool index out of range");
  HostPool& p = c->pools[pool];
  SF_REQUIRE(p.lead > 0, SF_EINVAL, "the pool has no lead slots");
  SF_REQUIRE(n >= 0 && (n == 0 || unit_ids), SF_EINVAL, "bad ids");
  hipStream_t s = (hipStream_t)stream_;
  hipLaunchKernelGGL(lead_plan_kernel, dim3(1), dim3(LEAD_T), 0, s, p.d_unit2slot, p.d.n_units,
                     (int32_t)p.d.capacity, p.lead, p.d_ring, unit_ids, n, p.d_plan);
  SF_LAUNCH_CHECK();
  hipLaunchKernelGGL(lead_copy_kernel, dim3((unsigned)std::max(1, std::min(p.lead, 1024))), dim3(256), 0, s,
                     p.host_dev, p.d_slots, p.d.unit_bytes, (const int32_t*)p.d_plan, p.lead);
  SF_LAUNCH_CHECK();
  hipLaunchKernelGGL(lead_map_kernel, dim3(1), dim3(256), 0, s, p.d_unit2slot, (const int32_t*)p.d_plan, p.lead);
  SF_LAUNCH_CHECK();
  return SF_OK;
}

namespace {

// Fetch lag: delta[b][n] = sum over the selected channels k that missed of
// x[b][k] * s[n][k/128] * c_lo[n][k], the refinement words read straight from the
// pinned host store (channel-major units: unit k holds c_lo[0..N)[k], LSB first).
// A thread per output row; the late channels are listed in LDS first (in selection
// order) and their words requested LAG_U at a time.
constexpr int LAG_T = 256, LAG_LIST = 2048, LAG_U = 8, LAG_MAXB = 16;

__global__ __launch_bounds__(LAG_T) void lag_delta_kernel(const uint8_t* store, int64_t unit_bytes,
                                                         const uint32_t* sz, int n_out, int k_in, int r,
                                                         const uint16_t* x, int batch, int k_sel,
                                                         const int32_t* sel, const int32_t* hit, float* delta) {
  __shared__ int s_k[LAG_LIST];
  __shared__ int s_n;
  const int tid = threadIdx.x;
  const int n = blockIdx.x * LAG_T + tid;
  const int ngr = k_in / 128;
  float acc[LAG_MAXB];
#pragma unroll
  for (int b = 0; b < LAG_MAXB; ++b) acc[b] = 0.f;
  for (int j0 = 0; j0 < k_sel; j0 += LAG_LIST) {
    const int jn = min(LAG_LIST, k_sel - j0);
    if (tid == 0) s_n = 0;
    __syncthreads();
    // late entries of this round, in selection order (one wave compacts by ballot)
    if (tid < 64) {
      int base = 0;
      for (int j = tid; j - tid < jn; j += 64) {
        const int kq = j < jn ? sel[j0 + j] : -1;
        const bool late = j < jn && hit[j0 + j] < 0 && kq >= 0 && kq < k_in;
        const uint64_t m = __ballot(late);
        const int pos = base + __popcll(m & ((1ull << tid) - 1ull));
        if (late) s_k[pos] = kq;
        base += __popcll(m);
      }
      if (tid == 0) s_n = base;
    }
    __syncthreads();
    const int nl = s_n;
    for (int i0 = 0; i0 < nl; i0 += LAG_U) {
      uint64_t wv[LAG_U];
      float sv[LAG_U];
      int kk[LAG_U];
#pragma unroll
      for (int u = 0; u < LAG_U; ++u) {
        kk[u] = i0 + u < nl ? s_k[i0 + u] : -1;
        wv[u] = 0;
        sv[u] = 0.f;
        if (kk[u] >= 0 && n < n_out) {
          const uint32_t* uw = (const uint32_t*)(store + (int64_t)kk[u] * unit_bytes);
          const int bit = n * r, wi = bit >> 5;
          const int nw = (int)(unit_bytes / 4);
          const uint32_t lo = uw[wi];
          const uint32_t hi2 = wi + 1 < nw ? uw[wi + 1] : 0u;
          wv[u] = (((uint64_t)hi2 << 32) | lo) >> (bit & 31);
          sv[u] = sf_h2f(sz[(int64_t)n * ngr + kk[u] / 128] & 0xFFFFu);
        }
      }
#pragma unroll
      for (int u = 0; u < LAG_U; ++u) {
        if (kk[u] < 0) break;
        const float c = (float)(uint32_t)(wv[u] & ((1u << r) - 1u));
        const float sc = sv[u] * c;
#pragma unroll
        for (int b = 0; b < LAG_MAXB; ++b)
          if (b < batch) acc[b] = fmaf(sf_h2f(x[(int64_t)b * k_in + kk[u]]), sc, acc[b]);
      }
    }
    __syncthreads();  // s_k is rewritten by the next round
  }
  if (n < n_out)
#pragma unroll
    for (int b = 0; b < LAG_MAXB; ++b)
      if (b < batch) delta[(int64_t)b * n_out + n] = acc[b];
}

}  // namespace

extern "C" sf_status sf_refine_lag_delta(sf_refine_cache* c, int32_t pool, const sf_qweight* w, const uint16_t* x_f16,
                                         int32_t batch, int32_t k_sel, const int32_t* sel, const int32_t* hit,
                                         float* delta_out, sf_stream stream) {
  SF_REQUIRE(c && w && x_f16 && delta_out, SF_EINVAL, "null argument");
  SF_REQUIRE(pool >= 0 && pool < (int32_t)c->pools.size(), SF_EINVAL, "pool index out of range");
  SF_REQUIRE(batch >= 1 && batch <= LAG_MAXB, SF_EINVAL, "batch must be 1..16");
  SF_REQUIRE(k_sel >= 0 && k_sel <= w->k_in && (k_sel == 0 || (sel && hit)), SF_EINVAL, "bad k_sel / sel / hit");
  SF_REQUIRE(w->fmt.r >= 1 && w->fmt.group == 128 && w->k_in % 128 == 0 && w->n_out > 0, SF_EINVAL, "bad weight");
  const HostPool& p = c->pools[pool];
  SF_REQUIRE(p.d.n_units == w->k_in && p.d.unit_bytes == (int64_t)w->n_out * w->fmt.r / 8 &&
                 ((int64_t)w->n_out * w->fmt.r) % 32 == 0,
             SF_EINVAL, "the pool's units are not this weight's channel-major refinement units");
  const uint8_t* store = p.resident ? p.d.device_store : (p.d.host_store ? p.host_dev : nullptr);
  SF_REQUIRE(store, SF_EUNSUPPORTED, "fetch lag needs a pinned host-RAM (or resident) store, not a store file");
  hipLaunchKernelGGL(lag_delta_kernel, dim3((unsigned)((w->n_out + LAG_T - 1) / LAG_T)), dim3(LAG_T), 0,
                     (hipStream_t)stream, store, p.d.unit_bytes, w->sz, (int)w->n_out,
                     (int)w->k_in, (int)w->fmt.r, x_f16, (int)batch, (int)k_sel, sel, hit, delta_out);
  SF_LAUNCH_CHECK();
  return SF_OK;
}

namespace {

// FP16 fetch: y[b][n] += sum over the selected channels k whose fp16 column is in a
// slot of x[b][k] * (w16[n][k] - resident[n][k]).  A thread per output row; the
// resident code of (n, k) is read from row n of the packed codes.
__global__ __launch_bounds__(LAG_T) void fp16_fetch_kernel(const uint8_t* slots, int64_t unit_bytes,
                                                          const uint8_t* res, const uint32_t* sz, int n_out, int k_in,
                                                          int b, int r, const uint16_t* x, int batch, int k_sel,
                                                          const int32_t* sel, const int32_t* slot, float* y) {
  __shared__ int s_k[LAG_LIST], s_s[LAG_LIST];
  __shared__ int s_n;
  const int tid = threadIdx.x;
  const int n = blockIdx.x * LAG_T + tid;
  const int ngr = k_in / 128;
  const int64_t row_bytes = (int64_t)k_in * b / 8;
  const uint32_t cmask = (1u << b) - 1u;
  float acc[LAG_MAXB];
#pragma unroll
  for (int q = 0; q < LAG_MAXB; ++q) acc[q] = 0.f;
  for (int j0 = 0; j0 < k_sel; j0 += LAG_LIST) {
    const int jn = min(LAG_LIST, k_sel - j0);
    __syncthreads();
    if (tid < 64) {
      int base = 0;
      for (int j = tid; j - tid < jn; j += 64) {
        const int kq = j < jn ? sel[j0 + j] : -1;
        const int sq = j < jn ? slot[j0 + j] : -1;
        const bool on = sq >= 0 && kq >= 0 && kq < k_in;
        const uint64_t m = __ballot(on);
        const int pos = base + __popcll(m & ((1ull << tid) - 1ull));
        if (on) {
          s_k[pos] = kq;
          s_s[pos] = sq;
        }
        base += __popcll(m);
      }
      if (tid == 0) s_n = base;
    }
    __syncthreads();
    const int nl = s_n;
    for (int i0 = 0; i0 < nl; i0 += LAG_U) {
      float dv[LAG_U];
      int kk[LAG_U];
#pragma unroll
      for (int u = 0; u < LAG_U; ++u) {
        kk[u] = i0 + u < nl ? s_k[i0 + u] : -1;
        dv[u] = 0.f;
        if (kk[u] >= 0 && n < n_out) {
          const int k = kk[u];
          const uint16_t w16 = ((const uint16_t*)(slots + (int64_t)s_s[i0 + u] * unit_bytes))[n];
          const int64_t bit = (int64_t)k * b;
          const uint8_t* cp = res + (int64_t)n * row_bytes + (bit >> 3);
          uint32_t cv = cp[0];
          if ((int)(bit & 7) + b > 8) cv |= (uint32_t)cp[1] << 8;
          const uint32_t c = (cv >> (bit & 7)) & cmask;
          const uint32_t w = sz[(int64_t)n * ngr + k / 128];
          const float st = sf_h2f(w & 0xFFFFu) * (float)(1u << r);
          dv[u] = sf_h2f(w16) - fmaf(st, (float)c, sf_h2f(w >> 16));
        }
      }
#pragma unroll
      for (int u = 0; u < LAG_U; ++u) {
        if (kk[u] < 0) break;
#pragma unroll
        for (int q = 0; q < LAG_MAXB; ++q)
          if (q < batch) acc[q] = fmaf(sf_h2f(x[(int64_t)q * k_in + kk[u]]), dv[u], acc[q]);
      }
    }
  }
  if (n < n_out)
#pragma unroll
    for (int q = 0; q < LAG_MAXB; ++q)
      if (q < batch) y[(int64_t)q * n_out + n] += acc[q];
}

}  // namespace

extern "C" sf_status sf_fp16_fetch_delta(sf_refine_cache* c, int32_t pool, const sf_qweight* w, const uint16_t* x_f16,
                                         int32_t batch, int32_t k_sel, const int32_t* sel, const int32_t* slot,
                                         float* y, sf_stream stream) {
  SF_REQUIRE(c && w && x_f16 && y, SF_EINVAL, "null argument");
  SF_REQUIRE(pool >= 0 && pool < (int32_t)c->pools.size(), SF_EINVAL, "pool index out of range");
  SF_REQUIRE(batch >= 1 && batch <= LAG_MAXB, SF_EINVAL, "batch must be 1..16");
  SF_REQUIRE(k_sel >= 0 && k_sel <= w->k_in && (k_sel == 0 || (sel && slot)), SF_EINVAL, "bad k_sel / sel / slot");
  SF_REQUIRE(w->fmt.group == 128 && w->k_in % 128 == 0 && w->n_out > 0 && w->fmt.b >= 1 && w->fmt.b <= 8 &&
                 w->resident && w->sz,
             SF_EINVAL, "bad weight");
  const HostPool& p = c->pools[pool];
  SF_REQUIRE(p.d.n_units == w->k_in && p.d.unit_bytes == 2 * w->n_out, SF_EINVAL,
             "the pool's units are not this weight's fp16 columns (n_units = k_in, unit_bytes = 2 * n_out)");
  if (k_sel == 0 || !p.d_slots) return SF_OK;
  hipLaunchKernelGGL(fp16_fetch_kernel, dim3((unsigned)((w->n_out + LAG_T - 1) / LAG_T)), dim3(LAG_T), 0,
                     (hipStream_t)stream, p.d_slots, p.d.unit_bytes, w->resident, w->sz, (int)w->n_out, (int)w->k_in,
                     (int)w->fmt.b, (int)w->fmt.r, x_f16, (int)batch, (int)k_sel, sel, slot, y);
  SF_LAUNCH_CHECK();
  return SF_OK;
}

extern "C" sf_status sf_refine_cache_io_stats(sf_refine_cache* c, int32_t pool, int64_t* reads, int64_t* bytes,
                                              double* p50_us, double* p99_us, double* read_ms) {
  SF_REQUIRE(c, SF_EINVAL, "null cache");
  SF_REQUIRE(pool < (int32_t)c->pools.size(), SF_EINVAL, "pool index out of range");
  int64_t n = 0, by = 0;
  double ms = 0.0;
  std::vector<float> lat;
  for (int i = 0; i < (int)c->pools.size(); ++i) {
    if (pool >= 0 && i != pool) continue;
    const HostPool& p = c->pools[i];
    n += p.io_reads;
    by += p.io_bytes;
    ms += p.io_ms;
    lat.insert(lat.end(), p.lat_us.begin(), p.lat_us.end());
  }
  double q50 = 0.0, q99 = 0.0;
  if (!lat.empty()) {
    std::sort(lat.begin(), lat.end());
    q50 = lat[(lat.size() - 1) / 2];
    q99 = lat[std::min(lat.size() - 1, (size_t)((double)(lat.size() - 1) * 0.99 + 0.5))];
  }
  if (reads) *reads = n;
  if (bytes) *bytes = by;
  if (p50_us) *p50_us = q50;
  if (p99_us) *p99_us = q99;
  if (read_ms) *read_ms = ms;
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
