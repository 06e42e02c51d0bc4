// Internal declarations shared by the libstrataflux sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/strataflux.h"

// ---- error reporting -------------------------------------------------------------
void sf_set_error(const std::string& msg);

#define SF_REQUIRE(cond, code, msg)            \
  do {                                         \
    if (!(cond)) {                             \
      sf_set_error(std::string(__func__) + ": " + (msg)); \
      return (code);                           \
    }                                          \
  } while (0)

#define SF_HIP(call)                                                              \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess) {                                                       \
      sf_set_error(std::string(__func__) + ": " #call ": " + hipGetErrorString(e_)); \
      return SF_EHIP;                                                             \
    }                                                                             \
  } while (0)

#define SF_LAUNCH_CHECK() SF_HIP(hipGetLastError())

// ---- workspace -------------------------------------------------------------------
// Control words at the start of every workspace (device memory).  Kernels that hand
// data from one workgroup to another inside a launch keep their flags and counters
// here; every launch leaves them as it found them (zero), and sf_workspace_check
// clears them all after a bounded wait has given up.
struct WsControl {
  uint32_t sel_state;   // 0 idle, 1 selection in progress, 2 published
  uint32_t done;        // workgroups finished (last one resets the words)
  uint32_t timeout;     // set when a bounded device wait gave up
  uint32_t spin_limit;  // polls a bounded wait makes before it gives up (0: 1 << 22)
  uint32_t pad[60];     // keeps the data area 256-byte aligned
  uint32_t row_ctr[1024];  // batched GEMV: slices finished per row block (last one resets)
  // split GEMV: the published selection in SPLIT_COPIES copies (word j = channel,
  // then per matrix word k_sel * (1 + op) + j = slot), valid while sel_flag is
  // raised; per group g = tile mod 64, flag word 32 g and reader count word 32 g
  // (one 128-byte line each, so that no single line takes every tile's requests)
  uint32_t hit[32768];
  uint32_t sel_flag[64 * 32];
  uint32_t rd_ctr[64 * 32];
};

struct sf_workspace {
  uint8_t* base = nullptr;  // device
  size_t bytes = 0;
  int device = 0;
};

// ---- cache (device view used by kernels) ------------------------------------------
struct PoolDev {
  const int32_t* unit2slot;  // [n_units], -1 = absent
  const uint8_t* slots;      // [capacity][unit_bytes]
  int32_t* log_units;        // lookup log: unit ids, in lookup order
  int32_t* log_slots;        // slot seen by each logged lookup (-1 = miss)
  uint32_t* log_count;       // entries used this step
  int32_t log_cap;           // entries available
  int32_t resident;          // every unit u is in slot u (unit2slot is the identity)
  int32_t unit_bytes;
  int64_t n_units;
};

// Resident workgroups per CU of `kernel` at `threads` threads and `lds` bytes of
// dynamic LDS on the current device (at least 1), cached per (device, kernel,
// threads, lds): the query costs microseconds of host time per launch otherwise.
int sf_occupancy(const void* kernel, int threads, size_t lds);

// Returns the device view of a pool, or a pool that misses everything if c is
// NULL or pool < 0.  Fails with SF_EINVAL for a bad pool index.
sf_status sf_cache_pool_view(sf_refine_cache* c, int32_t pool, PoolDev* out);

// Reserves n entries of a pool's lookup log (count word: entries reserved in bits
// 0..30, never more than cap; bit 31 set once a reservation did not fit).  Returns
// the first entry, or -1 if the n entries do not fit (nothing is reserved then, so
// every entry below the count has been written by its reserver).
__device__ __forceinline__ int sf_log_reserve(uint32_t* count, uint32_t n, uint32_t cap) {
  uint32_t old = __hip_atomic_load(count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (;;) {
    const uint32_t used = old & 0x7FFFFFFFu;
    if (used + n > cap) {
      (void)__hip_atomic_fetch_or(count, 0x80000000u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return -1;
    }
    if (__hip_atomic_compare_exchange_weak(count, &old, old + n, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT))
      return (int)used;
  }
}

// ---- fp16 helpers ------------------------------------------------------------------
__device__ __forceinline__ float sf_h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits16 & 0xFFFFu));
}

// Cross-workgroup hand-off inside one launch.  Data published by one workgroup for
// others is written with agent-scope atomic stores and read with agent-scope atomic
// loads, which are performed at the device coherence point (no L2 writeback or
// invalidation of the data itself).  The flag that announces the data is a release
// store after the data stores, and the reader's poll of the flag is an acquire
// load: the memory model then orders the data before the flag for any reader that
// sees the flag.
__device__ __forceinline__ void sf_put(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void sf_put(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void sf_put(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t sf_get(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t sf_get(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float sf_get(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// flag store that releases this thread's earlier stores, and the matching acquire poll
__device__ __forceinline__ void sf_put_release(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t sf_get_acquire(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
// counter increment that releases this thread's earlier stores (a workgroup's
// contribution is complete once its thread 0 counts it after a barrier)
__device__ __forceinline__ uint32_t sf_add_release(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t sf_add_acq_rel(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup barrier that orders LDS accesses only: this thread's global loads stay
// in flight (a plain __syncthreads() waits for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// All of this thread's memory operations have completed.
__device__ __forceinline__ void sf_drain() { __builtin_amdgcn_s_waitcnt(0); }

// Polls a bounded wait makes before it gives up: the workspace's spin-limit word,
// which follows its timeout word (0 means 1 << 22, about a second).
__device__ __forceinline__ uint32_t sf_spin_limit(const uint32_t* timeout_flag) {
  const uint32_t v = __hip_atomic_load(timeout_flag + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v ? v : (1u << 22);
}

// Bounded spin on a word raised by another workgroup of the same launch (acquire:
// what the other workgroup stored before it raised the word is visible after a
// true return).  Returns false if it gave up; the caller then skips the work that
// needed the word and the timeout flag reports it.
__device__ __forceinline__ bool sf_wait_word(uint32_t* p, uint32_t want, uint32_t* timeout_flag) {
  const uint32_t lim = sf_spin_limit(timeout_flag);
  for (uint32_t it = 0; it < lim; ++it) {
    if (sf_get(p) == want) {
      (void)sf_get_acquire(p);
      return true;
    }
    __builtin_amdgcn_s_sleep(4);
  }
  sf_put(timeout_flag, 1u);
  return false;
}

// Inclusive prefix sum over the 64 lanes of a wave by DPP: row-local Hillis-Steele
// steps (row_shr 1, 2, 4, 8 with zeros shifted in), then rows 1 and 3 add the totals
// of rows 0 and 2 (row_bcast15) and rows 2 and 3 the total of rows 0-1 (row_bcast31).
// Every lane must be active.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int sf_dpp_z(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, true);
}
__device__ __forceinline__ int sf_wave_incl_scan(int v) {
  v += sf_dpp_z<0x111>(v);
  v += sf_dpp_z<0x112>(v);
  v += sf_dpp_z<0x114>(v);
  v += sf_dpp_z<0x118>(v);
  v += sf_dpp_z<0x142, 0xA>(v);
  v += sf_dpp_z<0x143, 0xC>(v);
  return v;
}

static inline size_t sf_align256(size_t v) { return (v + 255) & ~size_t(255); }
