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
// Control words at the start of every workspace (device memory).
struct WsControl {
  uint32_t sel_state;  // 0 idle, 1 selection in progress, 2 published
  uint32_t done;       // workgroups finished (last one resets the words)
  uint32_t timeout;    // set when a bounded device wait gave up
  uint32_t pad[61];    // keeps the data area 256-byte aligned
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

// Returns the device view of a pool, or a pool that misses everything if c is
// NULL or pool < 0.  Fails with SF_EINVAL for a bad pool index.
sf_status sf_cache_pool_view(sf_refine_cache* c, int32_t pool, PoolDev* out);

// ---- fp16 helpers ------------------------------------------------------------------
__device__ __forceinline__ float sf_h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits16 & 0xFFFFu));
}

// Cross-workgroup hand-off inside one launch.  Data published by one workgroup for
// others is written with agent-scope atomic stores and read with agent-scope
// atomic loads, which are performed at the device coherence point (no L2 writeback
// or invalidation, which on a multi-XCD device would be needed for plain accesses
// and are costly).  The writer waits for its stores to complete (s_waitcnt) and
// passes a workgroup barrier before one thread raises the flag.
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
// Workgroup barrier that orders LDS accesses only: this thread's global loads stay
// in flight (a plain __syncthreads() waits for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// All of this thread's memory operations have completed.
__device__ __forceinline__ void sf_drain() { __builtin_amdgcn_s_waitcnt(0); }

// Bounded spin on a flag raised by another workgroup of the same launch.  Returns
// false if it gave up (after about a second); the caller then skips the work that
// needed the flag.
__device__ __forceinline__ bool sf_wait_word(uint32_t* p, uint32_t want, uint32_t* timeout_flag) {
  for (uint32_t it = 0; it < (1u << 22); ++it) {
    if (sf_get(p) == want) return true;
    __builtin_amdgcn_s_sleep(4);
  }
  sf_put(timeout_flag, 1u);
  return false;
}

// Phase timestamps for performance analysis.  Compiled in only with -DSF_PROBE
// (a separate build); SF_TS(i) records the wall clock of thread 0 of each
// workgroup in slot i (0..15) of that workgroup's row of the probe buffer.
#ifdef SF_PROBE
// one copy of the buffer pointer per translation unit (no relocatable device code),
// in constant memory: a scalar load, which does not wait for the vector loads in flight
static __constant__ long long* sf_probe_buf = nullptr;
void sf_probe_register(void (*install)(long long*));
namespace {
struct SfProbeInstaller {
  static void install(long long* p) { (void)hipMemcpyToSymbol(HIP_SYMBOL(sf_probe_buf), &p, sizeof(p)); }
  SfProbeInstaller() { sf_probe_register(&install); }
};
static SfProbeInstaller sf_probe_installer;
}  // namespace
#define SF_TS(i)                                                                          \
  do {                                                                                    \
    if (threadIdx.x == 0 && sf_probe_buf)                                                 \
      sf_probe_buf[((size_t)blockIdx.y * gridDim.x + blockIdx.x) * 16 + (i)] = wall_clock64(); \
  } while (0)
// the same, recorded by thread t of the workgroup
#define SF_TS_T(i, t)                                                                     \
  do {                                                                                    \
    if (threadIdx.x == (t) && sf_probe_buf)                                               \
      sf_probe_buf[((size_t)blockIdx.y * gridDim.x + blockIdx.x) * 16 + (i)] = wall_clock64(); \
  } while (0)
#else
#define SF_TS(i) ((void)0)
#define SF_TS_T(i, t) ((void)0)
#endif

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
