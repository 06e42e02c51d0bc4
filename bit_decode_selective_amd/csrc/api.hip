// Error reporting, version and workspace management of libstrataflux.
#include <string>

#include <map>
#include <mutex>
#include <tuple>

#include "sf_internal.h"

namespace {
thread_local std::string g_last_error;

__global__ void ws_zero_kernel(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}
}  // namespace

void sf_set_error(const std::string& msg) { g_last_error = msg; }

extern "C" int32_t sf_abi_version(void) { return SF_ABI_VERSION; }

extern "C" const char* sf_last_error(void) { return g_last_error.c_str(); }

extern "C" const char* sf_status_string(sf_status s) {
  switch (s) {
    case SF_OK: return "ok";
    case SF_EINVAL: return "invalid argument";
    case SF_EUNSUPPORTED: return "unsupported";
    case SF_ENOMEM: return "out of memory / buffer too small";
    case SF_EHIP: return "HIP runtime error";
    case SF_ESTATE: return "bad state";
    default: return "unknown status";
  }
}

extern "C" sf_status sf_workspace_create(size_t bytes, sf_workspace** out) {
  SF_REQUIRE(out, SF_EINVAL, "null out");
  *out = nullptr;
  if (bytes < sizeof(WsControl)) bytes = sizeof(WsControl);
  bytes = sf_align256(bytes);
  sf_workspace* w = new sf_workspace();
  hipGetDevice(&w->device);
  hipError_t e = hipMalloc((void**)&w->base, bytes);
  if (e != hipSuccess) {
    delete w;
    sf_set_error(std::string("sf_workspace_create: hipMalloc: ") + hipGetErrorString(e));
    return e == hipErrorOutOfMemory ? SF_ENOMEM : SF_EHIP;
  }
  w->bytes = bytes;
  const int words = (int)(sizeof(WsControl) / 4);
  hipLaunchKernelGGL(ws_zero_kernel, dim3(64), dim3(256), 0, 0, (uint32_t*)w->base, words);
  e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    hipFree(w->base);
    delete w;
    sf_set_error(std::string("sf_workspace_create: ") + hipGetErrorString(e));
    return SF_EHIP;
  }
  *out = w;
  return SF_OK;
}

extern "C" sf_status sf_workspace_destroy(sf_workspace* ws) {
  if (!ws) return SF_OK;
  hipDeviceSynchronize();
  hipFree(ws->base);
  delete ws;
  return SF_OK;
}

extern "C" sf_status sf_workspace_check(sf_workspace* ws) {
  SF_REQUIRE(ws, SF_EINVAL, "null workspace");
  SF_HIP(hipDeviceSynchronize());
  WsControl ctl;
  SF_HIP(hipMemcpy(&ctl, ws->base, sizeof(ctl), hipMemcpyDeviceToHost));
  if (ctl.timeout) {
    // a wait gave up: clear every flag and counter the kernels hand over with (the
    // control block and the per-call words in the data area), keeping the spin limit
    SF_HIP(hipMemset(ws->base, 0, ws->bytes));
    SF_HIP(hipMemcpy(ws->base + offsetof(WsControl, spin_limit), &ctl.spin_limit, 4, hipMemcpyHostToDevice));
    SF_HIP(hipDeviceSynchronize());
    sf_set_error("a device-side wait timed out; the affected rows carry no refinement");
    return SF_ESTATE;
  }
  return SF_OK;
}

extern "C" sf_status sf_workspace_set_spin_limit(sf_workspace* ws, uint32_t polls) {
  SF_REQUIRE(ws, SF_EINVAL, "null workspace");
  SF_HIP(hipDeviceSynchronize());
  SF_HIP(hipMemcpy(ws->base + offsetof(WsControl, spin_limit), &polls, 4, hipMemcpyHostToDevice));
  return SF_OK;
}

int sf_occupancy(const void* kernel, int threads, size_t lds) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, int, size_t>, int> memo;
  int dev = 0;
  (void)hipGetDevice(&dev);
  const auto key = std::make_tuple(dev, kernel, threads, lds);
  {
    std::lock_guard<std::mutex> g(mu);
    auto it = memo.find(key);
    if (it != memo.end()) return it->second;
  }
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, threads, lds) != hipSuccess || occ < 1) {
    (void)hipGetLastError();
    occ = 1;
  }
  std::lock_guard<std::mutex> g(mu);
  memo[key] = occ;
  return occ;
}
