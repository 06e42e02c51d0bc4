// Workgroup-wide helpers for 256-thread workgroups (4 waves of 64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Exclusive prefix sum over the 256 threads of a workgroup, thread order.
// `lds` needs 4 ints.  Returns the exclusive prefix; *total receives the sum.
__device__ __forceinline__ int wg_exclusive_scan(int v, int* lds, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) lds[wave] = incl;
  __syncthreads();
  int base = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int t = lds[w];
    if (w < wave) base += t;
    sum += t;
  }
  __syncthreads();
  *total = sum;
  return base + incl - v;
}

// Suffix sums of a 256-entry histogram held in LDS (in place: h[i] = sum h[j>=i]).
__device__ __forceinline__ void wg_suffix_sum256(uint32_t* h, int* lds4) {
  const int t = threadIdx.x;
  // thread t takes bin 255 - t so a forward scan gives suffix sums
  int v = (int)h[255 - t];
  int total;
  const int ex = wg_exclusive_scan(v, lds4, &total);
  h[255 - t] = (uint32_t)(ex + v);
  __syncthreads();
}

// Largest index i in [0, n) with h[i] >= need, for non-increasing suffix sums h
// (h[0] >= need is required).  Every thread gets the answer.
__device__ __forceinline__ int wg_find_threshold(const uint32_t* h, int n, uint32_t need, int* lds1) {
  const int t = threadIdx.x;
  if (t == 0) *lds1 = 0;
  __syncthreads();
  for (int i = t; i < n; i += 256) {
    const bool here = h[i] >= need && (i + 1 == n || h[i + 1] < need);
    if (here) *lds1 = i;
  }
  __syncthreads();
  const int r = *lds1;
  __syncthreads();
  return r;
}
