// Top-k channel selection inside one workgroup: the channels of largest magnitude
// (max over the batch rows of |x|), ties to the lower channel, written in ascending
// channel order.
//
// Method: rag-lover.com StrataFlux summary, explainer dialogue (解説) -- weight
// refinements are chosen by the magnitude of the input activation.  Readings: one
// selection per GEMV input shared by its batch rows (the key of a channel is the
// largest |x| over the rows), k_sel = ceil(p * n / 100), ties to the lower channel.
//
// Keys are |x| as 15-bit fp16 patterns, which order like the values.  Thread t of NT
// holds channels 8m .. 8m+7 for m = t + NT i (i < MI), two keys per register (word
// 4i + q: channel 8m + 2q in the low half, 8m + 2q + 1 in the high half).  The k-th
// largest key T is found digit by digit from the top (3, 4, 4, 4 bits): in each pass
// every thread counts its keys at or above the 7 or 15 candidate thresholds of the
// next digit and one block reduction gives the totals -- no atomics, so keys that
// crowd a few values cost nothing extra.  Per round i, ballots then place the keys
// above T and the first `need` keys equal to T (lowest channels first) in channel
// order.  Included by the GEMV sources and by the glue kernels that produce a GEMV's
// input and select its channels in the same launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfsel {

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Channel-order prefix of per-channel flags f[q] (this thread's 8 consecutive
// channels of one round) over the workgroup: flags in earlier channels; *total = all.
template <int NW>
__device__ __forceinline__ int flag_prefix(const bool (&f)[8], int* lds, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int below = 0, wtot = 0;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint64_t m = __ballot(f[q]);
    below += lanes_below(m);
    wtot += __popcll(m);
  }
  __syncthreads();
  if (lane == 0) lds[wave] = wtot;
  __syncthreads();
  int base = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = lds[w];
    if (w < wave) base += t;
    sum += t;
  }
  *total = sum;
  return base + below;
}

// Sum over the 64 lanes of a wave (every lane active), by DPP: row-local shifts, then
// row broadcasts, then the last lane's inclusive sum.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_z(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, true);
}
__device__ __forceinline__ uint32_t wave_total(uint32_t u) {
  int v = (int)u;
  v += dpp_z<0x111>(v);
  v += dpp_z<0x112>(v);
  v += dpp_z<0x114>(v);
  v += dpp_z<0x118>(v);
  v += dpp_z<0x142, 0xA>(v);
  v += dpp_z<0x143, 0xC>(v);
  return (uint32_t)__builtin_amdgcn_readlane(v, 63);
}

// Packs the keys of 8 consecutive fp16 values (4 words, two per word) into kw
// (max with what kw holds: call once per batch row).
__device__ __forceinline__ void key_max8(uint32_t* kw4, const uint32_t (&x)[4]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t a = x[q] & 0x7FFF7FFFu;
    kw4[q] = max(kw4[q] & 0xFFFFu, a & 0xFFFFu) | (max(kw4[q] >> 16, a >> 16) << 16);
  }
}

// The ks channels of largest key among channels [0, K) (K a multiple of 8, K <= 8 NT
// MI), ascending, into out[0..ks).  Every thread of the NT-thread workgroup calls it
// with its keys in the layout above (keys of channels >= K are never read).  ks
// must satisfy 0 < ks < K.  Ends with a barrier.
template <int NT, int MI>
__device__ void topk_keys(const uint32_t (&kw)[4 * MI], int K, int ks, int32_t* out) {
  constexpr int NW = NT / 64;
  __shared__ uint32_t red[NW][16];
  __shared__ uint32_t tot[16];
  __shared__ int lds[24];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // T = prefix P grown by one digit per pass; above = keys > the interval of P
  uint32_t P = 0u, above = 0u;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 12 - 4 * pass;       // digit bits [shift, shift + dbits)
    const int nd = pass == 0 ? 8 : 16;     // digit values
    // counts of thresholds v = 1..15, two 16-bit counts per word (a wave counts at
    // most 64 * 8 * MI <= 2048 keys, a workgroup at most 32768)
    uint32_t c[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) c[v] = 0u;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      if (tid + NT * i >= K / 8) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t key = (kw[4 * i + (e >> 1)] >> (16 * (e & 1))) & 0xFFFFu;
#pragma unroll
        for (int v = 1; v < 16; ++v)
          c[v >> 1] += key >= (((P << 4) | (uint32_t)v) << shift) ? (1u << (16 * (v & 1))) : 0u;
      }
    }
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const uint32_t x = wave_total(c[v]);
      if (lane == 0) red[wave][v] = x;
    }
    __syncthreads();
    if (tid < 8) {
      uint32_t x = 0u;
#pragma unroll
      for (int w = 0; w < NW; ++w) x += red[w][tid];
      // unpack: word j holds thresholds 2j (low half; none for j = 0) and 2j + 1
      if (tid > 0) tot[2 * tid - 1] = x & 0xFFFFu;
      tot[2 * tid] = x >> 16;
    }
    __syncthreads();
    // the largest digit whose threshold still has ks keys at or above it
    uint32_t d = 0u, hi = above;
#pragma unroll
    for (int v = 1; v < 16; ++v)
      if (v < nd && tot[v - 1] >= (uint32_t)ks) d = (uint32_t)v;
#pragma unroll
    for (int v = 1; v < 16; ++v)
      if ((uint32_t)v == d + 1u && v < nd) hi = tot[v - 1];
    above = hi;
    P = (P << 4) | d;
    __syncthreads();  // tot read by every thread before the next pass writes it
  }
  const uint32_t T = P;
  int need = ks - (int)above;  // keys equal to T that are taken, lowest channels first
  int written = 0, eq_seen = 0;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    if (NT * 8 * i >= K) break;
    const bool ok = tid + NT * i < K / 8;
    bool gt[8], eq[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = kw[4 * i + q] & 0xFFFFu, hi = kw[4 * i + q] >> 16;
      gt[2 * q] = ok && lo > T;
      gt[2 * q + 1] = ok && hi > T;
      eq[2 * q] = ok && lo == T;
      eq[2 * q + 1] = ok && hi == T;
    }
    int tot_eq;
    int eb = eq_seen + flag_prefix<NW>(eq, lds, &tot_eq);
    bool take[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      take[q] = gt[q] || (eq[q] && eb < need);
      eb += eq[q];
    }
    int tot;
    int pos = written + flag_prefix<NW>(take, lds, &tot);
    const int k0 = 8 * (tid + NT * i);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (take[q]) {
        if (pos < ks) out[pos] = k0 + q;
        ++pos;
      }
    written += tot;
    eq_seen += tot_eq;
  }
  __syncthreads();
}

}  // namespace sfsel
