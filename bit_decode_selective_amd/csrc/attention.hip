// Refined GQA decode attention over a nested low-bit KV cache.
//
// Method: rag-lover.com StrataFlux summary, explainer dialogue (解説) -- the KV
// cache is resident in low-bit form; the tokens that get refinement bits are
// chosen by the attention weight computed from the low-bit keys; limitations
// section -- a token whose refinement is missing keeps resident precision.
// Readings: one selection per (batch, kv head) with score = softmax weight summed
// over the kv head's query heads; for selected tokens that hit, both key and value
// use the (b+r)-bit value; the output softmax runs over all tokens after that.
//
// Three launches per call:
//   qk     : streams the resident keys (T split over workgroups), logits of the G
//            query heads of each KV head on MFMA (codes expanded into fp16
//            mantissas, value 1 + c/2^b, times q), per-split softmax max / sum;
//   select : merges the split statistics, forms the selection scores, builds a
//            2048-bin histogram of their bit patterns (many workgroups); the last
//            workgroup of each KV head finishes an exact radix select (ties to the
//            lower token), compacts the selection in token order, looks it up in
//            the refinement cache and overwrites the logits of the hit tokens with
//            their refined values l' = l + scale * s_K * (q . cK_lo);
//   pv     : streams the resident values with the final weights exp(l - m'),
//            adds s_V * cV_lo for the hit tokens of its split, and the last
//            workgroup of each KV head merges the split sums into the output.
// All weights are positive and final before they are accumulated, so fp32 sums
// carry no cancellation.
#include "block_scan.h"
#include "sf_internal.h"

namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int HD = 128;       // head dim
constexpr int SPLIT2 = 4096;  // tokens per select workgroup
constexpr int SEL_T = 1024;   // threads of a select workgroup
constexpr int SPR = 32;       // scores per thread per round in the finishing workgroup
constexpr int NBINS = 2048;   // first-level radix bins (top 11 bits of the score)

// qk: 16-token MFMA tiles; each wave loads TPW tiles up front
__host__ __device__ constexpr int qk_tpw(int b) { return b <= 2 ? 8 : (b == 4 ? 8 : 4); }
__host__ __device__ constexpr int qk_split(int b) { return 4 * 16 * qk_tpw(b); }
// pv: tokens per workgroup, their codes staged in LDS (16 KB)
__host__ __device__ constexpr int pv_split(int b) { return 1024 / b; }

__device__ __forceinline__ uint32_t field(const uint32_t* w, int bit, int width) {
  const int wi = bit >> 5, off = bit & 31;
  uint32_t v = w[wi] >> off;
  if (off + width > 32) v |= w[wi + 1] << (32 - off);
  return v & ((1u << width) - 1u);
}

__device__ __forceinline__ float h2f16(uint16_t bits) { return (float)__builtin_bit_cast(_Float16, bits); }

struct AttnArgs {
  const uint16_t* q;  // [batch][n_q][HD] fp16 bits
  const uint8_t* k_res;
  const uint32_t* k_sz;
  const uint8_t* v_res;
  const uint32_t* v_sz;
  int batch, n_q, n_kv, G, T, t_cap, b, r, k_sel, s1, s2, s3;
  float scale;
  float* logits;    // [batch*n_q][T]
  float* scores;    // [batch*n_kv][T rounded up to 4]
  float* k1part;    // [bh][s1][G][2]: split max, split sum of exp
  uint32_t* hist;   // [bh][NBINS]
  uint32_t* cnt;    // [bh][2]: select, pv workgroups done
  int32_t* sel;     // [bh][KS]
  int32_t* hit_t;   // [bh][KS]
  int32_t* hit_s;   // [bh][KS]
  int32_t* n_hit;   // [bh]
  float* mref;      // [bh][G]: max logit after refinement
  float* k3part;    // [bh][s3][G][1 + HD]
  const int32_t* sel_in;
  int32_t* sel_out;
  int32_t* hit_out;
  float* out;       // [batch][n_q][HD]
  PoolDev pool;
};

// ---- block helpers (256 threads) ------------------------------------------------
__device__ __forceinline__ float wg_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ float wg_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Suffix sums in place over n bins (n a multiple of 256) held in LDS.
__device__ void wg_suffix_sum(uint32_t* h, int n, int* lds4) {
  const int per = n / 256, t = threadIdx.x;
  const int hi = n - per * t;  // this thread sums bins [hi - per, hi)
  int s = 0;
  for (int i = hi - 1; i >= hi - per; --i) s += (int)h[i];
  int tot;
  int run = wg_exclusive_scan(s, lds4, &tot);
  for (int i = hi - 1; i >= hi - per; --i) {
    run += (int)h[i];
    h[i] = (uint32_t)run;
  }
  __syncthreads();
}

// ---- qk: logits + per-split softmax statistics -----------------------------------
template <int B, int G>
__global__ __launch_bounds__(256) void attn_qk_kernel(AttnArgs a) {
  __shared__ float st[4][16][2];
  __shared__ uint32_t s_ksz[qk_split(B)];
  constexpr int P = 32 / B, HP = P / 2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x, bh = blockIdx.y;
  const int bi = bh / a.n_kv, kvh = bh - bi * a.n_kv;
  const int T = a.T;
  constexpr int TPW = qk_tpw(B);
  const int t_begin = split * qk_split(B), t_end = min(T, t_begin + qk_split(B));

  // this call's selection histogram and counters start at zero
  for (int i = split * 256 + tid; i < NBINS; i += a.s1 * 256) a.hist[(size_t)bh * NBINS + i] = 0;
  if (split == 0 && tid < 2) a.cnt[bh * 2 + tid] = 0;

  // B operand: q of head n = lane % 16 (zero for n >= G) over the 32 dims of lane
  // group qg = lane / 16, in the same pair order as the key codes
  const int n = lane & 15, qg = lane >> 4;
  const uint16_t* qrow = a.q + ((size_t)bi * a.n_q + (size_t)kvh * G + (n < G ? n : 0)) * HD;
  uint16_t q32[32];
  {
    const u32x4* qv = (const u32x4*)(qrow + 32 * qg);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 v = qv[i];
      const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) q32[8 * i + e] = (uint16_t)(wds[e >> 1] >> (16 * (e & 1)));
    }
  }
  h8_t bq[4];
  float qpart = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int p = 4 * j + (e >> 1), h = e & 1;
      const int w = p / HP, i = p % HP;
      const float v = n < G ? h2f16(q32[P * w + i + h * HP]) : 0.f;
      bq[j][e] = (_Float16)v;
      qpart += v;
    }
  qpart += __shfl_xor(qpart, 16, 64);
  qpart += __shfl_xor(qpart, 32, 64);
  const float qsum = qpart;  // sum of q_n over all 128 dims

  const size_t tok0 = (size_t)bh * a.t_cap;
  const float scl = (float)(1u << (a.r + B));
  constexpr uint32_t m1 = ((1u << B) - 1u) << (10 - B);
  float run_m = -INFINITY, run_z = 0.f;
  SF_TS(0);
  for (int i = tid; i < t_end - t_begin; i += 256) s_ksz[i] = a.k_sz[tok0 + t_begin + i];
  // each wave: TPW tiles of 16 tokens, all loads issued first
  const int tw = t_begin + wave * 16 * TPW;
  uint32_t wv[TPW][B];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int tm = tw + 16 * u + (lane & 15);
    if (tm < t_end) {
      const uint32_t* src = (const uint32_t*)(a.k_res + (tok0 + tm) * (HD * B / 8)) + qg * B;
      if constexpr (B == 1) {
        wv[u][0] = __builtin_nontemporal_load(src);
      } else if constexpr (B == 2) {
        const u32x2 v = __builtin_nontemporal_load((const u32x2*)src);
        wv[u][0] = v.x; wv[u][1] = v.y;
      } else {
#pragma unroll
        for (int q4 = 0; q4 < B / 4; ++q4) {
          const u32x4 v = __builtin_nontemporal_load((const u32x4*)src + q4);
          wv[u][4 * q4] = v.x; wv[u][4 * q4 + 1] = v.y; wv[u][4 * q4 + 2] = v.z; wv[u][4 * q4 + 3] = v.w;
        }
      }
    } else {
#pragma unroll
      for (int w = 0; w < B; ++w) wv[u][w] = 0;
    }
  }
  __syncthreads();  // s_ksz
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    if (tw + 16 * u >= t_end) break;
    f4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t pr[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int p = 4 * j + v, w = p / HP, i = p % HP;
        const int sh = (10 - B) - i * B;
        const uint32_t t = sh >= 0 ? (wv[u][w] << sh) : (wv[u][w] >> (-sh));
        pr[v] = (t & (m1 | (m1 << 16))) | 0x3C003C00u;
      }
      const u32x4 pv = {pr[0], pr[1], pr[2], pr[3]};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, pv), bq[j], acc, 0, 0, 0);
    }
    if (n < G) {
      const int tb = tw + 16 * u + 4 * qg;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = tb + v;
        if (t < t_end) {
          const uint32_t szw = s_ksz[t - t_begin];
          const float s = sf_h2f(szw), z = sf_h2f(szw >> 16);
          const float l = a.scale * (z * qsum + (s * scl) * (acc[v] - qsum));
          a.logits[((size_t)bi * a.n_q + kvh * G + n) * T + t] = l;
          const float nm = fmaxf(run_m, l);
          run_z = run_z * __expf(run_m - nm) + __expf(l - nm);
          run_m = nm;
        }
      }
    }
  }
  SF_TS(1);
  // combine (m, z) over the 4 lane groups of each head, then over the waves
#pragma unroll
  for (int o = 16; o <= 32; o <<= 1) {
    const float om = __shfl_xor(run_m, o, 64), oz = __shfl_xor(run_z, o, 64);
    const float nm = fmaxf(run_m, om);
    run_z = (run_m > -INFINITY ? run_z * __expf(run_m - nm) : 0.f) + (om > -INFINITY ? oz * __expf(om - nm) : 0.f);
    run_m = nm;
  }
  if (lane < 16) {
    st[wave][lane][0] = run_m;
    st[wave][lane][1] = run_z;
  }
  __syncthreads();
  if (tid < G) {
    float m = -INFINITY;
    for (int w = 0; w < 4; ++w) m = fmaxf(m, st[w][tid][0]);
    float z = 0.f;
    for (int w = 0; w < 4; ++w)
      if (st[w][tid][0] > -INFINITY) z += st[w][tid][1] * __expf(st[w][tid][0] - m);
    float* P2 = a.k1part + (((size_t)bh * a.s1 + split) * G + tid) * 2;
    P2[0] = m;
    P2[1] = z;
  }
}

// ---- select ------------------------------------------------------------------------
// q_h . cK_lo for one head, cK_lo = the HD r-bit K refinement codes at the start of
// a KV unit (16-byte aligned); r = 1 and 2 keep the unit's words in registers.
template <int R>
__device__ __forceinline__ float kref_dot_r(const uint8_t* unit, const float* qh) {
  constexpr int NW = HD * R / 32;
  uint32_t w[NW];
  const u32x4* u4 = (const u32x4*)unit;
#pragma unroll
  for (int i = 0; i < NW / 4; ++i) {
    const u32x4 v = u4[i];
    w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
  }
  float dot = 0.f;
#pragma unroll
  for (int i = 0; i < HD; ++i) dot = fmaf(qh[i], (float)((w[(i * R) >> 5] >> ((i * R) & 31)) & ((1u << R) - 1u)), dot);
  return dot;
}

__device__ __forceinline__ float kref_dot(const uint8_t* unit, int r, const float* qh) {
  if (r == 2) return kref_dot_r<2>(unit, qh);
  if (r == 1) return kref_dot_r<1>(unit, qh);
  const uint32_t* w = (const uint32_t*)unit;
  float dot = 0.f;
  for (int i = 0; i < HD; ++i) dot = fmaf(qh[i], (float)field(w, i * r, r), dot);
  return dot;
}

__device__ __forceinline__ float wgN_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float m = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) m = fmaxf(m, red[w]);
  return m;
}

__device__ __forceinline__ float wgN_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float m = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) m += red[w];
  return m;
}

__device__ __forceinline__ int wgN_exclusive_scan(int v, int* lds, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  __syncthreads();
  if (lane == 63) lds[wave] = incl;
  __syncthreads();
  int base = 0, sum = 0;
  for (int w = 0; w < nw; ++w) {
    const int t = lds[w];
    if (w < wave) base += t;
    sum += t;
  }
  *total = sum;
  return base + incl - v;
}

// Suffix sums over NBINS bins with SEL_T threads (2 bins each), then the largest
// bin whose suffix count is >= need; *above = suffix count of the next bin.
__device__ int sel_threshold_bin(uint32_t* h, int nb, int need, int* lds, int* above) {
  const int t = threadIdx.x;
  const int i0 = NBINS - 1 - 2 * t, i1 = i0 - 1;
  const int v0 = (int)h[i0], v1 = (int)h[i1];
  int tot;
  const int ex = wgN_exclusive_scan(v0 + v1, lds, &tot);
  __syncthreads();
  h[i0] = (uint32_t)(ex + v0);
  h[i1] = (uint32_t)(ex + v0 + v1);
  if (t == 0) lds[40] = 0;
  __syncthreads();
  for (int i = t; i < nb; i += SEL_T)
    if ((int)h[i] >= need && (i + 1 == nb || (int)h[i + 1] < need)) lds[40] = i;
  __syncthreads();
  const int bin = lds[40];
  *above = bin + 1 < nb ? (int)h[bin + 1] : 0;
  __syncthreads();
  return bin;
}

template <int G>
__global__ __launch_bounds__(SEL_T) void attn_select_kernel(AttnArgs a) {
  __shared__ uint32_t lh[NBINS];
  __shared__ float s_m[G], s_iz[G], s_mref[G];
  __shared__ float red[16];
  __shared__ int lds[48];
  __shared__ float qf[G][HD];
  const int tid = threadIdx.x;
  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int bi = bh / a.n_kv, kvh = bh - bi * a.n_kv;
  const int T = a.T, ks = a.k_sel;
  const int KS = ks > 0 ? ks : 1;

  SF_TS(4);
  // global softmax statistics of the resident logits: split partials -> LDS,
  // then one thread per head combines them
  {
    float* pm = (float*)lh;  // reuse the histogram area: [G][s1] max, then sums
    const int n = G * a.s1;
    for (int i = tid; i < n && i < NBINS / 2; i += SEL_T) {
      const float* P2 = a.k1part + ((size_t)bh * a.s1 * G + i) * 2;  // (split, head) order
      pm[i] = P2[0];
      pm[NBINS / 2 + i] = P2[1];
    }
    __syncthreads();
    if (tid < G) {
      float m = -INFINITY;
      for (int sp = 0; sp < a.s1; ++sp) m = fmaxf(m, pm[sp * G + tid]);
      float z = 0.f;
      for (int sp = 0; sp < a.s1; ++sp) {
        const float ms = pm[sp * G + tid];
        if (ms > -INFINITY) z += pm[NBINS / 2 + sp * G + tid] * __expf(ms - m);
      }
      s_m[tid] = m;
      s_iz[tid] = 1.f / z;
    }
    __syncthreads();
  }

  if (ks == 0) {
    if (chunk == 0 && tid < G) a.mref[bh * G + tid] = s_m[tid];
    if (chunk == 0 && tid == 0) a.n_hit[bh] = 0;
    return;
  }

  int* sel = a.sel + (size_t)bh * KS;
  float* sc = a.scores + (size_t)bh * ((T + 3) & ~3);  // rows padded to 16 bytes
  if (a.sel_in == nullptr) {
    SF_TS(5);
    // scores of this chunk + first-level histogram
    for (int i = tid; i < NBINS; i += SEL_T) lh[i] = 0;
    __syncthreads();
    const int c0 = chunk * SPLIT2, c1 = min(T, c0 + SPLIT2);
    for (int t = c0 + tid; t < c1; t += SEL_T) {
      float v = 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h)
        v += expf(a.logits[((size_t)bi * a.n_q + kvh * G + h) * T + t] - s_m[h]) * s_iz[h];
      sf_put(sc + t, v);
      atomicAdd(&lh[__float_as_uint(v) >> 21], 1u);
    }
    __syncthreads();
    for (int i = tid; i < NBINS; i += SEL_T)
      if (lh[i]) atomicAdd(&a.hist[(size_t)bh * NBINS + i], lh[i]);
    sf_drain();
    __syncthreads();
    if (tid == 0)
      lds[44] = __hip_atomic_fetch_add(&a.cnt[bh * 2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                (uint32_t)(a.s2 - 1);
    __syncthreads();
    SF_TS(6);
    if (!lds[44]) return;

    // ---- last workgroup of this KV head: exact threshold by radix select ----
    // thread t holds tokens [round*SEL_T*SPR + t*SPR, +SPR) of each round
    const int rounds = (T + SEL_T * SPR - 1) / (SEL_T * SPR);
    float sv[SPR];
#define SF_LOAD_ROUND(rd)                                                                 \
  do {                                                                                    \
    const int base_ = (rd) * SEL_T * SPR + tid * SPR;                                     \
    _Pragma("unroll") for (int i_ = 0; i_ < SPR; i_ += 4) {                               \
      _Pragma("unroll") for (int e_ = 0; e_ < 4; ++e_) sv[i_ + e_] = base_ + i_ + e_ < T ? sf_get(sc + base_ + i_ + e_) : -1.f; \
    }                                                                                     \
  } while (0)
    for (int i = tid; i < NBINS; i += SEL_T) lh[i] = sf_get(a.hist + (size_t)bh * NBINS + i);
    __syncthreads();
    int above;
    uint32_t prefix;
    int need = ks;
    {
      const int bin = sel_threshold_bin(lh, NBINS, need, lds, &above);
      need -= above;
      prefix = (uint32_t)bin << 21;
    }
    if (rounds == 1) SF_LOAD_ROUND(0);
    for (int level = 0; level < 2; ++level) {
      const int sh = level == 0 ? 10 : 0, nb = level == 0 ? 2048 : 1024;
      const uint32_t pmask = level == 0 ? 0xFFE00000u : 0xFFFFFC00u;
      for (int i = tid; i < NBINS; i += SEL_T) lh[i] = 0;
      __syncthreads();
      for (int rd = 0; rd < rounds; ++rd) {
        if (rounds > 1) SF_LOAD_ROUND(rd);
#pragma unroll
        for (int i = 0; i < SPR; ++i) {
          const uint32_t key = __float_as_uint(sv[i]);
          if (sv[i] >= 0.f && (key & pmask) == prefix) atomicAdd(&lh[(key >> sh) & (uint32_t)(nb - 1)], 1u);
        }
      }
      __syncthreads();
      const int bin = sel_threshold_bin(lh, nb, need, lds, &above);
      need -= above;
      prefix |= (uint32_t)bin << sh;
    }
    SF_TS(7);
    const uint32_t thr = prefix;
    // ordered compaction, round by round
    int written = 0, eq_seen_total = 0;
    for (int rd = 0; rd < rounds; ++rd) {
      if (rounds > 1) SF_LOAD_ROUND(rd);
      int gt = 0, eq = 0;
#pragma unroll
      for (int i = 0; i < SPR; ++i) {
        const uint32_t key = __float_as_uint(sv[i]);
        const bool valid = sv[i] >= 0.f;
        gt += valid && key > thr;
        eq += valid && key == thr;
      }
      int tot_eq, tot;
      const int eq_before = eq_seen_total + wgN_exclusive_scan(eq, lds, &tot_eq);
      const int take_eq = max(0, min(eq, need - eq_before));
      int off = written + wgN_exclusive_scan(gt + take_eq, lds, &tot);
      int seen = 0;
      const int base = rd * SEL_T * SPR + tid * SPR;
#pragma unroll
      for (int i = 0; i < SPR; ++i) {
        const uint32_t key = __float_as_uint(sv[i]);
        if (!(sv[i] >= 0.f)) continue;
        if (key > thr) {
          sel[off++] = base + i;
        } else if (key == thr) {
          if (seen < take_eq) sel[off++] = base + i;
          ++seen;
        }
      }
      written += tot;
      eq_seen_total += tot_eq;
    }
#undef SF_LOAD_ROUND
  } else {
    if (chunk != 0) return;
    for (int j = tid; j < ks; j += SEL_T) sel[j] = a.sel_in[(size_t)bh * ks + j];
  }
  // sel[] is read back by other threads of this workgroup
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");

  SF_TS(8);
  // ---- lookup in selection order ----
  const size_t unit0 = (size_t)bh * a.t_cap;
  const int r = a.r;
  (void)r;
  int* hit_t = a.hit_t + (size_t)bh * KS;
  int* hit_s = a.hit_s + (size_t)bh * KS;
  if (tid == 0) {
    int base = -1;
    if (a.pool.log_count) {
      const uint32_t bse = atomicAdd(a.pool.log_count, (uint32_t)ks);
      base = (bse + (uint32_t)ks <= (uint32_t)a.pool.log_cap) ? (int)bse : -1;
    }
    lds[45] = base;
  }
  __syncthreads();
  const int base = lds[45];
  const int jpt = (ks + SEL_T - 1) / SEL_T;
  const int j0 = tid * jpt, j1 = min(ks, j0 + jpt);
  int nh = 0;
  for (int j = j0; j < j1; ++j) {
    const int t = sel[j];
    const int slot = (a.pool.unit2slot && t >= 0 && t < T) ? a.pool.unit2slot[unit0 + t] : -1;
    nh += slot >= 0;
  }
  int n_hits;
  int pos = wgN_exclusive_scan(nh, lds, &n_hits);
  for (int j = j0; j < j1; ++j) {
    const int t = sel[j];
    const bool ok = t >= 0 && t < T;
    const int slot = (a.pool.unit2slot && ok) ? a.pool.unit2slot[unit0 + t] : -1;
    if (a.sel_out) a.sel_out[(size_t)bh * ks + j] = t;
    if (a.hit_out) a.hit_out[(size_t)bh * ks + j] = slot;
    if (base >= 0) {
      a.pool.log_units[base + j] = ok ? (int)(unit0 + t) : -1;
      a.pool.log_slots[base + j] = slot;
    }
    if (slot >= 0) {
      hit_t[pos] = t;
      hit_s[pos] = slot;
      ++pos;
    }
  }
  for (int i = tid; i < G * HD; i += SEL_T) {
    const int h = i / HD, d = i - h * HD;
    qf[h][d] = h2f16(a.q[((size_t)bi * a.n_q + kvh * G + h) * HD + d]);
  }
  if (tid < G) s_mref[tid] = s_m[tid];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  SF_TS(9);
  // ---- refined logits of the hit tokens: l' = l + scale * s_K * (q . cK_lo) ----
  float mloc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) mloc[h] = -INFINITY;
  for (int m = tid; m < n_hits * G; m += SEL_T) {
    const int hh = m % G, mi = m / G;
    const int t = hit_t[mi];
    const float dot = kref_dot(a.pool.slots + (size_t)hit_s[mi] * a.pool.unit_bytes, a.r, qf[hh]);
    const float s = sf_h2f(a.k_sz[unit0 + t]);
    float* lp = a.logits + ((size_t)bi * a.n_q + kvh * G + hh) * T + t;
    const float l2 = *lp + a.scale * (s * dot);
    *lp = l2;
#pragma unroll
    for (int h = 0; h < G; ++h)
      if (h == hh) mloc[h] = fmaxf(mloc[h], l2);
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float v = wgN_max(mloc[h], red);
    if (tid == 0) s_mref[h] = fmaxf(s_mref[h], v);
  }
  __syncthreads();
  if (tid < G) a.mref[bh * G + tid] = s_mref[tid];
  if (tid == 0) a.n_hit[bh] = n_hits;
  SF_TS(10);
}

// ---- pv: weighted value sums with the final weights ------------------------------
template <int B, int G>
__global__ __launch_bounds__(256) void attn_pv_kernel(AttnArgs a) {
  constexpr int SPLIT3 = pv_split(B);
  constexpr int WPT = HD * B / 32;  // code words per token
  __shared__ float w[G][SPLIT3];
  __shared__ uint32_t s_vsz[SPLIT3];
  __shared__ uint32_t s_code[SPLIT3 * WPT];
  __shared__ float accr[4][G][HD];
  __shared__ float red[4];
  __shared__ float s_z[G], s_zz[G], s_m[G];
  __shared__ int flag;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x, bh = blockIdx.y;
  const int bi = bh / a.n_kv, kvh = bh - bi * a.n_kv;
  const int T = a.T;
  const int t_begin = split * SPLIT3, t_end = min(T, t_begin + SPLIT3);
  const int n_here = max(0, t_end - t_begin);
  const size_t tok0 = (size_t)bh * a.t_cap;
  SF_TS(11);
  // stage this split's value codes (16-byte loads) and scale words
  {
    const u32x4* src = (const u32x4*)(a.v_res + (tok0 + t_begin) * (HD * B / 8));
    const int nv = n_here * WPT / 4;
    for (int i = tid; i < nv; i += 256) {
      const u32x4 v = __builtin_nontemporal_load(src + i);
      s_code[4 * i] = v.x; s_code[4 * i + 1] = v.y; s_code[4 * i + 2] = v.z; s_code[4 * i + 3] = v.w;
    }
  }
  if (tid < G) s_m[tid] = a.mref[bh * G + tid];
  __syncthreads();
  // weights, their sum, and the sum of weight * zero-point per head
  float zs[G], zz[G];
#pragma unroll
  for (int h = 0; h < G; ++h) zs[h] = zz[h] = 0.f;
  for (int tl = tid; tl < n_here; tl += 256) {
    const int t = t_begin + tl;
    const uint32_t vsz = a.v_sz[tok0 + t];
    s_vsz[tl] = vsz;
    const float zv = sf_h2f(vsz >> 16);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float e = __expf(a.logits[((size_t)bi * a.n_q + kvh * G + h) * T + t] - s_m[h]);
      w[h][tl] = e;
      zs[h] += e;
      zz[h] = fmaf(e, zv, zz[h]);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float v1 = wg_sum(zs[h], red);
    if (tid == 0) s_z[h] = v1;
    const float v2 = wg_sum(zz[h], red);
    if (tid == 0) s_zz[h] = v2;
  }
  __syncthreads();
  SF_TS(12);
  // sum_t (w_t * s'_t) * c_t[d]; lane owns dims 2*lane, 2*lane+1; wave w takes tokens w, w+4, ...
  float acc0[G], acc1[G];
#pragma unroll
  for (int h = 0; h < G; ++h) acc0[h] = acc1[h] = 0.f;
  const float sres = (float)(1u << a.r);
  const int bit0 = 2 * lane * B;
#pragma unroll 4
  for (int tl = wave; tl < n_here; tl += 4) {
    const uint32_t word = s_code[tl * WPT + (bit0 >> 5)];
    const float sv = sf_h2f(s_vsz[tl]) * sres;
    const float c0 = (float)((word >> (bit0 & 31)) & ((1u << B) - 1u));
    const float c1 = (float)((word >> ((bit0 & 31) + B)) & ((1u << B) - 1u));
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float we = w[h][tl] * sv;
      acc0[h] = fmaf(we, c0, acc0[h]);
      acc1[h] = fmaf(we, c1, acc1[h]);
    }
  }
  // refinement of the hit tokens that fall in this split: + w * s_V * cV_lo
  if (wave == 0 && a.k_sel > 0) {
    const int nh = a.n_hit[bh];
    const int KS = a.k_sel;
    const int* hit_t = a.hit_t + (size_t)bh * KS;
    const int* hit_s = a.hit_s + (size_t)bh * KS;
    const int r = a.r;
    int lo = 0, hi = nh;  // first hit with token >= t_begin (hit tokens ascend)
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (hit_t[mid] < t_begin) lo = mid + 1; else hi = mid;
    }
    for (int m = lo; m < nh; ++m) {
      const int t = hit_t[m];
      if (t >= t_end) break;
      const uint32_t* unit = (const uint32_t*)(a.pool.slots + (size_t)hit_s[m] * a.pool.unit_bytes);
      const float sv = sf_h2f(s_vsz[t - t_begin]);
      const float c0 = (float)field(unit, HD * r + 2 * lane * r, r);
      const float c1 = (float)field(unit, HD * r + (2 * lane + 1) * r, r);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float we = w[h][t - t_begin] * sv;
        acc0[h] = fmaf(we, c0, acc0[h]);
        acc1[h] = fmaf(we, c1, acc1[h]);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    accr[wave][h][2 * lane] = acc0[h];
    accr[wave][h][2 * lane + 1] = acc1[h];
  }
  __syncthreads();
  float* P3 = a.k3part + (((size_t)bh * a.s3 + split) * G) * (1 + HD);
  for (int i = tid; i < G * HD; i += 256) {
    const int h = i / HD, d = i - h * HD;
    sf_put(P3 + h * (1 + HD) + 1 + d, ((accr[0][h][d] + accr[1][h][d]) + (accr[2][h][d] + accr[3][h][d])) + s_zz[h]);
  }
  if (tid < G) sf_put(P3 + tid * (1 + HD), s_z[tid]);
  SF_TS(13);
  // last workgroup of this KV head: out = sum_s N_s / sum_s Z_s
  sf_drain();
  __syncthreads();
  if (tid == 0)
    flag = __hip_atomic_fetch_add(&a.cnt[bh * 2 + 1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           (uint32_t)(a.s3 - 1);
  __syncthreads();
  if (!flag) return;
  SF_TS(14);
  const float* Pb = a.k3part + (size_t)bh * a.s3 * G * (1 + HD);
  for (int i = tid; i < G * HD; i += 256) {
    const int h = i / HD, d = i - h * HD;
    float num = 0.f, den = 0.f;
#pragma unroll 8
    for (int s = 0; s < a.s3; ++s) {
      num += sf_get(Pb + (s * G + h) * (1 + HD) + 1 + d);
      den += sf_get(Pb + (s * G + h) * (1 + HD));
    }
    a.out[((size_t)bi * a.n_q + kvh * G + h) * HD + d] = num / den;
  }
  SF_TS(15);
}

size_t attn_layout(int batch, int n_q, int n_kv, int T, int k_sel, size_t off[12]) {
  const int G = n_kv > 0 ? n_q / n_kv : 1;
  const int bh = batch * n_kv;
  const size_t s1 = (T + 255) / 256, s3 = (T + 127) / 128;  // bounds for every b
  const size_t KS = k_sel > 0 ? k_sel : 1;
  const size_t sizes[12] = {
      (size_t)batch * n_q * T * 4,    // logits
      (size_t)bh * ((T + 3) & ~3) * 4,  // scores (rows padded to 16 bytes)
      (size_t)bh * s1 * G * 2 * 4,    // k1part
      (size_t)bh * NBINS * 4,         // hist
      (size_t)bh * 2 * 4,             // cnt
      (size_t)bh * KS * 4,            // sel
      (size_t)bh * KS * 4,            // hit_t
      (size_t)bh * KS * 4,            // hit_s
      (size_t)bh * 4,                 // n_hit
      (size_t)bh * G * 4,             // mref
      (size_t)bh * s3 * G * (1 + HD) * 4,  // k3part
      0};
  size_t o = sf_align256(sizeof(WsControl));
  for (int i = 0; i < 12; ++i) {
    off[i] = o;
    o += sf_align256(sizes[i]);
  }
  return o;
}

template <int B, int G>
sf_status launch_attn(AttnArgs& a, hipStream_t s) {
  const int bh = a.batch * a.n_kv;
  hipLaunchKernelGGL((attn_qk_kernel<B, G>), dim3(a.s1, bh), dim3(256), 0, s, a);
  SF_LAUNCH_CHECK();
  hipLaunchKernelGGL((attn_select_kernel<G>), dim3(a.s2, bh), dim3(SEL_T), 0, s, a);
  SF_LAUNCH_CHECK();
  hipLaunchKernelGGL((attn_pv_kernel<B, G>), dim3(a.s3, bh), dim3(256), 0, s, a);
  SF_LAUNCH_CHECK();
  return SF_OK;
}

template <int B>
sf_status dispatch_g(AttnArgs& a, hipStream_t s) {
  switch (a.G) {
    case 1: return launch_attn<B, 1>(a, s);
    case 2: return launch_attn<B, 2>(a, s);
    case 4: return launch_attn<B, 4>(a, s);
    case 8: return launch_attn<B, 8>(a, s);
    default:
      sf_set_error("sf_refined_attn_decode: n_q / n_kv must be 1, 2, 4 or 8");
      return SF_EUNSUPPORTED;
  }
}

}  // namespace

extern "C" size_t sf_workspace_bytes_attn(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                          int32_t t_len, int32_t k_sel) {
  size_t off[12];
  return attn_layout(batch, n_q_heads, n_kv_heads, t_len, k_sel, off);
}

extern "C" sf_status sf_refined_attn_decode(const uint16_t* q_f16, int32_t n_q_heads, const sf_qkv* kv,
                                            float softmax_scale, int32_t k_sel, const int32_t* sel_in,
                                            sf_refine_cache* cache, int32_t pool, float* out,
                                            int32_t* sel_out, int32_t* hit_out, sf_workspace* ws,
                                            sf_stream stream) {
  SF_REQUIRE(q_f16 && kv && out && ws, SF_EINVAL, "null argument");
  SF_REQUIRE(kv->head_dim == HD, SF_EUNSUPPORTED, "head_dim must be 128");
  SF_REQUIRE(kv->fmt.group == 128 && kv->fmt.b >= 1 && kv->fmt.r >= 0 && kv->fmt.b + kv->fmt.r <= 8,
             SF_EUNSUPPORTED, "bad format");
  SF_REQUIRE(kv->batch > 0 && kv->n_kv_heads > 0 && n_q_heads % kv->n_kv_heads == 0, SF_EINVAL,
             "n_q_heads must be a multiple of n_kv_heads");
  SF_REQUIRE(kv->t_len >= 1 && kv->t_len <= kv->t_cap, SF_EINVAL, "need 1 <= t_len <= t_cap");
  SF_REQUIRE(k_sel >= 0 && k_sel <= kv->t_len, SF_EINVAL, "k_sel out of range");
  SF_REQUIRE(k_sel == 0 || kv->fmt.r > 0, SF_EINVAL, "k_sel > 0 needs r > 0");
  AttnArgs a = {};
  a.q = q_f16;
  a.k_res = kv->k_res;
  a.k_sz = kv->k_sz;
  a.v_res = kv->v_res;
  a.v_sz = kv->v_sz;
  a.batch = kv->batch;
  a.n_q = n_q_heads;
  a.n_kv = kv->n_kv_heads;
  a.G = n_q_heads / kv->n_kv_heads;
  a.T = kv->t_len;
  a.t_cap = kv->t_cap;
  a.b = kv->fmt.b;
  a.r = kv->fmt.r;
  a.k_sel = k_sel;
  a.scale = softmax_scale;
  a.s1 = (a.T + qk_split(a.b) - 1) / qk_split(a.b);
  a.s2 = (a.T + SPLIT2 - 1) / SPLIT2;
  a.s3 = (a.T + pv_split(a.b) - 1) / pv_split(a.b);
  size_t off[12];
  const size_t need = attn_layout(a.batch, a.n_q, a.n_kv, a.T, k_sel, off);
  SF_REQUIRE(ws->bytes >= need, SF_ENOMEM, "workspace too small");
  uint8_t* w = ws->base;
  a.logits = (float*)(w + off[0]);
  a.scores = (float*)(w + off[1]);
  a.k1part = (float*)(w + off[2]);
  a.hist = (uint32_t*)(w + off[3]);
  a.cnt = (uint32_t*)(w + off[4]);
  a.sel = (int32_t*)(w + off[5]);
  a.hit_t = (int32_t*)(w + off[6]);
  a.hit_s = (int32_t*)(w + off[7]);
  a.n_hit = (int32_t*)(w + off[8]);
  a.mref = (float*)(w + off[9]);
  a.k3part = (float*)(w + off[10]);
  a.sel_in = sel_in;
  a.sel_out = sel_out;
  a.hit_out = hit_out;
  a.out = out;
  if (k_sel > 0) {
    sf_status st = sf_cache_pool_view(cache, cache ? pool : -1, &a.pool);
    if (st != SF_OK) return st;
    if (a.pool.unit2slot) {
      SF_REQUIRE(a.pool.unit_bytes == 2 * HD * a.r / 8, SF_EINVAL, "pool unit size is not a KV unit");
      SF_REQUIRE(a.pool.n_units >= (int64_t)a.batch * a.n_kv * a.t_cap, SF_EINVAL,
                 "pool has fewer units than batch * n_kv * t_cap");
    }
  }
  hipStream_t s = (hipStream_t)stream;
  switch (a.b) {
    case 1: return dispatch_g<1>(a, s);
    case 2: return dispatch_g<2>(a, s);
    case 4: return dispatch_g<4>(a, s);
    case 8: return dispatch_g<8>(a, s);
    default:
      sf_set_error("sf_refined_attn_decode: resident KV width b must be 1, 2, 4 or 8");
      return SF_EUNSUPPORTED;
  }
}
