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
constexpr int SPLIT1 = 256;   // tokens per qk workgroup (4 waves x 4 MFMA tiles of 16)
constexpr int SPLIT2 = 2048;  // tokens per select workgroup
constexpr int SPLIT3 = 256;   // tokens per pv workgroup
constexpr int NBINS = 2048;   // first-level radix bins (top 11 bits of the score)

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
  float* scores;    // [batch*n_kv][T]
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
  constexpr int P = 32 / B, HP = P / 2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x, bh = blockIdx.y;
  const int bi = bh / a.n_kv, kvh = bh - bi * a.n_kv;
  const int T = a.T;
  const int t_begin = split * SPLIT1, t_end = min(T, t_begin + SPLIT1);

  // this call's selection histogram and counters start at zero
  for (int i = split * 256 + tid; i < NBINS; i += a.s1 * 256) a.hist[(size_t)bh * NBINS + i] = 0;
  if (split == 0 && tid < 2) a.cnt[bh * 2 + tid] = 0;

  // B operand: q of head n = lane % 16 (zero for n >= G) over the 32 dims of lane
  // group qg = lane / 16, in the same pair order as the key codes
  const int n = lane & 15, qg = lane >> 4;
  const uint16_t* qrow = a.q + ((size_t)bi * a.n_q + (size_t)kvh * G + (n < G ? n : 0)) * HD;
  h8_t bq[4];
  float qpart = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int p = 4 * j + (e >> 1), h = e & 1;
      const int w = p / HP, i = p % HP;
      const int dim = 32 * qg + P * w + i + h * HP;
      const float v = n < G ? h2f16(qrow[dim]) : 0.f;
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
  // each wave: 4 tiles of 16 tokens
  const int tw = t_begin + wave * 64;
  uint32_t wv[4][B];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
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
#pragma unroll
  for (int u = 0; u < 4; ++u) {
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
          const uint32_t szw = a.k_sz[tok0 + t];
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
template <int G>
__global__ __launch_bounds__(256) void attn_select_kernel(AttnArgs a) {
  __shared__ uint32_t lh[NBINS];
  __shared__ float s_m[G], s_iz[G], s_mref[G];
  __shared__ float red[4];
  __shared__ int lds[16];
  __shared__ float qf[G][HD];
  const int tid = threadIdx.x;
  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int bi = bh / a.n_kv, kvh = bh - bi * a.n_kv;
  const int T = a.T, ks = a.k_sel;
  const int KS = ks > 0 ? ks : 1;

  // global softmax statistics of the resident logits
  for (int h = 0; h < G; ++h) {
    float m = -INFINITY;
    for (int s = tid; s < a.s1; s += 256) m = fmaxf(m, a.k1part[(((size_t)bh * a.s1 + s) * G + h) * 2]);
    m = wg_max(m, red);
    float z = 0.f;
    for (int s = tid; s < a.s1; s += 256) {
      const float* P2 = a.k1part + (((size_t)bh * a.s1 + s) * G + h) * 2;
      if (P2[0] > -INFINITY) z += P2[1] * __expf(P2[0] - m);
    }
    z = wg_sum(z, red);
    if (tid == 0) {
      s_m[h] = m;
      s_iz[h] = 1.f / z;
    }
  }
  __syncthreads();

  if (ks == 0) {
    if (chunk == 0 && tid < G) a.mref[bh * G + tid] = s_m[tid];
    if (chunk == 0 && tid == 0) a.n_hit[bh] = 0;
    return;
  }

  int* sel = a.sel + (size_t)bh * KS;
  if (a.sel_in == nullptr) {
    // scores of this chunk + first-level histogram
    for (int i = tid; i < NBINS; i += 256) lh[i] = 0;
    __syncthreads();
    const int c0 = chunk * SPLIT2, c1 = min(T, c0 + SPLIT2);
    float* sc = a.scores + (size_t)bh * T;
    for (int t = c0 + tid; t < c1; t += 256) {
      float v = 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h)
        v += expf(a.logits[((size_t)bi * a.n_q + kvh * G + h) * T + t] - s_m[h]) * s_iz[h];
      sc[t] = v;
      atomicAdd(&lh[__float_as_uint(v) >> 21], 1u);
    }
    __syncthreads();
    for (int i = tid; i < NBINS; i += 256)
      if (lh[i]) atomicAdd(&a.hist[(size_t)bh * NBINS + i], lh[i]);
    __threadfence();
    __syncthreads();
    if (tid == 0) lds[8] = atomicAdd(&a.cnt[bh * 2], 1u) == (uint32_t)(a.s2 - 1);
    __syncthreads();
    if (!lds[8]) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

    // ---- last workgroup of this KV head: exact threshold ----
    for (int i = tid; i < NBINS; i += 256) lh[i] = a.hist[(size_t)bh * NBINS + i];
    __syncthreads();
    wg_suffix_sum(lh, NBINS, lds);
    uint32_t prefix = 0;
    int need = ks;
    {
      const int bin = wg_find_threshold(lh, NBINS, (uint32_t)need, lds + 4);
      need -= bin + 1 < NBINS ? (int)lh[bin + 1] : 0;
      prefix = (uint32_t)bin << 21;
      __syncthreads();
    }
    // levels 2 and 3: bits 20..10 and 9..0 of the keys that share the prefix
    for (int level = 0; level < 2; ++level) {
      const int sh = level == 0 ? 10 : 0, nb = level == 0 ? 2048 : 1024;
      const uint32_t pmask = level == 0 ? 0xFFE00000u : 0xFFFFFC00u;
      for (int i = tid; i < NBINS; i += 256) lh[i] = 0;
      __syncthreads();
      for (int t = tid; t < T; t += 256) {
        const uint32_t key = __float_as_uint(sc[t]);
        if ((key & pmask) == prefix) atomicAdd(&lh[(key >> sh) & (uint32_t)(nb - 1)], 1u);
      }
      __syncthreads();
      wg_suffix_sum(lh, NBINS, lds);
      const int bin = wg_find_threshold(lh, nb, (uint32_t)need, lds + 4);
      need -= bin + 1 < nb ? (int)lh[bin + 1] : 0;
      prefix |= (uint32_t)bin << sh;
      __syncthreads();
    }
    const uint32_t thr = prefix;
    // ordered compaction: thread owns tokens [tid*tpt, (tid+1)*tpt)
    const int tpt = (T + 255) / 256;
    const int t0 = tid * tpt, t1 = min(T, t0 + tpt);
    int gt = 0, eq = 0;
    for (int t = t0; t < t1; ++t) {
      const uint32_t key = __float_as_uint(sc[t]);
      gt += key > thr;
      eq += key == thr;
    }
    int tot;
    const int eq_before = wg_exclusive_scan(eq, lds, &tot);
    const int take_eq = max(0, min(eq, need - eq_before));
    int off = wg_exclusive_scan(gt + take_eq, lds, &tot);
    int seen = 0;
    for (int t = t0; t < t1; ++t) {
      const uint32_t key = __float_as_uint(sc[t]);
      if (key > thr) {
        sel[off++] = t;
      } else if (key == thr) {
        if (seen < take_eq) sel[off++] = t;
        ++seen;
      }
    }
  } else {
    if (chunk != 0) return;
    for (int j = tid; j < ks; j += 256) sel[j] = a.sel_in[(size_t)bh * ks + j];
  }
  __threadfence();
  __syncthreads();
  __threadfence();

  // ---- lookup in selection order ----
  const size_t unit0 = (size_t)bh * a.t_cap;
  int* hit_t = a.hit_t + (size_t)bh * KS;
  int* hit_s = a.hit_s + (size_t)bh * KS;
  if (tid == 0) {
    int base = -1;
    if (a.pool.log_count) {
      const uint32_t bse = atomicAdd(a.pool.log_count, (uint32_t)ks);
      base = (bse + (uint32_t)ks <= (uint32_t)a.pool.log_cap) ? (int)bse : -1;
    }
    lds[9] = base;
  }
  __syncthreads();
  const int base = lds[9];
  const int jpt = (ks + 255) / 256;
  const int j0 = tid * jpt, j1 = min(ks, j0 + jpt);
  int nh = 0;
  for (int j = j0; j < j1; ++j) {
    const int t = sel[j];
    const int slot = (a.pool.unit2slot && t >= 0 && t < T) ? a.pool.unit2slot[unit0 + t] : -1;
    nh += slot >= 0;
  }
  int n_hits;
  int pos = wg_exclusive_scan(nh, lds, &n_hits);
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
  for (int i = tid; i < G * HD; i += 256) {
    const int h = i / HD, d = i - h * HD;
    qf[h][d] = h2f16(a.q[((size_t)bi * a.n_q + kvh * G + h) * HD + d]);
  }
  if (tid < G) s_mref[tid] = s_m[tid];
  __threadfence();
  __syncthreads();
  __threadfence();
  // ---- refined logits of the hit tokens: l' = l + scale * s_K * (q . cK_lo) ----
  const int r = a.r;
  float mloc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) mloc[h] = -INFINITY;
  for (int m = tid; m < n_hits * G; m += 256) {
    const int hh = m % G, mi = m / G;
    const int t = hit_t[mi];
    const uint32_t* unit = (const uint32_t*)(a.pool.slots + (size_t)hit_s[mi] * a.pool.unit_bytes);
    float dot = 0.f;
    for (int i = 0; i < HD; ++i) dot = fmaf(qf[hh][i], (float)field(unit, i * r, r), dot);
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
    const float v = wg_max(mloc[h], red);
    if (tid == 0) s_mref[h] = fmaxf(s_mref[h], v);
  }
  __syncthreads();
  if (tid < G) a.mref[bh * G + tid] = s_mref[tid];
  if (tid == 0) a.n_hit[bh] = n_hits;
}

// ---- pv: weighted value sums with the final weights ------------------------------
template <int B, int G>
__global__ __launch_bounds__(256) void attn_pv_kernel(AttnArgs a) {
  __shared__ float w[G][SPLIT3];
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
  if (tid < G) s_m[tid] = a.mref[bh * G + tid];
  __syncthreads();
  // weights, their sum, and the sum of weight * zero-point per head
  float zs[G], zz[G];
#pragma unroll
  for (int h = 0; h < G; ++h) zs[h] = zz[h] = 0.f;
  for (int tl = tid; tl < n_here; tl += 256) {
    const int t = t_begin + tl;
    const float zv = sf_h2f(a.v_sz[tok0 + t] >> 16);
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
  // sum_t (w_t * s'_t) * c_t[d]; lane owns dims 2*lane, 2*lane+1; wave w takes tokens w, w+4, ...
  float acc0[G], acc1[G];
#pragma unroll
  for (int h = 0; h < G; ++h) acc0[h] = acc1[h] = 0.f;
  const float sres = (float)(1u << a.r);
  const int bit0 = 2 * lane * B;
  constexpr int U = 8;
  for (int tl0 = wave; tl0 < n_here; tl0 += 4 * U) {
    uint32_t word[U], szw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tl = tl0 + 4 * u;
      if (tl < n_here) {
        const size_t tok = tok0 + t_begin + tl;
        word[u] = ((const uint32_t*)(a.v_res + tok * (HD * B / 8)))[bit0 >> 5];
        szw[u] = a.v_sz[tok];
      } else {
        word[u] = 0;
        szw[u] = 0;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tl = tl0 + 4 * u;
      if (tl < n_here) {
        const float sv = sf_h2f(szw[u]) * sres;
        const float c0 = (float)((word[u] >> (bit0 & 31)) & ((1u << B) - 1u));
        const float c1 = (float)((word[u] >> ((bit0 & 31) + B)) & ((1u << B) - 1u));
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float we = w[h][tl] * sv;
          acc0[h] = fmaf(we, c0, acc0[h]);
          acc1[h] = fmaf(we, c1, acc1[h]);
        }
      }
    }
  }
  // refinement of the hit tokens that fall in this split: + w * s_V * cV_lo
  if (wave == 0 && a.k_sel > 0) {
    const int nh = a.n_hit[bh];
    const int KS = a.k_sel;
    const int* hit_t = a.hit_t + (size_t)bh * KS;
    const int* hit_s = a.hit_s + (size_t)bh * KS;
    const int r = a.r;
    for (int m = 0; m < nh; ++m) {
      const int t = hit_t[m];
      if (t < t_begin || t >= t_end) continue;
      const uint32_t* unit = (const uint32_t*)(a.pool.slots + (size_t)hit_s[m] * a.pool.unit_bytes);
      const float sv = sf_h2f(a.v_sz[tok0 + t]);
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
    P3[h * (1 + HD) + 1 + d] = ((accr[0][h][d] + accr[1][h][d]) + (accr[2][h][d] + accr[3][h][d])) + s_zz[h];
  }
  if (tid < G) P3[tid * (1 + HD)] = s_z[tid];
  // last workgroup of this KV head: out = sum_s N_s / sum_s Z_s
  __threadfence();
  __syncthreads();
  if (tid == 0) flag = atomicAdd(&a.cnt[bh * 2 + 1], 1u) == (uint32_t)(a.s3 - 1);
  __syncthreads();
  if (!flag) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const float* Pb = a.k3part + (size_t)bh * a.s3 * G * (1 + HD);
  for (int i = tid; i < G * HD; i += 256) {
    const int h = i / HD, d = i - h * HD;
    float num = 0.f, den = 0.f;
    for (int s = 0; s < a.s3; ++s) {
      num += Pb[(s * G + h) * (1 + HD) + 1 + d];
      den += Pb[(s * G + h) * (1 + HD)];
    }
    a.out[((size_t)bi * a.n_q + kvh * G + h) * HD + d] = num / den;
  }
}

size_t attn_layout(int batch, int n_q, int n_kv, int T, int k_sel, size_t off[12]) {
  const int G = n_kv > 0 ? n_q / n_kv : 1;
  const int bh = batch * n_kv;
  const size_t s1 = (T + SPLIT1 - 1) / SPLIT1, s3 = (T + SPLIT3 - 1) / SPLIT3;
  const size_t KS = k_sel > 0 ? k_sel : 1;
  const size_t sizes[12] = {
      (size_t)batch * n_q * T * 4,    // logits
      (size_t)bh * T * 4,             // scores
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
  hipLaunchKernelGGL((attn_select_kernel<G>), dim3(a.s2, bh), dim3(256), 0, s, a);
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
  a.s1 = (a.T + SPLIT1 - 1) / SPLIT1;
  a.s2 = (a.T + SPLIT2 - 1) / SPLIT2;
  a.s3 = (a.T + SPLIT3 - 1) / SPLIT3;
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
