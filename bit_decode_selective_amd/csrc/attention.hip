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
// The refinement is additive, so the refined output is the unrefined flash-decoding
// result plus a correction over the (few) hit tokens:
//   l'_t = l_t + scale * s_K,t * (q . cK_lo,t)           (t in E)
//   Z'   = Z + sum_E (e^{l'-m} - e^{l-m})
//   N'   = N + sum_E ((e^{l'-m} - e^{l-m}) * V_b,t + e^{l'-m} * s_V,t * cV_lo,t)
//   out  = N' / Z'
// Kernel A streams the resident K and V once (split over T) and writes the logits
// and per-split (m, Z, N) partials.  Kernel B, one workgroup per (batch, kv head),
// merges the partials, forms the selection scores, radix-selects the top-k tokens
// (ties to the lower token), looks them up in the refinement cache and applies the
// correction.
#include "block_scan.h"
#include "sf_internal.h"

namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }

constexpr int HD = 128;       // head dim
constexpr int MAX_G = 8;      // query heads per kv head
constexpr int MAX_SPLITS = 256;

// b in {1,2,4,8}: codes i and i + P/2 of a word share one and-or into fp16 lanes.
template <int B>
struct KCodec {
  static constexpr int P = 32 / B, HP = P / 2;
  static constexpr int WORDS = HD * B / 32;  // words per token-head
  static constexpr int PAIRS = HD / 2;
  __device__ static int pair_k0(int j) { return (j / HP) * P + (j % HP); }
  __device__ static int pair_k1(int j) { return pair_k0(j) + HP; }
  __device__ static __forceinline__ uint32_t pair(const uint32_t* w, int j) {
    const int wi = j / HP, i = j % HP;
    const int sh = (10 - B) - i * B;
    const uint32_t t = sh >= 0 ? (w[wi] << sh) : (w[wi] >> (-sh));
    constexpr uint32_t m = ((1u << B) - 1u) << (10 - B);
    return (t & (m | (m << 16))) | 0x3C003C00u;
  }
};

__device__ __forceinline__ uint32_t field(const uint32_t* w, int bit, int width) {
  const int wi = bit >> 5, off = bit & 31;
  uint32_t v = w[wi] >> off;
  if (off + width > 32) v |= w[wi + 1] << (32 - off);
  return v & ((1u << width) - 1u);
}

struct AttnArgs {
  const uint16_t* q;  // [batch][n_q][HD] fp16 bits
  const uint8_t* k_res;
  const uint32_t* k_sz;
  const uint8_t* v_res;
  const uint32_t* v_sz;
  int batch, n_q, n_kv, G, T, t_cap, b, r, splits, split_len, k_sel;
  float scale;
  float* logits;  // [batch][n_q][T]
  float* scores;  // [batch][n_kv][T]
  double* part;   // [batch*n_kv][splits][G][2 + HD]: m, Z, N[HD] (fp64)
  const int32_t* sel_in;
  int32_t* sel_out;
  int32_t* hit_out;
  int32_t* lists;   // per (batch, kv head): sel, hit token, hit slot [k_sel] each
  double* ee;       // per (batch, kv head): [k_sel][G][2]: weight added by the stream pass, e'
  float* out;       // [batch][n_q][HD]
  PoolDev pool;
};

// ---- kernel A: logits + per-split flash partials ---------------------------------
template <int B, int G>
__global__ __launch_bounds__(256) void attn_stream_kernel(AttnArgs a) {
  extern __shared__ float sm[];
  float* lg = sm;  // [G][split_len]
  __shared__ uint32_t qs[G][KCodec<B>::PAIRS];
  __shared__ float qsum[G];
  __shared__ float red[4][G];
  __shared__ double dred[4][G][2];
  __shared__ double acc_red[4][G][HD];

  using C = KCodec<B>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x, bh = blockIdx.y;
  const int bi = bh / a.n_kv, kvh = bh - bi * a.n_kv;
  const int L = a.split_len;
  const int t_begin = split * L;
  const int t_end = min(a.T, t_begin + L);
  const int n_here = max(0, t_end - t_begin);
  const uint16_t* qg = a.q + ((size_t)bi * a.n_q + (size_t)kvh * G) * HD;

  for (int p = tid; p < G * C::PAIRS; p += 256) {
    const int h = p / C::PAIRS, j = p - h * C::PAIRS;
    qs[h][j] = (uint32_t)qg[h * HD + C::pair_k0(j)] | ((uint32_t)qg[h * HD + C::pair_k1(j)] << 16);
  }
  if (tid < G) {
    float s = 0.f;
    for (int i = 0; i < HD; ++i) s += (float)__builtin_bit_cast(_Float16, qg[tid * HD + i]);
    qsum[tid] = s;
  }
  __syncthreads();

  const size_t tok0 = (size_t)bh * a.t_cap;
  const float scl = (float)(1u << (a.r + B));
  // A1: logits, one token per thread
  for (int tl = tid; tl < n_here; tl += 256) {
    const size_t tok = tok0 + t_begin + tl;
    uint32_t w[C::WORDS];
    const u32x4* src = (const u32x4*)(a.k_res + tok * (HD * B / 8));
#pragma unroll
    for (int i = 0; i < C::WORDS / 4; ++i) {
      const u32x4 v = __builtin_nontemporal_load(src + i);
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
    const uint32_t szw = a.k_sz[tok];
    const float s = sf_h2f(szw), z = sf_h2f(szw >> 16);
    float d[G];
#pragma unroll
    for (int h = 0; h < G; ++h) d[h] = 0.f;
#pragma unroll
    for (int j = 0; j < C::PAIRS; ++j) {
      const uint32_t pr = C::pair(w, j);
#pragma unroll
      for (int h = 0; h < G; ++h) d[h] = __builtin_amdgcn_fdot2(as_h2(pr), as_h2(qs[h][j]), d[h], false);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float l = a.scale * (z * qsum[h] + (s * scl) * (d[h] - qsum[h]));
      lg[h * L + tl] = l;
      a.logits[((size_t)bi * a.n_q + kvh * G + h) * a.T + t_begin + tl] = l;
    }
  }
  __syncthreads();
  // A2: split max; exponentials; Z and sum_t e_t z_t in fp64 (token-parallel)
  float m[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float v = -INFINITY;
    for (int tl = tid; tl < n_here; tl += 256) v = fmaxf(v, lg[h * L + tl]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    if (lane == 0) red[wave][h] = v;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) m[h] = fmaxf(fmaxf(red[0][h], red[1][h]), fmaxf(red[2][h], red[3][h]));
  double zs[G], zz[G];
#pragma unroll
  for (int h = 0; h < G; ++h) zs[h] = zz[h] = 0.0;
  for (int tl = tid; tl < n_here; tl += 256) {
    const double zv = (double)sf_h2f(a.v_sz[tok0 + t_begin + tl] >> 16);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float e = __expf(lg[h * L + tl] - m[h]);
      lg[h * L + tl] = e;
      zs[h] += (double)e;
      zz[h] = fma((double)e, zv, zz[h]);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    double v = zs[h], w = zz[h];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      v += __shfl_xor(v, o, 64);
      w += __shfl_xor(w, o, 64);
    }
    if (lane == 0) {
      dred[wave][h][0] = v;
      dred[wave][h][1] = w;
    }
  }
  __syncthreads();
  // A3: sum_t (e_t * s'_t) * c_t[d] in fp64; lane owns dims 2*lane, 2*lane+1
  double acc0[G], acc1[G];
#pragma unroll
  for (int h = 0; h < G; ++h) acc0[h] = acc1[h] = 0.0;
  const float sres = (float)(1u << a.r);
  const int bit0 = 2 * lane * B;
  for (int tl = wave; tl < n_here; tl += 4) {
    const size_t tok = tok0 + t_begin + tl;
    const uint32_t* vw = (const uint32_t*)(a.v_res + tok * (HD * B / 8));
    const uint32_t word = vw[bit0 >> 5];
    const double sv = (double)(sf_h2f(a.v_sz[tok]) * sres);
    const double c0 = (double)((word >> (bit0 & 31)) & ((1u << B) - 1u));
    const double c1 = (double)((word >> ((bit0 & 31) + B)) & ((1u << B) - 1u));
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const double we = (double)lg[h * L + tl] * sv;
      acc0[h] = fma(we, c0, acc0[h]);
      acc1[h] = fma(we, c1, acc1[h]);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    acc_red[wave][h][2 * lane] = acc0[h];
    acc_red[wave][h][2 * lane + 1] = acc1[h];
  }
  __syncthreads();
  double* P = a.part + (((size_t)bh * a.splits + split) * G) * (2 + HD);
  for (int i = tid; i < G * HD; i += 256) {
    const int h = i / HD, dd = i - h * HD;
    const double zt = (dred[0][h][1] + dred[1][h][1]) + (dred[2][h][1] + dred[3][h][1]);
    P[h * (2 + HD) + 2 + dd] =
        ((acc_red[0][h][dd] + acc_red[1][h][dd]) + (acc_red[2][h][dd] + acc_red[3][h][dd])) + zt;
  }
  if (tid < G) {
    P[tid * (2 + HD) + 0] = (double)m[tid];
    P[tid * (2 + HD) + 1] = (dred[0][tid][0] + dred[1][tid][0]) + (dred[2][tid][0] + dred[3][tid][0]);
  }
}

// ---- kernel B: merge, select, look up, correct ------------------------------------
constexpr int BT = 1024;  // threads of kernel B

__device__ __forceinline__ int wg1024_exclusive_scan(int v, int* lds, int* total) {
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
  for (int w = 0; w < BT / 64; ++w) {
    const int t = lds[w];
    if (w < wave) base += t;
    sum += t;
  }
  __syncthreads();
  *total = sum;
  return base + incl - v;
}

template <int B, int G>
__global__ __launch_bounds__(BT) void attn_select_correct_kernel(AttnArgs a) {
  __shared__ float s_m[G];
  __shared__ double s_Z[G], s_dZ[G];
  __shared__ double s_num[G][HD];
  __shared__ uint32_t hist[2048];
  __shared__ int lds[32];
  __shared__ float qf[G][HD];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int bi = bh / a.n_kv, kvh = bh - bi * a.n_kv;
  const int T = a.T, ks = a.k_sel;
  const int KS = ks > 0 ? ks : 1;
  int* sel = a.lists + (size_t)bh * 3 * KS;
  int* hit_t = sel + KS;
  int* hit_s = sel + 2 * KS;
  double* ee = a.ee + (size_t)bh * KS * G * 2;

  // 1. merge split partials (fp64); split s is scaled by f_s = exp(m_s - m)
  const double* P = a.part + (size_t)bh * a.splits * G * (2 + HD);
  if (tid < G) {
    float m = -INFINITY;
    for (int s = 0; s < a.splits; ++s) m = fmaxf(m, (float)P[(s * G + tid) * (2 + HD)]);
    double z = 0.0;
    for (int s = 0; s < a.splits; ++s) {
      const float ms = (float)P[(s * G + tid) * (2 + HD)];
      if (ms > -INFINITY) z += (double)__expf(ms - m) * P[(s * G + tid) * (2 + HD) + 1];
    }
    s_m[tid] = m;
    s_Z[tid] = z;
    s_dZ[tid] = 0.0;
  }
  for (int i = tid; i < G * HD; i += BT) {
    const int h = i / HD, d = i - h * HD;
    qf[h][d] = (float)__builtin_bit_cast(_Float16, a.q[((size_t)bi * a.n_q + kvh * G + h) * HD + d]);
  }
  __syncthreads();
  for (int i = tid; i < G * HD; i += BT) {
    const int h = i / HD, d = i - h * HD;
    double n = 0.0;
    for (int s = 0; s < a.splits; ++s) {
      const float ms = (float)P[(s * G + h) * (2 + HD)];
      if (ms > -INFINITY) n += (double)__expf(ms - s_m[h]) * P[(s * G + h) * (2 + HD) + 2 + d];
    }
    s_num[h][d] = n;
  }
  __syncthreads();

  if (ks > 0) {
    // 2. selection
    if (a.sel_in) {
      for (int j = tid; j < ks; j += BT) sel[j] = a.sel_in[(size_t)bh * ks + j];
    } else {
      float* sc = a.scores + (size_t)bh * T;
      float inv[G];
#pragma unroll
      for (int h = 0; h < G; ++h) inv[h] = (float)(1.0 / s_Z[h]);
      for (int t = tid; t < T; t += BT) {
        float v = 0.f;
#pragma unroll
        for (int h = 0; h < G; ++h)
          v += expf(a.logits[((size_t)bi * a.n_q + kvh * G + h) * T + t] - s_m[h]) * inv[h];
        sc[t] = v;
      }
      __threadfence();
      __syncthreads();
      __threadfence();
      // radix select over the fp32 bit patterns (scores are >= 0): 11 + 11 + 10 bits
      uint32_t prefix = 0, above = 0;
      int need = ks;
      const int shifts[3] = {21, 10, 0};
      const int widths[3] = {11, 11, 10};
      for (int pass = 0; pass < 3; ++pass) {
        const int sh = shifts[pass], nb = 1 << widths[pass];
        for (int i = tid; i < 2048; i += BT) hist[i] = 0;
        __syncthreads();
        const uint32_t pmask = pass == 0 ? 0u : (0xFFFFFFFFu << (sh + widths[pass]));
        for (int t = tid; t < T; t += BT) {
          const uint32_t key = __float_as_uint(sc[t]);
          if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & (nb - 1)], 1u);
        }
        __syncthreads();
        // suffix sums over nb bins: thread i takes bins 2i, 2i+1 in reverse order
        int v0 = 0, v1 = 0;
        const int i0 = nb - 1 - 2 * tid, i1 = i0 - 1;
        if (i0 >= 0) v0 = (int)hist[i0];
        if (i1 >= 0) v1 = (int)hist[i1];
        int tot;
        const int ex = wg1024_exclusive_scan(v0 + v1, lds, &tot);
        if (i0 >= 0) hist[i0] = (uint32_t)(ex + v0);
        if (i1 >= 0) hist[i1] = (uint32_t)(ex + v0 + v1);
        __syncthreads();
        if (tid == 0) lds[31] = 0;
        __syncthreads();
        for (int i = tid; i < nb; i += BT) {
          if ((int)hist[i] >= need && (i + 1 == nb || (int)hist[i + 1] < need)) lds[31] = i;
        }
        __syncthreads();
        const int bin = lds[31];
        const int more = (bin + 1 < nb) ? (int)hist[bin + 1] : 0;
        __syncthreads();
        above += more;
        need -= more;
        prefix |= (uint32_t)bin << sh;
      }
      const uint32_t thr = prefix;  // exact key of the k-th largest score
      // ordered compaction: thread owns tokens [tid*tpt, (tid+1)*tpt)
      const int tpt = (T + BT - 1) / BT;
      const int t0 = tid * tpt, t1 = min(T, t0 + tpt);
      int gt = 0, eq = 0;
      for (int t = t0; t < t1; ++t) {
        const uint32_t key = __float_as_uint(sc[t]);
        gt += key > thr;
        eq += key == thr;
      }
      int tot;
      const int eq_before = wg1024_exclusive_scan(eq, lds, &tot);
      const int take_eq = max(0, min(eq, need - eq_before));
      int off = wg1024_exclusive_scan(gt + take_eq, lds, &tot);
      int seen = 0;
      for (int t = t0; t < t1; ++t) {
        const uint32_t key = __float_as_uint(sc[t]);
        if (key > thr) sel[off++] = t;
        else if (key == thr) {
          if (seen < take_eq) sel[off++] = t;
          ++seen;
        }
      }
    }
    __threadfence();
    __syncthreads();
    __threadfence();
    // 3. lookup (units of this (batch, kv head)), in selection order
    const size_t unit0 = (size_t)bh * a.t_cap;
    if (tid == 0) {
      int base = -1;
      if (a.pool.log_count) {
        const uint32_t bse = atomicAdd(a.pool.log_count, (uint32_t)ks);
        base = (bse + (uint32_t)ks <= (uint32_t)a.pool.log_cap) ? (int)bse : -1;
      }
      lds[30] = base;
    }
    __syncthreads();
    const int base = lds[30];
    const int jpt = (ks + BT - 1) / BT;
    const int j0 = tid * jpt, j1 = min(ks, j0 + jpt);
    int nh = 0;
    for (int j = j0; j < j1; ++j) {
      const int t = sel[j];
      const bool ok = t >= 0 && t < T;
      const int slot = (a.pool.unit2slot && ok) ? a.pool.unit2slot[unit0 + t] : -1;
      nh += slot >= 0;
    }
    int n_hits;
    int pos = wg1024_exclusive_scan(nh, lds, &n_hits);
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
    __threadfence();
    __syncthreads();
    __threadfence();
    // 4. per hit: logit change from the K refinement, e and e'
    const int r = a.r;
    for (int m = tid; m < n_hits * G; m += BT) {
      const int hh = m / n_hits, mi = m - hh * n_hits;
      const int t = hit_t[mi];
      const uint32_t* unit = (const uint32_t*)(a.pool.slots + (size_t)hit_s[mi] * a.pool.unit_bytes);
      float dot = 0.f;
      for (int i = 0; i < HD; ++i) dot = fmaf(qf[hh][i], (float)field(unit, i * r, r), dot);
      const uint32_t szk = a.k_sz[unit0 + t];
      const float l = a.logits[((size_t)bi * a.n_q + kvh * G + hh) * T + t];
      const float l2 = l + a.scale * (sf_h2f(szk) * dot);
      // the weight the stream pass gave t: exp(l - m_split) scaled by exp(m_split - m)
      const int sp = t / a.split_len;
      const float ms = (float)P[(sp * G + hh) * (2 + HD)];
      const double w_old = (double)__expf(ms - s_m[hh]) * (double)__expf(l - ms);
      ee[2 * (mi * G + hh)] = w_old;
      ee[2 * (mi * G + hh) + 1] = (double)__expf(l2 - s_m[hh]);
    }
    __threadfence();
    __syncthreads();
    __threadfence();
    if (tid < G) {
      double dz = 0.0;
      for (int mi = 0; mi < n_hits; ++mi) dz += ee[2 * (mi * G + tid) + 1] - ee[2 * (mi * G + tid)];
      s_dZ[tid] = dz;
    }
    // 5. numerator correction, thread per (head, dim):
    //    N' = N - w_old * V_b,t + e' * V_B,t  over the hit tokens t
    const double sres = (double)(1u << r);
    for (int i = tid; i < G * HD; i += BT) {
      const int hh = i / HD, d = i - hh * HD;
      double dn = 0.0;
      for (int mi = 0; mi < n_hits; ++mi) {
        const int t = hit_t[mi];
        const uint32_t* vw = (const uint32_t*)(a.v_res + (unit0 + t) * (HD * B / 8));
        const uint32_t szv = a.v_sz[unit0 + t];
        const double sv = (double)sf_h2f(szv), zv = (double)sf_h2f(szv >> 16);
        const double chi = (double)field(vw, d * B, B);
        const uint32_t* unit = (const uint32_t*)(a.pool.slots + (size_t)hit_s[mi] * a.pool.unit_bytes);
        const double clo = (double)field(unit, HD * r + d * r, r);
        const double w_old = ee[2 * (mi * G + hh)], e2 = ee[2 * (mi * G + hh) + 1];
        const double vb = zv + (sv * sres) * chi;
        dn += e2 * (vb + sv * clo) - w_old * vb;
      }
      s_num[hh][d] += dn;
    }
    __syncthreads();
  }
  // 6. output
  for (int i = tid; i < G * HD; i += BT) {
    const int hh = i / HD, d = i - hh * HD;
    a.out[((size_t)bi * a.n_q + kvh * G + hh) * HD + d] = (float)(s_num[hh][d] / (s_Z[hh] + s_dZ[hh]));
  }
}

int choose_splits(int T) {
  int s = (T + 511) / 512;
  if (s < 1) s = 1;
  if (s > MAX_SPLITS) s = MAX_SPLITS;
  return s;
}

size_t attn_layout(int batch, int n_q, int n_kv, int T, int k_sel, size_t* o_log, size_t* o_sc,
                   size_t* o_part, size_t* o_lists, size_t* o_ee) {
  const int G = n_kv > 0 ? n_q / n_kv : 1;
  const int S = choose_splits(T);
  size_t off = sf_align256(sizeof(WsControl));
  *o_log = off;
  off += sf_align256((size_t)batch * n_q * T * 4);
  *o_sc = off;
  off += sf_align256((size_t)batch * n_kv * T * 4);
  *o_part = off;
  off += sf_align256((size_t)batch * n_kv * S * G * (2 + HD) * 8);
  const size_t KS = k_sel > 0 ? k_sel : 1;
  *o_lists = off;
  off += sf_align256((size_t)batch * n_kv * 3 * KS * 4);
  *o_ee = off;
  off += sf_align256((size_t)batch * n_kv * KS * G * 2 * 8);
  return off;
}

template <int B, int G>
sf_status launch_attn(AttnArgs& a, hipStream_t s) {
  const size_t lds_a = (size_t)G * a.split_len * 4;
  SF_REQUIRE(lds_a + (size_t)4 * G * HD * 8 <= 60 * 1024, SF_EUNSUPPORTED, "split too long");
  hipLaunchKernelGGL((attn_stream_kernel<B, G>), dim3(a.splits, a.batch * a.n_kv), dim3(256), lds_a, s, a);
  SF_LAUNCH_CHECK();
  hipLaunchKernelGGL((attn_select_correct_kernel<B, G>), dim3(a.batch * a.n_kv), dim3(BT), 0, s, a);
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
  size_t a, b, c, d, e;
  return attn_layout(batch, n_q_heads, n_kv_heads, t_len, k_sel, &a, &b, &c, &d, &e);
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
  a.splits = choose_splits(a.T);
  a.split_len = ((a.T + a.splits - 1) / a.splits + 63) / 64 * 64;
  a.k_sel = k_sel;
  a.scale = softmax_scale;
  size_t o_log, o_sc, o_part, o_lists, o_ee;
  const size_t need = attn_layout(a.batch, a.n_q, a.n_kv, a.T, k_sel, &o_log, &o_sc, &o_part, &o_lists, &o_ee);
  SF_REQUIRE(ws->bytes >= need, SF_ENOMEM, "workspace too small");
  a.logits = (float*)(ws->base + o_log);
  a.scores = (float*)(ws->base + o_sc);
  a.part = (double*)(ws->base + o_part);
  a.lists = (int32_t*)(ws->base + o_lists);
  a.ee = (double*)(ws->base + o_ee);
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
