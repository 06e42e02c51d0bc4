// Refined low-bit GEMV: resident b-bit weights everywhere, plus the refinement
// bits of the selected input channels that are present in the device cache.
//
// Method: rag-lover.com StrataFlux summary, explainer dialogue (解説) -- weight
// refinements are chosen by input-activation magnitude and are extra bits between
// resident levels; limitations section -- a channel whose refinement is missing
// keeps its resident value.  Paper abstract (arXiv 2611.08363): only the selected
// precision is streamed and it is reused across decoding steps.
//
// Because the refinement is additive (W_eff = W_res + s * c_lo on refined
// channels), y = x W_res^T + sum over hit channels k of x_k * s[:, g(k)] * c_lo[:, k].
// One launch computes, for up to SF_MAX_OPS matrices that share x:
//   * the channel selection (top-k of max-over-batch |x|, ties to the lower index)
//     and its cache lookup, done once by whichever workgroup starts first and
//     published to the others through the workspace;
//   * the resident GEMV, streamed from HBM with 16-byte loads, codes expanded into
//     fp16 lanes by mask-and-or into the mantissa (value 1 + c/2^b) and reduced with
//     v_dot2_f32_f16; sum_k c*x = 2^b * (dot - sum_k x) per chunk;
//   * the sparse refinement delta for each workgroup's rows.
#include "block_scan.h"
#include "sf_internal.h"

#define SF_MAX_OPS 4

namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }

struct GemvOpDev {
  const uint8_t* res;
  const uint32_t* sz;
  float* y;
  int32_t* hit_out;
  PoolDev pool;
  int32_t n_out;
  int32_t tile_begin;
};

struct GemvArgs {
  GemvOpDev ops[SF_MAX_OPS];
  const uint16_t* x;
  const int32_t* sel_in;
  int32_t* sel_out;
  WsControl* ctl;
  int32_t* ws_sel;       // [k_sel]
  int32_t* ws_hit_k;     // [n_ops][k_sel]
  int32_t* ws_hit_slot;  // [n_ops][k_sel]
  int32_t* ws_nhit;      // [n_ops]
  int32_t n_ops, k_in, batch, batch_off, k_sel, r, total_tiles, do_log;
};

// ---- code layouts ----------------------------------------------------------------
// A "chunk" is the run of codes one lane loads at once.  Pairs are the (k0, k1)
// channel pairs that one v_dot2 consumes; x is staged in LDS in pair order.

// b in {1, 2, 4, 8}: a 16-byte chunk of 4 words, P = 32/b codes per word.  Codes i
// and i + P/2 of a word are 16 bits apart, so one shift and one and-or put both in
// the top mantissa bits of the two fp16 halves.
template <int B>
struct CodecPow2 {
  static constexpr int WORDS = 4;
  static constexpr int CODES = 32 * WORDS / B;
  static constexpr int PAIRS = CODES / 2;
  static constexpr int P = 32 / B, HP = P / 2;
  __device__ static int pair_k0(int j) { return (j / HP) * P + (j % HP); }
  __device__ static int pair_k1(int j) { return pair_k0(j) + HP; }
  // pair index and half of channel kk (0 <= kk < CODES) of a chunk
  __device__ static __forceinline__ void locate(int kk, int* j, int* hi) {
    const int w = kk / P, q = kk % P;
    *hi = q >= HP;
    *j = w * HP + (q - (*hi) * HP);
  }
  __device__ static __forceinline__ uint32_t pair(const uint32_t* w, int j) {
    const int wi = j / HP, i = j % HP;
    const int sh = (10 - B) - i * B;
    const uint32_t t = sh >= 0 ? (w[wi] << sh) : (w[wi] >> (-sh));
    constexpr uint32_t m = ((1u << B) - 1u) << (10 - B);
    return (t & (m | (m << 16))) | 0x3C003C00u;
  }
};

// b in {3, 5, 6, 7}: a chunk is 32 codes = b words, codes straddle word boundaries;
// pairs are consecutive channels.
template <int B>
struct CodecStream {
  static constexpr int WORDS = B;
  static constexpr int CODES = 32;
  static constexpr int PAIRS = 16;
  __device__ static int pair_k0(int j) { return 2 * j; }
  __device__ static int pair_k1(int j) { return 2 * j + 1; }
  __device__ static __forceinline__ void locate(int kk, int* j, int* hi) {
    *j = kk >> 1;
    *hi = kk & 1;
  }
  __device__ static __forceinline__ uint32_t code(const uint32_t* w, int k) {
    const int bit = k * B, wi = bit >> 5, off = bit & 31;
    uint32_t v = w[wi] >> off;
    if (off + B > 32) v |= w[wi + 1] << (32 - off);
    return v & ((1u << B) - 1u);
  }
  __device__ static __forceinline__ uint32_t pair(const uint32_t* w, int j) {
    const uint32_t c0 = code(w, 2 * j), c1 = code(w, 2 * j + 1);
    return ((c0 | (c1 << 16)) << (10 - B)) | 0x3C003C00u;
  }
};

__device__ __forceinline__ uint32_t read_field(const uint8_t* unit, uint32_t bitpos, int width) {
  const uint32_t* w = (const uint32_t*)unit;
  const uint32_t wi = bitpos >> 5, off = bitpos & 31;
  uint32_t v = w[wi] >> off;
  if (off + width > 32) v |= w[wi + 1] << (32 - off);
  return v & ((1u << width) - 1u);
}

// ---- channel selection + lookup (one workgroup) ---------------------------------
// Thread t owns channels [t*cpt, (t+1)*cpt), cpt = 2*ceil(K/512) <= 64; their keys
// (max over the batch of |x| as 15-bit fp16 patterns, which order like the values)
// are read once, kept two per register, and radix-selected in two histogram passes
// (top 8 bits, then the low 7; one LDS histogram per wave), then compacted in
// channel order into `sel` (LDS when it fits, else the workspace).
constexpr int KEYW = 32;

__device__ void gemv_select_and_lookup(const GemvArgs& a, uint32_t* hist4, int* lds, int32_t* sel) {
  const int K = a.k_in, ks = a.k_sel, tid = threadIdx.x, wave = tid >> 6;
  if (a.sel_in) {
    for (int j = tid; j < ks; j += 256) sel[j] = a.sel_in[j];
  } else if (ks >= K) {
    for (int j = tid; j < ks; j += 256) sel[j] = j;
  } else {
    const int cpt = 2 * ((K + 511) / 512);
    const int k0 = tid * cpt;
    uint32_t kw[KEYW];
#pragma unroll
    for (int i = 0; i < KEYW; ++i) kw[i] = 0;
    for (int bb = 0; bb < a.batch; ++bb) {
      const uint32_t* xr = (const uint32_t*)(a.x + (size_t)bb * K);
#pragma unroll
      for (int i = 0; i < KEYW; ++i) {
        if (2 * i < cpt && k0 + 2 * i < K) {
          const uint32_t v = xr[(k0 >> 1) + i] & 0x7FFF7FFFu;
          const uint32_t lo = max(kw[i] & 0xFFFFu, v & 0xFFFFu), hi = max(kw[i] >> 16, v >> 16);
          kw[i] = lo | (hi << 16);
        }
      }
    }
    SF_TS(8);
    // T = the ks-th largest key: the largest v with count(key >= v) >= ks, found by
    // binary search over the 15-bit key range (15 block-wide counts)
    (void)hist4;
    int lo_v = 0, hi_v = 32768;  // count(>= lo_v) >= ks > count(>= hi_v)
    while (hi_v - lo_v > 1) {
      const int mid = (lo_v + hi_v) >> 1;
      int c = 0;
#pragma unroll
      for (int i = 0; i < KEYW; ++i)
        if (2 * i < cpt && k0 + 2 * i < K) c += ((int)(kw[i] & 0xFFFFu) >= mid) + ((int)(kw[i] >> 16) >= mid);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o, 64);
      __syncthreads();
      if ((tid & 63) == 0) lds[wave] = c;
      __syncthreads();
      const int tot4 = (lds[0] + lds[1]) + (lds[2] + lds[3]);
      if (tot4 >= ks) lo_v = mid; else hi_v = mid;
    }
    const uint32_t T = (uint32_t)lo_v;
    SF_TS(9);
    int above_l = 0;
#pragma unroll
    for (int i = 0; i < KEYW; ++i)
      if (2 * i < cpt && k0 + 2 * i < K) above_l += ((kw[i] & 0xFFFFu) > T) + ((kw[i] >> 16) > T);
    int above;
    (void)wg_exclusive_scan(above_l, lds, &above);
    const int need = ks - above;
    int gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < KEYW; ++i)
      if (2 * i < cpt && k0 + 2 * i < K) {
        const uint32_t lo = kw[i] & 0xFFFFu, hi = kw[i] >> 16;
        gt += (lo > T) + (hi > T);
        eq += (lo == T) + (hi == T);
      }
    int tot;
    const int eq_before = wg_exclusive_scan(eq, lds, &tot);
    const int take_eq = max(0, min(eq, need - eq_before));
    int off = wg_exclusive_scan(gt + take_eq, lds, &tot);
    int seen = 0;
#pragma unroll
    for (int i = 0; i < KEYW; ++i)
      if (2 * i < cpt && k0 + 2 * i < K) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t key = h ? (kw[i] >> 16) : (kw[i] & 0xFFFFu);
          const int k = k0 + 2 * i + h;
          if (key > T) {
            sel[off++] = k;
          } else if (key == T) {
            if (seen < take_eq) sel[off++] = k;
            ++seen;
          }
        }
      }
  }
  // sel[] is read back below by other threads of this workgroup
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  if (a.sel_out && a.do_log)
    for (int j = tid; j < ks; j += 256) a.sel_out[j] = sel[j];
  SF_TS(10);
  // lookups, per op, in selection order
  const int jpt = (ks + 255) / 256;
  const int j0 = tid * jpt, j1 = min(ks, j0 + jpt);
  for (int op = 0; op < a.n_ops; ++op) {
    const PoolDev pool = a.ops[op].pool;
    int32_t* hit_out = a.ops[op].hit_out;
    if (tid == 0) {
      int base = -1;
      if (pool.log_count && a.do_log) {
        const uint32_t bse = atomicAdd(pool.log_count, (uint32_t)ks);
        base = (bse + (uint32_t)ks <= (uint32_t)pool.log_cap) ? (int)bse : -1;
      }
      lds[6] = base;
    }
    __syncthreads();
    const int base = lds[6];
    int nh = 0;
    for (int j = j0; j < j1; ++j) {
      const int k = sel[j];
      const int slot = (pool.unit2slot && k >= 0 && k < K) ? pool.unit2slot[k] : -1;
      nh += slot >= 0;
    }
    int tot;
    int pos = wg_exclusive_scan(nh, lds, &tot);
    for (int j = j0; j < j1; ++j) {
      const int k = sel[j];
      const int slot = (pool.unit2slot && k >= 0 && k < K) ? pool.unit2slot[k] : -1;
      if (hit_out && a.do_log) hit_out[j] = slot;
      if (base >= 0) {
        pool.log_units[base + j] = k;
        pool.log_slots[base + j] = slot;
      }
      if (slot >= 0) {
        sf_put(a.ws_hit_k + op * ks + pos, k);
        sf_put(a.ws_hit_slot + op * ks + pos, slot);
        ++pos;
      }
    }
    if (tid == 0) sf_put(a.ws_nhit + op, tot);
    __syncthreads();
  }
}

// ---- the GEMV kernel -------------------------------------------------------------
// When refining, workgroup 0 only selects, looks up and publishes the hit lists.
// The other (tile) workgroups are persistent, 4 waves each: row tiles of 4R rows
// (R per wave) are dealt round-robin; lane l of a wave owns chunks l, l+64, ... of
// each of the wave's R rows.  The first chunk is requested before x is staged, and
// the next tile's first chunk before the current tile is reduced.  x is staged
// once per workgroup (16-byte loads scattered into pair order in LDS, chunk sums
// by shuffles).  NB batch rows [batch_off, batch_off + NB) per launch.
// Dynamic LDS: x pairs [NB][K/2] | x chunk sums [NB][nchunks] | delta staging:
// tile scale words [4R][K/128] and per-hit refinement words [HIT_CAP][SW].
constexpr int HIT_CAP = 512;  // hits staged in LDS per batch of the delta
constexpr int SW = 4;         // refinement words staged per hit (a tile's rows)

template <class C, int R>
__device__ __forceinline__ void load_chunk(const GemvOpDev& o, int row0, int c, size_t rowbytes, int ngr,
                                           uint32_t (&cw)[R][C::WORDS], uint32_t (&szw)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = row0 + r;
    if (row < o.n_out) {
      const uint32_t* src = (const uint32_t*)(o.res + row * rowbytes + (size_t)c * (4 * C::WORDS));
      if constexpr (C::WORDS == 4) {
        const u32x4 v = __builtin_nontemporal_load((const u32x4*)src);
        cw[r][0] = v.x; cw[r][1] = v.y; cw[r][2] = v.z; cw[r][3] = v.w;
      } else {
#pragma unroll
        for (int w = 0; w < C::WORDS; ++w) cw[r][w] = __builtin_nontemporal_load(src + w);
      }
      szw[r] = o.sz[(size_t)row * ngr + (c * C::CODES) / 128];
    } else {
#pragma unroll
      for (int w = 0; w < C::WORDS; ++w) cw[r][w] = 0;
      szw[r] = 0;
    }
  }
}

__device__ __forceinline__ int op_of_tile(const GemvArgs& a, int tile_g) {
  int op = 0;
  for (int i = 1; i < a.n_ops; ++i)
    if (tile_g >= a.ops[i].tile_begin) op = i;
  return op;
}

template <class C, int B, int R, int NB>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a) {
  extern __shared__ uint32_t smem[];
  __shared__ uint32_t s_hist[1024];
  __shared__ int s_lds[8];
  __shared__ float s_red[NB][256];
  __shared__ int s_hk[HIT_CAP], s_hs[HIT_CAP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.k_in;
  const int nchunks = K / C::CODES;
  const int xpairs = K / 2;
  const int rows_wg = 4 * R;
  const int ngr = K / 128;
  uint32_t* xs = smem;                              // [NB][K/2] fp16 pairs
  float* xsum = (float*)(smem + NB * xpairs);       // [NB][nchunks]
  uint32_t* s_sz = smem + NB * xpairs + NB * nchunks;  // [rows_wg][ngr]
  uint32_t* s_w = s_sz + rows_wg * ngr;                // [HIT_CAP][SW]
  const bool refine = a.k_sel > 0;
  const size_t rowbytes = (size_t)K * B / 8;

  SF_TS(0);
  if (refine && blockIdx.x == 0) {
    // the selecting workgroup: its sel list lives in the (otherwise unused) LDS
    // staging area when it fits
    int32_t* sel = (a.k_sel <= NB * xpairs) ? (int32_t*)smem : a.ws_sel;
    gemv_select_and_lookup(a, s_hist, s_lds, sel);
    SF_TS(2);
    sf_drain();
    __syncthreads();
    if (tid == 0) {
      sf_put(&a.ctl->sel_state, 2u);
      const uint32_t prev = __hip_atomic_fetch_add(&a.ctl->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (prev == gridDim.x - 1u) {
        sf_put(&a.ctl->done, 0u);
        sf_put(&a.ctl->sel_state, 0u);
      }
    }
    return;
  }
  const int twg = (int)blockIdx.x - (refine ? 1 : 0);  // tile workgroup index
  const int n_twg = (int)gridDim.x - (refine ? 1 : 0);

  // request the first chunk of this wave before anything else
  uint32_t cw[R][C::WORDS];
  uint32_t szw[R];
  bool have = false;
  if (twg < a.total_tiles && lane < nchunks) {
    const int op = op_of_tile(a, twg);
    load_chunk<C, R>(a.ops[op], (twg - a.ops[op].tile_begin) * rows_wg + wave * R, lane, rowbytes, ngr, cw, szw);
    have = true;
  }

  // stage x in pair order (16-byte loads, 2-byte LDS stores); the CODES/8 threads
  // that load one chunk sum it with shuffles
  {
    uint16_t* xh = (uint16_t*)xs;
    constexpr int TPC = C::CODES / 8;  // threads per chunk
    for (int bb = 0; bb < NB; ++bb) {
      const u32x4* xr = (const u32x4*)(a.x + (size_t)(a.batch_off + bb) * K);
      for (int m0 = 0; m0 < K / 8; m0 += 256) {
        const int m = m0 + tid;
        float part = 0.f;
        if (m < K / 8) {
          const u32x4 v = xr[m];
          const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int k = 8 * m + e;
            const int c = k / C::CODES, kk = k - c * C::CODES;
            int j, hi;
            C::locate(kk, &j, &hi);
            const uint16_t hb = (uint16_t)(wds[e >> 1] >> (16 * (e & 1)));
            xh[2 * (bb * xpairs + c * C::PAIRS + j) + hi] = hb;
            part += (float)__builtin_bit_cast(_Float16, hb);
          }
        }
#pragma unroll
        for (int o = TPC / 2; o >= 1; o >>= 1) part += __shfl_xor(part, o, TPC);
        if (m < K / 8 && (m % TPC) == 0) xsum[bb * nchunks + m / TPC] = part;
      }
    }
  }
  __syncthreads();

  SF_TS(1);
  const float scl = (float)(1u << (a.r + B));
  for (int tile_g = twg; tile_g < a.total_tiles; tile_g += n_twg) {
    const int op = op_of_tile(a, tile_g);
    const GemvOpDev& o = a.ops[op];
    const int tile = tile_g - o.tile_begin;
    const int row0 = tile * rows_wg + wave * R;
    float acc[NB][R];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[bb][r] = 0.f;
    for (int c = lane; c < nchunks; c += 64) {
      if (!have) load_chunk<C, R>(o, row0, c, rowbytes, ngr, cw, szw);
      have = false;
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        uint32_t xv[C::PAIRS];
        const u32x4* xp = (const u32x4*)(xs + bb * xpairs + c * C::PAIRS);
#pragma unroll
        for (int j = 0; j < C::PAIRS / 4; ++j) {
          const u32x4 v = xp[j];
          xv[4 * j] = v.x; xv[4 * j + 1] = v.y; xv[4 * j + 2] = v.z; xv[4 * j + 3] = v.w;
        }
        const float X = xsum[bb * nchunks + c];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float d = 0.f;
#pragma unroll
          for (int j = 0; j < C::PAIRS; ++j)
            d = __builtin_amdgcn_fdot2(as_h2(C::pair(cw[r], j)), as_h2(xv[j]), d, false);
          const float s = sf_h2f(szw[r]), z = sf_h2f(szw[r] >> 16);
          acc[bb][r] += (s * scl) * (d - X) + z * X;
        }
      }
    }
    // request the next tile's first chunk before reducing this one
    const int next = tile_g + n_twg;
    if (next < a.total_tiles && lane < nchunks) {
      const int op2 = op_of_tile(a, next);
      load_chunk<C, R>(a.ops[op2], (next - a.ops[op2].tile_begin) * rows_wg + wave * R, lane, rowbytes, ngr,
                       cw, szw);
      have = true;
    }
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float v = acc[bb][r];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        acc[bb][r] = v;
      }
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = row0 + r;
        if (row < o.n_out)
#pragma unroll
          for (int bb = 0; bb < NB; ++bb) o.y[(size_t)(a.batch_off + bb) * o.n_out + row] = acc[bb][r];
      }
    }
  }

  SF_TS(3);
  // sparse refinement delta over this workgroup's tiles: y += sum over hit
  // channels k of x_k * s[row][k/128] * c_lo[row][k]
  if (!refine) return;
  int ok = 1;
  if (tid == 0) s_lds[5] = sf_wait_word(&a.ctl->sel_state, 2u, &a.ctl->timeout) ? 1 : 0;
  __syncthreads();
  ok = s_lds[5];
  SF_TS(4);
  if (ok) {
    const int r = a.r;
    // the refinement bits of a tile's rows: rows_wg * r bits from bit tile*rows_wg*r
    // of each unit; staged in LDS when they span at most SW words
    const int nw = (rows_wg * r + 31) / 32 + 1;
    const bool staged = nw <= SW;
    for (int tile_g = twg; tile_g < a.total_tiles; tile_g += n_twg) {
      const int op = op_of_tile(a, tile_g);
      const GemvOpDev& o = a.ops[op];
      const int tile = tile_g - o.tile_begin;
      const int nh = sf_get(a.ws_nhit + op);
      const int* ghk = a.ws_hit_k + op * a.k_sel;
      const int* ghs = a.ws_hit_slot + op * a.k_sel;
      const uint32_t w0 = ((uint32_t)(tile * rows_wg) * r) >> 5;
      const int wpu = o.pool.unit_bytes / 4;
      // scale words of the tile's rows
      for (int i = tid; i < rows_wg * ngr; i += 256) {
        const int rr = i / ngr, g = i - rr * ngr;
        const int row = tile * rows_wg + rr;
        s_sz[i] = row < o.n_out ? o.sz[(size_t)row * ngr + g] : 0u;
      }
      const int i = tid % rows_wg, mstep = 256 / rows_wg;
      const int row = tile * rows_wg + i;
      float part[NB];
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) part[bb] = 0.f;
      for (int m0 = 0; m0 < nh; m0 += HIT_CAP) {
        const int mn = min(HIT_CAP, nh - m0);
        __syncthreads();
        for (int m = tid; m < mn; m += 256) {
          const int k = sf_get(ghk + m0 + m), slot = sf_get(ghs + m0 + m);
          s_hk[m] = k;
          s_hs[m] = slot;
          if (staged) {
            const uint32_t* u = (const uint32_t*)(o.pool.slots + (size_t)slot * o.pool.unit_bytes);
#pragma unroll
            for (int q = 0; q < SW; ++q)
              s_w[SW * m + q] = (q < nw && (int)w0 + q < wpu) ? u[w0 + q] : 0u;
          }
        }
        __syncthreads();
        if (row < o.n_out) {
          for (int m = tid / rows_wg; m < mn; m += mstep) {
            const int k = s_hk[m];
            uint32_t clo_u;
            if (staged) {
              const uint32_t p = (uint32_t)row * r - (w0 << 5);  // bit within the staged words
              const uint32_t q = p >> 5;
              const uint64_t w2 = (uint64_t)s_w[SW * m + q] | ((uint64_t)(q + 1 < (uint32_t)SW ? s_w[SW * m + q + 1] : 0u) << 32);
              clo_u = (uint32_t)(w2 >> (p & 31)) & ((1u << r) - 1u);
            } else {
              clo_u = read_field(o.pool.slots + (size_t)s_hs[m] * o.pool.unit_bytes, (uint32_t)row * r, r);
            }
            const float sv = sf_h2f(s_sz[i * ngr + (k >> 7)]);
            const int c = k / C::CODES, kk = k - c * C::CODES;
            int jj, hi;
            C::locate(kk, &jj, &hi);
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) {
              const h2_t xh = as_h2(xs[bb * xpairs + c * C::PAIRS + jj]);
              const float xk = hi ? (float)xh.y : (float)xh.x;
              part[bb] += (xk * sv) * (float)clo_u;
            }
          }
        }
      }
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) s_red[bb][tid] = part[bb];
      __syncthreads();
      // lane 0 of wave w wrote rows [w*R, w*R + R) of the tile: it adds their deltas
      if (lane == 0) {
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
          const int ii = wave * R + rr;
          const int rrow = tile * rows_wg + ii;
          if (rrow < o.n_out) {
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) {
              float sum = 0.f;
              for (int j = ii; j < 256; j += rows_wg) sum += s_red[bb][j];
              float* yp = o.y + (size_t)(a.batch_off + bb) * o.n_out + rrow;
              *yp = *yp + sum;
            }
          }
        }
      }
      __syncthreads();
    }
  }
  __syncthreads();
  SF_TS(5);
  if (tid == 0) {
    // the last workgroup to finish resets the words for the next launch
    const uint32_t prev = __hip_atomic_fetch_add(&a.ctl->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == gridDim.x - 1u) {
      sf_put(&a.ctl->done, 0u);
      sf_put(&a.ctl->sel_state, 0u);
    }
  }
}

int env_int(const char* name, int dflt) {
  const char* e = getenv(name);
  return e ? atoi(e) : dflt;
}

template <class C, int B, int R, int NB>
sf_status launch_gemv(GemvArgs& a, hipStream_t s) {
  const size_t lds = ((size_t)NB * (a.k_in / 2) + (size_t)NB * (a.k_in / C::CODES) +
                      (size_t)4 * R * (a.k_in / 128) + (size_t)SW * HIT_CAP) * 4;
  SF_REQUIRE(lds <= 52 * 1024, SF_EUNSUPPORTED, "k_in too large for the LDS staging of x");
  // persistent tile workgroups: as many as are resident at once (at most
  // SF_GEMV_WGS_PER_CU per CU if set), each with an equal number of tiles
  static int occ = 0, n_cu = 0;
  if (occ == 0) {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, (const void*)gemv_kernel<C, B, R, NB>, 256, lds) != hipSuccess || v < 1)
      v = 2;
    int dev = 0, cus = 0;
    (void)hipGetDevice(&dev);
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    occ = v;
    n_cu = cus;
  }
  const int per_cu = env_int("SF_GEMV_WGS_PER_CU", occ);
  const int cap = n_cu * (per_cu > 0 ? min(per_cu, occ) : occ) - (a.k_sel > 0 ? 1 : 0);
  const int tiles_per_wg = (a.total_tiles + cap - 1) / cap;
  const int grid = (a.total_tiles + tiles_per_wg - 1) / tiles_per_wg + (a.k_sel > 0 ? 1 : 0);
  hipLaunchKernelGGL((gemv_kernel<C, B, R, NB>), dim3((unsigned)grid), dim3(256), lds, s, a);
  SF_LAUNCH_CHECK();
  return SF_OK;
}

template <class C, int B, int R>
sf_status dispatch_nb(GemvArgs& a, int nb, hipStream_t s) {
  if (nb == 2) return launch_gemv<C, B, R, 2>(a, s);
  return launch_gemv<C, B, R, 1>(a, s);
}

template <class C, int B>
sf_status dispatch_r(GemvArgs& a, int R, int nb, hipStream_t s) {
  switch (R) {
    case 1: return dispatch_nb<C, B, 1>(a, nb, s);
    case 2: return dispatch_nb<C, B, 2>(a, nb, s);
    case 4: return dispatch_nb<C, B, 4>(a, nb, s);
    default: return dispatch_nb<C, B, 8>(a, nb, s);
  }
}

sf_status dispatch_b(GemvArgs& a, int b, int R, int nb, hipStream_t s) {
  switch (b) {
    case 1: return dispatch_r<CodecPow2<1>, 1>(a, R, nb, s);
    case 2: return dispatch_r<CodecPow2<2>, 2>(a, R, nb, s);
    case 3: return dispatch_r<CodecStream<3>, 3>(a, R, nb, s);
    case 4: return dispatch_r<CodecPow2<4>, 4>(a, R, nb, s);
    case 8: return dispatch_r<CodecPow2<8>, 8>(a, R, nb, s);
    default:
      sf_set_error("sf_refined_gemv: resident width b must be 1, 2, 3, 4 or 8");
      return SF_EUNSUPPORTED;
  }
}

}  // namespace

size_t sf_gemv_ws_layout(int32_t n_ops, int64_t k_in, int32_t k_sel, size_t* off_sel,
                         size_t* off_hk, size_t* off_hs, size_t* off_nh) {
  size_t off = sf_align256(sizeof(WsControl));
  *off_sel = off;
  off += sf_align256((size_t)(k_sel > 0 ? k_sel : 1) * 4);
  *off_hk = off;
  off += sf_align256((size_t)n_ops * (k_sel > 0 ? k_sel : 1) * 4);
  *off_hs = off;
  off += sf_align256((size_t)n_ops * (k_sel > 0 ? k_sel : 1) * 4);
  *off_nh = off;
  off += sf_align256((size_t)n_ops * 4);
  (void)k_in;
  return off;
}

extern "C" size_t sf_workspace_bytes_gemv(int32_t n_ops, int64_t k_in, int32_t k_sel) {
  size_t a, b, c, d;
  return sf_gemv_ws_layout(n_ops, k_in, k_sel, &a, &b, &c, &d);
}

extern "C" sf_status sf_refined_gemv(const sf_gemv_op* ops, int32_t n_ops, const uint16_t* x_f16,
                                     int32_t batch, int32_t k_sel, const int32_t* sel_in,
                                     int32_t* sel_out, sf_refine_cache* cache, sf_workspace* ws,
                                     sf_stream stream) {
  SF_REQUIRE(ops && n_ops >= 1 && n_ops <= SF_MAX_OPS, SF_EINVAL, "need 1..4 ops");
  SF_REQUIRE(x_f16 && batch >= 1, SF_EINVAL, "bad x / batch");
  SF_REQUIRE(ws, SF_EINVAL, "workspace required");
  const sf_qfmt f = ops[0].w.fmt;
  const int64_t K = ops[0].w.k_in;
  SF_REQUIRE(f.group == 128 && f.b >= 1 && f.r >= 0 && f.b + f.r <= 8, SF_EUNSUPPORTED, "bad format");
  SF_REQUIRE(K > 0 && K % 128 == 0 && K <= (1 << 20), SF_EINVAL, "k_in must be a multiple of 128");
  SF_REQUIRE(k_sel >= 0 && k_sel <= K, SF_EINVAL, "k_sel out of range");
  SF_REQUIRE(k_sel == 0 || f.r > 0, SF_EINVAL, "k_sel > 0 needs r > 0");
  GemvArgs a = {};
  // rows per wave (SF_GEMV_ROWS_PER_WAVE = 1, 2, 4 or 8 overrides the default)
  int rpw = env_int("SF_GEMV_ROWS_PER_WAVE", 0);
  int64_t rows_total = 0;
  for (int i = 0; i < n_ops; ++i) rows_total += ops[i].w.n_out;
  if (rpw != 1 && rpw != 2 && rpw != 4 && rpw != 8)
    rpw = rows_total <= 8192 ? 2 : (rows_total <= 16384 ? 4 : 8);
  const int rows_wg = 4 * rpw;
  int tiles = 0;
  for (int i = 0; i < n_ops; ++i) {
    const sf_gemv_op& o = ops[i];
    SF_REQUIRE(o.w.k_in == K && o.w.fmt.b == f.b && o.w.fmt.r == f.r && o.w.fmt.group == 128,
               SF_EINVAL, "ops must share k_in and format");
    SF_REQUIRE(o.w.resident && o.w.sz && o.y && o.w.n_out > 0 && o.w.n_out < (1 << 28), SF_EINVAL,
               "bad op tensors");
    GemvOpDev& d = a.ops[i];
    d.res = o.w.resident;
    d.sz = o.w.sz;
    d.y = o.y;
    d.hit_out = o.hit_out;
    d.n_out = (int32_t)o.w.n_out;
    d.tile_begin = tiles;
    if (k_sel > 0) {
      sf_status st = sf_cache_pool_view(cache, cache ? o.pool : -1, &d.pool);
      if (st != SF_OK) return st;
      if (d.pool.unit2slot) {
        SF_REQUIRE((int64_t)d.pool.unit_bytes * 8 >= o.w.n_out * f.r, SF_EINVAL, "pool unit too small for this matrix");
        SF_REQUIRE(d.pool.n_units >= K, SF_EINVAL, "pool has fewer units than input channels");
      }
    }
    tiles += (int)((o.w.n_out + rows_wg - 1) / rows_wg);
  }
  size_t o_sel, o_hk, o_hs, o_nh;
  const size_t need = sf_gemv_ws_layout(n_ops, K, k_sel, &o_sel, &o_hk, &o_hs, &o_nh);
  SF_REQUIRE(ws->bytes >= need, SF_ENOMEM, "workspace too small");
  a.x = x_f16;
  a.sel_in = sel_in;
  a.sel_out = sel_out;
  a.ctl = (WsControl*)ws->base;
  a.ws_sel = (int32_t*)(ws->base + o_sel);
  a.ws_hit_k = (int32_t*)(ws->base + o_hk);
  a.ws_hit_slot = (int32_t*)(ws->base + o_hs);
  a.ws_nhit = (int32_t*)(ws->base + o_nh);
  a.n_ops = n_ops;
  a.k_in = (int32_t)K;
  a.batch = batch;
  a.k_sel = k_sel;
  a.r = f.r;
  a.total_tiles = tiles;
  hipStream_t s = (hipStream_t)stream;
  // two batch rows per launch when both fit the LDS staging of x, else one
  const int max_nb = ((size_t)2 * K * 2 + 2 * K * 4 / 16 + 32 * (K / 128) * 4 + SW * HIT_CAP * 4) <= 52 * 1024 ? 2 : 1;
  for (int b0 = 0; b0 < batch; b0 += max_nb) {
    const int nb = (batch - b0) >= max_nb ? max_nb : 1;
    a.batch_off = b0;
    a.do_log = b0 == 0;
    sf_status st = dispatch_b(a, f.b, rpw, nb, s);
    if (st != SF_OK) return st;
  }
  return SF_OK;
}
