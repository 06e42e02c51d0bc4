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
// A call computes, for up to SF_MAX_OPS matrices that share x:
//   * select (one 1024-thread workgroup, its own launch): the channel selection
//     (top-k of max-over-batch |x|, ties to the lower index) by a two-pass LDS
//     radix select, and its cache lookup per matrix, into the workspace.  On its
//     own the workgroup has the CU to itself; inside the streaming launch the same
//     few thousand dependent LDS steps run several times slower;
//   * gemv: the resident GEMV, streamed from HBM with 16-byte loads, codes
//     expanded into fp16 lanes by mask-and-or into the mantissa (value 1 + c/2^b)
//     and reduced with v_dot2_f32_f16 (sum_k c*x = 2^b * (dot - sum_k x) per
//     chunk), plus the sparse refinement delta of each row tile before it is
//     written: the refinement words of the tile's rows in every hit slot are
//     requested when the tile starts and consumed after its chunks.
#include <algorithm>
#include <cstddef>

#include "sf_internal.h"

#define SF_MAX_OPS 4

namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }

constexpr int SEL_NT = 1024;          // threads of the selection workgroup
constexpr int MAX_SEL_K = 8 * SEL_NT * 4;  // k_in with a computed selection: 4 x 8 channels per thread

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
  int32_t* ws_sel;   // [k_sel]: selection, ascending
  int32_t* ws_slot;  // [n_ops][k_sel]: slot per op, -1 = miss
  int32_t n_ops, k_in, batch, batch_off, k_sel, r, total_tiles, hits_in_lds;
  // batched (MFMA) variant: channel slices per row block, groups per slice, hit
  // capacity per slice, padded rows, slice partials [ns][batch][rows_pad], and one
  // counter per row block
  int32_t ns, gs, nhp, rows_pad;
  int32_t report;  // fused kernel: report the selection, hits and lookup log
  float* part;
  uint32_t* ctr;
  // overlapped kernel: workgroup 0 selects (sel_wg = 1) and publishes through the
  // workspace control words ctl (WsControl: sel_state, done, timeout)
  int32_t sel_wg;
  uint32_t* ctl;
};

// ---- code layouts ----------------------------------------------------------------
// A "chunk" is the run of codes one lane loads at once.  Pairs are the (k0, k1)
// channel pairs that one v_dot2 consumes; x is staged in LDS in pair order.

// b in {1, 2, 4, 8}: a 16-byte chunk of 4 words, P = 32/b codes per word.  Codes i
// and i + P/2 of a word are 16 bits apart, so one shift and one and-or put both in
// the top mantissa bits of the two fp16 halves.
// Constants of the code expansion held in VGPRs: with both in VGPRs the mask-and-or
// is one v_and_or_b32 (a 32-bit literal cannot be a VOP3 operand here, which would
// split it into v_and_b32 + v_or_b32).
struct PairK {
  uint32_t m, e;
};
__device__ __forceinline__ PairK pair_k(uint32_t m) {
  PairK k{m, 0x3C003C00u};
  asm volatile("" : "+v"(k.m), "+v"(k.e));
  return k;
}

template <int B>
struct CodecPow2 {
  static constexpr int WORDS = 4;
  static constexpr int CODES = 32 * WORDS / B;
  static constexpr int PAIRS = CODES / 2;
  static constexpr int P = 32 / B, HP = P / 2;
  // pair index and half of channel kk (0 <= kk < CODES) of a chunk
  __device__ static __forceinline__ void locate(int kk, int* j, int* hi) {
    const int w = kk / P, q = kk % P;
    *hi = q >= HP;
    *j = w * HP + (q - (*hi) * HP);
  }
  // channels (within the chunk) of the low and high half of pair j
  __host__ __device__ static constexpr int lo(int j) { return (j / HP) * P + j % HP; }
  __host__ __device__ static constexpr int hi(int j) { return (j / HP) * P + HP + j % HP; }
  __device__ static __forceinline__ uint32_t pair(const uint32_t* w, int j) {
    const int wi = j / HP, i = j % HP;
    const int sh = (10 - B) - i * B;
    const uint32_t t = sh >= 0 ? (w[wi] << sh) : (w[wi] >> (-sh));
    constexpr uint32_t m = ((1u << B) - 1u) << (10 - B);
    return (t & (m | (m << 16))) | 0x3C003C00u;
  }
  __device__ static __forceinline__ PairK consts() {
    constexpr uint32_t m = ((1u << B) - 1u) << (10 - B);
    return pair_k(m | (m << 16));
  }
  __device__ static __forceinline__ uint32_t pair(const uint32_t* w, int j, const PairK& k) {
    const int wi = j / HP, i = j % HP;
    const int sh = (10 - B) - i * B;
    const uint32_t t = sh >= 0 ? (w[wi] << sh) : (w[wi] >> (-sh));
    return (t & k.m) | k.e;
  }
};

// b in {3, 5, 6, 7}: a chunk is 32 codes = b words, codes straddle word boundaries;
// pairs are consecutive channels.
template <int B>
struct CodecStream {
  static constexpr int WORDS = B;
  static constexpr int CODES = 32;
  static constexpr int PAIRS = 16;
  __device__ static __forceinline__ void locate(int kk, int* j, int* hi) {
    *j = kk >> 1;
    *hi = kk & 1;
  }
  __host__ __device__ static constexpr int lo(int j) { return 2 * j; }
  __host__ __device__ static constexpr int hi(int j) { return 2 * j + 1; }
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
  __device__ static __forceinline__ PairK consts() { return pair_k(0u); }
  __device__ static __forceinline__ uint32_t pair(const uint32_t* w, int j, const PairK& k) {
    const uint32_t c0 = code(w, 2 * j), c1 = code(w, 2 * j + 1);
    return ((c0 | (c1 << 16)) << (10 - B)) | k.e;
  }
};

// Words per chunk of x pairs in LDS: the pairs plus 4 words of padding, so that the
// lanes' 16-byte reads of consecutive chunks start in different banks.
template <class C>
__host__ __device__ constexpr int x_chunk_words() { return C::PAIRS + 4; }

// ---- selection + lookup (one 1024-thread workgroup) ----------------------------------
// Wave 0 scans NBIN = 64 * PER histogram bins from the top: the largest bin whose
// suffix count reaches `need`; lds[20] = bin, lds[21] = count above it.
template <int PER>
__device__ __forceinline__ void wave_threshold(const uint32_t* h, int need, int* lds) {
  constexpr int NBIN = 64 * PER;
  const int lane = threadIdx.x & 63;
  int c[PER], s = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = (int)h[NBIN - 1 - PER * lane - i];
    s += c[i];
  }
  int incl = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  int run = incl - s;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (run < need && run + c[i] >= need) {
      lds[20] = NBIN - 1 - PER * lane - i;
      lds[21] = run;
    }
    run += c[i];
  }
}

// number of set bits of m in the lanes below this one
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Channel-order prefix of per-channel flags f[q] (q = 0..7: this thread's 8
// consecutive channels) over the whole workgroup: returns the number of flags in
// earlier channels; *total = all flags.  One LDS round (lds[0..15]).
template <int NW = SEL_NT / 64>
__device__ __forceinline__ int blk_flag_prefix(const bool (&f)[8], int* lds, int* total) {
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

// Keys are max over the batch of |x| as 15-bit fp16 patterns, which order like the
// values.  Thread t holds channels 8m..8m+7 for m = t + 1024 i, two per register
// (word 4i + q: channel 8m + 2q low half, 8m + 2q + 1 high half).  The k-th largest
// key T comes from two histogram passes (top 8 bits, then the low 7), each wave
// counting into its own LDS histogram (the keys concentrate in a few bins, so one
// shared histogram would serialise the atomics) before the 16 are summed; then,
// per i, ballots place the keys above T and the first `need` keys equal to T
// (lowest channels first) in channel order.
__global__ __launch_bounds__(SEL_NT) void gemv_select_kernel(GemvArgs a) {
  constexpr int NW = SEL_NT / 64;
  __shared__ uint32_t whist[NW][256];
  __shared__ uint32_t hist[384];
  __shared__ int lds[24];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.k_in, ks = a.k_sel;
  int32_t* sel = a.ws_sel;
  SF_TS(6);
  if (a.sel_in) {
    for (int j = tid; j < ks; j += SEL_NT) sel[j] = a.sel_in[j];
  } else if (ks >= K) {
    for (int j = tid; j < ks; j += SEL_NT) sel[j] = j;
  } else {
    constexpr int MI = 4;
    uint32_t kw[4 * MI];
#pragma unroll
    for (int i = 0; i < 4 * MI; ++i) kw[i] = 0;
    for (int bb = 0; bb < a.batch; ++bb) {
      const u32x4* xr = (const u32x4*)(a.x + (size_t)bb * K);
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int m = tid + SEL_NT * i;
        if (m < K / 8) {
          const u32x4 v = xr[m];
          const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t x2 = wv[q] & 0x7FFF7FFFu;
            kw[4 * i + q] = max(kw[4 * i + q] & 0xFFFFu, x2 & 0xFFFFu) | (max(kw[4 * i + q] >> 16, x2 >> 16) << 16);
          }
        }
      }
    }
    uint32_t* wh = whist[wave];
    for (int i = lane; i < 256; i += 64) wh[i] = 0;
    __syncthreads();
    SF_TS(7);
#pragma unroll
    for (int i = 0; i < MI; ++i)
      if (tid + SEL_NT * i < K / 8)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          atomicAdd(&wh[(kw[4 * i + q] & 0xFFFFu) >> 7], 1u);
          atomicAdd(&wh[kw[4 * i + q] >> 23], 1u);
        }
    __syncthreads();
    if (tid < 256) {
      uint32_t c = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) c += whist[w][tid];
      hist[tid] = c;
    }
    __syncthreads();
    for (int i = lane; i < 128; i += 64) wh[i] = 0;  // every wave has been summed
    if (tid < 64) wave_threshold<4>(hist, ks, lds);
    __syncthreads();
    const uint32_t b1 = (uint32_t)lds[20];
    int need = ks - lds[21];
#pragma unroll
    for (int i = 0; i < MI; ++i)
      if (tid + SEL_NT * i < K / 8)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo = kw[4 * i + q] & 0xFFFFu, hi = kw[4 * i + q] >> 16;
          if ((lo >> 7) == b1) atomicAdd(&wh[lo & 127u], 1u);
          if ((hi >> 7) == b1) atomicAdd(&wh[hi & 127u], 1u);
        }
    __syncthreads();
    if (tid < 128) {
      uint32_t c = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) c += whist[w][tid];
      hist[256 + tid] = c;
    }
    __syncthreads();
    if (tid < 64) wave_threshold<2>(hist + 256, need, lds);
    __syncthreads();
    const uint32_t T = (b1 << 7) | (uint32_t)lds[20];
    need -= lds[21];  // keys equal to T that are taken, lowest channels first
    SF_TS(11);
    int written = 0, eq_seen = 0;
    for (int i = 0; i < MI; ++i) {
      if (SEL_NT * 8 * i >= K) break;
      const bool ok = tid + SEL_NT * i < K / 8;
      bool gt[8], eq[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = kw[4 * i + q] & 0xFFFFu, hi = kw[4 * i + q] >> 16;
        gt[2 * q] = ok && lo > T;
        gt[2 * q + 1] = ok && hi > T;
        eq[2 * q] = ok && lo == T;
        eq[2 * q + 1] = ok && hi == T;
      }
      // equal keys before each of this thread's channels, then the taken ones
      int tot_eq;
      int eb = eq_seen + blk_flag_prefix(eq, lds, &tot_eq);
      bool take[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        take[q] = gt[q] || (eq[q] && eb < need);
        eb += eq[q];
      }
      int tot;
      int pos = written + blk_flag_prefix(take, lds, &tot);
      const int k0 = 8 * (tid + SEL_NT * i);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (take[q]) {
          if (pos < ks) sel[pos] = k0 + q;
          ++pos;
        }
      written += tot;
      eq_seen += tot_eq;
    }
  }
  // sel[] is read back below by other threads of this workgroup
  __syncthreads();
  SF_TS(12);
  // lookups, per op, in selection order (with the report and the lookup log)
  if (tid < a.n_ops) {
    const PoolDev& pool = a.ops[tid].pool;
    int base = -1;
    if (pool.log_count) {
      const uint32_t bse = atomicAdd(pool.log_count, (uint32_t)ks);
      base = (bse + (uint32_t)ks <= (uint32_t)pool.log_cap) ? (int)bse : -1;
    }
    lds[tid] = base;
  }
  __syncthreads();
  for (int j = tid; j < ks; j += SEL_NT) {
    const int k = sel[j];
    if (a.sel_out) a.sel_out[j] = k;
    int slot[SF_MAX_OPS];
#pragma unroll
    for (int op = 0; op < SF_MAX_OPS; ++op)  // all loads first
      slot[op] = (op < a.n_ops && a.ops[op].pool.unit2slot && k >= 0 && k < K) ? a.ops[op].pool.unit2slot[k] : -1;
#pragma unroll
    for (int op = 0; op < SF_MAX_OPS; ++op) {
      if (op >= a.n_ops) break;
      a.ws_slot[op * ks + j] = slot[op];
      if (a.ops[op].hit_out) a.ops[op].hit_out[j] = slot[op];
      if (lds[op] >= 0) {
        a.ops[op].pool.log_units[lds[op] + j] = k;
        a.ops[op].pool.log_slots[lds[op] + j] = slot[op];
      }
    }
  }
  SF_TS(13);
}

// ---- the GEMV kernel -------------------------------------------------------------
// Persistent workgroups, 4 waves each: row tiles of 4R rows (R per wave) are dealt
// round-robin; lane l of a wave owns chunks l, l+64, ... of each of the wave's R
// rows.  The first chunk is requested before x is staged in LDS (16-byte loads
// scattered into pair order, chunk sums by shuffles), the next tile's first chunk
// before the current tile is reduced.  With refinement the hit list (selection
// and slots, from the select launch) is copied to LDS with the staging; each tile
// requests the refinement words of its rows in HPF hits per lane when it starts,
// records its rows' scale words per group while streaming, and adds the deltas
// before the wave reduction.  NB batch rows [batch_off, batch_off + NB) per launch.
// Dynamic LDS: x pairs [NB][K/2] | x chunk sums [NB][nchunks] | scale words
// [4][R][K/128] | (selection [k_sel] | slots [n_ops][k_sel] when they fit).
constexpr int HPF = 8;  // hits per lane whose refinement words are requested at tile start
// Words of a tile's refinement window: 4R rows of up to 7 bits, plus misalignment.
__host__ __device__ constexpr int wtm_of(int R) { return (31 + 4 * R * 7 + 31) / 32; }

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

// The same, unconditionally: rows past the matrix read its last row (their sums
// are never written); the caller clamps c.
template <class C, int R>
__device__ __forceinline__ void load_chunk_clamped(const GemvOpDev& o, int row0, int c, size_t rowbytes, int ngr,
                                                   uint32_t (&cw)[R][C::WORDS], uint32_t (&szw)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = min(row0 + r, o.n_out - 1);
    const uint32_t* src = (const uint32_t*)(o.res + row * rowbytes + (size_t)c * (4 * C::WORDS));
    if constexpr (C::WORDS == 4) {
      const u32x4 v = __builtin_nontemporal_load((const u32x4*)src);
      cw[r][0] = v.x; cw[r][1] = v.y; cw[r][2] = v.z; cw[r][3] = v.w;
    } else {
#pragma unroll
      for (int w = 0; w < C::WORDS; ++w) cw[r][w] = __builtin_nontemporal_load(src + w);
    }
    szw[r] = o.sz[(size_t)row * ngr + (c * C::CODES) / 128];
  }
}

__device__ __forceinline__ int op_of_tile(const GemvArgs& a, int tile_g) {
  int op = 0;
  for (int i = 1; i < a.n_ops; ++i)
    if (tile_g >= a.ops[i].tile_begin) op = i;
  return op;
}

// bits [p, p + width) of the 64-bit (w1:w0)
__device__ __forceinline__ uint32_t bits64(uint32_t w0, uint32_t w1, int p, int width) {
  return (uint32_t)((((uint64_t)w1 << 32) | w0) >> p) & ((1u << width) - 1u);
}

template <class C, int B, int R, int NB>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a) {
  extern __shared__ uint32_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.k_in;
  const int nchunks = K / C::CODES;
  const int xpairs = K / 2;
  const int rows_wg = 4 * R;
  const int ngr = K / 128;
  const int ks = a.k_sel;
  uint32_t* xs = smem;                                   // [NB][K/2] fp16 pairs
  float* xsum = (float*)(smem + NB * xpairs);            // [NB][nchunks]
  uint32_t* s_szw = (uint32_t*)(xsum + NB * nchunks);    // [4][R][ngr]
  int32_t* l_sel = (int32_t*)(s_szw + (ks > 0 ? 4 * R * ngr : 0));  // [k_sel] if hits_in_lds
  int32_t* l_slot = l_sel + ks;                                     // [n_ops][k_sel]
  const bool refine = ks > 0;
  const int32_t* hsel = a.hits_in_lds ? l_sel : a.ws_sel;
  const int32_t* hslot = a.hits_in_lds ? l_slot : a.ws_slot;
  const size_t rowbytes = (size_t)K * B / 8;

  SF_TS(0);
  // request the first chunk of this wave
  uint32_t cw[R][C::WORDS];
  uint32_t szw[R];
  bool have = false;
  if ((int)blockIdx.x < a.total_tiles && lane < nchunks) {
    const int op = op_of_tile(a, blockIdx.x);
    load_chunk<C, R>(a.ops[op], (blockIdx.x - a.ops[op].tile_begin) * rows_wg + wave * R, lane, rowbytes, ngr,
                     cw, szw);
    have = true;
  }
  // the hit list, when it fits in LDS
  if (refine && a.hits_in_lds) {
    for (int j = tid; j < ks * (1 + a.n_ops); j += 256) l_sel[j] = j < ks ? a.ws_sel[j] : a.ws_slot[j - ks];
  }
  // stage x in pair order (16-byte loads, all issued first; 2-byte LDS stores); the
  // CODES/8 threads that load one chunk sum it with shuffles
  {
    uint16_t* xh = (uint16_t*)xs;
    constexpr int TPC = C::CODES / 8;  // threads per chunk
    constexpr int XB = 8;              // 16-byte x loads in flight per thread
    for (int m0 = 0; m0 < K / 8; m0 += 256 * XB) {
      u32x4 xv[NB][XB];
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        const u32x4* xr = (const u32x4*)(a.x + (size_t)(a.batch_off + bb) * K);
#pragma unroll
        for (int i = 0; i < XB; ++i) {
          const int m = m0 + 256 * i + tid;
          if (m < K / 8) xv[bb][i] = xr[m];
        }
      }
#pragma unroll
      for (int i = 0; i < XB; ++i) {
        const int m = m0 + 256 * i + tid;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
          float part = 0.f;
          if (m < K / 8) {
            const uint32_t wds[4] = {xv[bb][i].x, xv[bb][i].y, xv[bb][i].z, xv[bb][i].w};
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
  }
  __syncthreads();
  SF_TS(1);

  const float scl = (float)(1u << (a.r + B));
  const int r = a.r;
  uint32_t* szrow = s_szw + wave * R * ngr;  // this wave's rows' scale words, [R][ngr]
  for (int tile_g = blockIdx.x; tile_g < a.total_tiles; tile_g += gridDim.x) {
    const int op = op_of_tile(a, tile_g);
    const GemvOpDev& o = a.ops[op];
    const int tile = tile_g - o.tile_begin;
    const int row0 = tile * rows_wg + wave * R;
    // the wave's R rows occupy bits [row0 * r, (row0 + R) * r) of every unit
    const int ubit = row0 * r, uwi = ubit >> 5, uoff = ubit & 31;
    const int wpu = o.pool.unit_bytes >> 2;
    const uint32_t* units = (const uint32_t*)o.pool.slots;
    const int32_t* slots = hslot + op * ks;
    // refinement words of the first HPF hits per lane, requested now, used after
    // the chunks
    int pslot[HPF];
    uint32_t pw0[HPF], pw1[HPF];
    if (refine) {
#pragma unroll
      for (int i = 0; i < HPF; ++i) {
        const int j = lane + 64 * i;
        pslot[i] = j < ks ? slots[j] : -1;
        pw0[i] = pw1[i] = 0u;
        if (pslot[i] >= 0) {
          const uint32_t* u = units + (size_t)pslot[i] * wpu;
          if (uwi < wpu) pw0[i] = u[uwi];
          if (uwi + 1 < wpu) pw1[i] = u[uwi + 1];
        }
      }
    }
    const PairK pk = C::consts();
    float acc[NB][R];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
      for (int rr = 0; rr < R; ++rr) acc[bb][rr] = 0.f;
    for (int c = lane; c < nchunks; c += 64) {
      if (!have) load_chunk<C, R>(o, row0, c, rowbytes, ngr, cw, szw);
      have = false;
      if (refine && (c * C::CODES) % 128 == 0)
#pragma unroll
        for (int rr = 0; rr < R; ++rr) szrow[rr * ngr + (c * C::CODES) / 128] = szw[rr];
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        const u32x4* xp = (const u32x4*)(xs + bb * xpairs + c * C::PAIRS);
        float d[R];
#pragma unroll
        for (int rr = 0; rr < R; ++rr) d[rr] = 0.f;
#pragma unroll
        for (int jb = 0; jb < C::PAIRS / 4; ++jb) {
          const u32x4 xv = xp[jb];
#pragma unroll
          for (int rr = 0; rr < R; ++rr)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              d[rr] = __builtin_amdgcn_fdot2(as_h2(C::pair(cw[rr], 4 * jb + q, pk)), as_h2(xv[q]), d[rr], false);
        }
        const float X = xsum[bb * nchunks + c];
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
          const float s = sf_h2f(szw[rr]), z = sf_h2f(szw[rr] >> 16);
          acc[bb][rr] += (s * scl) * (d[rr] - X) + z * X;
        }
      }
    }
    // refinement of the hit channels: + x_k * s[row][k/128] * c_lo[row][k]
    if (refine) {
      // the rows' scale words were recorded by other lanes of this wave
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      for (int j = lane; j < ks; j += 64) {
        const int i = (j - lane) >> 6;
        int slot;
        uint32_t w0, w1, w2 = 0u;
        if (i < HPF) {
          slot = pslot[0];
          w0 = pw0[0];
          w1 = pw1[0];
#pragma unroll
          for (int q = 1; q < HPF; ++q)
            if (q == i) {
              slot = pslot[q];
              w0 = pw0[q];
              w1 = pw1[q];
            }
          if (slot >= 0 && uoff + R * r > 64 && uwi + 2 < wpu) w2 = units[(size_t)slot * wpu + uwi + 2];
        } else {
          slot = slots[j];
          w0 = w1 = 0u;
          if (slot >= 0) {
            const uint32_t* u = units + (size_t)slot * wpu;
            if (uwi < wpu) w0 = u[uwi];
            if (uwi + 1 < wpu) w1 = u[uwi + 1];
            if (uwi + 2 < wpu) w2 = u[uwi + 2];
          }
        }
        if (slot < 0) continue;
        const int k = hsel[j];
        const int c = k / C::CODES, kk = k - c * C::CODES;
        int jj, hi;
        C::locate(kk, &jj, &hi);
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
          const int p = uoff + rr * r;
          const uint32_t clo = p + r <= 64 ? bits64(w0, w1, p, r) : bits64(w1, w2, p - 32, r);
          const float sv = sf_h2f(szrow[rr * ngr + (k >> 7)]) * (float)clo;
#pragma unroll
          for (int bb = 0; bb < NB; ++bb) {
            const h2_t xh = as_h2(xs[bb * xpairs + c * C::PAIRS + jj]);
            acc[bb][rr] = fmaf(hi ? (float)xh.y : (float)xh.x, sv, acc[bb][rr]);
          }
        }
      }
    }
    // request the next tile's first chunk before reducing this one
    const int next = tile_g + gridDim.x;
    if (next < a.total_tiles && lane < nchunks) {
      const int op2 = op_of_tile(a, next);
      load_chunk<C, R>(a.ops[op2], (next - a.ops[op2].tile_begin) * rows_wg + wave * R, lane, rowbytes, ngr,
                       cw, szw);
      have = true;
    }
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        float v = acc[bb][rr];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        acc[bb][rr] = v;
      }
    if (lane == 0) {
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        const int row = row0 + rr;
        if (row < o.n_out)
#pragma unroll
          for (int bb = 0; bb < NB; ++bb) o.y[(size_t)(a.batch_off + bb) * o.n_out + row] = acc[bb][rr];
      }
    }
    // the next tile records its scale words over this one's
    if (refine) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  SF_TS(3);
}




// ---- cross-lane sums by DPP -------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF,
                                                               false));
}
// Sum over groups of N = 2, 4, 8 or 16 consecutive lanes; every lane of a group
// gets its group's sum (quad swaps, then half-row and row mirrors).
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) v += dpp_mov<0x141>(v);  // row_half_mirror
  if constexpr (N >= 16) v += dpp_mov<0x140>(v); // row_mirror
  return v;
}
// Sum over the wave, complete in lane 63 (rows 1 and 3 take row 0 / row 2 by
// row_bcast15, then row 3 takes rows 0-1 by row_bcast31).
__device__ __forceinline__ float wave_sum63(float v) {
  v = group_sum<16>(v);
  v += dpp_mov<0x142, 0xA>(v);
  v += dpp_mov<0x143, 0xC>(v);
  return v;
}

// Inclusive prefix sum over the 64 lanes: row-local Hillis-Steele steps (row_shr
// 1, 2, 4, 8 with zeros shifted in), then rows 1 and 3 add the totals of rows 0
// and 2 (row_bcast15) and rows 2 and 3 the total of rows 0-1 (row_bcast31).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_mov_z(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, true);
}
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_mov_z<0x111>(v);  // row_shr:1
  v += dpp_mov_z<0x112>(v);  // row_shr:2
  v += dpp_mov_z<0x114>(v);  // row_shr:4
  v += dpp_mov_z<0x118>(v);  // row_shr:8
  v += dpp_mov_z<0x142, 0xA>(v);
  v += dpp_mov_z<0x143, 0xC>(v);
  return v;
}

// Largest bin b of the sum of four per-wave histograms h[w][0..nbin) whose suffix
// count (bins >= b) reaches `need`; *above = count in bins above b.  Every wave
// computes it from the histograms itself.  nbin = 256 or 128.
__device__ __forceinline__ void wave_threshold4(const uint32_t (*h)[256], int nbin, int need, int* bin,
                                                int* above) {
  const int lane = threadIdx.x & 63;
  const int per = nbin / 64;
  int c[4] = {0, 0, 0, 0}, s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i < per) {
      const int b = nbin - 1 - per * lane - i;
      c[i] = (int)((h[0][b] + h[1][b]) + (h[2][b] + h[3][b]));
      s += c[i];
    }
  const int incl = wave_incl_scan(s);
  int run = incl - s, hit = -1, hab = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i < per) {
      if (run < need && run + c[i] >= need) {
        hit = nbin - 1 - per * lane - i;
        hab = run;
      }
      run += c[i];
    }
  const uint64_t m = __ballot(hit >= 0);
  const int src = m ? __builtin_ctzll(m) : 0;
  *bin = __builtin_amdgcn_readlane(hit, src);
  *above = __builtin_amdgcn_readlane(hab, src);
}
__device__ __forceinline__ void wave_threshold4(const uint32_t (*h)[128], int nbin, int need, int* bin,
                                                int* above) {
  const int lane = threadIdx.x & 63;
  int c[2], s = 0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int b = 127 - 2 * lane - i;
    c[i] = (int)((h[0][b] + h[1][b]) + (h[2][b] + h[3][b]));
    s += c[i];
  }
  (void)nbin;
  const int incl = wave_incl_scan(s);
  int run = incl - s, hit = -1, hab = 0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (run < need && run + c[i] >= need) {
      hit = 127 - 2 * lane - i;
      hab = run;
    }
    run += c[i];
  }
  const uint64_t m = __ballot(hit >= 0);
  const int src = m ? __builtin_ctzll(m) : 0;
  *bin = __builtin_amdgcn_readlane(hit, src);
  *above = __builtin_amdgcn_readlane(hab, src);
}

// Keys of 8 channels (4 words of two 15-bit keys): (#keys > T) | (#keys == T) << 16.
__device__ __forceinline__ uint32_t gt_eq_count(const uint32_t* kp, uint32_t T) {
  const u32x4 kv = *(const u32x4*)kp;
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t lo = kv[q] & 0xFFFFu, hi = kv[q] >> 16;
    gt += (lo > T) + (hi > T);
    eq += (lo == T) + (hi == T);
  }
  return gt | (eq << 16);
}

// Sum of c (0 <= c < 256) over the lanes below this one, by ballots of its bits;
// *total = the sum over the wave.
__device__ __forceinline__ uint32_t wave_excl_sum8(uint32_t c, uint32_t* total) {
  uint32_t ex = 0, tot = 0;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const uint64_t m = __ballot((c >> b) & 1u);
    ex += (uint32_t)lanes_below(m) << b;
    tot += (uint32_t)__popcll(m) << b;
  }
  *total = tot;
  return ex;
}

// Sum of c (0 <= c < 16) over the lanes below this one, by ballots of its bits;
// *total = the sum over the wave.
__device__ __forceinline__ uint32_t wave_excl_small(uint32_t c, uint32_t* total) {
  uint32_t ex = 0, tot = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint64_t m = __ballot((c >> b) & 1u);
    ex += (uint32_t)lanes_below(m) << b;
    tot += (uint32_t)__popcll(m) << b;
  }
  *total = tot;
  return ex;
}


size_t fused_lds_bytes(int k_in, int codes, int nb, int k_sel, int rpw) {
  size_t w = (size_t)nb * (k_in / codes) * (codes / 2 + 4) + (size_t)nb * (((k_in / codes) + 3) & ~3);
  if (k_sel > 0) w += (size_t)(k_in / 2) + (size_t)4 * rpw * (k_in / 128) + (size_t)k_sel + (size_t)(k_in / 16);
  return w * 4;
}

size_t split_sel_lds_words(int k_in, int k_sel) {
  return (size_t)(k_in / 2) + 2 * (size_t)(k_in / 32) + (((size_t)k_sel + 3) & ~(size_t)3) + 4 * 256 + 4 * 128 + 16;
}

// The fused kernel with workgroup 0 selecting: x staged as in the fused kernel, the
// hits (channel, x, the tile's window words) after the scale words; the selecting
// workgroup's own layout may be larger.
size_t fused_sw_lds_bytes(int k_in, int codes, int nb, int k_sel, int rpw) {
  size_t tile = (size_t)nb * (k_in / codes) * (codes / 2 + 4) + (size_t)nb * (((k_in / codes) + 3) & ~3);
  if (k_sel > 0) tile += (size_t)4 * rpw * (k_in / 128) + (size_t)k_sel * (1 + nb + wtm_of(rpw));
  const size_t sel = k_sel > 0 ? split_sel_lds_words(k_in, k_sel) : 0;
  return std::max(tile, sel) * 4;
}

// ---- batch-1/2 GEMV with one selecting workgroup ---------------------------------
// Workgroup 0 selects the channels (the same two-pass radix select as the other
// kernels, on its 4 waves), looks up their slots per matrix and publishes both
// through the workspace with agent-scope stores before raising sel_state.  Every
// other workgroup is one row tile (4 waves x R rows) and needs the selection only
// at its end: it requests x and the tile's codes, stages x in LDS (pair order,
// chunk stride padded by 4 words so that the lanes' 16-byte reads of consecutive
// chunks fall in different banks), runs the resident dot products, then waits for
// the selection, fetches the refinement words of its rows at the hit channels and
// adds them before the row sums (DPP) are written.  The last tile to read the
// selection resets sel_state for the next launch.
// Dynamic LDS, tiles: x pairs [NB][nchunks][PAIRS + 4] | chunk sums [NB][nchunks]
// | scale words [4][R][K/128]; selector: keys [K/2] | bitmaps [2][K/32] |
// selection [k_sel] | histograms [4][256] + [4][128] | 16 words.
size_t split_lds_bytes(int k_in, int pairs, int codes, int nb, int k_sel, int rpw) {
  (void)pairs;
  (void)codes;
  size_t tile = 0;
  if (k_sel > 0) tile += (size_t)4 * rpw * (k_in / 128) + (size_t)k_sel * (1 + nb + (31 + 4 * rpw * 7 + 31) / 32);
  size_t sel = 0;
  if (k_sel > 0) sel = (size_t)(k_in / 2) + 2 * (size_t)(k_in / 32) + (((size_t)k_sel + 3) & ~(size_t)3) + 4 * 256 + 4 * 128 + 16;
  return std::max(tile, sel) * 4;
}

// Copies of the published words (tile t reads copy t mod SPLIT_COPIES), and the
// stride of one copy in words.
constexpr int SPLIT_COPIES = 8;
__host__ __device__ inline int split_copy_words(int k_sel, int n_ops) { return ((k_sel * (1 + n_ops)) + 31) & ~31; }

// A tile that has seen the flag counts itself (no return value).
__device__ __forceinline__ void count_reader(const GemvArgs& a, int grp) {
  uint32_t* c = a.ctl + offsetof(WsControl, rd_ctr) / 4 + 32 * grp;
  (void)__hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Lane 0 of a wave polls its group's flag (bounded); the result is wave-uniform.
__device__ __forceinline__ bool wait_published(const GemvArgs& a, int grp) {
  const uint32_t* f = a.ctl + offsetof(WsControl, sel_flag) / 4 + 32 * grp;
  for (uint32_t it = 0;; ++it) {
    uint32_t v = 0u;
    if ((threadIdx.x & 63) == 0) v = sf_get(f);
    if (__builtin_amdgcn_readfirstlane(v) != 0u) return true;
    if (it >= (1u << 22)) {
      if ((threadIdx.x & 63) == 0) sf_put(a.ctl + 2, 1u);
      return false;
    }
    __builtin_amdgcn_s_sleep(8);
  }
}

// Workgroup 0, after publishing: waits until every tile has seen the flag, then
// lowers the flags and clears the counts for the next launch.
__device__ __forceinline__ void split_retire(const GemvArgs& a) {
  const int tid = threadIdx.x;
  if (tid >= 64) return;
  uint32_t* ctr = a.ctl + offsetof(WsControl, rd_ctr) / 4 + 32 * tid;
  uint32_t* flag = a.ctl + offsetof(WsControl, sel_flag) / 4 + 32 * tid;
  const uint32_t tiles = (uint32_t)a.total_tiles;
  const uint32_t want = (uint32_t)tid < tiles ? (tiles - (uint32_t)tid + 63u) / 64u : 0u;
  for (uint32_t it = 0;; ++it) {
    if (__all(sf_get(ctr) >= want)) break;
    if (it >= (1u << 22)) {
      sf_put(a.ctl + 2, 1u);
      return;  // the timeout flag reports it
    }
    __builtin_amdgcn_s_sleep(8);
  }
  sf_put(flag, 0u);
  sf_put(ctr, 0u);
}

// Workgroup 0: selection into l_sel (LDS), then the lookups, the published copy in
// the workspace and the reports.
__device__ __forceinline__ void split_select_and_publish(const GemvArgs& a, uint32_t* smem) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.k_in, ks = a.k_sel, n8 = K / 8;
  uint32_t* keys = smem;                       // [K/2]
  uint32_t* bm_sure = keys + K / 2;            // [K/32]
  uint32_t* bm_bnd = bm_sure + K / 32;         // [K/32]
  int32_t* l_sel = (int32_t*)(bm_bnd + K / 32);  // [ks]
  uint32_t (*whist)[256] = (uint32_t (*)[256])(l_sel + ((ks + 3) & ~3));
  uint32_t (*whist2)[128] = (uint32_t (*)[128])(whist[4]);
  int* sc = (int*)(whist2[4]);  // [16]
  SF_TS(6);
  if (a.sel_in) {
    for (int j = tid; j < ks; j += 256) l_sel[j] = a.sel_in[j];
  } else if (ks >= K) {
    for (int j = tid; j < ks; j += 256) l_sel[j] = j;
  } else {
    for (int i = lane; i < 256; i += 64) whist[wave][i] = 0u;
    for (int i = lane; i < 128; i += 64) whist2[wave][i] = 0u;
    // keys (max over the batch of |x| as 15-bit patterns) and pass 1: top 8 key bits;
    // 8 loads a thread in flight (K <= 16384 in one round)
    for (int m0 = 0; m0 < n8; m0 += 256 * 8) {
      u32x4 kv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) kv[i] = u32x4{0u, 0u, 0u, 0u};
      for (int bb = 0; bb < a.batch; ++bb) {
        const u32x4* xr = (const u32x4*)(a.x + (size_t)bb * K);
        u32x4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = xr[min(m0 + 256 * i + tid, n8 - 1)];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t x2 = v[i][q] & 0x7FFF7FFFu;
            kv[i][q] = max(kv[i][q] & 0xFFFFu, x2 & 0xFFFFu) | (max(kv[i][q] >> 16, x2 >> 16) << 16);
          }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int m = m0 + 256 * i + tid;
        if (m < n8) {
          *(u32x4*)(keys + 4 * m) = kv[i];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            atomicAdd(&whist[wave][(kv[i][q] & 0xFFFFu) >> 7], 1u);
            atomicAdd(&whist[wave][kv[i][q] >> 23], 1u);
          }
        }
      }
    }
    lds_barrier();
    SF_TS(7);
    int b1, above1;
    wave_threshold4(whist, 256, ks, &b1, &above1);
    // pass 2: low 7 bits of the keys in bin b1; bitmaps of the keys above bin b1
    // (all taken) and in bin b1
    {
      uint8_t* bs = (uint8_t*)bm_sure;
      uint8_t* bb = (uint8_t*)bm_bnd;
      for (int m = tid; m < n8; m += 256) {
        const u32x4 kv = *(const u32x4*)(keys + 4 * m);
        uint32_t sure = 0u, bnd = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t key = (kv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
          const int bin = (int)(key >> 7);
          sure |= (uint32_t)(bin > b1) << e;
          if (bin == b1) {
            bnd |= 1u << e;
            atomicAdd(&whist2[wave][key & 127u], 1u);
          }
        }
        bs[m] = (uint8_t)sure;
        bb[m] = (uint8_t)bnd;
      }
    }
    lds_barrier();
    SF_TS(11);
    int b2, above2;
    wave_threshold4(whist2, 128, ks - above1, &b2, &above2);
    const uint32_t need = (uint32_t)(ks - above1 - above2);  // keys equal to T taken, lowest channels first
    // compaction in channel order (thread t owns bitmap words [t W, t W + W))
    const int nw = K / 32, W = (nw + 255) / 256;
    const uint16_t* key16 = (const uint16_t*)keys;
    uint32_t sg[4], eqm[4], cs = 0u, ce = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sg[i] = eqm[i] = 0u;
      const int w = tid * W + i;
      if (i < W && w < nw) {
        uint32_t bnd = bm_bnd[w], gtw = 0u, eqw = 0u;
        while (bnd) {
          const int bit = __builtin_ctz(bnd);
          bnd &= bnd - 1u;
          const uint32_t lo = key16[32 * w + bit] & 127u;
          gtw |= (uint32_t)(lo > (uint32_t)b2) << bit;
          eqw |= (uint32_t)(lo == (uint32_t)b2) << bit;
        }
        sg[i] = bm_sure[w] | gtw;
        eqm[i] = eqw;
        cs += __popc(sg[i]);
        ce += __popc(eqm[i]);
      }
    }
    uint32_t ts, te;
    uint32_t sbefore = wave_excl_sum8(cs, &ts), ebefore = wave_excl_sum8(ce, &te);
    if (lane == 0) sc[wave] = (int)(ts | (te << 16));
    lds_barrier();
    for (int w = 0; w < wave; ++w) {
      sbefore += (uint32_t)sc[w] & 0xFFFFu;
      ebefore += (uint32_t)sc[w] >> 16;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t all = sg[i] | eqm[i];
      while (all) {
        const int bit = __builtin_ctz(all);
        all &= all - 1u;
        const int c = 32 * (tid * W + i) + bit;
        if ((sg[i] >> bit) & 1u) {
          l_sel[sbefore + min(ebefore, need)] = c;
          ++sbefore;
        } else {
          if (ebefore < need) l_sel[sbefore + ebefore] = c;
          ++ebefore;
        }
      }
    }
  }
  lds_barrier();
  SF_TS(12);
  // the published words first: the channels and, per matrix without resident
  // units, the slots, in SPLIT_COPIES copies
  uint32_t* hw = a.ctl + offsetof(WsControl, hit) / 4;
  const int cst = split_copy_words(ks, a.n_ops);
  for (int j = tid; j < ks; j += 256) {
    const int k = l_sel[j];
#pragma unroll
    for (int c = 0; c < SPLIT_COPIES; ++c) sf_put(hw + c * cst + j, (uint32_t)k);
#pragma unroll
    for (int op = 0; op < SF_MAX_OPS; ++op) {
      if (op >= a.n_ops) break;
      const PoolDev& pool = a.ops[op].pool;
      if (pool.resident) continue;
      const int slot = pool.unit2slot ? pool.unit2slot[k] : -1;
#pragma unroll
      for (int c = 0; c < SPLIT_COPIES; ++c) sf_put(hw + c * cst + ks * (1 + op) + j, (uint32_t)slot);
    }
  }
  // the words are complete at the coherence point before any flag goes up
  sf_drain();
  __syncthreads();
  if (tid < 64) sf_put(a.ctl + offsetof(WsControl, sel_flag) / 4 + 32 * tid, 1u);
  SF_TS(13);
  // the reports (selection, hits, lookup log: one reservation per matrix) after
  // the flags, off the tiles' path
  if (!a.report) return;
  if (tid < a.n_ops) {
    const PoolDev& pool = a.ops[tid].pool;
    int base = -1;
    if (pool.log_count) {
      const uint32_t bse = atomicAdd(pool.log_count, (uint32_t)ks);
      base = (bse + (uint32_t)ks <= (uint32_t)pool.log_cap) ? (int)bse : -1;
    }
    sc[8 + tid] = base;
  }
  lds_barrier();
  for (int j = tid; j < ks; j += 256) {
    const int k = l_sel[j];
    if (a.sel_out) a.sel_out[j] = k;
#pragma unroll
    for (int op = 0; op < SF_MAX_OPS; ++op) {
      if (op >= a.n_ops) break;
      const PoolDev& pool = a.ops[op].pool;
      const int slot = pool.resident ? k : (pool.unit2slot ? pool.unit2slot[k] : -1);
      if (a.ops[op].hit_out) a.ops[op].hit_out[j] = slot;
      const int base = sc[8 + op];
      if (base >= 0) {
        pool.log_units[base + j] = k;
        pool.log_slots[base + j] = slot;
      }
    }
  }
}


// Refinement of one row tile from workgroup 0's published selection: wave 0 waits
// for its flag group and counts the tile; the tile gathers per hit the words that
// hold its 4R rows' refinement bits (one request per hit and tile) and x at the hit
// into LDS; each wave adds x_k * s[row][k/128] * c_lo[row][k] for its R rows.
// szrow: this wave's rows' scale words [R][K/128] (LDS, complete for all lanes
// before the first barrier here); sflag: one LDS word.
template <class C, int R, int NB, int WTM>
__device__ __forceinline__ void split_refine_tile(const GemvArgs& a, const GemvOpDev& o, int op, int tile_g, int row0,
                                                  const uint32_t* szrow, int32_t* l_hk, float* l_hx, uint32_t* l_hw,
                                                  float (&acc)[NB][R], int* sflag) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ks = a.k_sel, K = a.k_in, ngr = K / 128, r = a.r;
  if (wave == 0) {
    const bool ok0 = wait_published(a, tile_g & 63);
    if (lane == 0) {
      count_reader(a, tile_g & 63);
      *sflag = ok0 ? 1 : 0;
    }
  }
  lds_barrier();
  const int tb = (tile_g - o.tile_begin) * 4 * R * r, tw0 = tb >> 5, toff = tb & 31;
  const int wt = (toff + 4 * R * r + 31) >> 5;  // words of the tile's window (<= WTM)
  const int wpu = o.pool.unit_bytes >> 2;
  const uint32_t* units = (const uint32_t*)o.pool.slots;
  const bool resident = o.pool.resident != 0;
  const bool any = *sflag != 0 && (resident || o.pool.unit2slot != nullptr);
  if (any) {
    const uint32_t* hc = a.ctl + offsetof(WsControl, hit) / 4 + (tile_g % SPLIT_COPIES) * split_copy_words(ks, a.n_ops);
    for (int j = tid; j < ks; j += 256) {
      const int k = (int)sf_get(hc + j);
      const int slot = resident ? k : (int)sf_get(hc + ks * (1 + op) + j);
      l_hk[j] = slot >= 0 ? k : -1;
      if (slot >= 0) {
        const uint32_t* u = units + (size_t)slot * wpu + tw0;
        if (wt <= 2 && tw0 + 1 < wpu && ((uintptr_t)u & 7u) == 0) {  // one 8-byte request
          const u32x2 v = *(const u32x2*)u;
          l_hw[j * WTM] = v.x;
          if (WTM > 1) l_hw[j * WTM + 1] = v.y;
        } else {
#pragma unroll
          for (int w = 0; w < WTM; ++w)
            if (w < wt) l_hw[j * WTM + w] = tw0 + w < wpu ? u[w] : 0u;
        }
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) l_hx[j * NB + bb] = sf_h2f(a.x[(size_t)(a.batch_off + bb) * K + k]);
      }
    }
  }
  lds_barrier();  // the hits
  SF_TS(5);
  if (!any) return;
  const int pw = toff + wave * R * r;  // this wave's first row in the window
  const int wi0 = pw >> 5, sh0 = pw & 31;
  if (sh0 + R * r <= 64) {
    // the wave's R * r bits lie in two consecutive window words (wave-uniform
    // position): one 64-bit shift per hit, then a field per row
    const uint32_t fmask = (1u << r) - 1u;
    for (int j = lane; j < ks; j += 64) {
      const int k = l_hk[j];
      if (k < 0) continue;
      const uint32_t lo = l_hw[j * WTM + wi0];
      const uint32_t hi = wi0 + 1 < WTM ? l_hw[j * WTM + min(wi0 + 1, WTM - 1)] : 0u;
      const uint64_t bits = ((((uint64_t)hi) << 32) | lo) >> sh0;  // a word past the window only feeds unused bits
      float xq[NB];
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) xq[bb] = l_hx[j * NB + bb];
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        const uint32_t clo = (uint32_t)(bits >> (rr * r)) & fmask;
        const float sv = sf_h2f(szrow[rr * ngr + (k >> 7)]) * (float)clo;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) acc[bb][rr] = fmaf(xq[bb], sv, acc[bb][rr]);
      }
    }
    SF_TS(9);
    return;
  }
  for (int j = lane; j < ks; j += 64) {
    const int k = l_hk[j];
    if (k < 0) continue;
    uint32_t wv[WTM];
#pragma unroll
    for (int w = 0; w < WTM; ++w) wv[w] = w < wt ? l_hw[j * WTM + w] : 0u;
    float xq[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) xq[bb] = l_hx[j * NB + bb];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      const int p = pw + rr * r, wi = p >> 5;
      uint32_t lo = wv[0], hi = wv[1 < WTM ? 1 : 0];
#pragma unroll
      for (int w = 1; w < WTM; ++w)
        if (w == wi) {
          lo = wv[w];
          hi = w + 1 < WTM ? wv[w + 1 < WTM ? w + 1 : w] : 0u;
        }
      const uint32_t clo = bits64(lo, hi, p & 31, r);
      const float sv = sf_h2f(szrow[rr * ngr + (k >> 7)]) * (float)clo;
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) acc[bb][rr] = fmaf(xq[bb], sv, acc[bb][rr]);
    }
  }
  SF_TS(9);
}

// ---- batch-1/2 GEMV with the selection in every workgroup ----------------------
// One row tile per workgroup (4 waves x R rows).  All code loads of the tile are
// issued first (a window of D chunks per lane when a row has more than 64 chunks).
// While they are in flight the workgroup stages x in LDS and selects the channels
// itself, exactly as the selection workgroup does: keys max-over-batch |x| as
// 15-bit fp16 patterns (kept in LDS in channel order), the k-th largest by two
// histogram passes (one histogram per wave), the selected channels in channel
// order by ballot prefixes.  Each lane then looks up the slots of its hits and
// requests their refinement words for its wave's rows; the resident dot products
// run meanwhile and the deltas are added before the row sums are written.  The
// first workgroup of each matrix reports its hits and lookup log, workgroup 0 the
// selection.
// SW = true: workgroup 0 selects for all (as in the split kernel) and the tiles
// take the selection from its published words after their resident dot products.
template <class C, int B, int R, int NB, int D, int XB, bool SW>
__global__ __launch_bounds__(256) void gemv_fused_kernel(GemvArgs a) {
  extern __shared__ uint32_t smem[];
  __shared__ uint32_t whist[4][256];
  __shared__ uint32_t whist2[4][128];
  __shared__ uint32_t s_cnt[4 * (MAX_SEL_K / 2048)];
  __shared__ int lds[24];
  if constexpr (SW) {
    if (blockIdx.x == 0) {
      __builtin_amdgcn_s_setprio(3);
      split_select_and_publish(a, smem);
      __builtin_amdgcn_s_setprio(0);
      split_retire(a);
      return;
    }
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // each wave clears the histograms it counts into (its own, before its atomics)
  for (int i = lane; i < 256; i += 64) whist[wave][i] = 0u;
  for (int i = lane; i < 128; i += 64) whist2[wave][i] = 0u;
  const int K = a.k_in, nchunks = K / C::CODES, xpairs = K / 2, ngr = K / 128, n8 = K / 8;
  const int ks = a.k_sel;
  const bool refine = ks > 0;
  constexpr int XCS = x_chunk_words<C>();                      // words per chunk of x pairs
  uint32_t* xs = smem;                                         // [NB][nchunks][XCS] fp16 pairs
  float* xsum = (float*)(smem + NB * nchunks * XCS);           // [NB][nchunks]
  uint32_t* keys = (uint32_t*)(xsum + NB * ((nchunks + 3) & ~3));  // [K/2]: channel-order key pairs
  uint32_t* s_szw = keys + ((refine && !SW) ? xpairs : 0);     // [4][R][ngr]
  int32_t* l_sel = (int32_t*)(s_szw + (refine ? 4 * R * ngr : 0));  // [ks]
  uint32_t* bm_sure = (uint32_t*)(l_sel + (refine ? ks : 0));      // [K/32]: keys above the boundary bin
  uint32_t* bm_bnd = bm_sure + (refine ? K / 32 : 0);               // [K/32]: keys in the boundary bin
  const bool computed = !SW && refine && !a.sel_in && ks < K;      // the selection is computed here
  const int tile_g = blockIdx.x - (SW ? 1 : 0);
  const int op = op_of_tile(a, tile_g);
  const GemvOpDev& o = a.ops[op];
  const int row0 = (tile_g - o.tile_begin) * 4 * R + wave * R;
  const size_t rowbytes = (size_t)K * B / 8;
  SF_TS(0);

  // x first (the selection needs it early; loads complete in order), then the
  // tile's codes; both unconditional (clamped addresses, unused values), so that
  // staging x waits for the x loads only
  u32x4 xv0[NB][XB];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    const u32x4* xr = (const u32x4*)(a.x + (size_t)(a.batch_off + bb) * K);
#pragma unroll
    for (int i = 0; i < XB; ++i) xv0[bb][i] = xr[min(256 * i + tid, n8 - 1)];
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the x loads ahead of the code loads
  // the first D chunks of every row of this lane
  uint32_t cw[D][R][C::WORDS];
  uint32_t szw[D][R];
#pragma unroll
  for (int u = 0; u < D; ++u) load_chunk_clamped<C, R>(o, row0, min(lane + 64 * u, nchunks - 1), rowbytes, ngr, cw[u], szw[u]);

  // x in pair order; chunk sums; selection keys in channel order
  uint16_t* xh = (uint16_t*)xs;
  auto stage = [&](const u32x4 (&xv)[NB][XB], int m0) {
    constexpr int TPC = C::CODES / 8;  // threads per chunk
#pragma unroll
    for (int i = 0; i < XB; ++i) {
      const int m = m0 + 256 * i + tid;
      u32x4 kv = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        float part = 0.f;
        if (m < n8) {
          const uint32_t wds[4] = {xv[bb][i].x, xv[bb][i].y, xv[bb][i].z, xv[bb][i].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t x2 = wds[q] & 0x7FFF7FFFu;
            kv[q] = max(kv[q] & 0xFFFFu, x2 & 0xFFFFu) | (max(kv[q] >> 16, x2 >> 16) << 16);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int k = 8 * m + e;
            const int c = k / C::CODES, kk = k - c * C::CODES;
            int j, hi;
            C::locate(kk, &j, &hi);
            const uint16_t hb = (uint16_t)(wds[e >> 1] >> (16 * (e & 1)));
            xh[2 * ((bb * nchunks + c) * XCS + j) + hi] = hb;
            part += (float)__builtin_bit_cast(_Float16, hb);
          }
        }
        part = group_sum<TPC>(part);
        if (m < n8 && (m % TPC) == 0) xsum[bb * nchunks + m / TPC] = part;
      }
      if (!SW && refine && m < n8) *(u32x4*)(keys + 4 * m) = kv;
      if (computed && m < n8)  // selection pass 1: top 8 key bits, one histogram per wave
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          atomicAdd(&whist[wave][(kv[q] & 0xFFFFu) >> 7], 1u);
          atomicAdd(&whist[wave][kv[q] >> 23], 1u);
        }
    }
  };
  stage(xv0, 0);
  for (int m0 = 256 * XB; m0 < n8; m0 += 256 * XB) {  // x longer than XB loads a thread
    u32x4 xv[NB][XB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const u32x4* xr = (const u32x4*)(a.x + (size_t)(a.batch_off + bb) * K);
#pragma unroll
      for (int i = 0; i < XB; ++i) xv[bb][i] = xr[min(m0 + 256 * i + tid, n8 - 1)];
    }
    stage(xv, m0);
  }
  SF_TS(1);

  // the selection, ascending, into l_sel
  if (!SW && refine) {
    if (a.sel_in) {
      for (int j = tid; j < ks; j += 256) l_sel[j] = a.sel_in[j];
    } else if (ks >= K) {
      for (int j = tid; j < ks; j += 256) l_sel[j] = j;
    } else {
      lds_barrier();  // keys and the pass-1 histograms
      // every wave finds the boundary bin itself (no further barrier)
      int b1, above1;
      wave_threshold4(whist, 256, ks, &b1, &above1);
      SF_TS(5);
      // pass 2: low 7 bits of the keys in bin b1; bitmaps of the keys above bin b1
      // (all taken) and in bin b1 (decided by the low bits)
      {
        uint8_t* bs = (uint8_t*)bm_sure;
        uint8_t* bb = (uint8_t*)bm_bnd;
        for (int m = tid; m < n8; m += 256) {
          const u32x4 kv = *(const u32x4*)(keys + 4 * m);
          uint32_t sure = 0u, bnd = 0u;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t key = (kv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
            const int bin = (int)(key >> 7);
            sure |= (uint32_t)(bin > b1) << e;
            if (bin == b1) {
              bnd |= 1u << e;
              atomicAdd(&whist2[wave][key & 127u], 1u);
            }
          }
          bs[m] = (uint8_t)sure;
          bb[m] = (uint8_t)bnd;
        }
      }
      lds_barrier();
      int b2, above2;
      wave_threshold4(whist2, 128, ks - above1, &b2, &above2);
      SF_TS(8);
      const uint32_t need = (uint32_t)(ks - above1 - above2);  // keys equal to T taken, lowest channels first
      // compaction in channel order: thread t owns words [t W, t W + W) of the
      // bitmaps; taken = above-bin | (boundary with low bits > b2) | the first
      // `need` boundary keys with low bits == b2
      const int nw = K / 32, W = (nw + 255) / 256;
      const uint16_t* key16 = (const uint16_t*)keys;
      uint32_t sg[4], eqm[4], cs = 0u, ce = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sg[i] = eqm[i] = 0u;
        const int w = tid * W + i;
        if (i < W && w < nw) {
          uint32_t bnd = bm_bnd[w], gtw = 0u, eqw = 0u;
          while (bnd) {
            const int bit = __builtin_ctz(bnd);
            bnd &= bnd - 1u;
            const uint32_t lo = key16[32 * w + bit] & 127u;
            gtw |= (uint32_t)(lo > (uint32_t)b2) << bit;
            eqw |= (uint32_t)(lo == (uint32_t)b2) << bit;
          }
          sg[i] = bm_sure[w] | gtw;
          eqm[i] = eqw;
          cs += __popc(sg[i]);
          ce += __popc(eqm[i]);
        }
      }
      uint32_t ts, te;
      uint32_t sbefore = wave_excl_sum8(cs, &ts), ebefore = wave_excl_sum8(ce, &te);
      if (lane == 0) s_cnt[wave] = ts | (te << 16);
      lds_barrier();
      for (int w = 0; w < wave; ++w) {
        sbefore += s_cnt[w] & 0xFFFFu;
        ebefore += s_cnt[w] >> 16;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t all = sg[i] | eqm[i];
        while (all) {
          const int bit = __builtin_ctz(all);
          all &= all - 1u;
          const int c = 32 * (tid * W + i) + bit;
          if ((sg[i] >> bit) & 1u) {
            l_sel[sbefore + min(ebefore, need)] = c;
            ++sbefore;
          } else {
            if (ebefore < need) l_sel[sbefore + ebefore] = c;
            ++ebefore;
          }
        }
      }
    }
  }
  lds_barrier();  // x, chunk sums and the selection
  SF_TS(2);

  const float scl = (float)(1u << (a.r + B));
  const int r = a.r;
  uint32_t* szrow = s_szw + wave * R * ngr;  // this wave's rows' scale words, [R][ngr]
  // the wave's R rows occupy bits [row0 * r, (row0 + R) * r) of every unit
  const int ubit = row0 * r, uwi = ubit >> 5, uoff = ubit & 31;
  const int wpu = o.pool.unit_bytes >> 2;
  const uint32_t* units = (const uint32_t*)o.pool.slots;
  const int32_t* u2s = o.pool.unit2slot;
  // slots of this lane's first HPF hits and their refinement words for the wave's rows
  int pslot[HPF];
  uint32_t pw0[HPF], pw1[HPF];
  if (!SW && refine) {
#pragma unroll
    for (int i = 0; i < HPF; ++i) {
      const int j = lane + 64 * i;
      pslot[i] = j < ks ? (o.pool.resident ? l_sel[j] : (u2s ? u2s[l_sel[j]] : -1)) : -1;
    }
#pragma unroll
    for (int i = 0; i < HPF; ++i) {
      pw0[i] = pw1[i] = 0u;
      if (pslot[i] >= 0) {
        const uint32_t* u = units + (size_t)pslot[i] * wpu;
        if (uwi < wpu) pw0[i] = u[uwi];
        if (uwi + 1 < wpu) pw1[i] = u[uwi + 1];
      }
    }
  }

  const PairK pk = C::consts();
  float acc[NB][R];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb)
#pragma unroll
    for (int rr = 0; rr < R; ++rr) acc[bb][rr] = 0.f;
  for (int c0 = 0; c0 < nchunks; c0 += 64 * D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int c = c0 + 64 * u + lane;
      if (c < nchunks) {
        if (refine && (c * C::CODES) % 128 == 0)
#pragma unroll
          for (int rr = 0; rr < R; ++rr) szrow[rr * ngr + (c * C::CODES) / 128] = szw[u][rr];
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
          const u32x4* xp = (const u32x4*)(xs + (bb * nchunks + c) * XCS);
          float d[R];
#pragma unroll
          for (int rr = 0; rr < R; ++rr) d[rr] = 0.f;
          // batch 1: fully unrolled (constant word indices, no indexed register
          // reads); the x pairs are read one step ahead and no further (the empty
          // asm keeps later LDS reads after it).  Batch 2 keeps a short loop, for
          // its register count.
          constexpr int JU = NB == 1 ? C::PAIRS / 4 : 2;
          u32x4 xn = xp[0];
#pragma unroll JU
          for (int jb = 0; jb < C::PAIRS / 4; ++jb) {
            const u32x4 xv = xn;
            if (jb + 1 < C::PAIRS / 4) xn = xp[jb + 1];
#pragma unroll
            for (int rr = 0; rr < R; ++rr)
#pragma unroll
              for (int q = 0; q < 4; ++q)
                d[rr] = __builtin_amdgcn_fdot2(as_h2(C::pair(cw[u][rr], 4 * jb + q, pk)), as_h2(xv[q]), d[rr], false);
            asm volatile("" ::: "memory");
          }
          const float X = xsum[bb * nchunks + c];
#pragma unroll
          for (int rr = 0; rr < R; ++rr) {
            const float sv = sf_h2f(szw[u][rr]), zv = sf_h2f(szw[u][rr] >> 16);
            acc[bb][rr] += (sv * scl) * (d[rr] - X) + zv * X;
          }
        }
      }
    }
    // the next chunks: a wave-uniform exit first, then unconditional loads (clamped
    // addresses; a lane past the end loads a chunk it never uses), so the loaded
    // words replace the current ones in place
    if (c0 + 64 * D >= nchunks) break;
#pragma unroll
    for (int u = 0; u < D; ++u)
      load_chunk_clamped<C, R>(o, row0, min(c0 + 64 * D + 64 * u + lane, nchunks - 1), rowbytes, ngr, cw[u], szw[u]);
  }
  SF_TS(3);
  if constexpr (SW) {
    if (refine) {
      int32_t* l_hk = (int32_t*)(s_szw + 4 * R * ngr);
      split_refine_tile<C, R, NB, wtm_of(R)>(a, o, op, tile_g, row0, szrow, l_hk, (float*)(l_hk + ks),
                                            (uint32_t*)(l_hk + ks + ks * NB), acc, &lds[23]);
    }
  }
  // refinement of the hit channels: + x_k * s[row][k/128] * c_lo[row][k]
  if (!SW && refine) {
    // the rows' scale words were recorded by other lanes of this wave
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int j = lane; j < ks; j += 64) {
      const int i = (j - lane) >> 6;
      int slot;
      uint32_t w0, w1, w2 = 0u;
      if (i < HPF) {
        slot = pslot[0];
        w0 = pw0[0];
        w1 = pw1[0];
#pragma unroll
        for (int q = 1; q < HPF; ++q)
          if (q == i) {
            slot = pslot[q];
            w0 = pw0[q];
            w1 = pw1[q];
          }
        if (slot >= 0 && uoff + R * r > 64 && uwi + 2 < wpu) w2 = units[(size_t)slot * wpu + uwi + 2];
      } else {
        slot = o.pool.resident ? l_sel[j] : (u2s ? u2s[l_sel[j]] : -1);
        w0 = w1 = 0u;
        if (slot >= 0) {
          const uint32_t* u = units + (size_t)slot * wpu;
          if (uwi < wpu) w0 = u[uwi];
          if (uwi + 1 < wpu) w1 = u[uwi + 1];
          if (uwi + 2 < wpu) w2 = u[uwi + 2];
        }
      }
      if (slot < 0) continue;
      const int k = l_sel[j];
      const int c = k / C::CODES, kk = k - c * C::CODES;
      int jj, hi;
      C::locate(kk, &jj, &hi);
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        const int p = uoff + rr * r;
        const uint32_t clo = p + r <= 64 ? bits64(w0, w1, p, r) : bits64(w1, w2, p - 32, r);
        const float sv = sf_h2f(szrow[rr * ngr + (k >> 7)]) * (float)clo;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
          const h2_t xh = as_h2(xs[(bb * nchunks + c) * XCS + jj]);
          acc[bb][rr] = fmaf(hi ? (float)xh.y : (float)xh.x, sv, acc[bb][rr]);
        }
      }
    }
  }
#pragma unroll
  for (int bb = 0; bb < NB; ++bb)
#pragma unroll
    for (int rr = 0; rr < R; ++rr) acc[bb][rr] = wave_sum63(acc[bb][rr]);
  SF_TS(10);
  if (lane == 63) {
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      const int row = row0 + rr;
      if (row < o.n_out)
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) o.y[(size_t)(a.batch_off + bb) * o.n_out + row] = acc[bb][rr];
    }
  }
  // reports (once per call): the selection, each matrix's hits and lookup log
  if (!SW && refine && a.report) {
    if (tile_g == 0 && a.sel_out)
      for (int j = tid; j < ks; j += 256) a.sel_out[j] = l_sel[j];
    if (tile_g == o.tile_begin && (o.hit_out || o.pool.log_count)) {
      if (tid == 0) {
        int base = -1;
        if (o.pool.log_count) {
          const uint32_t bse = atomicAdd(o.pool.log_count, (uint32_t)ks);
          base = (bse + (uint32_t)ks <= (uint32_t)o.pool.log_cap) ? (int)bse : -1;
        }
        lds[22] = base;
      }
      lds_barrier();
      const int base = lds[22];
      for (int j = tid; j < ks; j += 256) {
        const int k = l_sel[j];
        const int slot = o.pool.resident ? k : (u2s ? u2s[k] : -1);
        if (o.hit_out) o.hit_out[j] = slot;
        if (base >= 0) {
          o.pool.log_units[base + j] = k;
          o.pool.log_slots[base + j] = slot;
        }
      }
    }
  }
  SF_TS(4);
}

// x pair j of a chunk from the chunk's x in natural order (word t = channels 2t, 2t+1)
template <class C>
__device__ __forceinline__ uint32_t xpair(const uint32_t* X, int j) {
  const int l = C::lo(j), h = C::hi(j);
  if (l / 2 == h / 2 && l % 2 == 0 && h % 2 == 1) return X[l / 2];
  return __builtin_amdgcn_perm(X[h / 2], X[l / 2], ((h % 2 ? 0x0706u : 0x0504u) << 16) | (l % 2 ? 0x0302u : 0x0100u));
}

template <class C, int R, int NB>
__device__ __forceinline__ void load_x_chunk(const GemvArgs& a, int c, uint32_t (&xw)[NB][C::CODES / 2]) {
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    const u32x4* xr = (const u32x4*)(a.x + (size_t)(a.batch_off + bb) * a.k_in + (size_t)c * C::CODES);
#pragma unroll
    for (int i = 0; i < C::CODES / 8; ++i) {
      const u32x4 v = xr[i];
      xw[bb][4 * i] = v.x;
      xw[bb][4 * i + 1] = v.y;
      xw[bb][4 * i + 2] = v.z;
      xw[bb][4 * i + 3] = v.w;
    }
  }
}

constexpr int SPLIT_HPF = 8;  // hits per lane whose words are requested together

template <class C, int B, int R, int NB, int D>
__global__ __launch_bounds__(256) void gemv_split_kernel(GemvArgs a) {
  extern __shared__ uint32_t smem[];
  __shared__ int s_flag;
  const int ks = a.k_sel;
  const bool refine = ks > 0;
  if (a.sel_wg && blockIdx.x == 0) {
    __builtin_amdgcn_s_setprio(3);  // issue ahead of the streaming waves sharing the CU
    split_select_and_publish(a, smem);
    __builtin_amdgcn_s_setprio(0);
    split_retire(a);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.k_in, nchunks = K / C::CODES, ngr = K / 128;
  uint32_t* s_szw = smem;                                          // [4][R][ngr]
  int32_t* l_hk = (int32_t*)(s_szw + (refine ? 4 * R * ngr : 0));  // [k_sel] hit channel or -1
  float* l_hx = (float*)(l_hk + (refine ? ks : 0));                 // [k_sel][NB] x at the hit
  uint32_t* l_hw = (uint32_t*)(l_hx + (refine ? ks * NB : 0));      // [k_sel][wtm_of(R)] the tile's words
  const int tile_g = blockIdx.x - a.sel_wg;
  // the selecting workgroup's x requests reach the memory queues ahead of the tiles'
  // code streams (the tiles finish before the selection at these sizes)
  if (refine && a.sel_wg) __builtin_amdgcn_s_sleep(40);
  const int op = op_of_tile(a, tile_g);
  const GemvOpDev& o = a.ops[op];
  const int row0 = (tile_g - o.tile_begin) * 4 * R + wave * R;
  const size_t rowbytes = (size_t)K * B / 8;
  SF_TS(0);

  // the first D chunks of this lane: codes of the wave's rows, their scale words
  // and x (natural order; L1/L2-resident after the first wave), clamped so that
  // every load is unconditional
  uint32_t cw[D][R][C::WORDS];
  uint32_t szw[D][R];
  uint32_t xw[D][NB][C::CODES / 2];
#pragma unroll
  for (int u = 0; u < D; ++u) {
    const int c = min(lane + 64 * u, nchunks - 1);
    load_chunk_clamped<C, R>(o, row0, c, rowbytes, ngr, cw[u], szw[u]);
    load_x_chunk<C, R, NB>(a, c, xw[u]);
  }

  const float scl = (float)(1u << (a.r + B));
  const int r = a.r;
  uint32_t* szrow = s_szw + wave * R * ngr;  // this wave's rows' scale words, [R][ngr]
  const PairK pk = C::consts();
  float acc[NB][R];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb)
#pragma unroll
    for (int rr = 0; rr < R; ++rr) acc[bb][rr] = 0.f;
  for (int c0 = 0; c0 < nchunks; c0 += 64 * D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int c = c0 + 64 * u + lane;
      if (c < nchunks) {
        if (refine && (c * C::CODES) % 128 == 0)
#pragma unroll
          for (int rr = 0; rr < R; ++rr) szrow[rr * ngr + (c * C::CODES) / 128] = szw[u][rr];
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
          float X = 0.f;
#pragma unroll
          for (int t = 0; t < C::CODES / 2; ++t) X = __builtin_amdgcn_fdot2(as_h2(xw[u][bb][t]), as_h2(0x3C003C00u), X, false);
          float d[R];
#pragma unroll
          for (int rr = 0; rr < R; ++rr) d[rr] = 0.f;
#pragma unroll
          for (int jb = 0; jb < C::PAIRS; jb += 4) {
            // four pairs at a time keeps the live x pairs and expanded codes few
            uint32_t xp[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) xp[q] = xpair<C>(xw[u][bb], jb + q);
#pragma unroll
            for (int rr = 0; rr < R; ++rr)
#pragma unroll
              for (int q = 0; q < 4; ++q)
                d[rr] = __builtin_amdgcn_fdot2(as_h2(C::pair(cw[u][rr], jb + q, pk)), as_h2(xp[q]), d[rr], false);
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int rr = 0; rr < R; ++rr) {
            const float sv = sf_h2f(szw[u][rr]), zv = sf_h2f(szw[u][rr] >> 16);
            acc[bb][rr] += (sv * scl) * (d[rr] - X) + zv * X;
          }
        }
        const int cn = c + 64 * D;
        if (cn < nchunks) {
          load_chunk_clamped<C, R>(o, row0, cn, rowbytes, ngr, cw[u], szw[u]);
          load_x_chunk<C, R, NB>(a, cn, xw[u]);
        }
      }
    }
  }
  SF_TS(2);
  // refinement of the hit channels: + x_k * s[row][k/128] * c_lo[row][k]
  if (refine) split_refine_tile<C, R, NB, wtm_of(R)>(a, o, op, tile_g, row0, szrow, l_hk, l_hx, l_hw, acc, &s_flag);
#pragma unroll
  for (int bb = 0; bb < NB; ++bb)
#pragma unroll
    for (int rr = 0; rr < R; ++rr) acc[bb][rr] = wave_sum63(acc[bb][rr]);
  if (lane == 63) {
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      const int row = row0 + rr;
      if (row < o.n_out)
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) o.y[(size_t)(a.batch_off + bb) * o.n_out + row] = acc[bb][rr];
    }
  }
  SF_TS(4);
}

// ---- batched GEMV on MFMA (batch 3..16 per launch) --------------------------------
// With several batch rows the GEMV is a real contraction.  v_mfma_f32_16x16x32_f16
// takes A = x (row = batch row, fp16, exact) and B = codes expanded to fp16
// 1 + c/2^b (exact), giving C[batch][row] = X + sum_k c x / 2^b over its 32 k-slots.
// The 32 k-slots of one MFMA come from one group of 128 channels: lane (q, n)
// supplies 8 codes of weight row n from channels [32q, 32q + 32) of the group,
// four MFMAs cover the group, and the group's scale words are applied to the
// fp32 result: y += s' D + (z - s') X with s' = s 2^(r+b).  x is staged in LDS
// once per workgroup, in the order in which a word's half-pairs come out.  Hit
// refinements of the workgroup's channel slice are compacted, 32 to an MFMA:
// A = x at the hit channels, B = s * c_lo as a sum of two fp16 terms (exact), so
// the fp32 sum sees the full-precision value on hits.  A workgroup covers 64*RT
// rows (RT 16-row tiles per wave) by one channel slice; the slices of a row block
// are summed in slice order by the workgroup that finishes last.
constexpr int MPFG = 4;         // groups of codes in flight per tile
constexpr int MAX_ROW_BLOCKS = 1024;  // counters in the workspace control block

template <int W>
__device__ __forceinline__ void load_words(const uint8_t* src, uint32_t (&w)[W]) {
  if constexpr (W == 1) {
    w[0] = __builtin_nontemporal_load((const uint32_t*)src);
  } else if constexpr (W == 2) {
    const u32x2 v = __builtin_nontemporal_load((const u32x2*)src);
    w[0] = v.x; w[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      const u32x4 v = __builtin_nontemporal_load((const u32x4*)src + i);
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
  }
}

__host__ __device__ constexpr size_t mfma_lds_words(int nb, int gs, int rows_wg, int nhp) {
  return (size_t)nb * (gs * 64 + 4) + (size_t)gs * 16 + (size_t)rows_wg * (gs + 1) * 2 +
         ((size_t)nb * (nhp + 8) + 1) / 2 + (size_t)nhp * 2;
}

template <int B, int RT>
__global__ __launch_bounds__(256) void gemv_mfma_kernel(GemvArgs a) {
  using C = CodecPow2<B>;
  constexpr int WQ = B;  // words holding one lane's 32 codes of a group
  extern __shared__ uint32_t smem[];
  __shared__ int s_cnt[4][2];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, q = lane >> 4;
  const int ns = a.ns, GS = a.gs;
  const int slice = blockIdx.x % ns, tile_g = blockIdx.x / ns;
  const int op = op_of_tile(a, tile_g);
  const GemvOpDev& o = a.ops[op];
  constexpr int rows_wg = 64 * RT;
  const int row_wg0 = (tile_g - o.tile_begin) * rows_wg;
  const int K = a.k_in, ngr = K / 128;
  const int g0 = slice * GS, k0 = g0 * 128, KS = GS * 128;
  const int nb = min(16, a.batch - a.batch_off);
  const size_t rowbytes = (size_t)K * B / 8;
  const int XSTR = GS * 64 + 4;  // words per batch row of staged x
  const int SSTR = GS + 1;       // scale pairs per row
  const int HSTR = a.nhp + 8;    // fp16 per batch row of hit x
  uint32_t* xs = smem;                                  // [nb][XSTR]
  float* xsum = (float*)(xs + nb * XSTR);               // [GS][16]
  float2* sp = (float2*)(xsum + GS * 16);               // [rows_wg][SSTR]: (s', z - s')
  _Float16* hx = (_Float16*)(sp + rows_wg * SSTR);      // [nb][HSTR]
  int32_t* hk = (int32_t*)(xs + (mfma_lds_words(nb, GS, rows_wg, a.nhp) - 2 * a.nhp));  // [nhp]
  int32_t* hs = hk + a.nhp;                                                            // [nhp]
  const int wrow0 = wave * 16 * RT;  // this wave's first row within the block

  // codes of the first MPFG groups of every tile
  uint32_t cw[MPFG][RT][WQ];
  auto issue = [&](int u, int gl) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int row = row_wg0 + wrow0 + 16 * t + n;
      if (gl < GS && row < o.n_out) {
        load_words<WQ>(o.res + (size_t)row * rowbytes + (size_t)(g0 + gl) * (16 * B) + q * (4 * B), cw[u][t]);
      } else {
#pragma unroll
        for (int w = 0; w < WQ; ++w) cw[u][t][w] = 0u;
      }
    }
  };
#pragma unroll
  for (int u = 0; u < MPFG; ++u) issue(u, u);

  // x slice -> LDS in half-pair order, with its group sums
  {
    const int per_row = KS / 8;  // 16-byte loads per batch row (a multiple of 16)
    const int items = nb * per_row;
    constexpr int XB = 4;
    for (int i0 = 0; i0 < items; i0 += 256 * XB) {
      u32x4 xv[XB];
#pragma unroll
      for (int it = 0; it < XB; ++it) {
        const int i = i0 + 256 * it + tid;
        if (i < items) {
          const int bc = i / per_row, c8 = i - bc * per_row;
          xv[it] = *(const u32x4*)(a.x + (size_t)(a.batch_off + bc) * K + k0 + 8 * c8);
        }
      }
#pragma unroll
      for (int it = 0; it < XB; ++it) {
        const int i = i0 + 256 * it + tid;
        float part = 0.f;
        int bc = 0, c8 = 0;
        if (i < items) {
          bc = i / per_row;
          c8 = i - bc * per_row;
          const uint32_t wds[4] = {xv[it].x, xv[it].y, xv[it].z, xv[it].w};
          uint16_t* xh = (uint16_t*)(xs + bc * XSTR);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int kl = 8 * c8 + e, gl = kl >> 7, kg = kl & 127;
            int j, hi;
            C::locate(kg & 31, &j, &hi);
            const uint16_t hb = (uint16_t)(wds[e >> 1] >> (16 * (e & 1)));
            xh[2 * ((gl * 4 + (kg >> 5)) * 16 + j) + hi] = hb;
            part += (float)__builtin_bit_cast(_Float16, hb);
          }
        }
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) part += __shfl_xor(part, off, 16);
        if (i < items && (c8 & 15) == 0) xsum[(c8 >> 4) * 16 + bc] = part;
      }
    }
    for (int i = tid; i < GS * 16; i += 256)
      if ((i & 15) >= nb) xsum[i] = 0.f;
  }
  // scale words of the block's rows in the slice -> (s 2^(r+b), z - s 2^(r+b))
  {
    const float scl = (float)(1u << (a.r + B));
    constexpr int SB = 8;
    for (int i0 = 0; i0 < rows_wg * GS; i0 += 256 * SB) {
      uint32_t w[SB];
#pragma unroll
      for (int it = 0; it < SB; ++it) {
        const int i = i0 + 256 * it + tid;
        const int rl = i / GS, gl = i - rl * GS, row = row_wg0 + rl;
        w[it] = (i < rows_wg * GS && row < o.n_out) ? o.sz[(size_t)row * ngr + g0 + gl] : 0u;
      }
#pragma unroll
      for (int it = 0; it < SB; ++it) {
        const int i = i0 + 256 * it + tid;
        if (i < rows_wg * GS) {
          const int rl = i / GS, gl = i - rl * GS;
          const float sv = sf_h2f(w[it]) * scl, zv = sf_h2f(w[it] >> 16);
          sp[rl * SSTR + gl] = make_float2(sv, zv - sv);
        }
      }
    }
  }
  // selected channels inside the slice: positions [h0, h1) of the ascending list
  const int ks = a.k_sel;
  int h0 = 0, nh = 0;
  if (ks > 0) {
    int c0 = 0, c1 = 0;
    for (int j = tid; j < ks; j += 256) {
      const int k = a.ws_sel[j];
      c0 += k < k0;
      c1 += k < k0 + KS;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      c0 += __shfl_xor(c0, off, 64);
      c1 += __shfl_xor(c1, off, 64);
    }
    if (lane == 0) {
      s_cnt[wave][0] = c0;
      s_cnt[wave][1] = c1;
    }
  }
  lds_barrier();
  if (ks > 0) {
    h0 = (s_cnt[0][0] + s_cnt[1][0]) + (s_cnt[2][0] + s_cnt[3][0]);
    nh = (s_cnt[0][1] + s_cnt[1][1]) + (s_cnt[2][1] + s_cnt[3][1]) - h0;
    const int nhp = (nh + 31) & ~31;
    const int32_t* slots = a.ws_slot + (size_t)op * ks;
    for (int j = tid; j < nhp; j += 256) {
      const bool valid = j < nh;
      const int k = valid ? a.ws_sel[h0 + j] : k0;
      hk[j] = k;
      hs[j] = valid ? slots[h0 + j] : -1;
      for (int bc = 0; bc < nb; ++bc)
        hx[bc * HSTR + j] = valid ? __builtin_bit_cast(_Float16, a.x[(size_t)(a.batch_off + bc) * K + k])
                                  : (_Float16)0.f;
    }
  }

  // resident GEMV
  const PairK pk = C::consts();
  f4_t acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f4_t{0.f, 0.f, 0.f, 0.f};
  const bool arow = n < nb;  // this lane's A row is a real batch row
  for (int gb = 0; gb < GS; gb += MPFG) {
#pragma unroll
    for (int u = 0; u < MPFG; ++u) {
      const int gl = gb + u;
      if (gl < GS) {
        h8_t ax[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          if (arow) {
            ax[m] = *(const h8_t*)(xs + n * XSTR + (gl * 4 + q) * 16 + 4 * m);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) ax[m][e] = (_Float16)0.f;
          }
        }
        const f4_t X4 = *(const f4_t*)(xsum + gl * 16 + 4 * q);
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          f4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const u32x4 bv = {C::pair(cw[u][t], 4 * m, pk), C::pair(cw[u][t], 4 * m + 1, pk),
                              C::pair(cw[u][t], 4 * m + 2, pk), C::pair(cw[u][t], 4 * m + 3, pk)};
            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(ax[m], __builtin_bit_cast(h8_t, bv), d, 0, 0, 0);
          }
          const float2 sc = sp[(wrow0 + 16 * t + n) * SSTR + gl];
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[t][v] = fmaf(sc.x, d[v], fmaf(sc.y, X4[v], acc[t][v]));
        }
      }
      issue(u, gl + MPFG);
    }
  }

  // refinements of the hit channels in the slice, 32 channels per MFMA
  if (ks > 0 && nh > 0) {
    lds_barrier();  // hit lists staged
    const uint32_t* units = (const uint32_t*)o.pool.slots;
    const int wpu = o.pool.unit_bytes >> 2;
    const int r = a.r;
    const float sdown = 1.f / (float)(1u << (r + B));
    for (int blk = 0; blk * 32 < nh; ++blk) {
      h8_t ah;
      if (arow) {
        ah = *(const h8_t*)(hx + n * HSTR + blk * 32 + 8 * q);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) ah[e] = (_Float16)0.f;
      }
      int kk[8], sl[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kk[e] = hk[blk * 32 + 8 * q + e];
        sl[e] = hs[blk * 32 + 8 * q + e];
      }
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int rl = wrow0 + 16 * t + n, row = row_wg0 + rl;
        const int bit = row * r, wi = bit >> 5, off = bit & 31;
        uint32_t w0[8], w1[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          w0[e] = w1[e] = 0u;
          if (sl[e] >= 0 && row < o.n_out) {
            const uint32_t* u = units + (size_t)sl[e] * wpu;
            w0[e] = u[wi];
            if (off + r > 32 && wi + 1 < wpu) w1[e] = u[wi + 1];
          }
        }
        u32x4 hb, lb;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          uint32_t hp = 0u, lp = 0u;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int e = 2 * f + h;
            const float val = sp[rl * SSTR + ((kk[e] - k0) >> 7)].x * sdown * (float)bits64(w0[e], w1[e], off, r);
            const _Float16 vh = (_Float16)val;
            const _Float16 vl = (_Float16)(val - (float)vh);
            hp |= (uint32_t)__builtin_bit_cast(uint16_t, vh) << (16 * h);
            lp |= (uint32_t)__builtin_bit_cast(uint16_t, vl) << (16 * h);
          }
          hb[f] = hp;
          lb[f] = lp;
        }
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, __builtin_bit_cast(h8_t, hb), acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, __builtin_bit_cast(h8_t, lb), acc[t], 0, 0, 0);
      }
    }
  }

  // lane (q, n) holds batch rows 4q .. 4q+3 of weight row n of each tile
  if (ns == 1) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int row = row_wg0 + wrow0 + 16 * t + n;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int bc = 4 * q + v;
        if (bc < nb && row < o.n_out) o.y[(size_t)(a.batch_off + bc) * o.n_out + row] = acc[t][v];
      }
    }
    return;
  }
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int prow = tile_g * rows_wg + wrow0 + 16 * t + n;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int bc = 4 * q + v;
      if (bc < nb) sf_put(a.part + (size_t)(slice * nb + bc) * a.rows_pad + prow, acc[t][v]);
    }
  }
  sf_drain();
  __syncthreads();
  if (tid == 0)
    s_last = __builtin_amdgcn_atomic_inc32(a.ctr + tile_g, (uint32_t)(ns - 1), __ATOMIC_RELAXED, "agent") ==
             (uint32_t)(ns - 1);
  __syncthreads();
  if (!s_last) return;
  // last slice of this row block: y = sum of the slices' partials, in slice order
  for (int i = tid; i < nb * rows_wg; i += 256) {
    const int bc = i / rows_wg, rl = i - bc * rows_wg, row = row_wg0 + rl;
    if (row >= o.n_out) continue;
    const float* pp = a.part + (size_t)bc * a.rows_pad + tile_g * rows_wg + rl;
    const size_t sstride = (size_t)nb * a.rows_pad;
    float sum = 0.f;
    for (int s0 = 0; s0 < ns; s0 += 16) {
      float v[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) v[k] = s0 + k < ns ? sf_get(pp + (size_t)(s0 + k) * sstride) : 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) sum += v[k];
    }
    o.y[(size_t)(a.batch_off + bc) * o.n_out + row] = sum;
  }
}

int env_int(const char* name, int dflt) {
  const char* e = getenv(name);
  return e ? atoi(e) : dflt;
}

size_t gemv_lds_bytes(int k_in, int codes, int nb, int n_ops, int k_sel, int rpw, bool hits_in_lds) {
  size_t w = (size_t)nb * (k_in / 2) + (size_t)nb * (k_in / codes);
  if (k_sel > 0) w += (size_t)4 * rpw * (k_in / 128) + (hits_in_lds ? (size_t)k_sel * (1 + n_ops) : 0);
  return w * 4;
}

constexpr size_t MAX_DYN_LDS = 96 * 1024;
constexpr size_t HIT_LDS = 16 * 1024;  // hit lists up to this size are copied to LDS

template <class C, int B, int R, int NB>
sf_status launch_gemv(GemvArgs& a, hipStream_t s) {
  a.hits_in_lds = a.k_sel > 0 && (size_t)a.k_sel * (1 + a.n_ops) * 4 <= HIT_LDS;
  const size_t lds = gemv_lds_bytes(a.k_in, C::CODES, NB, a.n_ops, a.k_sel, R, a.hits_in_lds);
  SF_REQUIRE(lds <= MAX_DYN_LDS, SF_EUNSUPPORTED, "k_in too large for the LDS staging of x");
  // persistent workgroups: as many as are resident at once (at most
  // SF_GEMV_WGS_PER_CU per CU if set), each with an equal number of tiles
  static int n_cu = 0;
  if (n_cu == 0) {
    int dev = 0, cus = 0;
    (void)hipGetDevice(&dev);
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    n_cu = cus;
  }
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void*)gemv_kernel<C, B, R, NB>, 256, lds) != hipSuccess ||
      occ < 1)
    occ = 1;
  const int per_cu = env_int("SF_GEMV_WGS_PER_CU", occ);
  const int cap = n_cu * (per_cu > 0 ? min(per_cu, occ) : occ);
  const int tiles_per_wg = (a.total_tiles + cap - 1) / cap;
  const int grid = (a.total_tiles + tiles_per_wg - 1) / tiles_per_wg;
  hipLaunchKernelGGL((gemv_kernel<C, B, R, NB>), dim3((unsigned)grid), dim3(256), lds, s, a);
  SF_LAUNCH_CHECK();
  return SF_OK;
}

template <class C, int B, int R, int NB, bool SW = false>
sf_status launch_fused(GemvArgs& a, hipStream_t s) {
  constexpr int D = R >= 8 ? 1 : (R >= 4 ? 2 : 4);
  const size_t lds =
      SW ? fused_sw_lds_bytes(a.k_in, C::CODES, NB, a.k_sel, R) : fused_lds_bytes(a.k_in, C::CODES, NB, a.k_sel, R);
  SF_REQUIRE(lds <= MAX_DYN_LDS, SF_EUNSUPPORTED, "k_in too large for the LDS staging of x");
  const dim3 grid((unsigned)(a.total_tiles + (SW ? 1 : 0)));
  if (a.k_in <= 256 * 8 * 2)
    hipLaunchKernelGGL((gemv_fused_kernel<C, B, R, NB, D, 2, SW>), grid, dim3(256), lds, s, a);
  else
    hipLaunchKernelGGL((gemv_fused_kernel<C, B, R, NB, D, 8, SW>), grid, dim3(256), lds, s, a);
  SF_LAUNCH_CHECK();
  return SF_OK;
}


int device_cus();

template <class C, int B, int R, int NB>
sf_status launch_split(GemvArgs& a, hipStream_t s) {
  constexpr int D = R >= 8 ? 1 : 2;
  const size_t lds = split_lds_bytes(a.k_in, C::PAIRS, C::CODES, NB, a.k_sel, R);
  SF_REQUIRE(lds <= MAX_DYN_LDS, SF_EUNSUPPORTED, "k_in too large for the LDS staging of x");
  // the tiles wait for workgroup 0 only at their end, but a tile that has to wait
  // for a free slot adds a whole tile time: when the grid does not fit the device
  // at once, the fused kernel (selection in every workgroup) is used instead
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void*)gemv_split_kernel<C, B, R, NB, D>, 256, lds) !=
          hipSuccess ||
      occ < 1)
    occ = 1;
  // SF_GEMV_SPLIT=2 always takes the staged variant (x in LDS, workgroup 0 selecting)
  const bool staged = env_int("SF_GEMV_SPLIT", 1) == 2;
  if (staged || (long)occ * device_cus() < (long)a.total_tiles + a.sel_wg) {
    // the staged variant needs fewer registers; else the fused kernel
    constexpr int D2 = R >= 8 ? 1 : (R >= 4 ? 2 : 4);
    const size_t lds2 = fused_sw_lds_bytes(a.k_in, C::CODES, NB, a.k_sel, R);
    int occ2 = 0;
    const void* k2 = a.k_in <= 256 * 8 * 2 ? (const void*)gemv_fused_kernel<C, B, R, NB, D2, 2, true>
                                           : (const void*)gemv_fused_kernel<C, B, R, NB, D2, 8, true>;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ2, k2, 256, lds2) != hipSuccess || occ2 < 1) occ2 = 1;
    if (a.sel_wg && lds2 <= MAX_DYN_LDS && (staged || (long)occ2 * device_cus() >= (long)a.total_tiles + 1))
      return launch_fused<C, B, R, NB, true>(a, s);
    if (fused_lds_bytes(a.k_in, C::CODES, NB, a.k_sel, R) <= MAX_DYN_LDS) {
      a.sel_wg = 0;
      return launch_fused<C, B, R, NB>(a, s);
    }
  }
  const dim3 grid((unsigned)(a.total_tiles + a.sel_wg));
  hipLaunchKernelGGL((gemv_split_kernel<C, B, R, NB, D>), grid, dim3(256), lds, s, a);
  SF_LAUNCH_CHECK();
  return SF_OK;
}

enum GemvKind { KIND_PERSISTENT = 0, KIND_FUSED = 1, KIND_SPLIT = 2 };

template <class C, int B, int R>
sf_status dispatch_nb(GemvArgs& a, int nb, int kind, hipStream_t s) {
  if (kind == KIND_SPLIT) return nb == 2 ? launch_split<C, B, R, 2>(a, s) : launch_split<C, B, R, 1>(a, s);
  if (kind == KIND_FUSED) return nb == 2 ? launch_fused<C, B, R, 2>(a, s) : launch_fused<C, B, R, 1>(a, s);
  if (nb == 2) return launch_gemv<C, B, R, 2>(a, s);
  return launch_gemv<C, B, R, 1>(a, s);
}

template <class C, int B>
sf_status dispatch_r(GemvArgs& a, int R, int nb, int kind, hipStream_t s) {
  switch (R) {
    case 1: return dispatch_nb<C, B, 1>(a, nb, kind, s);
    case 2: return dispatch_nb<C, B, 2>(a, nb, kind, s);
    case 4: return dispatch_nb<C, B, 4>(a, nb, kind, s);
    default: return dispatch_nb<C, B, 8>(a, nb, kind, s);
  }
}

sf_status dispatch_b(GemvArgs& a, int b, int R, int nb, int kind, hipStream_t s) {
  switch (b) {
    case 1: return dispatch_r<CodecPow2<1>, 1>(a, R, nb, kind, s);
    case 2: return dispatch_r<CodecPow2<2>, 2>(a, R, nb, kind, s);
    case 3: return dispatch_r<CodecStream<3>, 3>(a, R, nb, kind, s);
    case 4: return dispatch_r<CodecPow2<4>, 4>(a, R, nb, kind, s);
    case 8: return dispatch_r<CodecPow2<8>, 8>(a, R, nb, kind, s);
    default:
      sf_set_error("sf_refined_gemv: resident width b must be 1, 2, 3, 4 or 8");
      return SF_EUNSUPPORTED;
  }
}

int codes_per_chunk(int b) { return (b == 1 || b == 2 || b == 4 || b == 8) ? 128 / b : 32; }

size_t gemv_ws_layout(int32_t n_ops, int32_t k_sel, size_t part_bytes, size_t* off_sel, size_t* off_slot,
                      size_t* off_part) {
  const size_t ks = k_sel > 0 ? (size_t)k_sel : 1;
  size_t o = sf_align256(sizeof(WsControl));
  *off_sel = o;
  o += sf_align256(ks * 4);
  *off_slot = o;
  o += sf_align256((size_t)(n_ops > 0 ? n_ops : 1) * ks * 4);
  *off_part = o;
  o += sf_align256(part_bytes);
  return o;
}

int device_cus() {
  static int n_cu = 0;
  if (n_cu == 0) {
    int dev = 0, cus = 0;
    (void)hipGetDevice(&dev);
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    n_cu = cus;
  }
  return n_cu;
}

// The batched MFMA kernel serves b in {1, 2, 4, 8} from three batch rows up
// (SF_GEMV_MFMA=0 / 1 forces it off / on).
bool mfma_wanted(int b, int batch) {
  if (b != 1 && b != 2 && b != 4 && b != 8) return false;
  const int e = env_int("SF_GEMV_MFMA", -1);
  if (e >= 0) return e != 0;
  return batch >= 3;
}

constexpr size_t MAX_MFMA_LDS = 64 * 1024;

struct MfmaPlan {
  int rt = 0, ns = 1, gs = 0, nhp = 0, tiles = 0;
  size_t part_bytes = 0;
};

// Rows per workgroup: 256 when that still gives a quarter of the CUs a row block,
// else 128, else 64.  Channel slices: the fewest (a divisor of the group count,
// at most 16 groups each, LDS within 64 KB) that give 1.5 workgroups per CU.
// SF_GEMV_MFMA_RT and SF_GEMV_MFMA_SLICES override the choices.
MfmaPlan mfma_plan(const int64_t* n_out, int n_ops, int K, int batch, int k_sel) {
  MfmaPlan p;
  const int n_cu = device_cus();
  const int nb = batch < 16 ? batch : 16;
  auto tiles_for = [&](int rows) {
    int t = 0;
    for (int i = 0; i < n_ops; ++i) t += (int)((n_out[i] + rows - 1) / rows);
    return t;
  };
  int rt = env_int("SF_GEMV_MFMA_RT", 0);
  if (rt != 1 && rt != 2 && rt != 4) rt = tiles_for(256) >= n_cu / 4 ? 4 : (tiles_for(128) >= n_cu / 4 ? 2 : 1);
  const int rows_wg = 64 * rt, tiles = tiles_for(rows_wg), ngr = K / 128;
  const int want_ns = env_int("SF_GEMV_MFMA_SLICES", 0);
  int best = -1;
  for (int ns = 1; ns <= ngr; ++ns) {
    if (ngr % ns) continue;
    const int gs = ngr / ns;
    if (gs > 16 || (ns > 1 && tiles > MAX_ROW_BLOCKS)) continue;
    const int nhp = k_sel > 0 ? ((std::min(k_sel, gs * 128) + 31) & ~31) : 0;
    if (mfma_lds_words(nb, gs, rows_wg, nhp) * 4 > MAX_MFMA_LDS) continue;
    best = ns;
    if (want_ns > 0 ? ns >= want_ns : (long)tiles * ns >= 3L * n_cu / 2) break;
  }
  if (best < 0) return p;
  p.rt = rt;
  p.ns = best;
  p.gs = ngr / best;
  p.nhp = k_sel > 0 ? ((std::min(k_sel, p.gs * 128) + 31) & ~31) : 0;
  p.tiles = tiles;
  p.part_bytes = best > 1 ? (size_t)best * nb * tiles * rows_wg * 4 : 0;
  return p;
}

template <int B>
sf_status launch_mfma_rt(GemvArgs& a, int rt, size_t lds, hipStream_t s) {
  const dim3 grid((unsigned)(a.total_tiles * a.ns));
  switch (rt) {
    case 1: hipLaunchKernelGGL((gemv_mfma_kernel<B, 1>), grid, dim3(256), lds, s, a); break;
    case 2: hipLaunchKernelGGL((gemv_mfma_kernel<B, 2>), grid, dim3(256), lds, s, a); break;
    default: hipLaunchKernelGGL((gemv_mfma_kernel<B, 4>), grid, dim3(256), lds, s, a); break;
  }
  SF_LAUNCH_CHECK();
  return SF_OK;
}

sf_status launch_mfma(GemvArgs& a, int b, int rt, size_t lds, hipStream_t s) {
  switch (b) {
    case 1: return launch_mfma_rt<1>(a, rt, lds, s);
    case 2: return launch_mfma_rt<2>(a, rt, lds, s);
    case 4: return launch_mfma_rt<4>(a, rt, lds, s);
    default: return launch_mfma_rt<8>(a, rt, lds, s);
  }
}

// The plan sf_refined_gemv uses for these ops (rt = 0: the per-row-pair kernel).
MfmaPlan plan_for(const sf_gemv_op* ops, int n_ops, int batch, int k_sel) {
  MfmaPlan p;
  if (!mfma_wanted(ops[0].w.fmt.b, batch)) return p;
  int64_t no[SF_MAX_OPS];
  for (int i = 0; i < n_ops; ++i) no[i] = ops[i].w.n_out;
  return mfma_plan(no, n_ops, (int)ops[0].w.k_in, batch, k_sel);
}

}  // namespace

extern "C" size_t sf_workspace_bytes_gemv(const sf_gemv_op* ops, int32_t n_ops, int32_t batch, int32_t k_sel) {
  size_t part = 0;
  if (ops && n_ops >= 1 && n_ops <= SF_MAX_OPS && batch >= 1 && ops[0].w.k_in > 0 && ops[0].w.k_in % 128 == 0)
    part = plan_for(ops, n_ops, batch, k_sel).part_bytes;
  size_t a, b, c;
  return gemv_ws_layout(n_ops, k_sel, part, &a, &b, &c);
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
  SF_REQUIRE(k_sel == 0 || sel_in || k_sel == K || K <= MAX_SEL_K, SF_EUNSUPPORTED,
             "computed selection needs k_in <= 32768");
  GemvArgs a = {};
  // rows per wave (SF_GEMV_ROWS_PER_WAVE = 1, 2, 4 or 8 overrides the default)
  int rpw = env_int("SF_GEMV_ROWS_PER_WAVE", 0);
  int64_t rows_total = 0;
  for (int i = 0; i < n_ops; ++i) rows_total += ops[i].w.n_out;
  if (rpw != 1 && rpw != 2 && rpw != 4 && rpw != 8) {
    if (env_int("SF_GEMV_SPLIT", 1) != 0 || env_int("SF_GEMV_FUSED", 1) != 0)  // one row tile per workgroup, 8 rows a wave at most
      rpw = rows_total <= 8192 ? 4 : 8;
    else
      rpw = rows_total <= 8192 ? 2 : (rows_total <= 16384 ? 4 : 8);
  }
  const MfmaPlan mp = plan_for(ops, n_ops, batch, k_sel);
  const bool mfma = mp.rt > 0;
  const int rows_wg = mfma ? 64 * mp.rt : 4 * rpw;
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
  size_t o_sel, o_slot, o_part;
  SF_REQUIRE(ws->bytes >= gemv_ws_layout(n_ops, k_sel, mp.part_bytes, &o_sel, &o_slot, &o_part), SF_ENOMEM,
             "workspace too small");
  a.x = x_f16;
  a.sel_in = sel_in;
  a.sel_out = sel_out;
  a.ws_sel = (int32_t*)(ws->base + o_sel);
  a.ws_slot = (int32_t*)(ws->base + o_slot);
  a.n_ops = n_ops;
  a.k_in = (int32_t)K;
  a.batch = batch;
  a.k_sel = k_sel;
  a.r = f.r;
  a.total_tiles = tiles;
  hipStream_t s = (hipStream_t)stream;
  const int cpc = codes_per_chunk(f.b);
  // Batch 1-2 without the batched kernel: by default the split kernel (workgroup 0
  // selects while the others stream; SF_GEMV_SPLIT=0 falls back to the fused
  // kernel, which selects in every workgroup, and SF_GEMV_FUSED=0 then to the
  // separate selection launch and the persistent kernel).  With more rows than one
  // launch takes, the selection over all rows comes from the selection launch.
  int kind = KIND_PERSISTENT;
  if (!mfma) {
    if (env_int("SF_GEMV_SPLIT", 1) != 0 && split_lds_bytes((int)K, cpc / 2, cpc, 1, k_sel, rpw) <= MAX_DYN_LDS &&
        (size_t)SPLIT_COPIES * split_copy_words(k_sel, n_ops) <= sizeof(((WsControl*)nullptr)->hit) / 4)
      kind = KIND_SPLIT;
    else if (env_int("SF_GEMV_FUSED", 1) != 0 && fused_lds_bytes((int)K, cpc, 1, k_sel, rpw) <= MAX_DYN_LDS)
      kind = KIND_FUSED;
  }
  const size_t lds2 = kind == KIND_SPLIT   ? split_lds_bytes((int)K, cpc / 2, cpc, 2, k_sel, rpw)
                      : kind == KIND_FUSED ? fused_lds_bytes((int)K, cpc, 2, k_sel, rpw)
                                           : gemv_lds_bytes((int)K, cpc, 2, n_ops, k_sel, rpw, false);
  const int max_nb = lds2 <= 64 * 1024 ? 2 : 1;
  const bool one_launch = kind != KIND_PERSISTENT && batch <= max_nb;
  if (k_sel > 0 && !one_launch) {
    hipLaunchKernelGGL(gemv_select_kernel, dim3(1), dim3(SEL_NT), 0, s, a);
    SF_LAUNCH_CHECK();
  }
  if (mfma) {
    a.ns = mp.ns;
    a.gs = mp.gs;
    a.nhp = mp.nhp;
    a.rows_pad = tiles * rows_wg;
    a.part = (float*)(ws->base + o_part);
    a.ctr = (uint32_t*)(ws->base + offsetof(WsControl, row_ctr));
    for (int b0 = 0; b0 < batch; b0 += 16) {
      const int nb = batch - b0 < 16 ? batch - b0 : 16;
      a.batch_off = b0;
      sf_status st = launch_mfma(a, f.b, mp.rt, mfma_lds_words(nb, mp.gs, rows_wg, mp.nhp) * 4, s);
      if (st != SF_OK) return st;
    }
    return SF_OK;
  }
  // two batch rows per launch when both fit the LDS staging of x, else one
  if (kind != KIND_PERSISTENT) {
    a.report = one_launch ? 1 : 0;
    if (!one_launch && k_sel > 0) a.sel_in = a.ws_sel;
  }
  a.sel_wg = (kind == KIND_SPLIT && k_sel > 0) ? 1 : 0;
  a.ctl = (uint32_t*)ws->base;
  for (int b0 = 0; b0 < batch; b0 += max_nb) {
    const int nb = (batch - b0) >= max_nb ? max_nb : 1;
    a.batch_off = b0;
    sf_status st = dispatch_b(a, f.b, rpw, nb, kind, s);
    if (st != SF_OK) return st;
  }
  return SF_OK;
}
