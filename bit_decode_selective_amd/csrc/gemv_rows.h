// Row-tile kernels of the batch-1/2 refined GEMV and what they share with the rest
// of the GEMV sources (argument blocks, code layouts, selection helpers).  Included
// by gemv.hip and by one source per resident width, which instantiate the kernels
// for that width.  The method, readings and kernel designs are described at the top
// of gemv.hip.
#pragma once

#include <algorithm>
#include <cstddef>
#include <cstdlib>

#include "sf_internal.h"

#define SF_MAX_OPS 4

namespace sfg {

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
  int32_t n_ops, k_in, batch, batch_off, k_sel, r, total_tiles;
  // batched (MFMA) variant: channel slices per row block, groups per slice, hit
  // capacity per slice, padded rows, slice partials [ns][batch][rows_pad], and one
  // counter per row block
  int32_t ns, gs, nhp, rows_pad;
  int32_t report;  // fused kernel: report the selection, hits and lookup log
  float* part;
  uint32_t* ctr;
  // overlapped kernel: workgroup 0 selects (sel_wg = 1) and publishes through the
  // workspace control words ctl (WsControl: sel_state, done, timeout); n_readers:
  // the workgroups that read the published words (every other workgroup)
  int32_t sel_wg;
  int32_t n_readers;
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

// number of set bits of m in the lanes below this one
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// ---- the GEMV kernel -------------------------------------------------------------
// Shared pieces of the row-tile kernels: chunk loads of R rows, the op of a tile
// and the refinement window of a tile.
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

// One count into a per-wave LDS histogram.  The active lanes whose bin equals the
// first active lane's bin are added by one lane with their number: a whole wave
// adding to one address (all-equal keys, as an all-zero input gives) would
// otherwise serialise on it.
__device__ __forceinline__ void hist_add(uint32_t* h, uint32_t bin) {
  const uint32_t b0 = __builtin_amdgcn_readfirstlane(bin);
  const bool same = bin == b0;
  const uint64_t m = __ballot(same);
  const bool leader = same && lanes_below(m) == 0;
  if (!same || leader) atomicAdd(&h[bin], leader ? (uint32_t)__popcll(m) : 1u);
}

// Pass 1 of the selection: the top 8 bits of the 8 keys of each active lane into the
// wave's histogram.  When every active lane holds 8 copies of one key (an all-equal
// input, e.g. all zeros), one lane adds them all: a wave of same-address LDS atomics
// serialises; otherwise plain per-key atomics (cheaper than aggregating every key).
__device__ __forceinline__ void hist_add8(uint32_t* h, const u32x4& kv) {
  const uint32_t k0 = __builtin_amdgcn_readfirstlane(kv[0]);
  const bool same = kv[0] == k0 && kv[1] == k0 && kv[2] == k0 && kv[3] == k0 && (k0 & 0xFFFFu) == (k0 >> 16);
  const uint64_t act = __ballot(true);
  if (__ballot(same) == act) {
    if (lanes_below(act) == 0) atomicAdd(&h[(k0 & 0xFFFFu) >> 7], 8u * (uint32_t)__popcll(act));
    return;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    atomicAdd(&h[(kv[q] & 0xFFFFu) >> 7], 1u);
    atomicAdd(&h[kv[q] >> 23], 1u);
  }
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


inline size_t fused_lds_bytes(int k_in, int codes, int nb, int k_sel, int rpw) {
  size_t w = (size_t)nb * (k_in / codes) * (codes / 2 + 4) + (size_t)nb * (((k_in / codes) + 3) & ~3);
  if (k_sel > 0) w += (size_t)(k_in / 2) + (size_t)4 * rpw * (k_in / 128) + (size_t)k_sel + (size_t)(k_in / 16);
  return w * 4;
}

inline size_t split_sel_lds_words(int k_in, int k_sel) {
  return (size_t)(k_in / 2) + 2 * (size_t)(k_in / 32) + (((size_t)k_sel + 3) & ~(size_t)3) + 4 * 256 + 4 * 128 + 16;
}

// The fused kernel with workgroup 0 selecting: x staged as in the fused kernel, the
// hits (channel, x, the tile's window words) after the scale words; the selecting
// workgroup's own layout may be larger.
inline size_t fused_sw_lds_bytes(int k_in, int codes, int nb, int k_sel, int rpw) {
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
inline size_t split_lds_bytes(int k_in, int pairs, int codes, int nb, int k_sel, int rpw, bool selector = true) {
  (void)pairs;
  (void)codes;
  size_t tile = 0;
  if (k_sel > 0) tile += (size_t)4 * rpw * (k_in / 128) + (size_t)k_sel * (1 + nb + (31 + 4 * rpw * 7 + 31) / 32);
  size_t sel = 0;
  if (k_sel > 0 && selector)
    sel = (size_t)(k_in / 2) + 2 * (size_t)(k_in / 32) + (((size_t)k_sel + 3) & ~(size_t)3) + 4 * 256 + 4 * 128 + 16;
  return std::max(tile, sel) * 4;
}

// LDS of split_select alone (the selection launch of batches the row kernels do
// not take in one launch).
inline size_t select_lds_bytes(int k_in, int k_sel) {
  return ((size_t)(k_in / 2) + 2 * (size_t)(k_in / 32) + (((size_t)k_sel + 3) & ~(size_t)3) + 4 * 256 + 4 * 128 + 16) * 4;
}

// Copies of the published words (tile t reads copy t mod SPLIT_COPIES), and the
// stride of one copy in words.
constexpr int SPLIT_COPIES = 8;
__host__ __device__ inline int split_copy_words(int k_sel, int n_ops) { return ((k_sel * (1 + n_ops)) + 31) & ~31; }

// A tile that has seen the flag (or given up on it) counts itself.
__device__ __forceinline__ void count_reader(const GemvArgs& a, int grp) {
  uint32_t* c = a.ctl + offsetof(WsControl, rd_ctr) / 4 + 32 * grp;
  (void)__hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Published words carry their own validity: bit 31 set on a word the selecting
// workgroup has written in this launch, 0 on a cleared one.  A reader that sees bit
// 31 reads that writer's value (one location, one atomic store): the hand-off needs
// no ordering between different locations, so the flags are only a hint of when to
// start reading and no cache writeback or invalidation is needed.
__device__ __forceinline__ uint32_t pub_word(int v) { return 0x80000000u | ((uint32_t)v & 0x7FFFFFFFu); }
__device__ __forceinline__ int pub_value(uint32_t w) { return (int)(w << 1) >> 1; }  // sign from bit 30

// A published word, waited for (bounded); -1 if it never became valid.
__device__ __forceinline__ int read_published(const uint32_t* p, const GemvArgs& a) {
  uint32_t w = sf_get(p);
  if (w >> 31) return pub_value(w);
  const uint32_t lim = sf_spin_limit(a.ctl + 2);
  for (uint32_t it = 0; it < lim; ++it) {
    __builtin_amdgcn_s_sleep(2);
    w = sf_get(p);
    if (w >> 31) return pub_value(w);
  }
  sf_put(a.ctl + 2, 1u);
  return -1;
}

// Lane 0 of a wave polls its group's flag (bounded); the result is wave-uniform.
__device__ __forceinline__ bool wait_published(const GemvArgs& a, int grp) {
  const uint32_t* f = a.ctl + offsetof(WsControl, sel_flag) / 4 + 32 * grp;
  const uint32_t lim = sf_spin_limit(a.ctl + 2);
  for (uint32_t it = 0;; ++it) {
    uint32_t v = 0u;
    if ((threadIdx.x & 63) == 0) v = sf_get(f);
    if (__builtin_amdgcn_readfirstlane(v) != 0u) return true;
    if (it >= lim) {
      if ((threadIdx.x & 63) == 0) sf_put(a.ctl + 2, 1u);
      return false;
    }
    __builtin_amdgcn_s_sleep(8);
  }
}

// Workgroup 0, after publishing: waits until every tile has read the words, then
// clears them and lowers the flags and counts for the next launch.  If the wait
// gives up, it clears them all the same (a tile still to come then finds no valid
// word and keeps its rows unrefined) and the timeout word reports it; the workspace
// check clears any count such a late tile leaves behind.
__device__ __forceinline__ void split_retire(const GemvArgs& a) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    uint32_t* ctr = a.ctl + offsetof(WsControl, rd_ctr) / 4 + 32 * tid;
    const uint32_t tiles = (uint32_t)a.n_readers;
    const uint32_t want = (uint32_t)tid < tiles ? (tiles - (uint32_t)tid + 63u) / 64u : 0u;
    const uint32_t lim = sf_spin_limit(a.ctl + 2);
    for (uint32_t it = 0;; ++it) {
      if (__all(sf_get(ctr) >= want)) break;
      if (it >= lim) {
        sf_put(a.ctl + 2, 1u);
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
  }
  __syncthreads();
  uint32_t* hw = a.ctl + offsetof(WsControl, hit) / 4;
  const int n = SPLIT_COPIES * split_copy_words(a.k_sel, a.n_ops);
  for (int i = tid; i < n; i += 256) sf_put(hw + i, 0u);
  if (tid < 64) {
    sf_put(a.ctl + offsetof(WsControl, sel_flag) / 4 + 32 * tid, 0u);
    sf_put(a.ctl + offsetof(WsControl, rd_ctr) / 4 + 32 * tid, 0u);
  }
}

// key words of NI u32x4 slots a thread (channels 8m .. 8m+7, m = m0 + 256 i + tid):
// the running max over the batch rows of |x|, RG = 16 / NI rows' loads in flight at
// once (rows past the batch re-read the last row, which leaves the max unchanged)
__device__ __forceinline__ void key_max8x(u32x4& kv, const u32x4& v) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t x2 = v[q] & 0x7FFF7FFFu;
    kv[q] = max(kv[q] & 0xFFFFu, x2 & 0xFFFFu) | (max(kv[q] >> 16, x2 >> 16) << 16);
  }
}
template <int NI>
__device__ __forceinline__ void key_rows(const GemvArgs& a, int m0, int n8, int tid, u32x4 (&kv)[8]) {
  constexpr int RG = 16 / NI;
  const int K = a.k_in;
  for (int b0 = 0; b0 < a.batch; b0 += RG) {
    u32x4 v[RG][NI];
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const u32x4* xr = (const u32x4*)(a.x + (size_t)min(b0 + r, a.batch - 1) * K);
#pragma unroll
      for (int i = 0; i < NI; ++i) v[r][i] = xr[min(m0 + 256 * i + tid, n8 - 1)];
    }
#pragma unroll
    for (int r = 0; r < RG; ++r)
#pragma unroll
      for (int i = 0; i < NI; ++i) key_max8x(kv[i], v[r][i]);
  }
}

// The channel selection of one 256-thread workgroup into LDS (returned: k_sel
// channels, ascending; every thread returns after a barrier), by a two-pass radix
// select over per-wave LDS histograms of the 15-bit |x| keys (max over the batch
// rows).  smem: the selector layout of split_lds_bytes / select_lds_bytes.  ROWS:
// the key loads of several batch rows are issued together (the batched selection
// launch); otherwise row by row, 8 slots a thread (the split kernel, batch 1 or 2).
template <bool ROWS = false>
__device__ __forceinline__ int32_t* split_select(const GemvArgs& a, uint32_t* smem) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.k_in, ks = a.k_sel, n8 = K / 8;
  uint32_t* keys = smem;                       // [K/2]
  uint32_t* bm_sure = keys + K / 2;            // [K/32]
  uint32_t* bm_bnd = bm_sure + K / 32;         // [K/32]
  int32_t* l_sel = (int32_t*)(bm_bnd + K / 32);  // [ks]
  uint32_t (*whist)[256] = (uint32_t (*)[256])(l_sel + ((ks + 3) & ~3));
  uint32_t (*whist2)[128] = (uint32_t (*)[128])(whist[4]);
  int* sc = (int*)(whist2[4]);  // [16]
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
      if constexpr (ROWS) {
        switch (min(8, (n8 - m0 + 255) / 256)) {
          case 1: key_rows<1>(a, m0, n8, tid, kv); break;
          case 2: key_rows<2>(a, m0, n8, tid, kv); break;
          case 3: key_rows<3>(a, m0, n8, tid, kv); break;
          case 4: key_rows<4>(a, m0, n8, tid, kv); break;
          case 5: key_rows<5>(a, m0, n8, tid, kv); break;
          case 6: key_rows<6>(a, m0, n8, tid, kv); break;
          case 7: key_rows<7>(a, m0, n8, tid, kv); break;
          default: key_rows<8>(a, m0, n8, tid, kv); break;
        }
      } else {
        for (int bb = 0; bb < a.batch; ++bb) {
          const u32x4* xr = (const u32x4*)(a.x + (size_t)bb * K);
          u32x4 v[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = xr[min(m0 + 256 * i + tid, n8 - 1)];
#pragma unroll
          for (int i = 0; i < 8; ++i) key_max8x(kv[i], v[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int m = m0 + 256 * i + tid;
        if (m < n8) {
          *(u32x4*)(keys + 4 * m) = kv[i];
          hist_add8(whist[wave], kv[i]);
        }
      }
    }
    lds_barrier();
    int b1, above1;
    wave_threshold4(whist, 256, ks, &b1, &above1);
    // a crowded boundary bin (all-equal inputs) takes wave-aggregated counts below
    const bool crowd = (whist[0][b1] + whist[1][b1]) + (whist[2][b1] + whist[3][b1]) > 2048u;
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
          const uint32_t bin = ((kv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) >> 7;
          sure |= (uint32_t)(bin > (uint32_t)b1) << e;
          bnd |= (uint32_t)(bin == (uint32_t)b1) << e;
        }
        bs[m] = (uint8_t)sure;
        bb[m] = (uint8_t)bnd;
        if (crowd) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if ((bnd >> e) & 1u) hist_add(whist2[wave], (kv[e >> 1] >> (16 * (e & 1))) & 127u);
        } else {
          for (uint32_t r = bnd; r; r &= r - 1u) {  // the boundary bin's keys (few)
            const int e = __builtin_ctz(r);
            atomicAdd(&whist2[wave][(kv[e >> 1] >> (16 * (e & 1))) & 127u], 1u);
          }
        }
      }
    }
    lds_barrier();
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
  return l_sel;
}

// Workgroup 0: selection into LDS, then the lookups, the published copy in the
// workspace and the reports.
template <bool ROWS = false>
__device__ __forceinline__ void split_select_and_publish(const GemvArgs& a, uint32_t* smem) {
  const int tid = threadIdx.x;
  const int ks = a.k_sel;
  const int32_t* l_sel = split_select<ROWS>(a, smem);
  int* sc = (int*)(l_sel + ((ks + 3) & ~3) + 4 * 256 + 4 * 128);  // [16] (after the histograms)
  // the published words first: the channels and, per matrix without resident
  // units, the slots, in SPLIT_COPIES copies
  uint32_t* hw = a.ctl + offsetof(WsControl, hit) / 4;
  const int cst = split_copy_words(ks, a.n_ops);
  for (int j = tid; j < ks; j += 256) {
    const int k = l_sel[j];
#pragma unroll
    for (int c = 0; c < SPLIT_COPIES; ++c) sf_put(hw + c * cst + j, pub_word(k));
#pragma unroll
    for (int op = 0; op < SF_MAX_OPS; ++op) {
      if (op >= a.n_ops) break;
      const PoolDev& pool = a.ops[op].pool;
      if (pool.resident) continue;
      const int slot = pool.unit2slot ? pool.unit2slot[k] : -1;
#pragma unroll
      for (int c = 0; c < SPLIT_COPIES; ++c) sf_put(hw + c * cst + ks * (1 + op) + j, pub_word(slot));
    }
  }
  // the words are complete at the coherence point before any flag goes up
  sf_drain();
  __syncthreads();
  if (tid < 64) sf_put(a.ctl + offsetof(WsControl, sel_flag) / 4 + 32 * tid, 1u);
  // the reports (selection, hits, lookup log: one reservation per matrix) after
  // the flags, off the tiles' path
  if (!a.report) return;
  if (tid < a.n_ops) {
    const PoolDev& pool = a.ops[tid].pool;
    int base = -1;
    if (pool.log_count) {
      base = sf_log_reserve(pool.log_count, (uint32_t)ks, (uint32_t)pool.log_cap);
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
  const bool direct = a.sel_wg == 0;  // the selection is in sel_in, complete before the launch
  if (wave == 0) {
    const bool ok0 = direct || wait_published(a, tile_g & 63);
    if (lane == 0) *sflag = ok0 ? 1 : 0;
  }
  lds_barrier();
  const int tb = (tile_g - o.tile_begin) * 4 * R * r, tw0 = tb >> 5, toff = tb & 31;
  const int wt = (toff + 4 * R * r + 31) >> 5;  // words of the tile's window (<= WTM)
  const int wpu = o.pool.unit_bytes >> 2;
  const uint32_t* units = (const uint32_t*)o.pool.slots;
  const bool resident = o.pool.resident != 0;
  const bool any = *sflag != 0 && (resident || o.pool.unit2slot != nullptr);
  // direct: the first tile of each matrix reports its hits and logs its lookups
  // (one reservation per matrix); the first tile of matrix 0 reports the selection
  const bool reporter = direct && a.report && tile_g == o.tile_begin;
  int log_base = -1;
  if (reporter && o.pool.log_count) {
    if (tid == 0) sflag[1] = sf_log_reserve(o.pool.log_count, (uint32_t)ks, (uint32_t)o.pool.log_cap);
    lds_barrier();
    log_base = sflag[1];
  }
  if (any || reporter) {
    const uint32_t* hc = a.ctl + offsetof(WsControl, hit) / 4 + (tile_g % SPLIT_COPIES) * split_copy_words(ks, a.n_ops);
    for (int j = tid; j < ks; j += 256) {
      int k, slot;
      if (direct) {
        k = a.sel_in ? a.sel_in[j] : j;  // no sel_in: every channel (k_sel = k_in)
        slot = (unsigned)k >= (unsigned)K ? -1 : (resident ? k : (o.pool.unit2slot ? o.pool.unit2slot[k] : -1));
        if (reporter) {
          if (op == 0 && a.sel_out) a.sel_out[j] = k;
          if (o.hit_out) o.hit_out[j] = slot;
          if (log_base >= 0) {
            o.pool.log_units[log_base + j] = k;
            o.pool.log_slots[log_base + j] = slot;
          }
        }
        if (!any) continue;
      } else {
        k = read_published(hc + j, a);
        slot = resident ? k : read_published(hc + ks * (1 + op) + j, a);
      }
      if ((unsigned)k >= (unsigned)K) slot = -1;  // never read outside x or the units
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
  // counted only once every read of the published words has completed (their values
  // are in LDS): the selecting workgroup clears the words when all tiles are counted
  if (tid == 0 && !direct) count_reader(a, tile_g & 63);
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
  __shared__ int lds[25];
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
        hist_add8(whist[wave], kv);
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
      const bool crowd = (whist[0][b1] + whist[1][b1]) + (whist[2][b1] + whist[3][b1]) > 2048u;
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
            const uint32_t bin = ((kv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) >> 7;
            sure |= (uint32_t)(bin > (uint32_t)b1) << e;
            bnd |= (uint32_t)(bin == (uint32_t)b1) << e;
          }
          bs[m] = (uint8_t)sure;
          bb[m] = (uint8_t)bnd;
          if (crowd) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if ((bnd >> e) & 1u) hist_add(whist2[wave], (kv[e >> 1] >> (16 * (e & 1))) & 127u);
          } else {
            for (uint32_t r = bnd; r; r &= r - 1u) {  // the boundary bin's keys (few)
              const int e = __builtin_ctz(r);
              atomicAdd(&whist2[wave][(kv[e >> 1] >> (16 * (e & 1))) & 127u], 1u);
            }
          }
        }
      }
      lds_barrier();
      int b2, above2;
      wave_threshold4(whist2, 128, ks - above1, &b2, &above2);
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
          base = sf_log_reserve(o.pool.log_count, (uint32_t)ks, (uint32_t)o.pool.log_cap);
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
  __shared__ int s_flag[2];
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
  // refinement of the hit channels: + x_k * s[row][k/128] * c_lo[row][k]
  if (refine) split_refine_tile<C, R, NB, wtm_of(R)>(a, o, op, tile_g, row0, szrow, l_hk, l_hx, l_hw, acc, s_flag);
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
}

inline int env_int(const char* name, int dflt) {
  const char* e = getenv(name);
  return e ? atoi(e) : dflt;
}

constexpr size_t MAX_DYN_LDS = 96 * 1024;

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


inline int device_cus() {
  static int n_cu = 0;
  if (n_cu == 0) {
    int dev = 0, cus = 0;
    (void)hipGetDevice(&dev);
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    n_cu = cus;
  }
  return n_cu;
}

// Takes the arguments by value: a fallback below changes sel_wg for this launch
// only, never for the later batch-row launches of the same call.
template <class C, int B, int R, int NB>
sf_status launch_split(GemvArgs a, hipStream_t s) {
  constexpr int D = R >= 8 ? 1 : 2;
  const size_t lds = split_lds_bytes(a.k_in, C::PAIRS, C::CODES, NB, a.k_sel, R, a.sel_wg != 0);
  SF_REQUIRE(lds <= MAX_DYN_LDS, SF_EUNSUPPORTED, "k_in too large for the LDS staging of x");
  // without a selecting workgroup no workgroup waits for another: any grid size
  // the tiles wait for workgroup 0 only at their end, but a tile that has to wait
  // for a free slot adds a whole tile time: when the grid does not fit the device
  // at once, the fused kernel (selection in every workgroup) is used instead
  const int occ = sf_occupancy((const void*)gemv_split_kernel<C, B, R, NB, D>, 256, lds);
  // SF_GEMV_SPLIT=2 always takes the staged variant (x in LDS, workgroup 0 selecting)
  const bool staged = env_int("SF_GEMV_SPLIT", 1) == 2;
  if (a.sel_wg && (staged || (long)occ * device_cus() < (long)a.total_tiles + a.sel_wg)) {
    // the staged variant needs fewer registers; else the fused kernel
    constexpr int D2 = R >= 8 ? 1 : (R >= 4 ? 2 : 4);
    const size_t lds2 = fused_sw_lds_bytes(a.k_in, C::CODES, NB, a.k_sel, R);
    const void* k2 = a.k_in <= 256 * 8 * 2 ? (const void*)gemv_fused_kernel<C, B, R, NB, D2, 2, true>
                                           : (const void*)gemv_fused_kernel<C, B, R, NB, D2, 8, true>;
    const int occ2 = sf_occupancy(k2, 256, lds2);
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

enum GemvKind { KIND_NONE = 0, KIND_FUSED = 1, KIND_SPLIT = 2 };

template <class C, int B, int R>
sf_status dispatch_nb(GemvArgs& a, int nb, int kind, hipStream_t s) {
  if (kind == KIND_SPLIT) return nb == 2 ? launch_split<C, B, R, 2>(a, s) : launch_split<C, B, R, 1>(a, s);
  return nb == 2 ? launch_fused<C, B, R, 2>(a, s) : launch_fused<C, B, R, 1>(a, s);
}

template <class C, int B>
sf_status dispatch_r(GemvArgs& a, int R, int nb, int kind, hipStream_t s) {
  return R == 4 ? dispatch_nb<C, B, 4>(a, nb, kind, s) : dispatch_nb<C, B, 8>(a, nb, kind, s);
}

// Row-tile launch of one resident width (defined in gemv_rows_b<b>.hip).
sf_status gemv_rows_b1(GemvArgs& a, int R, int nb, int kind, hipStream_t s);
sf_status gemv_rows_b2(GemvArgs& a, int R, int nb, int kind, hipStream_t s);
sf_status gemv_rows_b3(GemvArgs& a, int R, int nb, int kind, hipStream_t s);
sf_status gemv_rows_b4(GemvArgs& a, int R, int nb, int kind, hipStream_t s);
sf_status gemv_rows_b8(GemvArgs& a, int R, int nb, int kind, hipStream_t s);

}  // namespace sfg
