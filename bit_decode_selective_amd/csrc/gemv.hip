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
__device__ __forceinline__ uint32_t chan_key(const uint16_t* x, int batch, int K, int k) {
  uint32_t m = 0;
  for (int bb = 0; bb < batch; ++bb) {
    const uint32_t v = x[(size_t)bb * K + k] & 0x7FFFu;
    m = v > m ? v : m;
  }
  return m;
}

__device__ void gemv_select_and_lookup(const GemvArgs& a, uint32_t* hist, int* lds) {
  const int K = a.k_in, ks = a.k_sel, tid = threadIdx.x;
  int32_t* sel = a.ws_sel;
  if (a.sel_in) {
    for (int j = tid; j < ks; j += 256) sel[j] = a.sel_in[j];
  } else if (ks >= K) {
    for (int j = tid; j < ks; j += 256) sel[j] = j;
  } else {
    // radix select on 15-bit keys |x| (fp16 bit patterns order like the values)
    for (int i = tid; i < 256; i += 256) hist[i] = 0;
    __syncthreads();
    for (int k = tid; k < K; k += 256) atomicAdd(&hist[chan_key(a.x, a.batch, K, k) >> 7], 1u);
    __syncthreads();
    wg_suffix_sum256(hist, lds);
    const int b1 = wg_find_threshold(hist, 256, (uint32_t)ks, lds + 4);
    const uint32_t above1 = b1 < 255 ? hist[b1 + 1] : 0u;
    __syncthreads();
    hist[tid] = 0;
    __syncthreads();
    for (int k = tid; k < K; k += 256) {
      const uint32_t kk = chan_key(a.x, a.batch, K, k);
      if ((int)(kk >> 7) == b1) atomicAdd(&hist[kk & 127u], 1u);
    }
    __syncthreads();
    wg_suffix_sum256(hist, lds);
    const int lo = wg_find_threshold(hist, 128, (uint32_t)ks - above1, lds + 4);
    const uint32_t above = above1 + (lo < 127 ? hist[lo + 1] : 0u);
    const uint32_t T = ((uint32_t)b1 << 7) | (uint32_t)lo;
    const int need = ks - (int)above;
    __syncthreads();
    // ordered compaction: thread t owns channels [t*cpt, (t+1)*cpt)
    const int cpt = (K + 255) / 256;
    const int k0 = tid * cpt, k1 = min(K, k0 + cpt);
    int gt = 0, eq = 0;
    for (int k = k0; k < k1; ++k) {
      const uint32_t kk = chan_key(a.x, a.batch, K, k);
      gt += kk > T;
      eq += kk == T;
    }
    int tot;
    const int eq_before = wg_exclusive_scan(eq, lds, &tot);
    const int take_eq = max(0, min(eq, need - eq_before));
    int off = wg_exclusive_scan(gt + take_eq, lds, &tot);
    int eq_seen = 0;
    for (int k = k0; k < k1; ++k) {
      const uint32_t kk = chan_key(a.x, a.batch, K, k);
      if (kk > T) {
        sel[off++] = k;
      } else if (kk == T) {
        if (eq_seen < take_eq) sel[off++] = k;
        ++eq_seen;
      }
    }
  }
  __threadfence();
  __syncthreads();
  __threadfence();
  if (a.sel_out && a.do_log)
    for (int j = tid; j < ks; j += 256) a.sel_out[j] = sel[j];
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
        a.ws_hit_k[op * ks + pos] = k;
        a.ws_hit_slot[op * ks + pos] = slot;
        ++pos;
      }
    }
    if (tid == 0) a.ws_nhit[op] = tot;
    __syncthreads();
  }
}

// ---- the GEMV kernel -------------------------------------------------------------
// Persistent workgroups of 4 waves.  Row tiles of 4R rows (R per wave) are dealt to
// workgroups round-robin: workgroup g takes tiles g, g + grid, ...  Within a tile,
// lane l of a wave owns chunks l, l+64, ... of each of the wave's R rows.  x is
// staged once per workgroup.  NB batch rows [batch_off, batch_off + NB) per launch.
template <class C, int B, int R, int NB>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a) {
  extern __shared__ uint32_t smem[];
  __shared__ uint32_t s_hist[256];
  __shared__ int s_lds[8];
  __shared__ float s_y[NB][4 * R];
  __shared__ float s_red[NB][256];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.k_in;
  const int nchunks = K / C::CODES;
  const int xpairs = K / 2;
  uint32_t* xs = smem;                         // [NB][K/2] fp16 pairs
  float* xsum = (float*)(smem + NB * xpairs);  // [NB][nchunks]
  const bool refine = a.k_sel > 0;
  const int rows_wg = 4 * R;

  if (tid == 0) s_lds[7] = refine ? (atomicCAS(&a.ctl->sel_state, 0u, 1u) == 0u) : 0;

  // stage x in pair order; per-chunk sums of x by the lanes holding the chunk's pairs
  for (int bb = 0; bb < NB; ++bb) {
    const uint16_t* xr = a.x + (size_t)(a.batch_off + bb) * K;
    for (int p0 = 0; p0 < xpairs; p0 += 256) {
      const int p = p0 + tid;
      float v = 0.f;
      if (p < xpairs) {
        const int c = p / C::PAIRS, j = p - c * C::PAIRS;
        const int kb = c * C::CODES;
        const uint32_t pr = (uint32_t)xr[kb + C::pair_k0(j)] | ((uint32_t)xr[kb + C::pair_k1(j)] << 16);
        xs[bb * xpairs + p] = pr;
        const h2_t h = as_h2(pr);
        v = (float)h.x + (float)h.y;
      }
#pragma unroll
      for (int o = C::PAIRS / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, C::PAIRS);
      if (p < xpairs && (p % C::PAIRS) == 0) xsum[bb * nchunks + p / C::PAIRS] = v;
    }
  }
  __syncthreads();

  const bool selector = s_lds[7] != 0;
  if (selector) {
    gemv_select_and_lookup(a, s_hist, s_lds);
    __threadfence();
    __syncthreads();
    if (tid == 0) __hip_atomic_store(&a.ctl->sel_state, 2u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }

  const size_t rowbytes = (size_t)K * B / 8;
  const int ngr = K / 128;
  const float scl = (float)(1u << (a.r + B));

  // resident GEMV over this workgroup's tiles; y = x W_res^T written per tile
  for (int tile_g = blockIdx.x; tile_g < a.total_tiles; tile_g += gridDim.x) {
    int op = 0;
    for (int i = 1; i < a.n_ops; ++i)
      if (tile_g >= a.ops[i].tile_begin) op = i;
    const GemvOpDev& o = a.ops[op];
    const int tile = tile_g - o.tile_begin;
    const int row0 = tile * rows_wg + wave * R;
    float acc[NB][R];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[bb][r] = 0.f;

    for (int c = lane; c < nchunks; c += 64) {
      uint32_t cw[R][C::WORDS];
      uint32_t szw[R];
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

  // sparse refinement delta over this workgroup's tiles: y += sum over hit
  // channels of x_k * s * c_lo (each row is read back by the lane that wrote it)
  if (refine) {
    int ok = 1;
    if (!selector) {
      if (tid == 0) s_lds[5] = sf_wait_word(&a.ctl->sel_state, 2u, &a.ctl->timeout) ? 1 : 0;
      __syncthreads();
      ok = s_lds[5];
    }
    // y rows written above by lane 0 of each wave are read back below by other
    // threads of this workgroup
    __threadfence();
    __syncthreads();
    if (ok) {
      for (int tile_g = blockIdx.x; tile_g < a.total_tiles; tile_g += gridDim.x) {
        int op = 0;
        for (int i = 1; i < a.n_ops; ++i)
          if (tile_g >= a.ops[i].tile_begin) op = i;
        const GemvOpDev& o = a.ops[op];
        const int tile = tile_g - o.tile_begin;
        const int nh = a.ws_nhit[op];
        const int i = tid % rows_wg, mstep = 256 / rows_wg;
        const int row = tile * rows_wg + i;
        float part[NB];
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) part[bb] = 0.f;
        if (row < o.n_out) {
          const int* hk = a.ws_hit_k + op * a.k_sel;
          const int* hs = a.ws_hit_slot + op * a.k_sel;
          for (int m = tid / rows_wg; m < nh; m += mstep) {
            const int k = hk[m];
            const uint8_t* unit = o.pool.slots + (size_t)hs[m] * o.pool.unit_bytes;
            const float clo = (float)read_field(unit, (uint32_t)row * a.r, a.r);
            const float sv = sf_h2f(o.sz[(size_t)row * ngr + k / 128]);
            const int c = k / C::CODES, kk = k - c * C::CODES;
            int jj, hi;
            C::locate(kk, &jj, &hi);
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) {
              const h2_t xh = as_h2(xs[bb * xpairs + c * C::PAIRS + jj]);
              const float xk = hi ? (float)xh.y : (float)xh.x;
              part[bb] += (xk * sv) * clo;
            }
          }
        }
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) s_red[bb][tid] = part[bb];
        __syncthreads();
        if (tid < rows_wg && row < o.n_out) {
#pragma unroll
          for (int bb = 0; bb < NB; ++bb) {
            float sum = 0.f;
            for (int j = tid; j < 256; j += rows_wg) sum += s_red[bb][j];
            float* yp = o.y + (size_t)(a.batch_off + bb) * o.n_out + row;
            *yp = *yp + sum;
          }
        }
        __syncthreads();
      }
    }
    __syncthreads();
    if (tid == 0) {
      const uint32_t prev = atomicAdd(&a.ctl->done, 1u);
      if (prev == gridDim.x - 1u) {
        __hip_atomic_store(&a.ctl->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&a.ctl->sel_state, 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

int env_int(const char* name, int dflt) {
  const char* e = getenv(name);
  return e ? atoi(e) : dflt;
}

template <class C, int B, int R, int NB>
sf_status launch_gemv(GemvArgs& a, hipStream_t s) {
  const size_t lds = (size_t)NB * (a.k_in / 2) * 4 + (size_t)NB * (a.k_in / C::CODES) * 4;
  SF_REQUIRE(lds <= 64 * 1024, SF_EUNSUPPORTED, "k_in too large for the LDS staging of x");
  // persistent grid: about SF_GEMV_WGS_PER_CU workgroups per CU, each taking an
  // equal number of tiles
  const int per_cu = env_int("SF_GEMV_WGS_PER_CU", 4);
  const int cap = 256 * (per_cu > 0 ? per_cu : 4);
  const int tiles_per_wg = (a.total_tiles + cap - 1) / cap;
  const int grid = (a.total_tiles + tiles_per_wg - 1) / tiles_per_wg;
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
    default: return dispatch_nb<C, B, 4>(a, nb, s);
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
  // rows per wave (SF_GEMV_ROWS_PER_WAVE = 1, 2 or 4 overrides the default)
  int rpw = env_int("SF_GEMV_ROWS_PER_WAVE", 0);
  int64_t rows_total = 0;
  for (int i = 0; i < n_ops; ++i) rows_total += ops[i].w.n_out;
  if (rpw != 1 && rpw != 2 && rpw != 4) rpw = rows_total <= 8192 ? 1 : (rows_total <= 16384 ? 2 : 4);
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
  for (int b0 = 0; b0 < batch; b0 += 2) {
    const int nb = (batch - b0) >= 2 ? 2 : 1;
    a.batch_off = b0;
    a.do_log = b0 == 0;
    sf_status st = dispatch_b(a, f.b, rpw, nb, s);
    if (st != SF_OK) return st;
  }
  return SF_OK;
}
