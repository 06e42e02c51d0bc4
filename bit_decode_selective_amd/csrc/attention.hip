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
// Kernels (per call, one KV head = one (batch, kv head) pair):
//   split  : a workgroup per 256 tokens streams the resident keys: logits of the G
//            query heads on MFMA (key codes expanded into fp16 mantissas, value
//            1 + c/2^b, times q), split-local softmax max m_s and sum z_s.  Without
//            refinement it also streams the values and forms the split's value sum
//            N_s = sum_t e^(l - m_s) V_b[t] (flash-decoding partials).
//   select : a 1024-thread workgroup per 4096-token chunk.  Merges the split
//            statistics into the softmax max / sum of each head.  Without
//            refinement it merges the partials and the last chunk writes the output.
//            With refinement it scores its chunk (softmax weight summed over the G
//            heads) and, with the other chunks of the KV head, finds the exact k-th
//            score by a radix select over shared histograms (ties to the lower
//            token); each chunk writes its part of the ascending selection, looks it
//            up in the refinement cache and replaces the logits of its hits by
//            l' = l + scale * s_K * (q . cK_lo) and records its max logit after
//            replacement.
//   pv     : (refinement only) a workgroup per 512 tokens (256 for b = 8) forms
//            the final weights e^(l - max), sums weight * V_b on MFMA
//            and adds weight * s_V * cV_lo for its hits; the last workgroup of the
//            KV head divides numerator by denominator.
// Weights are final and positive before anything is accumulated, so no sum
// cancels a large term.  Value sums on MFMA use the weight as an fp16 high part
// plus an fp16 low part (about 22 bits) times codes in the 1 + c/2^b form.
// The chunks of one KV head in `select` wait for each other at up to four points
// (bounded spins).  Workgroups are dispatched in order and a KV head has at most
// 256 chunks, so the chunks of a KV head are resident together.
#include "group_quant.h"
#include "sf_internal.h"

namespace {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int HD = 128;          // head dim
constexpr int SA = 256;          // tokens per split workgroup
constexpr int CB = 4096;         // tokens per select workgroup (chunk)
constexpr int SEL_T = 1024;      // threads of a select workgroup
constexpr int TPT = CB / SEL_T;  // tokens per select thread
constexpr int PW = HD + 4;       // partial record: N[HD], max, sum, pad
constexpr int NBIN = 2048;       // histogram bins (levels: key bits 30..20, 19..10, 9..0)
constexpr int MAX_CHUNKS = 256;
constexpr int PV_NR = 8;                // value-sum records per KV head (pv split s adds into record s % PV_NR)
constexpr float SCORE_CUTOFF = -64.f;  // logit below the head's max past which a weight scores 0

__host__ __device__ constexpr int pv_tokens(int b) { return b <= 4 ? 512 : 256; }

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
  int batch, n_q, n_kv, G, T, LT, t_cap, b, r, k_sel, nsa, s2, nsp;
  int variant;  // SF_ATTN_NESTED, SF_ATTN_FP16_TOKENS or SF_ATTN_DROP_UNSELECTED
  int spw;      // pv splits per workgroup
  float scale;
  float* logits;    // [batch*n_q][LT] (rows padded to 4 floats)
  float* part_a;    // [bh][nsa][G][PW]: split max / sum (+ value sums without refinement)
  float2* part_ms;  // [bh][nsa][G]: split max / sum again, packed (the select kernel's merge reads these)
  float* part_c;    // [bh][s2][G][PW]: chunk sums (without refinement)
  float* part_p;    // [bh][PV_NR][G][PW]: value sums of the splits (with refinement)
  float* cmax;      // [bh][s2][G]: chunk max of the replaced logits
  int32_t* sel_ws;  // [bh][KS]: selection
  int32_t* slot_ws; // [bh][KS]: slot of each selected token, -1 = miss
  uint32_t* hist;   // [bh][3][NBIN]
  uint32_t* ctl;    // [bh][8]: arrival counters 0..4 and 6; word 5 of KV head 0: lookup-log base
  uint32_t* cnts;   // [bh][s2][2]: per chunk (above, equal) counts
  const int32_t* sel_in;
  int32_t* sel_out;
  int32_t* hit_out;
  float* out;       // [batch][n_q][HD]
  uint16_t* out16;  // the same as fp16 bits (round to nearest even), or null
  uint32_t* timeout;
  PoolDev pool;
  // appending the new token at position T - 1 in the split pass (k_new non-null):
  // its K and V rows [bh][HD] fp32, and where its refinement units go (the unit of
  // KV head bh at ap_refine + bh * ap_refine_ld * unit_bytes; may be null)
  const float* k_new;
  const float* v_new;
  uint8_t* ap_refine;
  int64_t ap_refine_ld;
};

__device__ __forceinline__ void merge_ms(float& m, float& z, float om, float oz) {
  const float nm = fmaxf(m, om);
  if (nm == -INFINITY) return;
  z = (m > -INFINITY ? z * __expf(m - nm) : 0.f) + (om > -INFINITY ? oz * __expf(om - nm) : 0.f);
  m = nm;
}

typedef _Float16 h2v_t __attribute__((ext_vector_type(2)));

// Two codes (low, high half) as the exact fp16 values c/2^B: built as 1 + c/2^B in
// the mantissa, then one exact packed fp16 subtraction of 1.  A value sum on MFMA is
// then the sum itself, not the difference of two larger sums.
template <int B>
__device__ __forceinline__ uint32_t code_pair(uint32_t c_lo, uint32_t c_hi) {
  const h2v_t one = {(_Float16)1.f, (_Float16)1.f};
  const uint32_t x = (((c_hi << 16) | c_lo) << (10 - B)) | 0x3C003C00u;
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2v_t, x) - one);
}

// B operand of a value-sum MFMA: the codes of dim d for this lane's 8 tokens
// tk0..tk0+7 (rows of the LDS-staged codes, stride WPTP words), as c/2^B.
template <int B, int WPTP>
__device__ __forceinline__ u32x4 code_operand(const uint32_t* s_vc, int tk0, int d) {
  constexpr uint32_t cmask = (1u << B) - 1u;
  const int bit = d * B, wi = bit >> 5, sh = bit & 31;
  uint32_t c[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) c[e] = (s_vc[(tk0 + e) * WPTP + wi] >> sh) & cmask;
  u32x4 bv;
#pragma unroll
  for (int e = 0; e < 4; ++e) bv[e] = code_pair<B>(c[2 * e], c[2 * e + 1]);
  return bv;
}

// ---- split: logits, split softmax statistics (and value sums) --------------------
template <int B, int G, bool PV>
__global__ __launch_bounds__(256) void attn_split_kernel(AttnArgs a) {
  constexpr int WPT = HD * B / 32;  // code words per token
  constexpr int WPTP = WPT + 1;     // padded LDS row (conflict-free column reads)
  constexpr int UP = SA + 8;        // padded A-operand row (halves)
  constexpr int P = 32 / B, HP = P / 2;
  __shared__ uint32_t s_vc[PV ? SA * WPTP : 1];
  __shared__ uint32_t s_ksz[SA], s_vsz[PV ? SA : 1];
  __shared__ float s_l[G][SA];
  __shared__ _Float16 s_u[PV ? 2 * G : 1][UP];
  __shared__ float s_red[4][3 * G + 1];
  __shared__ float s_st[3 * G + 1];
  __shared__ uint8_t s_aq[2][256];       // the appended token's codes (quantiser scratch)
  __shared__ uint32_t s_nk[2][4 * B];    // its resident words, K and V
  __shared__ uint32_t s_nsz[2];          // its sz words
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x, bh = blockIdx.y;
  const int bi = bh / a.n_kv, kvh = bh - bi * a.n_kv;
  const int T = a.T;
  const int t_begin = split * SA, n_here = min(SA, T - t_begin);
  const size_t tok0 = (size_t)bh * a.t_cap + t_begin;

  // the new token, when this call appends it and this split holds position T - 1:
  // waves 0 and 1 quantise its K and V rows exactly as the KV append does (codes,
  // sz words and refinement units into the cache), and this workgroup takes the
  // token's words from LDS rather than reading back what it has just written
  const int tnew = a.k_new ? T - 1 - t_begin : -1;
  const bool app = tnew >= 0 && tnew < SA;
  if (app) {
    if (wave < 2) {
      const size_t pos = (size_t)bh * a.t_cap + (T - 1);
      uint8_t* res = const_cast<uint8_t*>(wave ? a.v_res : a.k_res);
      uint32_t* szp = const_cast<uint32_t*>(wave ? a.v_sz : a.k_sz);
      uint32_t* ref = a.ap_refine && a.r > 0
                          ? (uint32_t*)(a.ap_refine + (size_t)bh * a.ap_refine_ld * (2 * 16 * a.r) + wave * 16 * a.r)
                          : nullptr;
      sfq::quantize_group_wave((wave ? a.v_new : a.k_new) + (size_t)bh * HD, B, a.r, s_aq[wave], s_aq[wave] + 128,
                               (uint32_t*)(res + pos * 16 * B), szp + pos, ref, s_nk[wave], &s_nsz[wave]);
    }
    __syncthreads();
  }

  // this call's selection histograms, counters and lookup-log base
  if (a.k_sel > 0) {
    uint32_t* h = a.hist + (size_t)bh * 3 * NBIN;
    for (int i = split * 256 + tid; i < 3 * NBIN; i += a.nsa * 256) h[i] = 0;
    float* pp = a.part_p + (size_t)bh * PV_NR * G * PW;  // the value-sum records of the KV head
    for (int i = split * 256 + tid; i < PV_NR * G * PW; i += a.nsa * 256) pp[i] = 0.f;
    if (split == 0 && tid == 0) {
      for (int i = 0; i < 8; ++i)
        if (i != 5) a.ctl[bh * 8 + i] = 0;
      if (bh == 0) {
        int base = -1;
        if (a.pool.log_count) {
          const uint32_t n = (uint32_t)(a.batch * a.n_kv) * (uint32_t)a.k_sel;
          base = sf_log_reserve(a.pool.log_count, n, (uint32_t)a.pool.log_cap);
        }
        a.ctl[5] = (uint32_t)base;
      }
    }
  } else if (split == 0 && tid == 0) {
    a.ctl[bh * 8 + 4] = 0;
  }

  // loads: (value codes -> LDS), scale words -> LDS, key codes -> registers
  if constexpr (PV) {
    const u32x4* src = (const u32x4*)(a.v_res + tok0 * (HD * B / 8));
    const int nv = n_here * WPT / 4;
    for (int i = tid; i < nv; i += 256) {
      const int w = 4 * i, tk = w / WPT, c = w - tk * WPT;
      if (tk == tnew) continue;
      const u32x4 v = __builtin_nontemporal_load(src + i);
      uint32_t* d = s_vc + tk * WPTP + c;
      d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    }
    if (app && tid < WPT) s_vc[tnew * WPTP + tid] = s_nk[1][tid];
    s_vsz[tid] = tid == tnew ? s_nsz[1] : (tid < n_here ? a.v_sz[tok0 + tid] : 0u);
  }
  s_ksz[tid] = tid == tnew ? s_nsz[0] : (tid < n_here ? a.k_sz[tok0 + tid] : 0u);
  const int n = lane & 15, qg = lane >> 4;
  uint32_t kw[4][B];  // wave: 4 tiles of 16 tokens; lane: token n of each tile, dims 32qg..
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int tl = wave * 64 + 16 * u + n;
    if (tl == tnew) {
#pragma unroll
      for (int w = 0; w < B; ++w) kw[u][w] = s_nk[0][qg * B + w];
    } else if (tl < n_here) {
      const uint32_t* src = (const uint32_t*)(a.k_res + (tok0 + tl) * (HD * B / 8)) + qg * B;
      if constexpr (B == 1) {
        kw[u][0] = __builtin_nontemporal_load(src);
      } else if constexpr (B == 2) {
        const u32x2 v = __builtin_nontemporal_load((const u32x2*)src);
        kw[u][0] = v.x; kw[u][1] = v.y;
      } else {
#pragma unroll
        for (int q4 = 0; q4 < B / 4; ++q4) {
          const u32x4 v = __builtin_nontemporal_load((const u32x4*)src + q4);
          kw[u][4 * q4] = v.x; kw[u][4 * q4 + 1] = v.y; kw[u][4 * q4 + 2] = v.z; kw[u][4 * q4 + 3] = v.w;
        }
      }
    } else {
#pragma unroll
      for (int w = 0; w < B; ++w) kw[u][w] = 0;
    }
  }
  // B operand: q of head n (zero for n >= G) over dims 32qg.., in the codes' pair order
  h8_t bq[4];
  float qsum;
  {
    const uint16_t* qrow = a.q + ((size_t)bi * a.n_q + (size_t)kvh * G + (n < G ? n : 0)) * HD;
    uint16_t q32[32];
    const u32x4* qv = (const u32x4*)(qrow + 32 * qg);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 v = qv[i];
      const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) q32[8 * i + e] = (uint16_t)(wds[e >> 1] >> (16 * (e & 1)));
    }
    float qpart = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int p = 4 * j + (e >> 1), hh = e & 1;
        const int w = p / HP, i = p % HP;
        const float v = n < G ? h2f16(q32[P * w + i + hh * HP]) : 0.f;
        bq[j][e] = (_Float16)v;
        qpart += v;
      }
    qpart += __shfl_xor(qpart, 16, 64);
    qpart += __shfl_xor(qpart, 32, 64);
    qsum = qpart;
  }
  __syncthreads();  // s_ksz (s_vsz, s_vc)

  // ---- logits on MFMA ----
  const float kscl = (float)(1u << (a.r + B));
  constexpr uint32_t m1 = ((1u << B) - 1u) << (10 - B);
  const bool want_logits = a.k_sel > 0;
  float* lrow = a.logits + ((size_t)bi * a.n_q + kvh * G + (n < G ? n : 0)) * a.LT + t_begin;
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
        const uint32_t t = sh >= 0 ? (kw[u][w] << sh) : (kw[u][w] >> (-sh));
        pr[v] = (t & (m1 | (m1 << 16))) | 0x3C003C00u;
      }
      const u32x4 pv = {pr[0], pr[1], pr[2], pr[3]};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, pv), bq[j], acc, 0, 0, 0);
    }
    if (n < G) {
      const int tb = wave * 64 + 16 * u + 4 * qg;
      float l4[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint32_t szw = s_ksz[tb + v];
        const float s = sf_h2f(szw), z = sf_h2f(szw >> 16);
        l4[v] = tb + v < n_here ? a.scale * (z * qsum + (s * kscl) * (acc[v] - qsum)) : -INFINITY;
        s_l[n][tb + v] = l4[v];
      }
      if (want_logits) {
        if (tb + 3 < n_here) {
          *(f4_t*)(lrow + tb) = f4_t{l4[0], l4[1], l4[2], l4[3]};
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (tb + v < n_here) lrow[tb + v] = l4[v];
        }
      }
    }
  }
  __syncthreads();  // s_l

  // ---- split max per head (and the largest value scale) ----
  const int t = tid;  // this thread's token within the split
  float sv = 0.f, zv = 0.f;
  if constexpr (PV) {
    const uint32_t vsz = s_vsz[t];
    sv = sf_h2f(vsz);
    zv = sf_h2f(vsz >> 16);
  }
  {
    float mx[G + 1];
#pragma unroll
    for (int h = 0; h < G; ++h) mx[h] = s_l[h][t];
    mx[G] = t < n_here ? sv : 0.f;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
#pragma unroll
      for (int h = 0; h <= G; ++h) mx[h] = fmaxf(mx[h], __shfl_xor(mx[h], o, 64));
    if (lane == 0)
#pragma unroll
      for (int h = 0; h <= G; ++h) s_red[wave][h] = mx[h];
    __syncthreads();
    if (tid <= G) s_st[tid] = fmaxf(fmaxf(s_red[0][tid], s_red[1][tid]), fmaxf(s_red[2][tid], s_red[3][tid]));
    __syncthreads();
  }
  // fp16 A operand scaled by 2^shift so that the largest weight * scale is below 2^14
  const float smax = s_st[G] * (float)(1u << a.r);
  int e2 = 0;
  if (smax > 0.f) (void)frexpf(smax, &e2);
  const int shift = smax > 0.f ? 14 - e2 : 0;
  const float uscale = ldexpf((float)(1u << a.r), shift);
  float ms[G], acc3[3 * G];
#pragma unroll
  for (int h = 0; h < G; ++h) ms[h] = s_st[h];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float w = t < n_here ? __expf(s_l[h][t] - ms[h]) : 0.f;
    acc3[3 * h] = w;
    acc3[3 * h + 1] = acc3[3 * h + 2] = 0.f;
    if constexpr (PV) {
      const float u = w * sv * uscale;
      // weight * scale as an fp16 high part plus a low part scaled by 2^11, which
      // stays a normal fp16 (about 22 bits for weights down to 2^-28 of the largest)
      const _Float16 hi = (_Float16)u;
      const _Float16 lo = (_Float16)((u - (float)hi) * 2048.f);
      s_u[2 * h][t] = hi;
      s_u[2 * h + 1][t] = lo;
      acc3[3 * h + 1] = w * zv;
    }
  }
  __syncthreads();  // s_u written; s_red free
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1)
#pragma unroll
    for (int i = 0; i < 3 * G; ++i) acc3[i] += __shfl_xor(acc3[i], o, 64);
  if (lane == 0)
#pragma unroll
    for (int i = 0; i < 3 * G; ++i) s_red[wave][i] = acc3[i];

  f4_t pacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  if constexpr (PV) {
    // value sums on MFMA; wave w: dims [32w, 32w+32) as two 16-dim blocks; A rows
    // 2h / 2h+1 = high / low part of head h's scaled weights
#pragma unroll 2
    for (int kb = 0; kb < SA / 32; ++kb) {
      const int tk0 = 32 * kb + 8 * qg;
      h8_t av;
      if (n < 2 * G) {
        av = *(const h8_t*)(&s_u[n][tk0]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) av[e] = (_Float16)0.f;
      }
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const u32x4 bv = code_operand<B, WPTP>(s_vc, tk0, 32 * wave + 16 * db + n);
        pacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(h8_t, bv), pacc[db], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // s_red
  if (tid < 3 * G) s_st[tid] = (s_red[0][tid] + s_red[1][tid]) + (s_red[2][tid] + s_red[3][tid]);
  __syncthreads();
  float* PS = a.part_a + ((size_t)bh * a.nsa + split) * G * PW;
  if constexpr (PV) {
    // lane group qg holds rows 4qg..4qg+3 = head 2qg (rows 0, 1) and head 2qg+1 (rows 2, 3)
    const float back = ldexpf(1.f, B - shift);  // 2^B undoes the c/2^B form, 2^-shift the scaling
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int d = 32 * wave + 16 * db + n;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int h = 2 * qg + hh;
        if (h < G) {
          const float D = pacc[db][2 * hh] + pacc[db][2 * hh + 1] * (1.f / 2048.f);
          PS[h * PW + d] = s_st[3 * h + 1] + back * D;
        }
      }
    }
  }
  if (tid < G) {
    PS[tid * PW + HD] = ms[tid];
    PS[tid * PW + HD + 1] = s_st[3 * tid];
    a.part_ms[((size_t)bh * a.nsa + split) * G + tid] = make_float2(ms[tid], s_st[3 * tid]);
  }
}

// ---- select / merge ----------------------------------------------------------------
__device__ __forceinline__ int blk_exclusive_scan(int v, int* lds, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int NW = SEL_T / 64;
  const int incl = sf_wave_incl_scan(v);
  __syncthreads();
  if (lane == 63) lds[wave] = incl;
  __syncthreads();
  int base = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = lds[w];
    if (w < wave) base += t;
    sum += t;
  }
  *total = sum;
  return base + incl - v;
}

// Over nb bins in LDS (nb = 1024 or 2048): the largest bin whose suffix count
// reaches `need`.  Returns the bin; *above = count of the bins after it, *inbin =
// its own count.  Every thread gets the answer.
__device__ int blk_threshold(const uint32_t* h, int nb, int need, int* lds, int* above, int* inbin) {
  const int per = nb / SEL_T;  // 1 or 2
  const int t = threadIdx.x;
  const int top = nb - 1 - per * t;  // this thread's bins: top, top-1, ..
  if (t == 0) {
    lds[32] = 0;
    lds[33] = 0;
    lds[34] = 0;
  }
  int s = 0;
  for (int i = 0; i < per; ++i) s += (int)h[top - i];
  int tot;
  const int ex = blk_exclusive_scan(s, lds, &tot);
  int run = ex;
  for (int i = 0; i < per; ++i) {
    const int c = (int)h[top - i];
    if (run < need && run + c >= need) {
      lds[32] = top - i;
      lds[33] = run;
      lds[34] = c;
    }
    run += c;
  }
  __syncthreads();
  const int bin = lds[32];
  *above = lds[33];
  *inbin = lds[34];
  __syncthreads();
  return bin;
}

// This workgroup's contribution is written; count it and wait until all n chunks
// of the KV head have arrived.
__device__ __forceinline__ void chunk_barrier(uint32_t* ctr, uint32_t n, uint32_t* timeout) {
  sf_drain();
  __syncthreads();
  if (threadIdx.x == 0) {
    (void)sf_add_release(ctr, 1u);
    (void)sf_wait_word(ctr, n, timeout);
  }
  __syncthreads();
}

// q_h . cK_lo for the G heads h, over the HD r-bit key refinement codes at the start
// of a unit (each code extracted once; dims summed in order)
template <int G, int R>
__device__ __forceinline__ void kref_dots_r(const uint8_t* unit, const float (*qf)[HD], float (&dot)[G]) {
  constexpr int NW = HD * R / 32;
  uint32_t w[NW];
  const u32x4* u4 = (const u32x4*)unit;
#pragma unroll
  for (int i = 0; i < NW / 4; ++i) {
    const u32x4 v = u4[i];
    w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
  }
#pragma unroll
  for (int h = 0; h < G; ++h) dot[h] = 0.f;
  // one code word per step (the words shift down, so every index is static)
#pragma unroll 1
  for (int wi = 0; wi < NW; ++wi) {
    const uint32_t wv = w[0];
#pragma unroll
    for (int k = 0; k + 1 < NW; ++k) w[k] = w[k + 1];
#pragma unroll
    for (int e = 0; e < 32 / R; ++e) {
      const float c = (float)((wv >> (e * R)) & ((1u << R) - 1u));
      const int i = wi * (32 / R) + e;
#pragma unroll
      for (int h = 0; h < G; ++h) dot[h] = fmaf(qf[h][i], c, dot[h]);
    }
  }
}

template <int G>
__device__ __forceinline__ void kref_dots(const uint8_t* unit, int r, const float (*qf)[HD], float (&dot)[G]) {
  if (r == 2) return kref_dots_r<G, 2>(unit, qf, dot);
  if (r == 1) return kref_dots_r<G, 1>(unit, qf, dot);
  const uint32_t* w = (const uint32_t*)unit;
#pragma unroll
  for (int h = 0; h < G; ++h) dot[h] = 0.f;
  for (int i = 0; i < HD; ++i) {
    const float c = (float)field(w, i * r, r);
#pragma unroll
    for (int h = 0; h < G; ++h) dot[h] = fmaf(qf[h][i], c, dot[h]);
  }
}

// q_h . K16 for the G heads h, over a unit that holds the key as HD fp16 values
// (then the value's)
template <int G>
__device__ __forceinline__ void k16_dots(const uint8_t* unit, const float (*qf)[HD], float (&dot)[G]) {
  const u32x4* u4 = (const u32x4*)unit;
#pragma unroll
  for (int h = 0; h < G; ++h) dot[h] = 0.f;
#pragma unroll 2
  for (int i = 0; i < HD / 8; ++i) {
    const u32x4 v = u4[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float k0 = h2f16((uint16_t)(v[e] & 0xFFFFu)), k1 = h2f16((uint16_t)(v[e] >> 16));
#pragma unroll
      for (int h = 0; h < G; ++h) {
        dot[h] = fmaf(qf[h][8 * i + 2 * e], k0, dot[h]);
        dot[h] = fmaf(qf[h][8 * i + 2 * e + 1], k1, dot[h]);
      }
    }
  }
}

template <int G>
__global__ __launch_bounds__(SEL_T) void attn_select_kernel(AttnArgs a) {
  __shared__ uint32_t lh[NBIN];
  __shared__ int s_tok[CB];
  __shared__ int s_slot[CB];
  __shared__ float qf[G][HD];
  __shared__ float s_m[G], s_iz[G];
  __shared__ float s_wm[SEL_T / 64][G][2];
  __shared__ int lds[40];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int bi = bh / a.n_kv, kvh = bh - bi * a.n_kv;
  const int T = a.T, ks = a.k_sel, s2 = a.s2;
  const int KS = ks > 0 ? ks : 1;
  const int c0 = chunk * CB;
  uint32_t* ctl = a.ctl + bh * 8;
  if (ks > 0)
    for (int i = tid; i < G * HD; i += SEL_T) {
      const int h = i / HD, d = i - h * HD;
      qf[h][d] = h2f16(a.q[((size_t)bi * a.n_q + kvh * G + h) * HD + d]);
    }

  // this thread's logits (TPT consecutive tokens per head), requested before the
  // split statistics are merged so that the two round trips overlap
  const int tb = c0 + TPT * tid;
  f4_t l4p[G];
  if (ks > 0 && a.sel_in == nullptr) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float* lr = a.logits + ((size_t)bi * a.n_q + kvh * G + h) * a.LT + tb;
      l4p[h] = f4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      if (tb + 3 < T) {
        l4p[h] = *(const f4_t*)lr;
      } else {
#pragma unroll
        for (int i = 0; i < TPT; ++i)
          if (tb + i < T) l4p[h][i] = lr[i];
      }
    }
  }

  // ---- softmax max / sum per head from the split statistics ----
  {
    constexpr int NJ = SEL_T / G;
    const int h = tid % G, j = tid / G;
    float m = -INFINITY, z = 0.f;
    const float2* PM = a.part_ms + (size_t)bh * a.nsa * G;
    for (int s0 = j; s0 < a.nsa; s0 += 4 * NJ) {  // four records requested at once
      float2 r[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) r[u] = s0 + u * NJ < a.nsa ? PM[(s0 + u * NJ) * G + h] : make_float2(-INFINITY, 0.f);
#pragma unroll
      for (int u = 0; u < 4; ++u) merge_ms(m, z, r[u].x, r[u].y);
    }
#pragma unroll
    for (int o = G; o < 64; o <<= 1) merge_ms(m, z, __shfl_xor(m, o, 64), __shfl_xor(z, o, 64));
    if (lane < G) {
      s_wm[wave][lane][0] = m;
      s_wm[wave][lane][1] = z;
    }
    __syncthreads();
    if (tid < G) {
      float mm = -INFINITY, zz = 0.f;
      for (int w = 0; w < SEL_T / 64; ++w) merge_ms(mm, zz, s_wm[w][tid][0], s_wm[w][tid][1]);
      s_m[tid] = mm;
      s_iz[tid] = 1.f / zz;
    }
    __syncthreads();
  }

  if (ks == 0) {
    // ---- no refinement: this chunk's value sums relative to the global max ----
    float* PC = a.part_c + ((size_t)bh * s2 + chunk) * G * PW;
    if (tid < G * HD) {
      const int s_lo = c0 / SA, s_hi = min(a.nsa, (c0 + CB) / SA);
      const int h = tid / HD, d = tid - h * HD;
      const float* PA = a.part_a + (size_t)bh * a.nsa * G * PW;
      float nc = 0.f, zc = 0.f;
      const float mh = s_m[h];
      for (int s = s_lo; s < s_hi; ++s) {
        const float* r = PA + (s * G + h) * PW;
        const float f = __expf(r[HD] - mh);
        nc = fmaf(f, r[d], nc);
        if (d == 0) zc = fmaf(f, r[HD + 1], zc);
      }
      sf_put(PC + h * PW + d, nc);
      if (d == 0) sf_put(PC + h * PW + HD + 1, zc);
    }
    sf_drain();
    __syncthreads();
    if (tid == 0)
      lds[36] = sf_add_acq_rel(ctl + 4, 1u) == (uint32_t)(s2 - 1);
    __syncthreads();
    if (!lds[36]) return;
    // last chunk: out = sum_c N_c / sum_c z_c (all relative to the same max)
    if (tid < G * HD) {
      const int h = tid / HD, d = tid - h * HD;
      const float* PB = a.part_c + (size_t)bh * s2 * G * PW;
      float num = 0.f, den = 0.f;
      for (int c0_ = 0; c0_ < s2; c0_ += 8) {
        float vn[8], vd[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int c = min(c0_ + k, s2 - 1);
          vn[k] = sf_get(PB + (c * G + h) * PW + d);
          vd[k] = sf_get(PB + (c * G + h) * PW + HD + 1);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (c0_ + k < s2) {
            num += vn[k];
            den += vd[k];
          }
      }
      const size_t oi = ((size_t)bi * a.n_q + kvh * G + h) * HD + d;
      a.out[oi] = num / den;
      if (a.out16) a.out16[oi] = __builtin_bit_cast(uint16_t, (_Float16)(num / den));
    }
    return;
  }

  int off = 0, cnt = 0;  // this chunk's range of selection positions
  float mx_uns[G];       // max logit of this thread's unselected tokens
#pragma unroll
  for (int h = 0; h < G; ++h) mx_uns[h] = -INFINITY;
  if (a.sel_in == nullptr) {
    // ---- scores of this chunk's tokens (TPT consecutive per thread) ----
    uint32_t key[TPT];
    float lgk[G][TPT];  // this thread's logits (for the max over the unselected tokens)
    {
      float sc[TPT] = {};
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const f4_t l4 = l4p[h];
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
          // a weight below e^-64 of the head's largest adds nothing (ties at zero
          // then go to the lower token)
          const float dl = l4[i] - s_m[h];
          sc[i] += dl >= SCORE_CUTOFF ? __expf(dl) * s_iz[h] : 0.f;
          lgk[h][i] = l4[i];
        }
      }
#pragma unroll
      for (int i = 0; i < TPT; ++i) key[i] = __float_as_uint(sc[i]);
    }
    // ---- radix select of the k-th key over all chunks of this KV head ----
    // selected: (key >> sh) > tv, or (key >> sh) == tv within the first `need`
    uint32_t* gh = a.hist + (size_t)bh * 3 * NBIN;
    int need = ks, sh = 31;
    uint32_t tv = 0;
    for (int level = 0; level < 3; ++level) {
      const int lsh = level == 0 ? 20 : (level == 1 ? 10 : 0);
      const int nb = level == 0 ? 2048 : 1024;
      for (int i = tid; i < nb; i += SEL_T) lh[i] = 0;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < TPT; ++i) {
        const bool valid = tb + i < T;
        if (level == 0) {
          // scores of exactly 0 (every head past the cutoff) are common in peaked
          // attention: counted by ballot, one LDS add per wave, not one per token
          const uint64_t zm = __ballot(valid && key[i] == 0u);
          if (lane == 0 && zm) atomicAdd(&lh[0], (uint32_t)__popcll(zm));
          if (valid && key[i] != 0u) atomicAdd(&lh[(key[i] >> lsh) & (uint32_t)(nb - 1)], 1u);
        } else if (valid && (key[i] >> sh) == tv) {
          atomicAdd(&lh[(key[i] >> lsh) & (uint32_t)(nb - 1)], 1u);
        }
      }
      __syncthreads();
      uint32_t* g = gh + level * NBIN;
      for (int i = tid; i < nb; i += SEL_T)
        if (lh[i]) atomicAdd(&g[i], lh[i]);
      chunk_barrier(ctl + level, (uint32_t)s2, a.timeout);
      for (int i = tid; i < nb; i += SEL_T) lh[i] = sf_get(g + i);
      __syncthreads();
      int above, inbin;
      const uint32_t bin = (uint32_t)blk_threshold(lh, nb, need, lds, &above, &inbin);
      need -= above;
      tv = level == 0 ? bin : ((tv << 10) | bin);
      sh = lsh;
      if (need == inbin) break;  // the whole bin is taken: no finer level needed
      // level-0 bin 0 holds exactly the zero scores (a nonzero score is at least
      // e^-64 / sum, far above the bin's bound): the k-th score is 0
      if (level == 0 && bin == 0u) break;
    }
    // ---- counts above / at the threshold, exchanged between the chunks ----
    int gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const bool valid = tb + i < T;
      gt += valid && (key[i] >> sh) > tv;
      eq += valid && (key[i] >> sh) == tv;
    }
    int gt_c, eq_c;
    (void)blk_exclusive_scan(gt, lds, &gt_c);
    const int eq_before = blk_exclusive_scan(eq, lds, &eq_c);
    if (tid == 0) {
      sf_put(a.cnts + ((size_t)bh * s2 + chunk) * 2, (uint32_t)gt_c);
      sf_put(a.cnts + ((size_t)bh * s2 + chunk) * 2 + 1, (uint32_t)eq_c);
    }
    chunk_barrier(ctl + 3, (uint32_t)s2, a.timeout);
    if (wave == 0) {
      // prefix over chunks; equal keys are taken in token (= chunk) order
      int run_sel = 0, run_eq = 0;
      for (int cb = 0; cb < s2; cb += 64) {
        const int c = cb + lane;
        int g_ = 0, e_ = 0;
        if (c < s2) {
          g_ = (int)sf_get(a.cnts + ((size_t)bh * s2 + c) * 2);
          e_ = (int)sf_get(a.cnts + ((size_t)bh * s2 + c) * 2 + 1);
        }
        const int ie = sf_wave_incl_scan(e_);
        const int eb = run_eq + ie - e_;  // equal keys before chunk c
        const int tk = max(0, min(e_, need - eb));
        const int is = sf_wave_incl_scan(g_ + tk);
        if (c == chunk) {
          lds[37] = run_sel + is - (g_ + tk);
          lds[38] = g_ + tk;
          lds[39] = eb;
        }
        run_sel += __builtin_amdgcn_readlane(is, 63);
        run_eq += __builtin_amdgcn_readlane(ie, 63);
      }
    }
    __syncthreads();
    off = lds[37];
    cnt = lds[38];
    const int eq_chunk_before = lds[39];
    // ---- ordered compaction of this chunk's selection into LDS ----
    int nsel = 0;
    bool take[TPT];
    {
      int eseen = eq_chunk_before + eq_before;
#pragma unroll
      for (int i = 0; i < TPT; ++i) {
        const bool valid = tb + i < T;
        const bool g_ = valid && (key[i] >> sh) > tv;
        const bool e_ = valid && (key[i] >> sh) == tv;
        take[i] = g_ || (e_ && eseen < need);
        eseen += e_;
        nsel += take[i];
      }
    }
    int tot;
    int pos = blk_exclusive_scan(nsel, lds, &tot);
#pragma unroll
    for (int i = 0; i < TPT; ++i)
      if (take[i] && pos < CB) s_tok[pos++] = tb + i;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < TPT; ++i)
        if (!take[i]) mx_uns[h] = fmaxf(mx_uns[h], lgk[h][i]);  // invalid tokens hold -inf
  } else {
    // external selection: chunk c takes positions [c*ks/s2, (c+1)*ks/s2)
    off = (int)(((long long)chunk * ks) / s2);
    cnt = (int)(((long long)(chunk + 1) * ks) / s2) - off;
    for (int j = tid; j < cnt; j += SEL_T) s_tok[j] = a.sel_in[(size_t)bh * ks + off + j];
    // the max over the tokens of this chunk that no chunk selected
    uint32_t* selbits = lh;  // [CB / 32] (the histograms are unused on this path)
    for (int i = tid; i < CB / 32; i += SEL_T) selbits[i] = 0u;
    __syncthreads();
    for (int j = tid; j < ks; j += SEL_T) {
      const int t = a.sel_in[(size_t)bh * ks + j] - c0;
      if (t >= 0 && t < CB) atomicOr(&selbits[t >> 5], 1u << (t & 31));
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int t = tb + i;
      if (t < T && !((selbits[(t - c0) >> 5] >> ((t - c0) & 31)) & 1u))
#pragma unroll
        for (int h = 0; h < G; ++h)
          mx_uns[h] = fmaxf(mx_uns[h], a.logits[((size_t)bi * a.n_q + kvh * G + h) * a.LT + t]);
    }
  }
  // (off, cnt) are only out of range after a timed-out wait
  off = min(max(off, 0), ks);
  cnt = min(max(cnt, 0), min(CB, ks - off));
  __syncthreads();

  // ---- lookups, in selection order: every selected token's slot into LDS (all of a
  //      thread's lookups requested at once) ----
  const size_t unit0 = (size_t)bh * a.t_cap;
  const int base = a.pool.log_count ? (int)sf_get(a.ctl + 5) : -1;
  {
    constexpr int NR = CB / SEL_T;  // cnt <= CB: one pass
    int tk[NR], sl[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int j = tid + SEL_T * i;
      tk[i] = j < cnt ? s_tok[j] : -1;
      const bool ok = tk[i] >= 0 && tk[i] < T;
      // (a resident pool holds unit u in slot u)
      sl[i] = !ok ? -1
                  : (a.pool.resident ? (int)(unit0 + tk[i])
                                     : (a.pool.unit2slot ? a.pool.unit2slot[unit0 + tk[i]] : -1));
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int j = tid + SEL_T * i;
      if (j >= cnt) continue;
      const bool ok = tk[i] >= 0 && tk[i] < T;
      const size_t p = (size_t)bh * ks + off + j;
      s_slot[j] = sl[i];
      a.sel_ws[(size_t)bh * KS + off + j] = tk[i];
      a.slot_ws[(size_t)bh * KS + off + j] = sl[i];
      if (a.sel_out) a.sel_out[p] = tk[i];
      if (a.hit_out) a.hit_out[p] = sl[i];
      if (base >= 0) {
        a.pool.log_units[base + p] = ok ? (int)(unit0 + tk[i]) : -1;
        a.pool.log_slots[base + p] = sl[i];
      }
    }
  }
  __syncthreads();

  // ---- for the hits the logits of all G heads become l' = l + scale * s_K *
  //      (q_h . cK_lo) (one token a thread, its unit read once) ----
  // max after replacement: unselected tokens, selected misses (old logit), hits (new)
  // (dropping the unselected tokens: the max over the selected ones only)
  float mloc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) mloc[h] = a.variant == SF_ATTN_DROP_UNSELECTED ? -INFINITY : mx_uns[h];
#pragma nounroll
  for (int j = tid; j < cnt; j += SEL_T) {
    const int t = s_tok[j], slot = s_slot[j];
    if (t < 0 || t >= T) continue;
    float* lp[G];
    float l[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      lp[h] = a.logits + ((size_t)bi * a.n_q + kvh * G + h) * a.LT + t;
      l[h] = *lp[h];
    }
    if (slot < 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) mloc[h] = fmaxf(mloc[h], l[h]);
      continue;
    }
    const float s = sf_h2f(a.k_sz[unit0 + t]);
    const uint8_t* unit = a.pool.slots + (size_t)slot * a.pool.unit_bytes;
    float dot[G];
    // nested: l + scale * s_K * (q . cK_lo); fp16 tokens: scale * (q . K16)
    if (a.variant == SF_ATTN_FP16_TOKENS)
      k16_dots<G>(unit, qf, dot);
    else
      kref_dots<G>(unit, a.r, qf, dot);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float l2 = a.variant == SF_ATTN_FP16_TOKENS ? a.scale * dot[h] : l[h] + a.scale * (s * dot[h]);
      *lp[h] = l2;
      mloc[h] = fmaxf(mloc[h], l2);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mloc[h] = fmaxf(mloc[h], __shfl_xor(mloc[h], o, 64));
  }
  if (lane == 0)
#pragma unroll
    for (int h = 0; h < G; ++h) s_wm[wave][h][0] = mloc[h];
  __syncthreads();
  // this chunk's max after replacement; pv takes the max over the chunks
  if (tid < G) {
    float mm = -INFINITY;
    for (int w = 0; w < SEL_T / 64; ++w) mm = fmaxf(mm, s_wm[w][tid][0]);
    a.cmax[((size_t)bh * s2 + chunk) * G + tid] = mm;
  }
}

// ---- pv: final weights, value sums, hit refinements, merge ---------------------------
// Every load of the workgroup is issued first: its V codes (16 bytes a thread per
// step), scale words, final logits and the KV head's max.  V codes are staged
// column-major ([code word][token], padded), so a lane's B operand -- one dim of 8
// consecutive tokens -- is two 16-byte LDS reads.  The refinement of the hits is
// not done by the split that holds the token: in peaked attention the selection
// crowds into a few splits, so workgroup s of a KV head takes the equal share
// [s k / nsp, (s + 1) k / nsp) of the selection positions instead, with weights
// relative to the KV head's common max; the words of a batch of hits are requested
// at once.  All splits of a KV head use the same max, so their sums are added into
// one fp32 record per head (atomically); the last split divides.
constexpr int PV_HB = 256;   // hits staged in LDS together at most (one a thread)
constexpr int PV_HW = 1792;  // words of their staging (a batch holds fewer hits when a hit has more)
constexpr int PV_RWM = 28;   // value refinement words of a nested unit at most (HD * r / 32, r <= 7)

template <int B, int G>
__global__ __launch_bounds__(256) void attn_pv_kernel(AttnArgs a) {
  constexpr int SP = pv_tokens(B);
  constexpr int WPT = HD * B / 32;       // code words per token
  constexpr int CST = SP + 4;            // column stride (words), keeps 16-byte alignment
  constexpr int UP = SP + 8;
  constexpr int TPW = SP / 256;          // tokens per thread in the weight phase
  constexpr int NV = SP * WPT / 4 / 256; // 16-byte code loads per thread
  // The V codes and the fp16 weights are dead once the value sums are formed; the
  // hit staging then reuses the codes' space and the per-wave sums the weights'.
  constexpr int VC_BYTES = WPT * CST * 4;
  constexpr int HIT_BYTES = PV_HW * 4 + PV_HB * (G + 2) * 4;
  constexpr int U_BYTES = 2 * G * UP * 2, ACC_BYTES = 4 * G * HD * 4;
  __shared__ __attribute__((aligned(16))) uint8_t s_big[VC_BYTES > HIT_BYTES ? VC_BYTES : HIT_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_big2[U_BYTES > ACC_BYTES ? U_BYTES : ACC_BYTES];
  uint32_t* const s_vc = (uint32_t*)s_big;                                 // [WPT][CST]
  uint32_t* const s_hr = (uint32_t*)s_big;                                 // [PV_HW] hit words
  float(*const s_hw)[G] = (float(*)[G])(s_big + PV_HW * 4);                // [PV_HB][G] hit weights
  int* const s_hslot = (int*)(s_big + PV_HW * 4 + PV_HB * G * 4);          // [PV_HB] slot, -1 = none
  uint32_t* const s_hsz = (uint32_t*)(s_big + PV_HW * 4 + PV_HB * (G + 1) * 4);  // [PV_HB] scale words
  _Float16(*const s_u)[UP] = (_Float16(*)[UP])s_big2;                      // [2G][UP]
  float(*const s_acc)[G][HD] = (float(*)[G][HD])s_big2;                    // [4][G][HD]
  __shared__ uint32_t s_vsz[SP];
  __shared__ float s_red[4][3 * G + 1];
  __shared__ float s_st[3 * G + 1];
  __shared__ int s_rng[4][2];
  __shared__ int s_flag;
  __shared__ uint32_t s_selm[SP / 32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.y;
  const int bi = bh / a.n_kv, kvh = bh - bi * a.n_kv;
  const int T = a.T;
  // this workgroup's splits [sp0, sp1) (one, unless the grid would not fit at once)
  const int sp0 = blockIdx.x * a.spw, sp1 = min(a.nsp, sp0 + a.spw);
  // ---- loads ----
  // this workgroup's share of the hits (see the hit section): the first batch's
  // positions and slots, one a thread, before anything else
  const int* sel = a.sel_ws + (size_t)bh * a.k_sel;
  const int* slots = a.slot_ws + (size_t)bh * a.k_sel;
  const bool f16u = a.variant == SF_ATTN_FP16_TOKENS;
  const int RW = f16u ? HD / 2 : HD * a.r / 32;  // value words of a unit
  const int RS = RW + (f16u ? WPT : 0);          // words staged per hit
  const int HB = min(PV_HB, PV_HW / RS);
  const int p0 = (int)((long long)sp0 * a.k_sel / a.nsp), p1 = (int)((long long)sp1 * a.k_sel / a.nsp);
  int h_t = -1, h_slot = -1;
  if (tid < min(HB, p1 - p0)) {
    h_t = sel[p0 + tid];
    h_slot = slots[p0 + tid];
  }
  // one split's V codes (16 bytes a thread per step), scale words and final logits
  const int tl0 = TPW * tid;  // this thread's first token within a split
  u32x4 vc[NV];
  uint32_t vsz[TPW];
  float lg[G][TPW];
  const auto load_split = [&](int split) {
    const int t_begin = split * SP, n_here = min(SP, T - t_begin);
    const size_t tok0 = (size_t)bh * a.t_cap + t_begin;
    const u32x4* src = (const u32x4*)(a.v_res + tok0 * (HD * B / 8));
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = tid + 256 * i;
      vc[i] = idx < n_here * WPT / 4 ? __builtin_nontemporal_load(src + idx) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < TPW; ++i) vsz[i] = tl0 + i < n_here ? a.v_sz[tok0 + tl0 + i] : 0u;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float* lr = a.logits + ((size_t)bi * a.n_q + kvh * G + h) * a.LT + t_begin + tl0;
#pragma unroll
      for (int i = 0; i < TPW; ++i) lg[h][i] = tl0 + i < n_here ? lr[i] : -INFINITY;
    }
  };
  load_split(sp0);
  // the KV head's max logit after replacement: the max over its chunks' maxima
  // (every wave forms it, lanes over chunks)
  float mh[G];
#pragma unroll
  for (int h = 0; h < G; ++h) mh[h] = -INFINITY;
  for (int c = lane; c < a.s2; c += 64)
#pragma unroll
    for (int h = 0; h < G; ++h) mh[h] = fmaxf(mh[h], a.cmax[((size_t)bh * a.s2 + c) * G + h]);
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mh[h] = fmaxf(mh[h], __shfl_xor(mh[h], o, 64));
  // the first batch's logits, scale words and (nested) refinement words: they land
  // while the splits' own sums are formed
  float h_l[G];
  uint32_t h_sz = 0u;
  u32x4 h_w[PV_RWM / 4];
  const auto load_hit = [&]() {
    const bool ok = h_slot >= 0 && h_t >= 0 && h_t < T;
#pragma unroll
    for (int h = 0; h < G; ++h) h_l[h] = ok ? a.logits[((size_t)bi * a.n_q + kvh * G + h) * a.LT + h_t] : -INFINITY;
    h_sz = ok ? a.v_sz[(size_t)bh * a.t_cap + h_t] : 0u;
    const u32x4* uw = (const u32x4*)(a.pool.slots + (size_t)(ok ? h_slot : 0) * a.pool.unit_bytes) + RW / 4;
#pragma unroll
    for (int k = 0; k < PV_RWM / 4; ++k) h_w[k] = ok && !f16u && 4 * k < RW ? uw[k] : u32x4{0u, 0u, 0u, 0u};
  };
  load_hit();
  const bool drop = a.variant == SF_ATTN_DROP_UNSELECTED;
  const int r = a.r;
  const int n = lane & 15, qg = lane >> 4;
  constexpr uint32_t cmask = (1u << B) - 1u;
  // this workgroup's value sums (lane: dims 32 wave + 16 db + n of heads 2 qg + hh)
  // and weight sums (thread h < G), each split's rescaled to the common max
  float accv[2][2] = {{0.f, 0.f}, {0.f, 0.f}}, accz = 0.f;
  for (int split = sp0; split < sp1; ++split) {
    const int t_begin = split * SP, n_here = min(SP, T - t_begin);
    if (split > sp0) __syncthreads();  // the previous split's LDS reads are done
    // dropping the unselected tokens: the selected positions of this split's
    // tokens, [#sel < t_begin, #sel < t_end)
    int below0 = 0, below1 = 0;
    if (drop)
      for (int j = tid; j < a.k_sel; j += 256) {
        const int t = sel[j];
        below0 += t < t_begin;
        below1 += t < t_begin + n_here;
      }
    // ---- V codes into LDS, column-major ----
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int w = 4 * (tid + 256 * i), tk = w / WPT, c = w - tk * WPT;
#pragma unroll
      for (int e = 0; e < 4; ++e) s_vc[(c + e) * CST + tk] = vc[i][e];
    }
    // largest value scale of the split, the split's max logit per head, the hit range
    float smx = 0.f, lmx[G];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      s_vsz[tl0 + i] = vsz[i];
      smx = fmaxf(smx, sf_h2f(vsz[i]));
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      lmx[h] = lg[h][0];
#pragma unroll
      for (int i = 1; i < TPW; ++i) lmx[h] = fmaxf(lmx[h], lg[h][i]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      smx = fmaxf(smx, __shfl_xor(smx, o, 64));
#pragma unroll
      for (int h = 0; h < G; ++h) lmx[h] = fmaxf(lmx[h], __shfl_xor(lmx[h], o, 64));
      below0 += __shfl_xor(below0, o, 64);
      below1 += __shfl_xor(below1, o, 64);
    }
    if (lane == 0) {
      s_red[wave][0] = smx;
#pragma unroll
      for (int h = 0; h < G; ++h) s_red[wave][1 + h] = lmx[h];
      s_rng[wave][0] = below0;
      s_rng[wave][1] = below1;
    }
    __syncthreads();
    smx = fmaxf(fmaxf(s_red[0][0], s_red[1][0]), fmaxf(s_red[2][0], s_red[3][0]));
    // weights relative to the split's own max (full fp16 precision in the value
    // sums); the sums are rescaled to the KV head's common max before they are added
    float msp[G];
#pragma unroll
    for (int h = 0; h < G; ++h)
      msp[h] = fmaxf(fmaxf(s_red[0][1 + h], s_red[1][1 + h]), fmaxf(s_red[2][1 + h], s_red[3][1 + h]));
    if (drop) {
      // only the selected tokens are attended: the others get no weight, and the
      // split's reference max is taken over the selected ones (the selection ascends)
      const int hit_lo = (s_rng[0][0] + s_rng[1][0]) + (s_rng[2][0] + s_rng[3][0]);
      const int nh = min((s_rng[0][1] + s_rng[1][1]) + (s_rng[2][1] + s_rng[3][1]) - hit_lo, SP);
      if (tid < SP / 32) s_selm[tid] = 0u;
      __syncthreads();
      for (int j = tid; j < nh; j += 256) {
        const int t = sel[hit_lo + j] - t_begin;
        if (t >= 0 && t < n_here) atomicOr(&s_selm[t >> 5], 1u << (t & 31));
      }
      __syncthreads();
#pragma unroll
      for (int h = 0; h < G; ++h) lmx[h] = -INFINITY;
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int t = tl0 + i;
        const bool on = t < n_here && ((s_selm[t >> 5] >> (t & 31)) & 1u);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          if (!on) lg[h][i] = -INFINITY;
          lmx[h] = fmaxf(lmx[h], lg[h][i]);
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1)
#pragma unroll
        for (int h = 0; h < G; ++h) lmx[h] = fmaxf(lmx[h], __shfl_xor(lmx[h], o, 64));
      if (lane == 0)
#pragma unroll
        for (int h = 0; h < G; ++h) s_red[wave][1 + h] = lmx[h];
      __syncthreads();
#pragma unroll
      for (int h = 0; h < G; ++h)
        msp[h] = fmaxf(fmaxf(s_red[0][1 + h], s_red[1][1 + h]), fmaxf(s_red[2][1 + h], s_red[3][1 + h]));
      __syncthreads();
    }
    const float smax = smx * (float)(1u << r);
    int e2 = 0;
    if (smax > 0.f) (void)frexpf(smax, &e2);
    const int shift = smax > 0.f ? 14 - e2 : 0;
    const float uscale = ldexpf((float)(1u << r), shift);
    float acc3[3 * G];
#pragma unroll
    for (int i = 0; i < 3 * G; ++i) acc3[i] = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const float w = lg[h][i] == -INFINITY ? 0.f : __expf(lg[h][i] - msp[h]);
        const float u = w * sf_h2f(vsz[i]) * uscale;
        const _Float16 hi = (_Float16)u;
        const _Float16 lo = (_Float16)((u - (float)hi) * 2048.f);
        s_u[2 * h][tl0 + i] = hi;
        s_u[2 * h + 1][tl0 + i] = lo;
        acc3[3 * h] += w;
        acc3[3 * h + 1] = fmaf(w, sf_h2f(vsz[i] >> 16), acc3[3 * h + 1]);
      }
    // the next split's loads go out now and land during this split's value sums
    if (split + 1 < sp1) load_split(split + 1);
    __syncthreads();  // s_u, s_vc, s_vsz written; s_red free
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
#pragma unroll
      for (int i = 0; i < 3 * G; ++i) acc3[i] += __shfl_xor(acc3[i], o, 64);
    if (lane == 0)
#pragma unroll
      for (int i = 0; i < 3 * G; ++i) s_red[wave][i] = acc3[i];

    // e^(split max - common max) per head
    float fsc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) fsc[h] = msp[h] > -INFINITY ? __expf(msp[h] - mh[h]) : 0.f;

    // ---- value sums on MFMA; wave w: dims [32w, 32w+32) as two 16-dim blocks ----
    f4_t pacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll 2
    for (int kb = 0; kb < SP / 32; ++kb) {
      const int tk0 = 32 * kb + 8 * qg;
      h8_t av;
      if (n < 2 * G) {
        av = *(const h8_t*)(&s_u[n][tk0]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) av[e] = (_Float16)0.f;
      }
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const int d = 32 * wave + 16 * db + n;
        const int bit = d * B, wi = bit >> 5, sh = bit & 31;
        const u32x4 w0 = *(const u32x4*)(s_vc + wi * CST + tk0);
        const u32x4 w1 = *(const u32x4*)(s_vc + wi * CST + tk0 + 4);
        const uint32_t c[8] = {(w0.x >> sh) & cmask, (w0.y >> sh) & cmask, (w0.z >> sh) & cmask,
                               (w0.w >> sh) & cmask, (w1.x >> sh) & cmask, (w1.y >> sh) & cmask,
                               (w1.z >> sh) & cmask, (w1.w >> sh) & cmask};
        u32x4 bv;
#pragma unroll
        for (int e = 0; e < 4; ++e) bv[e] = code_pair<B>(c[2 * e], c[2 * e + 1]);
        pacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(h8_t, bv), pacc[db], 0, 0, 0);
      }
    }
    __syncthreads();  // s_red
    if (tid < 3 * G) s_st[tid] = (s_red[0][tid] + s_red[1][tid]) + (s_red[2][tid] + s_red[3][tid]);
    __syncthreads();
    // lane group qg holds rows 4qg..4qg+3 = head 2qg (rows 0, 1) and head 2qg+1 (rows 2, 3)
    const float back = ldexpf(1.f, B - shift);  // 2^B undoes the c/2^B form, 2^-shift the scaling
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int h = 2 * qg + hh;
        if (h < G) {
          float fh = fsc[0], sth = s_st[1];
#pragma unroll
          for (int h2 = 1; h2 < G; ++h2)
            if (h2 == h) {
              fh = fsc[h2];
              sth = s_st[3 * h2 + 1];
            }
          const float D = pacc[db][2 * hh] + pacc[db][2 * hh + 1] * (1.f / 2048.f);
          accv[db][hh] = fmaf(fh, sth + back * D, accv[db][hh]);
        }
      }
    if (tid < G) {
      float ft = fsc[0];
#pragma unroll
      for (int h2 = 1; h2 < G; ++h2)
        if (h2 == tid) ft = fsc[h2];
      accz = fmaf(ft, s_st[3 * tid], accz);
    }
  }

  // ---- this workgroup's share of the hits: + w * s_V * cV_lo; lane: dims 2l, 2l+1 ----
  // Positions [p0, p1) of the KV head's selection, in batches of HB (one a thread
  // while staged).  A hit whose weight is 0 in fp32 for every head adds nothing.
  // Nested units: the value's refinement words follow the key's (RW each); fp16
  // units: the value's HD fp16 values follow the key's (64 words), and a hit adds
  // w * (V16 - V_b), V_b from the token's resident codes (staged after the words).
  float hacc[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) hacc[h][0] = hacc[h][1] = 0.f;
  for (int j0 = p0; j0 < p1; j0 += HB) {
    const int nb = min(HB, p1 - j0);
    if (j0 > p0) {  // later batches: requested now
      h_t = h_slot = -1;
      if (tid < nb) {
        h_t = sel[j0 + tid];
        h_slot = slots[j0 + tid];
      }
      load_hit();
    }
    __syncthreads();  // the previous batch's staging has been read
    if (tid < nb) {
      bool any = false;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float w = h_l[h] == -INFINITY ? 0.f : __expf(h_l[h] - mh[h]);
        any = any || w != 0.f;
        s_hw[tid][h] = w;
      }
      s_hslot[tid] = any ? h_slot : -1;
      s_hsz[tid] = h_sz;
      if (!f16u)
#pragma unroll
        for (int k = 0; k < PV_RWM / 4; ++k)
          if (4 * k < RW) *(u32x4*)(s_hr + tid * RS + 4 * k) = h_w[k];
    }
    if (f16u) {
      __syncthreads();
      // the value's fp16 words and the token's resident codes of each live hit
      for (int i = tid; i < nb * RS; i += 256) {
        const int jj = i / RS, w2 = i - jj * RS;
        const int slot = s_hslot[jj];
        if (slot < 0) continue;
        const int t = sel[j0 + jj];
        s_hr[i] = w2 < RW ? ((const uint32_t*)(a.pool.slots + (size_t)slot * a.pool.unit_bytes))[RW + w2]
                          : ((const uint32_t*)(a.v_res + ((size_t)bh * a.t_cap + t) * (HD * B / 8)))[w2 - RW];
      }
    }
    __syncthreads();
    for (int jj = wave; jj < nb; jj += 4) {
      if (s_hslot[jj] < 0) continue;
      const uint32_t* vr = s_hr + jj * RS;
      const float sv = sf_h2f(s_hsz[jj]);
      float c0, c1;
      if (f16u) {
        constexpr uint32_t cm = (1u << B) - 1u;
        const float st = sv * (float)(1u << r), zv = sf_h2f(s_hsz[jj] >> 16);
        const int d0 = 2 * lane, d1 = 2 * lane + 1;
        const uint32_t q0 = (vr[RW + ((d0 * B) >> 5)] >> ((d0 * B) & 31)) & cm;
        const uint32_t q1 = (vr[RW + ((d1 * B) >> 5)] >> ((d1 * B) & 31)) & cm;
        c0 = h2f16((uint16_t)(vr[lane] & 0xFFFFu)) - fmaf(st, (float)q0, zv);
        c1 = h2f16((uint16_t)(vr[lane] >> 16)) - fmaf(st, (float)q1, zv);
      } else {
        c0 = sv * (float)field(vr, 2 * lane * r, r);
        c1 = sv * (float)field(vr, (2 * lane + 1) * r, r);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        hacc[h][0] = fmaf(s_hw[jj][h], c0, hacc[h][0]);
        hacc[h][1] = fmaf(s_hw[jj][h], c1, hacc[h][1]);
      }
    }
  }
  __syncthreads();  // every wave is past its reads of s_u and s_hr
#pragma unroll
  for (int h = 0; h < G; ++h) {
    s_acc[wave][h][2 * lane] = hacc[h][0];
    s_acc[wave][h][2 * lane + 1] = hacc[h][1];
  }
  __syncthreads();  // s_acc
  // this workgroup's sums, added into one of the KV head's records [PV_NR][G][PW]
  // (zeroed by the split launch; several records keep the adds per address few)
  float* PB = a.part_p + (size_t)bh * PV_NR * G * PW;
  float* PP = PB + (size_t)(blockIdx.x % PV_NR) * G * PW;
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    const int d = 32 * wave + 16 * db + n;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int h = 2 * qg + hh;
      if (h < G) {
        const float corr = (s_acc[0][h][d] + s_acc[1][h][d]) + (s_acc[2][h][d] + s_acc[3][h][d]);
        (void)__hip_atomic_fetch_add(PP + h * PW + d, accv[db][hh] + corr, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (tid < G)
    (void)__hip_atomic_fetch_add(PP + tid * PW + HD + 1, accz, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  sf_drain();
  __syncthreads();
  if (tid == 0)
    s_flag = sf_add_acq_rel(a.ctl + bh * 8 + 6, 1u) ==
             (uint32_t)(gridDim.x - 1);
  __syncthreads();
  if (!s_flag) return;
  // last workgroup of this KV head: out = N / z over the records
  for (int i = tid; i < G * HD; i += 256) {
    const int h = i / HD, d = i - h * HD;
    float vn[PV_NR], vz[PV_NR];
#pragma unroll
    for (int k = 0; k < PV_NR; ++k) {
      vn[k] = sf_get(PB + ((size_t)k * G + h) * PW + d);
      vz[k] = sf_get(PB + ((size_t)k * G + h) * PW + HD + 1);
    }
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int k = 0; k < PV_NR; ++k) {
      num += vn[k];
      den += vz[k];
    }
    const size_t oi = ((size_t)bi * a.n_q + kvh * G + h) * HD + d;
    a.out[oi] = num / den;
    if (a.out16) a.out16[oi] = __builtin_bit_cast(uint16_t, (_Float16)(num / den));
  }
}

size_t attn_layout(int batch, int n_q, int n_kv, int T, int k_sel, size_t off[12]) {
  const int G = n_kv > 0 ? n_q / n_kv : 1;
  const size_t bh = (size_t)batch * n_kv;
  const size_t nsa = (T + SA - 1) / SA, s2 = (T + CB - 1) / CB, nsp = (T + 255) / 256;  // nsp: bound for every b
  const size_t KS = k_sel > 0 ? k_sel : 1;
  const size_t LT = ((size_t)T + 3) & ~size_t(3);
  const size_t sizes[12] = {
      (size_t)batch * n_q * LT * 4,  // logits
      bh * nsa * G * PW * 4,         // split partials
      bh * s2 * G * PW * 4,          // chunk partials
      bh * PV_NR * G * PW * 4,       // value-sum records
      bh * s2 * G * 4,               // chunk max
      0,                             // (unused)
      bh * KS * 4,                   // selection
      bh * KS * 4,                   // slots
      bh * 3 * NBIN * 4,             // histograms
      bh * 8 * 4,                    // control words
      bh * s2 * 2 * 4,               // chunk counts
      bh * nsa * G * 8};             // split max / sum, compact
  size_t o = sf_align256(sizeof(WsControl));
  for (int i = 0; i < 12; ++i) {
    off[i] = o;
    o += sf_align256(sizes[i]);
  }
  return o;
}

int attn_device_cus() {
  static int n_cu = 0;
  if (n_cu == 0) {
    int dev = 0, cus = 0;
    (void)hipGetDevice(&dev);
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    n_cu = cus;
  }
  return n_cu;
}

template <int B, int G>
sf_status launch_attn(AttnArgs& a, hipStream_t s) {
  const int bh = a.batch * a.n_kv;
  // the chunks of one KV head wait for each other: all of them must be resident at
  // once (workgroups are dispatched in order, so the chunks of earlier KV heads
  // finish and make room for later ones)
  const int occ = std::max(1, sf_occupancy((const void*)attn_select_kernel<G>, SEL_T, 0));
  SF_REQUIRE((long)a.s2 <= (long)occ * attn_device_cus(), SF_EUNSUPPORTED,
             "t_len too long: the selection chunks of one KV head do not fit the device at once");
  if (a.k_sel == 0) {
    hipLaunchKernelGGL((attn_split_kernel<B, G, true>), dim3(a.nsa, bh), dim3(256), 0, s, a);
    SF_LAUNCH_CHECK();
    hipLaunchKernelGGL((attn_select_kernel<G>), dim3(a.s2, bh), dim3(SEL_T), 0, s, a);
    SF_LAUNCH_CHECK();
    return SF_OK;
  }
  hipLaunchKernelGGL((attn_split_kernel<B, G, false>), dim3(a.nsa, bh), dim3(256), 0, s, a);
  SF_LAUNCH_CHECK();
  hipLaunchKernelGGL((attn_select_kernel<G>), dim3(a.s2, bh), dim3(SEL_T), 0, s, a);
  SF_LAUNCH_CHECK();
  // pv: one split a workgroup, unless the grid would not fit the device at once;
  // then each workgroup takes consecutive splits (their loads overlap the previous
  // split's value sums)
  const long pv_cap = (long)std::max(1, sf_occupancy((const void*)attn_pv_kernel<B, G>, 256, 0)) * attn_device_cus();
  a.spw = (int)std::max<long>(1, ((long)a.nsp * bh + pv_cap - 1) / pv_cap);
  hipLaunchKernelGGL((attn_pv_kernel<B, G>), dim3((a.nsp + a.spw - 1) / a.spw, bh), dim3(256), 0, s, a);
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

static sf_status attn_decode(const uint16_t* q_f16, int32_t n_q_heads, const sf_qkv* kv, const float* k_new,
                             const float* v_new, uint8_t* refine_out, int64_t refine_ld, float softmax_scale,
                             int32_t k_sel, const int32_t* sel_in, sf_refine_cache* cache, int32_t pool, float* out,
                             uint16_t* out_f16, int32_t* sel_out, int32_t* hit_out, sf_workspace* ws,
                             sf_stream stream, int32_t variant);

extern "C" sf_status sf_refined_attn_decode(const uint16_t* q_f16, int32_t n_q_heads, const sf_qkv* kv,
                                            float softmax_scale, int32_t k_sel, const int32_t* sel_in,
                                            sf_refine_cache* cache, int32_t pool, float* out,
                                            int32_t* sel_out, int32_t* hit_out, sf_workspace* ws,
                                            sf_stream stream) {
  return attn_decode(q_f16, n_q_heads, kv, nullptr, nullptr, nullptr, 0, softmax_scale, k_sel, sel_in, cache, pool,
                     out, nullptr, sel_out, hit_out, ws, stream, SF_ATTN_NESTED);
}

static sf_status attn_decode(const uint16_t* q_f16, int32_t n_q_heads, const sf_qkv* kv, const float* k_new,
                             const float* v_new, uint8_t* refine_out, int64_t refine_ld, float softmax_scale,
                             int32_t k_sel, const int32_t* sel_in, sf_refine_cache* cache, int32_t pool, float* out,
                             uint16_t* out_f16, int32_t* sel_out, int32_t* hit_out, sf_workspace* ws,
                             sf_stream stream, int32_t variant) {
  SF_REQUIRE(q_f16 && kv && out && ws, SF_EINVAL, "null argument");
  SF_REQUIRE(variant == SF_ATTN_NESTED || variant == SF_ATTN_FP16_TOKENS || variant == SF_ATTN_DROP_UNSELECTED,
             SF_EINVAL, "unknown attention variant");
  SF_REQUIRE(variant != SF_ATTN_DROP_UNSELECTED || k_sel >= 1, SF_EINVAL,
             "dropping the unselected tokens needs k_sel >= 1");
  SF_REQUIRE(kv->head_dim == HD, SF_EUNSUPPORTED, "head_dim must be 128");
  SF_REQUIRE(kv->fmt.group == 128 && kv->fmt.b >= 1 && kv->fmt.r >= 0 && kv->fmt.b + kv->fmt.r <= 8,
             SF_EUNSUPPORTED, "bad format");
  SF_REQUIRE(kv->batch > 0 && kv->n_kv_heads > 0 && n_q_heads % kv->n_kv_heads == 0, SF_EINVAL,
             "n_q_heads must be a multiple of n_kv_heads");
  SF_REQUIRE(kv->t_len >= 1 && kv->t_len <= kv->t_cap, SF_EINVAL, "need 1 <= t_len <= t_cap");
  SF_REQUIRE((int64_t)kv->t_len <= (int64_t)MAX_CHUNKS * CB, SF_EUNSUPPORTED, "t_len above 1048576");
  SF_REQUIRE(k_sel >= 0 && k_sel <= kv->t_len, SF_EINVAL, "k_sel out of range");
  SF_REQUIRE(k_sel == 0 || kv->fmt.r > 0 || variant != SF_ATTN_NESTED, SF_EINVAL, "k_sel > 0 needs r > 0");
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
  a.LT = (a.T + 3) & ~3;
  a.t_cap = kv->t_cap;
  a.b = kv->fmt.b;
  a.r = kv->fmt.r;
  a.k_sel = k_sel;
  a.variant = variant;
  a.scale = softmax_scale;
  a.nsa = (a.T + SA - 1) / SA;
  a.s2 = (a.T + CB - 1) / CB;
  a.nsp = (a.T + pv_tokens(a.b) - 1) / pv_tokens(a.b);
  size_t off[12];
  const size_t need = attn_layout(a.batch, a.n_q, a.n_kv, a.T, k_sel, off);
  SF_REQUIRE(ws->bytes >= need, SF_ENOMEM, "workspace too small");
  uint8_t* w = ws->base;
  a.logits = (float*)(w + off[0]);
  a.part_a = (float*)(w + off[1]);
  a.part_c = (float*)(w + off[2]);
  a.part_p = (float*)(w + off[3]);
  a.cmax = (float*)(w + off[4]);
  a.sel_ws = (int32_t*)(w + off[6]);
  a.slot_ws = (int32_t*)(w + off[7]);
  a.hist = (uint32_t*)(w + off[8]);
  a.ctl = (uint32_t*)(w + off[9]);
  a.cnts = (uint32_t*)(w + off[10]);
  a.part_ms = (float2*)(w + off[11]);
  a.timeout = (uint32_t*)(w + offsetof(WsControl, timeout));
  a.sel_in = sel_in;
  a.sel_out = sel_out;
  a.hit_out = hit_out;
  a.out = out;
  a.out16 = out_f16;
  a.k_new = k_new;
  a.v_new = v_new;
  a.ap_refine = refine_out;
  a.ap_refine_ld = refine_ld;
  if (k_sel > 0) {
    sf_status st = sf_cache_pool_view(cache, cache ? pool : -1, &a.pool);
    if (st != SF_OK) return st;
    if (a.pool.unit2slot) {
      const int want = variant == SF_ATTN_FP16_TOKENS ? 2 * HD * 2 : 2 * HD * a.r / 8;
      SF_REQUIRE(a.pool.unit_bytes == want, SF_EINVAL,
                 "pool unit size is not a KV unit of this variant (nested: 2*128*r/8, fp16 tokens: 512 bytes)");
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

extern "C" sf_status sf_attn_decode_variant(const uint16_t* q_f16, int32_t n_q_heads, const sf_qkv* kv,
                                            float softmax_scale, int32_t k_sel, const int32_t* sel_in,
                                            sf_refine_cache* cache, int32_t pool, float* out,
                                            int32_t* sel_out, int32_t* hit_out, sf_workspace* ws,
                                            sf_stream stream, int32_t variant) {
  return attn_decode(q_f16, n_q_heads, kv, nullptr, nullptr, nullptr, 0, softmax_scale, k_sel, sel_in, cache, pool,
                     out, nullptr, sel_out, hit_out, ws, stream, variant);
}

extern "C" sf_status sf_refined_attn_decode_append(const uint16_t* q_f16, int32_t n_q_heads, const sf_qkv* kv,
                                                   const float* k_new, const float* v_new, uint8_t* refine_out,
                                                   int64_t refine_ld, float softmax_scale, int32_t k_sel,
                                                   const int32_t* sel_in, sf_refine_cache* cache, int32_t pool,
                                                   float* out, uint16_t* out_f16, int32_t* sel_out,
                                                   int32_t* hit_out, sf_workspace* ws, sf_stream stream) {
  SF_REQUIRE(k_new && v_new, SF_EINVAL, "null k_new / v_new");
  SF_REQUIRE(refine_out == nullptr || refine_ld >= 1, SF_EINVAL, "refine_ld must be >= 1");
  return attn_decode(q_f16, n_q_heads, kv, k_new, v_new, refine_out, refine_ld, softmax_scale, k_sel, sel_in, cache,
                     pool, out, out_f16, sel_out, hit_out, ws, stream, SF_ATTN_NESTED);
}
