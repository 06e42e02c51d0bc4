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

#include <mutex>
#include <string>

#include "gemv_rows.h"

namespace sfg {
// The channel selection over x read from memory (split_select: one 256-thread
// workgroup, two-pass radix select), then the lookups and reports of every matrix
// of the call.
__global__ __launch_bounds__(256) void gemv_select_kernel(GemvArgs a) {
  extern __shared__ uint32_t smem[];
  __shared__ int lds[24];
  const int tid = threadIdx.x;
  const int K = a.k_in, ks = a.k_sel;
  int32_t* sel = a.ws_sel;
  const int32_t* l_sel = split_select<true>(a, smem);
  for (int j = tid; j < ks; j += 256) sel[j] = l_sel[j];
  // sel[] is read back below by other threads of this workgroup
  __syncthreads();
  // lookups, per op, in selection order (with the report and the lookup log)
  if (tid < a.n_ops) {
    const PoolDev& pool = a.ops[tid].pool;
    int base = -1;
    if (pool.log_count) {
      base = sf_log_reserve(pool.log_count, (uint32_t)ks, (uint32_t)pool.log_cap);
    }
    lds[tid] = base;
  }
  __syncthreads();
  for (int j = tid; j < ks; j += 256) {
    const int k = l_sel[j];
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
constexpr int MAX_ROW_BLOCKS = 1024;  // counters in the workspace control block

// (plain loads: the lanes of one load take 32 of a line's 128 bytes and the next
// groups' loads the rest; with nontemporal loads the lines were fetched again)
template <int W>
__device__ __forceinline__ void load_words(const uint8_t* src, uint32_t (&w)[W]) {
  if constexpr (W == 1) {
    w[0] = *(const uint32_t*)src;
  } else if constexpr (W == 2) {
    const u32x2 v = *(const u32x2*)src;
    w[0] = v.x; w[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      const u32x4 v = *((const u32x4*)src + i);
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
  }
}

// uw: words of a refinement unit that hold the workgroup's rows (rows_wg r / 32;
// 0 without a selection)
__host__ __device__ constexpr size_t mfma_lds_words(int nb, int gs, int rows_wg, int nhp, int uw) {
  return (size_t)nb * (gs * 64 + 4) + (size_t)gs * 16 + (size_t)rows_wg * (gs + 1) * 2 +
         ((size_t)nb * (nhp + 8) + 1) / 2 + (size_t)nhp * 2 + (size_t)32 * uw;
}

// PAIR (b = 1, 2 and an even group count per slice): the 4 lanes of a row load
// two groups' codes together (8 b bytes a lane, 16 at b = 2, instead of 4 b) and
// swap one half with the lane 32 away, so that each lane holds one chunk of 32
// codes of each group (lanes q = 0, 1, 2, 3 chunks 0, 2, 1, 3); x is read in the
// same chunk order.  Measured on a streaming probe of the gate/up shape: 16-byte
// loads over 64-byte spans of a row move the bytes in 6.7 us against 9.1 us for
// 8-byte loads over 32-byte spans.
template <int B, int RT, bool PAIR>
__global__ __launch_bounds__(256) void gemv_mfma_kernel(GemvArgs a) {
  using C = CodecPow2<B>;
  constexpr int WQ = B;  // words holding one lane's 32 codes of a group
  static_assert(!PAIR || B <= 2, "paired loads serve b = 1 and 2");
  constexpr int MPFG = 4;  // groups of codes in flight per tile
  extern __shared__ uint32_t smem[];
  __shared__ int s_cnt[4][2];
  __shared__ int s_last;
  __shared__ int s_pub;
  // with sel_wg, workgroup 0 selects the channels over all batch rows and publishes
  // them (as the batch-1/2 split kernel's selecting workgroup); the others take the
  // selection after their resident pass
  if (a.sel_wg && blockIdx.x == 0) {
    __builtin_amdgcn_s_setprio(3);
    split_select_and_publish<false>(a, smem);
    __builtin_amdgcn_s_setprio(0);
    split_retire(a);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, q = lane >> 4;
  const int ns = a.ns, GS = a.gs;
  // workgroups go to the 8 XCDs in turn: the slices of a row block are given
  // workgroups of one XCD, so that the row block's scale lines are fetched into one
  // L2 (slices on different XCDs fetched each line once per XCD: 1.8x the bytes)
  const int wid = blockIdx.x - a.sel_wg, nwg = gridDim.x - a.sel_wg;  // this reader's index
  int wl = wid;
  if ((nwg & 7) == 0) wl = (wid & 7) * (nwg >> 3) + (wid >> 3);
  const int slice = wl % ns, tile_g = wl / ns;
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
  const int UW = a.nhp > 0 ? rows_wg * a.r / 32 : 0;  // unit words of the block's rows
  int32_t* hk = (int32_t*)(xs + (mfma_lds_words(nb, GS, rows_wg, a.nhp, UW) - 2 * a.nhp - 32 * UW));  // [nhp]
  int32_t* hs = hk + a.nhp;                                                                         // [nhp]
  uint32_t* hu = (uint32_t*)(hs + a.nhp);  // [32][UW]: one block of hits' unit words
  const int wrow0 = wave * 16 * RT;  // this wave's first row within the block

  // codes of the first MPFG groups of every tile (PAIR: unit u even and u + 1 hold
  // groups gl and gl + 1 as loaded until they are exchanged)
  const int cq = PAIR ? (((q & 1) << 1) | (q >> 1)) : q;  // the chunk of a group this lane holds
  uint32_t cw[MPFG][RT][WQ];
  auto issue = [&](int u, int gl) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int row = row_wg0 + wrow0 + 16 * t + n;
      if (gl < GS && row < o.n_out) {
        const uint8_t* src = o.res + (size_t)row * rowbytes + (size_t)(g0 + gl) * (16 * B);
        if constexpr (PAIR) {
          uint32_t v[2 * WQ];
          load_words<2 * WQ>(src + q * (8 * B), v);
#pragma unroll
          for (int w = 0; w < WQ; ++w) {
            cw[u][t][w] = v[w];
            cw[u + 1][t][w] = v[WQ + w];
          }
        } else {
          load_words<WQ>(src + q * (4 * B), cw[u][t]);
        }
      } else {
#pragma unroll
        for (int w = 0; w < WQ; ++w) {
          cw[u][t][w] = 0u;
          if constexpr (PAIR) cw[u + 1][t][w] = 0u;
        }
      }
    }
  };
#pragma unroll
  for (int u = 0; u < MPFG; u += PAIR ? 2 : 1) issue(u, u);
  // PAIR: lanes q < 2 hold chunks 2q, 2q + 1 of group gl, lanes q >= 2 chunks
  // 2(q-2), 2(q-2) + 1 of group gl + 1; each passes one chunk to the lane 32 away
  auto exchange = [&](int u) {
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int w = 0; w < WQ; ++w) {
        const uint32_t give = q < 2 ? cw[u + 1][t][w] : cw[u][t][w];
        const uint32_t got = (uint32_t)__shfl_xor((int)give, 32, 64);
        if (q < 2) cw[u + 1][t][w] = got;
        else cw[u][t][w] = got;
      }
  };

  // The first batch of every prologue load is requested before any of them is
  // used: the x slice, the scale words of the block's rows and the selection with
  // its slots (one round trip instead of four).
  const int per_row = KS / 8;  // 16-byte x loads per batch row (a multiple of 16)
  const int items = nb * per_row;
  constexpr int XB = 4, SB = 8, SU = 2;
  const int ks = a.k_sel;
  const int32_t* slots = a.ws_slot + (size_t)op * ks;
  u32x4 xv[XB];
  auto load_x = [&](int i0) {
#pragma unroll
    for (int it = 0; it < XB; ++it) {
      const int i = i0 + 256 * it + tid;
      if (i < items) {
        const int bc = i / per_row, c8 = i - bc * per_row;
        xv[it] = *(const u32x4*)(a.x + (size_t)(a.batch_off + bc) * K + k0 + 8 * c8);
      }
    }
  };
  uint32_t w[SB];
  auto load_sz = [&](int i0) {
#pragma unroll
    for (int it = 0; it < SB; ++it) {
      const int i = i0 + 256 * it + tid;
      const int rl = i / GS, gl = i - rl * GS, row = row_wg0 + rl;
      w[it] = (i < rows_wg * GS && row < o.n_out) ? o.sz[(size_t)row * ngr + g0 + gl] : 0u;
    }
  };
  // the selection and its slots: from the selection launch (complete before this
  // one), or published by workgroup 0 (read after the resident pass)
  const bool pub = a.sel_wg != 0;
  const uint32_t* hc = a.ctl + offsetof(WsControl, hit) / 4 + (wid % SPLIT_COPIES) * split_copy_words(ks, a.n_ops);
  const bool resident = o.pool.resident != 0;
  auto sel_k = [&](int j) { return pub ? read_published(hc + j, a) : a.ws_sel[j]; };
  auto sel_slot = [&](int j, int k) {
    return pub ? (resident ? k : read_published(hc + ks * (1 + op) + j, a)) : slots[j];
  };
  int selk[SU], sels[SU];
#pragma unroll
  for (int u = 0; u < SU; ++u) {
    const int j = tid + 256 * u;
    selk[u] = !pub && j < ks ? a.ws_sel[j] : INT32_MAX;
    sels[u] = !pub && j < ks ? slots[j] : -1;
  }
  load_x(0);
  load_sz(0);

  // x slice -> LDS in half-pair order, with its group sums
  for (int i0 = 0; i0 < items; i0 += 256 * XB) {
    if (i0 > 0) load_x(i0);
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
  // scale words of the block's rows in the slice -> (s 2^(r+b), z - s 2^(r+b))
  {
    const float scl = (float)(1u << (a.r + B));
    for (int i0 = 0; i0 < rows_wg * GS; i0 += 256 * SB) {
      if (i0 > 0) load_sz(i0);
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
  // selected channels inside the slice: positions [h0, h1) of the ascending list,
  // then the slice's hit list (channel, slot, x at each batch row) from the staged x
  int h0 = 0, nh = 0;
  auto find_hits = [&]() {
    int c0 = 0, c1 = 0;
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      c0 += selk[u] < k0;
      c1 += selk[u] < k0 + KS;
    }
    for (int j = tid + 256 * SU; j < ks; j += 256) {
      const int k = sel_k(j);
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
    lds_barrier();  // (x staged,) counts
    h0 = (s_cnt[0][0] + s_cnt[1][0]) + (s_cnt[2][0] + s_cnt[3][0]);
    nh = (s_cnt[0][1] + s_cnt[1][1]) + (s_cnt[2][1] + s_cnt[3][1]) - h0;
    const int nhp = (nh + 31) & ~31;
    auto stage = [&](int pos, int k, int slot) {
      hk[pos] = k;
      hs[pos] = slot;
      const int kl = k - k0, kg = kl & 127;
      int j, hi;
      C::locate(kg & 31, &j, &hi);
      const int hoff = 2 * (((kl >> 7) * 4 + (kg >> 5)) * 16 + j) + hi;
      for (int bc = 0; bc < nb; ++bc)
        hx[bc * HSTR + pos] = __builtin_bit_cast(_Float16, ((const uint16_t*)(xs + bc * XSTR))[hoff]);
    };
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      const int j = tid + 256 * u;
      if (j >= h0 && j < h0 + nh) stage(j - h0, selk[u], sels[u]);
    }
    for (int j = tid + 256 * SU; j < h0 + nh; j += 256)
      if (j >= h0) {
        const int k = sel_k(j);
        stage(j - h0, k, sel_slot(j, k));
      }
    for (int p = nh + tid; p < nhp; p += 256) {
      hk[p] = k0;
      hs[p] = -1;
      for (int bc = 0; bc < nb; ++bc) hx[bc * HSTR + p] = (_Float16)0.f;
    }
  };
  if (ks > 0 && !pub)
    find_hits();
  else
    lds_barrier();  // x staged

  // the unit words of the first 32 hits (the block's rows only) are requested
  // now and land during the resident pass
  const uint32_t* units = (const uint32_t*)o.pool.slots;
  const int wpu = o.pool.unit_bytes >> 2;
  const int wbase = row_wg0 / 32 * a.r;  // row_wg0 is a multiple of 64
  const int n_hw = 32 * UW;
  auto load_hw = [&](int blk, int idx) -> uint32_t {
    if (idx >= n_hw) return 0u;
    const int h = idx / UW, w = idx - h * UW, sl = hs[blk * 32 + h], wi = wbase + w;
    return (sl >= 0 && wi < wpu) ? units[(size_t)sl * wpu + wi] : 0u;
  };
  constexpr int HV = 4;  // prefetched words a thread (blocks of up to 1024 words)
  uint32_t hpre[HV];
  const bool pre = !pub && ks > 0 && nh > 0 && n_hw <= 256 * HV;
  if (!pub && ks > 0 && nh > 0) lds_barrier();  // hit lists staged
  if (pre) {
#pragma unroll
    for (int v = 0; v < HV; ++v) hpre[v] = load_hw(0, tid + 256 * v);
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
      if constexpr (PAIR) {
        if ((u & 1) == 0 && gl < GS) exchange(u);
      }
      if (gl < GS) {
        h8_t ax[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          if (arow) {
            ax[m] = *(const h8_t*)(xs + n * XSTR + (gl * 4 + cq) * 16 + 4 * m);
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
      if constexpr (PAIR) {
        if (u & 1) issue(u - 1, gl - 1 + MPFG);
      } else {
        issue(u, gl + MPFG);
      }
    }
  }

  // the published selection, after the resident pass: wave 0 waits for its flag group,
  // every thread reads its words, the hit list is staged, and once every read has
  // completed the workgroup counts itself for workgroup 0
  if (pub && ks > 0) {
    if (wave == 0) {
      const bool ok0 = wait_published(a, wid & 63);
      if (lane == 0) s_pub = ok0 ? 1 : 0;
    }
    lds_barrier();
    if (s_pub) {
#pragma unroll
      for (int u = 0; u < SU; ++u) {
        const int j = tid + 256 * u;
        selk[u] = j < ks ? sel_k(j) : INT32_MAX;
        sels[u] = j < ks ? sel_slot(j, selk[u]) : -1;
      }
      find_hits();
      lds_barrier();  // hit lists staged
    }
    if (tid == 0) count_reader(a, wid & 63);
  }

  // refinements of the hit channels in the slice, 32 channels per MFMA
  if (ks > 0 && nh > 0) {
    const int r = a.r;
    const float sdown = 1.f / (float)(1u << (r + B));
    for (int blk = 0; blk * 32 < nh; ++blk) {
      // this block's unit words -> LDS
      if (blk > 0) lds_barrier();  // the previous block's words are consumed
      if (blk == 0 && pre) {
#pragma unroll
        for (int v = 0; v < HV; ++v)
          if (tid + 256 * v < n_hw) hu[tid + 256 * v] = hpre[v];
      } else {
        for (int i0 = 0; i0 < n_hw; i0 += 256 * HV) {
          uint32_t v4[HV];
#pragma unroll
          for (int v = 0; v < HV; ++v) v4[v] = load_hw(blk, i0 + tid + 256 * v);
#pragma unroll
          for (int v = 0; v < HV; ++v)
            if (i0 + tid + 256 * v < n_hw) hu[i0 + tid + 256 * v] = v4[v];
        }
      }
      lds_barrier();
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
            // a row's bits end inside the block's span, which ends on a word boundary
            const uint32_t* u = hu + (8 * q + e) * UW - wbase;
            w0[e] = u[wi];
            if (off + r > 32) w1[e] = u[wi + 1];
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
    s_last = __builtin_amdgcn_atomic_inc32(a.ctr + tile_g, (uint32_t)(ns - 1), __ATOMIC_ACQ_REL, "agent") ==
             (uint32_t)(ns - 1);
  __syncthreads();
  if (!s_last) return;
  // last slice of this row block: y = sum of the slices' partials, in slice order;
  // 32 partials of the thread's items (at most 16 batch rows x rows_wg / 256 of
  // them) and consecutive slices are requested at once
  constexpr int MI = 4 * RT, SS = 32 / MI;
  const int n_items = nb * rows_wg;
  const size_t sstride = (size_t)nb * a.rows_pad;
  float sum[MI];
#pragma unroll
  for (int m = 0; m < MI; ++m) sum[m] = 0.f;
  for (int s0 = 0; s0 < ns; s0 += SS) {
    float v[SS][MI];
#pragma unroll
    for (int ss = 0; ss < SS; ++ss)
#pragma unroll
      for (int m = 0; m < MI; ++m) {
        const int i = tid + 256 * m, bc = i / rows_wg, rl = i - bc * rows_wg;
        const bool ok = s0 + ss < ns && i < n_items && row_wg0 + rl < o.n_out;
        v[ss][m] = ok ? sf_get(a.part + (size_t)bc * a.rows_pad + tile_g * rows_wg + rl + (size_t)(s0 + ss) * sstride)
                      : 0.f;
      }
#pragma unroll
    for (int ss = 0; ss < SS; ++ss)
#pragma unroll
      for (int m = 0; m < MI; ++m) sum[m] += v[ss][m];
  }
#pragma unroll
  for (int m = 0; m < MI; ++m) {
    const int i = tid + 256 * m, bc = i / rows_wg, rl = i - bc * rows_wg, row = row_wg0 + rl;
    if (i < n_items && row < o.n_out) o.y[(size_t)(a.batch_off + bc) * o.n_out + row] = sum[m];
  }
}

sf_status dispatch_b(GemvArgs& a, int b, int R, int nb, int kind, hipStream_t s) {
  switch (b) {
    case 1: return gemv_rows_b1(a, R, nb, kind, s);
    case 2: return gemv_rows_b2(a, R, nb, kind, s);
    case 3: return gemv_rows_b3(a, R, nb, kind, s);
    case 4: return gemv_rows_b4(a, R, nb, kind, s);
    case 8: return gemv_rows_b8(a, R, nb, kind, s);
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
MfmaPlan mfma_plan(const int64_t* n_out, int n_ops, int K, int batch, int k_sel, int r) {
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
    if (mfma_lds_words(nb, gs, rows_wg, nhp, k_sel > 0 ? rows_wg * r / 32 : 0) * 4 > MAX_MFMA_LDS) continue;
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

template <int B, bool PAIR>
sf_status launch_mfma_rt(GemvArgs& a, int rt, size_t lds, hipStream_t s) {
  const dim3 grid((unsigned)(a.total_tiles * a.ns + a.sel_wg));
  switch (rt) {
    case 1: hipLaunchKernelGGL((gemv_mfma_kernel<B, 1, PAIR>), grid, dim3(256), lds, s, a); break;
    case 2: hipLaunchKernelGGL((gemv_mfma_kernel<B, 2, PAIR>), grid, dim3(256), lds, s, a); break;
    default: hipLaunchKernelGGL((gemv_mfma_kernel<B, 4, PAIR>), grid, dim3(256), lds, s, a); break;
  }
  SF_LAUNCH_CHECK();
  return SF_OK;
}

sf_status launch_mfma(GemvArgs& a, int b, int rt, size_t lds, hipStream_t s) {
  switch (b) {
    case 1: return a.gs % 2 == 0 ? launch_mfma_rt<1, true>(a, rt, lds, s) : launch_mfma_rt<1, false>(a, rt, lds, s);
    case 2: return a.gs % 2 == 0 ? launch_mfma_rt<2, true>(a, rt, lds, s) : launch_mfma_rt<2, false>(a, rt, lds, s);
    case 4: return launch_mfma_rt<4, false>(a, rt, lds, s);
    default: return launch_mfma_rt<8, false>(a, rt, lds, s);
  }
}

// The plan sf_refined_gemv uses for these ops (rt = 0: the per-row-pair kernel).
MfmaPlan plan_for(const sf_gemv_op* ops, int n_ops, int batch, int k_sel) {
  MfmaPlan p;
  if (!mfma_wanted(ops[0].w.fmt.b, batch)) return p;
  int64_t no[SF_MAX_OPS];
  for (int i = 0; i < n_ops; ++i) no[i] = ops[i].w.n_out;
  return mfma_plan(no, n_ops, (int)ops[0].w.k_in, batch, k_sel, ops[0].w.fmt.r);
}

}  // namespace sfg

using namespace sfg;

extern "C" size_t sf_workspace_bytes_gemv(const sf_gemv_op* ops, int32_t n_ops, int32_t batch, int32_t k_sel) {
  size_t part = 0;
  if (ops && n_ops >= 1 && n_ops <= SF_MAX_OPS && batch >= 1 && ops[0].w.k_in > 0 && ops[0].w.k_in % 128 == 0)
    part = plan_for(ops, n_ops, batch, k_sel).part_bytes;
  size_t a, b, c;
  return gemv_ws_layout(n_ops, k_sel, part, &a, &b, &c);
}

// The refined GEMV on a workspace at ws_base (ws_bytes long, control block zeroed
// and left zeroed by every call).
static sf_status refined_gemv_on(const sf_gemv_op* ops, int32_t n_ops, const uint16_t* x_f16, int32_t batch,
                                 int32_t k_sel, const int32_t* sel_in, int32_t* sel_out, sf_refine_cache* cache,
                                 uint8_t* ws_base, size_t ws_bytes, sf_stream stream) {
  SF_REQUIRE(ops && n_ops >= 1 && n_ops <= SF_MAX_OPS, SF_EINVAL, "need 1..4 ops");
  SF_REQUIRE(x_f16 && batch >= 1, SF_EINVAL, "bad x / batch");
  const sf_qfmt f = ops[0].w.fmt;
  const int64_t K = ops[0].w.k_in;
  SF_REQUIRE(f.group == 128 && f.b >= 1 && f.r >= 0 && f.b + f.r <= 8, SF_EUNSUPPORTED, "bad format");
  SF_REQUIRE(K > 0 && K % 128 == 0 && K <= (1 << 20), SF_EINVAL, "k_in must be a multiple of 128");
  SF_REQUIRE(k_sel >= 0 && k_sel <= K, SF_EINVAL, "k_sel out of range");
  SF_REQUIRE(k_sel == 0 || f.r > 0, SF_EINVAL, "k_sel > 0 needs r > 0");
  SF_REQUIRE(k_sel == 0 || sel_in || k_sel == K || K <= MAX_SEL_K, SF_EUNSUPPORTED,
             "computed selection needs k_in <= 32768");
  GemvArgs a = {};
  // rows per wave: 4 up to 8192 rows per call, else 8 (one row tile per workgroup);
  // SF_GEMV_ROWS_PER_WAVE = 4 or 8 forces a value (a test hook)
  int rpw = env_int("SF_GEMV_ROWS_PER_WAVE", 0);
  int64_t rows_total = 0;
  for (int i = 0; i < n_ops; ++i) rows_total += ops[i].w.n_out;
  if (rpw != 4 && rpw != 8) rpw = rows_total <= 8192 ? 4 : 8;
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
  SF_REQUIRE(ws_bytes >= gemv_ws_layout(n_ops, k_sel, mp.part_bytes, &o_sel, &o_slot, &o_part), SF_ENOMEM,
             "workspace too small");
  a.x = x_f16;
  a.sel_in = sel_in;
  a.sel_out = sel_out;
  a.ws_sel = (int32_t*)(ws_base + o_sel);
  a.ws_slot = (int32_t*)(ws_base + o_slot);
  a.n_ops = n_ops;
  a.k_in = (int32_t)K;
  a.batch = batch;
  a.k_sel = k_sel;
  a.r = f.r;
  a.total_tiles = tiles;
  hipStream_t s = (hipStream_t)stream;
  const int cpc = codes_per_chunk(f.b);
  // Batch 1-2 without the batched kernel: the split kernel (workgroup 0 selects
  // while the others stream), or the fused kernel (selection in every workgroup)
  // where the split kernel's LDS or published copies do not fit.  SF_GEMV_SPLIT=0
  // forces the fused kernel and SF_GEMV_SPLIT=2 the staged split variant (test
  // hooks).  With more batch rows than one launch takes, the selection over all rows
  // comes from the selection launch.
  // A selection that is given (sel_in, or every channel) needs no selecting
  // workgroup: each tile looks its hits up itself ("direct").
  const bool given = k_sel == 0 || sel_in != nullptr || k_sel >= K;
  int kind = KIND_NONE;
  if (!mfma) {
    if (env_int("SF_GEMV_SPLIT", 1) != 0 && given && split_lds_bytes((int)K, cpc / 2, cpc, 1, k_sel, rpw, false) <= MAX_DYN_LDS)
      kind = KIND_SPLIT;
    else if (env_int("SF_GEMV_SPLIT", 1) != 0 && split_lds_bytes((int)K, cpc / 2, cpc, 1, k_sel, rpw) <= MAX_DYN_LDS &&
        (size_t)SPLIT_COPIES * split_copy_words(k_sel, n_ops) <= sizeof(((WsControl*)nullptr)->hit) / 4)
      kind = KIND_SPLIT;
    else if (fused_lds_bytes((int)K, cpc, 1, k_sel, rpw) <= MAX_DYN_LDS)
      kind = KIND_FUSED;
    SF_REQUIRE(kind != KIND_NONE, SF_EUNSUPPORTED, "k_in too large for the batch-1/2 kernels' LDS");
  }
  const size_t lds2 = kind == KIND_SPLIT ? split_lds_bytes((int)K, cpc / 2, cpc, 2, k_sel, rpw, !given)
                                         : fused_lds_bytes((int)K, cpc, 2, k_sel, rpw);
  const int max_nb = lds2 <= 64 * 1024 ? 2 : 1;
  const bool one_launch = !mfma && batch <= max_nb;
  // the batched kernel selects in its own workgroup 0 when one launch takes every
  // batch row and the selector's LDS and the published copies fit; else a selection
  // launch comes first
  const bool mfma_sw = mfma && !given && batch <= 16 && select_lds_bytes((int)K, k_sel) <= MAX_MFMA_LDS &&
                       (size_t)SPLIT_COPIES * split_copy_words(k_sel, n_ops) <= sizeof(((WsControl*)nullptr)->hit) / 4;
  if (k_sel > 0 && !one_launch && !mfma_sw) {
    hipLaunchKernelGGL(gemv_select_kernel, dim3(1), dim3(256), select_lds_bytes((int)K, k_sel), s, a);
    SF_LAUNCH_CHECK();
  }
  if (mfma) {
    a.ns = mp.ns;
    a.gs = mp.gs;
    a.nhp = mp.nhp;
    a.rows_pad = tiles * rows_wg;
    a.part = (float*)(ws_base + o_part);
    a.ctr = (uint32_t*)(ws_base + offsetof(WsControl, row_ctr));
    a.ctl = (uint32_t*)ws_base;
    a.sel_wg = mfma_sw ? 1 : 0;
    a.report = mfma_sw ? 1 : 0;
    a.n_readers = tiles * mp.ns;
    for (int b0 = 0; b0 < batch; b0 += 16) {
      const int nb = batch - b0 < 16 ? batch - b0 : 16;
      a.batch_off = b0;
      size_t lds = mfma_lds_words(nb, mp.gs, rows_wg, mp.nhp, mp.nhp > 0 ? rows_wg * f.r / 32 : 0) * 4;
      if (mfma_sw) lds = std::max(lds, select_lds_bytes((int)K, k_sel));
      sf_status st = launch_mfma(a, f.b, mp.rt, lds, s);
      if (st != SF_OK) return st;
    }
    return SF_OK;
  }
  // two batch rows per launch when both fit the LDS staging of x, else one
  a.report = one_launch ? 1 : 0;
  if (!one_launch && k_sel > 0) a.sel_in = a.ws_sel;
  // the selecting workgroup only where the selection is computed in this launch
  a.sel_wg = (kind == KIND_SPLIT && k_sel > 0 && a.sel_in == nullptr && k_sel < K) ? 1 : 0;
  a.ctl = (uint32_t*)ws_base;
  a.n_readers = tiles;
  for (int b0 = 0; b0 < batch; b0 += max_nb) {
    const int nb = (batch - b0) >= max_nb ? max_nb : 1;
    a.batch_off = b0;
    sf_status st = dispatch_b(a, f.b, rpw, nb, kind, s);
    if (st != SF_OK) return st;
  }
  return SF_OK;
}

extern "C" sf_status sf_refined_gemv(const sf_gemv_op* ops, int32_t n_ops, const uint16_t* x_f16,
                                     int32_t batch, int32_t k_sel, const int32_t* sel_in,
                                     int32_t* sel_out, sf_refine_cache* cache, sf_workspace* ws,
                                     sf_stream stream) {
  SF_REQUIRE(ws, SF_EINVAL, "workspace required");
  return refined_gemv_on(ops, n_ops, x_f16, batch, k_sel, sel_in, sel_out, cache, ws->base, ws->bytes, stream);
}

// ---- the same call without a workspace: a library-owned scratch array ------------
// For callers that cannot allocate (graph capture, serving loops).  The array is a
// file-scope device variable: each device the library runs on holds its own copy
// from module load until the process ends.  Host code never uses the array's name as
// an address: its device address comes from hipGetSymbolAddress, once per device.
namespace {
constexpr size_t SF_SCRATCH_BYTES = size_t(8) << 20;
__device__ __align__(256) uint8_t scratch[SF_SCRATCH_BYTES];
constexpr int SF_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[SF_MAX_DEVICES] = {};

// Clears the control block's flags and counters (the split kernel's hand-off words,
// the batched kernel's row-block counters and the timeout word) on the stream.
__global__ void scratch_clear_kernel(uint32_t* ctl) {
  WsControl* c = (WsControl*)ctl;
  for (int i = threadIdx.x; i < 64 * 32; i += blockDim.x) {
    c->sel_flag[i] = 0u;
    c->rd_ctr[i] = 0u;
  }
  for (int i = threadIdx.x; i < 1024; i += blockDim.x) c->row_ctr[i] = 0u;
  if (threadIdx.x == 0) {
    c->sel_state = 0u;
    c->done = 0u;
    c->timeout = 0u;
    c->spin_limit = 0u;
  }
}

sf_status scratch_of_device(uint8_t** out) {
  int dev = 0;
  SF_HIP(hipGetDevice(&dev));
  SF_REQUIRE(dev >= 0 && dev < SF_MAX_DEVICES, SF_EUNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    SF_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    SF_REQUIRE(p != nullptr, SF_EHIP, "no device address for the scratch array");
    g_scratch_ptr[dev] = (uint8_t*)p;
  }
  *out = g_scratch_ptr[dev];
  return SF_OK;
}
}  // namespace

extern "C" sf_status sf_refined_gemv_noalloc(const sf_gemv_op* ops, int32_t n_ops, const uint16_t* x_f16,
                                             int32_t batch, int32_t k_sel, const int32_t* sel_in,
                                             int32_t* sel_out, sf_refine_cache* cache, sf_stream stream) {
  SF_REQUIRE(ops && n_ops >= 1 && n_ops <= SF_MAX_OPS && batch >= 1, SF_EINVAL, "need 1..4 ops and batch >= 1");
  const size_t need = sf_workspace_bytes_gemv(ops, n_ops, batch, k_sel);
  SF_REQUIRE(need <= SF_SCRATCH_BYTES, SF_ENOMEM,
             "this call needs " + std::to_string(need) + " bytes of scratch; the scratch array holds " +
                 std::to_string(SF_SCRATCH_BYTES) + " (use sf_refined_gemv with a workspace)");
  uint8_t* base = nullptr;
  sf_status st = scratch_of_device(&base);
  if (st != SF_OK) return st;
  hipLaunchKernelGGL(scratch_clear_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream, (uint32_t*)base);
  SF_LAUNCH_CHECK();
  return refined_gemv_on(ops, n_ops, x_f16, batch, k_sel, sel_in, sel_out, cache, base, SF_SCRATCH_BYTES, stream);
}
