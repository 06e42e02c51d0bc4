// Decode-step glue around the refined GEMV and attention: embedding gather,
// residual add + RMSNorm, per-head q/k RMSNorm + rotary embedding, SwiGLU, fp16
// casts and greedy argmax.
//
// The pages describe only the refined GEMV and attention; a decoder step around
// them follows the public Llama-3.1 / Qwen3 layer definitions (RMSNorm, rotate-half
// rotary embedding, SwiGLU feed-forward, fp32 residual stream, fp16 GEMV inputs).
// These kernels move a few KB per call; each is one launch of small workgroups,
// with reductions inside a workgroup only.
#include <algorithm>

#include "select_core.h"
#include "sf_internal.h"

namespace {

__device__ __forceinline__ uint16_t f2h(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }

template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) s += red[w];
  __syncthreads();
  return s;
}

// h[b] = table[ids[b]] (fp16 -> fp32); an id outside [0, vocab) gives a zero row
__global__ __launch_bounds__(256) void embed_kernel(const uint16_t* table, int64_t vocab, int hidden, const int32_t* ids,
                                                    float* h) {
  const int b = blockIdx.x;
  const int id = ids[b];
  const bool ok = id >= 0 && id < vocab;
  const uint16_t* row = table + (ok ? (size_t)id : 0) * hidden;
  for (int i = threadIdx.x; i < hidden; i += 256) h[(size_t)b * hidden + i] = ok ? sf_h2f(row[i]) : 0.f;
}

// h[b] += y[b] (if y); x[b] = fp16(h[b] / sqrt(mean(h[b]^2) + eps) * w)
// General form: any hidden size, one strided pass to add and square, one to scale.
constexpr int NORM_T = 256;
__global__ __launch_bounds__(NORM_T) void add_rmsnorm_kernel(float* h, const float* y, const float* w, int hidden,
                                                             float eps, uint16_t* x) {
  __shared__ float red[NORM_T / 64];
  const int b = blockIdx.x;
  float* hr = h + (size_t)b * hidden;
  const float* yr = y ? y + (size_t)b * hidden : nullptr;
  float ss = 0.f;
  for (int i = threadIdx.x; i < hidden; i += NORM_T) {
    float v = hr[i];
    if (yr) {
      v += yr[i];
      hr[i] = v;
    }
    ss = fmaf(v, v, ss);
  }
  const float tot = block_sum<NORM_T>(ss, red);
  const float rstd = 1.f / sqrtf(tot / (float)hidden + eps);
  for (int i = threadIdx.x; i < hidden; i += NORM_T) x[(size_t)b * hidden + i] = f2h(hr[i] * rstd * w[i]);
}

// Row kept in registers: hidden % 4 == 0 and hidden <= 4 * NORMV_T * NORMV_N.  Every
// load of the row is issued before the first reduction, so a row costs about one
// memory latency instead of one per strided step.
constexpr int NORMV_T = 1024, NORMV_N = 4;
__global__ __launch_bounds__(NORMV_T) void add_rmsnorm_vec_kernel(float* __restrict__ h, const float* __restrict__ y,
                                                                  const float* __restrict__ w, int hidden, float eps,
                                                                  uint16_t* __restrict__ x) {
  __shared__ float red[NORMV_T / 64];
  const int b = blockIdx.x, n4 = hidden >> 2;
  float4* hr = (float4*)(h + (size_t)b * hidden);
  const float4* yr = y ? (const float4*)(y + (size_t)b * hidden) : nullptr;
  float4 v[NORMV_N];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < NORMV_N; ++k) {
    const int i = threadIdx.x + k * NORMV_T;
    v[k] = i < n4 ? hr[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    if (yr && i < n4) {
      const float4 t = yr[i];
      v[k].x += t.x;
      v[k].y += t.y;
      v[k].z += t.z;
      v[k].w += t.w;
    }
  }
#pragma unroll
  for (int k = 0; k < NORMV_N; ++k) {
    const int i = threadIdx.x + k * NORMV_T;
    if (yr && i < n4) hr[i] = v[k];
    ss = fmaf(v[k].x, v[k].x, ss);
    ss = fmaf(v[k].y, v[k].y, ss);
    ss = fmaf(v[k].z, v[k].z, ss);
    ss = fmaf(v[k].w, v[k].w, ss);
  }
  const float tot = block_sum<NORMV_T>(ss, red);
  const float rstd = 1.f / sqrtf(tot / (float)hidden + eps);
  const float4* wr = (const float4*)w;
  uint2* xr = (uint2*)(x + (size_t)b * hidden);
#pragma unroll
  for (int k = 0; k < NORMV_N; ++k) {
    const int i = threadIdx.x + k * NORMV_T;
    if (i < n4) {
      const float4 g = wr[i];
      const uint32_t lo = (uint32_t)f2h(v[k].x * rstd * g.x) | ((uint32_t)f2h(v[k].y * rstd * g.y) << 16);
      const uint32_t hi = (uint32_t)f2h(v[k].z * rstd * g.z) | ((uint32_t)f2h(v[k].w * rstd * g.w) << 16);
      xr[i] = make_uint2(lo, hi);
    }
  }
}

// One wave per (batch, head) of 128 dims; lane i owns the rotate-half pair (i, i + 64).
// Heads [0, n_q) are queries (written as fp16 to qh), the rest keys (written as
// fp32 to ko).  Optional per-head RMSNorm first.  Angles are formed and rotated in fp64
// (positions reach 2^17 radians and beyond).
__global__ __launch_bounds__(64) void qk_rope_kernel(const float* q, const float* k, int n_q, int n_kv, const float* qw,
                                                     const float* kw, float eps, int pos, double theta, uint16_t* qh,
                                                     float* ko) {
  const int b = blockIdx.y, head = blockIdx.x, i = threadIdx.x;
  const bool isq = head < n_q;
  const float* v = isq ? q + ((size_t)b * n_q + head) * 128 : k + ((size_t)b * n_kv + (head - n_q)) * 128;
  const float* nw = isq ? qw : kw;
  float x0 = v[i], x1 = v[i + 64];
  if (nw) {
    float ss = x0 * x0 + x1 * x1;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
    const float rstd = 1.f / sqrtf(ss / 128.f + eps);
    x0 = x0 * rstd * nw[i];
    x1 = x1 * rstd * nw[i + 64];
  }
  const double ang = (double)pos * pow(theta, -2.0 * (double)i / 128.0);
  double sn, cs;
  sincos(ang, &sn, &cs);
  const float r0 = (float)((double)x0 * cs - (double)x1 * sn);
  const float r1 = (float)((double)x1 * cs + (double)x0 * sn);
  if (isq) {
    uint16_t* o = qh + ((size_t)b * n_q + head) * 128;
    o[i] = f2h(r0);
    o[i + 64] = f2h(r1);
  } else {
    float* o = ko + ((size_t)b * n_kv + (head - n_q)) * 128;
    o[i] = r0;
    o[i + 64] = r1;
  }
}

// act = fp16(silu(gate) * up)
__global__ __launch_bounds__(256) void swiglu_kernel(const float* g, const float* u, int64_t n, uint16_t* act) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float gv = g[i];
    act[i] = f2h(gv / (1.f + expf(-gv)) * u[i]);
  }
}

__global__ __launch_bounds__(256) void residual_add_kernel(float* h, const float* d, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) h[i] += d[i];
}

__global__ __launch_bounds__(256) void to_f16_kernel(const float* x, int64_t n, uint16_t* out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) out[i] = f2h(x[i]);
}

// ids[b] = argmax over logits[b] (lowest index among equal maxima; NaN never wins).
// One workgroup per row; the row is read as 16-byte vectors, AMAX_U of them in
// flight per thread, so that a long vocabulary costs a few memory latencies.
constexpr int AMAX_T = 1024, AMAX_U = 8;

__device__ __forceinline__ void amax_take(float v, int64_t i, float& best, int64_t& bi) {
  if (v > best || (v == best && (bi < 0 || i < bi))) {
    best = v;
    bi = i;
  }
}

__global__ __launch_bounds__(AMAX_T) void argmax_kernel(const float* logits, int64_t vocab, int32_t* ids) {
  __shared__ float sv[AMAX_T / 64];
  __shared__ int64_t si[AMAX_T / 64];
  const int b = blockIdx.x, tid = threadIdx.x;
  const float* row = logits + (size_t)b * vocab;
  float best = -INFINITY;
  int64_t bi = -1;
  // scalar head up to 16-byte alignment, then vectors, then the scalar tail
  const int64_t head = std::min<int64_t>(vocab, (int64_t)((16 - ((uintptr_t)row & 15)) & 15) / 4);
  if (tid < head) amax_take(row[tid], tid, best, bi);
  const int64_t nv = (vocab - head) / 4;
  const float4* rv = (const float4*)(row + head);
  for (int64_t v0 = 0; v0 < nv; v0 += (int64_t)AMAX_T * AMAX_U) {
    float4 x[AMAX_U];
#pragma unroll
    for (int u = 0; u < AMAX_U; ++u) {
      const int64_t j = v0 + tid + (int64_t)AMAX_T * u;
      x[u] = j < nv ? rv[j] : make_float4(NAN, NAN, NAN, NAN);
    }
#pragma unroll
    for (int u = 0; u < AMAX_U; ++u) {
      const int64_t i0 = head + 4 * (v0 + tid + (int64_t)AMAX_T * u);
      amax_take(x[u].x, i0, best, bi);
      amax_take(x[u].y, i0 + 1, best, bi);
      amax_take(x[u].z, i0 + 2, best, bi);
      amax_take(x[u].w, i0 + 3, best, bi);
    }
  }
  const int64_t tail0 = head + 4 * nv;
  if (tail0 + tid < vocab) amax_take(row[tail0 + tid], tail0 + tid, best, bi);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int64_t oi = __shfl_xor(bi, o, 64);
    if (oi >= 0) amax_take(ov, oi, best, bi);
  }
  const int lane = tid & 63, wave = tid >> 6;
  if (lane == 0) {
    sv[wave] = best;
    si[wave] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < AMAX_T / 64; ++w)
      if (si[w] >= 0) amax_take(sv[w], si[w], best, bi);
    ids[b] = (int32_t)(bi < 0 ? 0 : bi);
  }
}

unsigned grid_for(int64_t n) { return (unsigned)std::min<int64_t>((n + 255) / 256, 4096); }

// ---- producers of a GEMV input that also select its channels ----------------------
// One 1024-thread workgroup forms the fp16 input x of `batch` rows of n channels and
// selects the k_sel channels of largest max-over-rows |x| (select_core.h), so that
// the GEMV that reads x starts with its selection ready.  Thread t owns channels
// 8m .. 8m+7 of every row, m = t + 1024 i (i < MI).  The element arithmetic is that
// of sf_add_rmsnorm, sf_swiglu and sf_to_f16.
constexpr int PS_T = 1024, PS_MAXB = 16;
enum ProdOp { PROD_NORM = 0, PROD_SWIGLU = 1, PROD_CAST = 2 };

struct ProdArgs {
  float* h;         // NORM: residual rows [batch][n] (h += y in place when y is given)
  const float* y;
  const float* w;   // NORM: gain [n]
  const float* a;   // SWIGLU: gate; CAST: x
  const float* b;   // SWIGLU: up
  int batch, n;
  float eps;
  uint16_t* out;    // [batch][n] fp16 bits
  int k_sel;
  int32_t* sel_out; // [k_sel]
};

__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const float4 a = ((const float4*)p)[0], b = ((const float4*)p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <int OP, int MI>
__global__ __launch_bounds__(PS_T) void produce_select_kernel(ProdArgs p) {
  __shared__ float red[PS_T / 64][PS_MAXB];
  __shared__ float rstd[PS_MAXB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = p.n, n8 = n / 8;
  // rows 0 and 1 of this thread's channels stay in registers between the passes
  float keep[2][MI][8];
  if constexpr (OP == PROD_NORM) {
    // h += y, and per row the sum of squares (all rows reduced together)
    float ss[PS_MAXB];
#pragma unroll
    for (int bb = 0; bb < PS_MAXB; ++bb) ss[bb] = 0.f;
#pragma unroll
    for (int bb = 0; bb < PS_MAXB; ++bb) {
      if (bb >= p.batch) break;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int m = tid + PS_T * i;
        if (m >= n8) continue;
        float v[8], t[8];
        load8(p.h + (size_t)bb * n + 8 * m, v);
        if (p.y) load8(p.y + (size_t)bb * n + 8 * m, t);
        if (p.y) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] += t[e];
          float4* hp = (float4*)(p.h + (size_t)bb * n + 8 * m);
          hp[0] = make_float4(v[0], v[1], v[2], v[3]);
          hp[1] = make_float4(v[4], v[5], v[6], v[7]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) ss[bb] = fmaf(v[e], v[e], ss[bb]);
        if (bb < 2)
#pragma unroll
          for (int e = 0; e < 8; ++e) keep[bb][i][e] = v[e];
      }
    }
#pragma unroll
    for (int bb = 0; bb < PS_MAXB; ++bb) {
      if (bb >= p.batch) break;
      float v = ss[bb];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
      if (lane == 0) red[wave][bb] = v;
    }
    __syncthreads();
    if (tid < p.batch) {
      float t = 0.f;
#pragma unroll
      for (int w = 0; w < PS_T / 64; ++w) t += red[w][tid];
      rstd[tid] = 1.f / sqrtf(t / (float)n + p.eps);
    }
    __syncthreads();
  }
  uint32_t kw[4 * MI];
#pragma unroll
  for (int i = 0; i < 4 * MI; ++i) kw[i] = 0u;
  for (int bb = 0; bb < p.batch; ++bb) {
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int m = tid + PS_T * i;
      if (m >= n8) continue;
      const size_t off = (size_t)bb * n + 8 * m;
      float v[8];
      if constexpr (OP == PROD_NORM) {
        float g[8];
        if (bb < 2) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = keep[bb < 1 ? 0 : 1][i][e];
        } else {
          load8(p.h + off, v);
        }
        load8(p.w + 8 * m, g);
        const float rs = rstd[bb];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = v[e] * rs * g[e];
      } else if constexpr (OP == PROD_SWIGLU) {
        float u[8];
        load8(p.a + off, v);
        load8(p.b + off, u);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = v[e] / (1.f + expf(-v[e])) * u[e];
      } else {
        load8(p.a + off, v);
      }
      uint32_t x[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) x[q] = (uint32_t)f2h(v[2 * q]) | ((uint32_t)f2h(v[2 * q + 1]) << 16);
      ((uint4*)(p.out + off))[0] = make_uint4(x[0], x[1], x[2], x[3]);
      sfsel::key_max8(kw + 4 * i, x);
    }
  }
  const int ks = p.k_sel;
  if (ks <= 0 || !p.sel_out) return;
  if (ks >= n) {
    for (int j = tid; j < ks; j += PS_T) p.sel_out[j] = j;
    return;
  }
  sfsel::topk_keys<PS_T, MI>(kw, n, ks, p.sel_out);
}

template <int OP>
sf_status launch_produce(const ProdArgs& p, hipStream_t s) {
  const int mi = (p.n / 8 + PS_T - 1) / PS_T;
  if (mi <= 1)
    hipLaunchKernelGGL((produce_select_kernel<OP, 1>), dim3(1), dim3(PS_T), 0, s, p);
  else if (mi <= 2)
    hipLaunchKernelGGL((produce_select_kernel<OP, 2>), dim3(1), dim3(PS_T), 0, s, p);
  else
    hipLaunchKernelGGL((produce_select_kernel<OP, 4>), dim3(1), dim3(PS_T), 0, s, p);
  SF_LAUNCH_CHECK();
  return SF_OK;
}

sf_status check_produce(const ProdArgs& p) {
  const auto al = [](const void* q, uintptr_t a) { return q == nullptr || ((uintptr_t)q & (a - 1)) == 0; };
  SF_REQUIRE(p.out && p.batch >= 1 && p.batch <= PS_MAXB, SF_EINVAL, "need an output and 1 <= batch <= 16");
  SF_REQUIRE(p.n > 0 && p.n % 8 == 0 && p.n <= 8 * PS_T * 4, SF_EINVAL, "n must be a multiple of 8, at most 32768");
  SF_REQUIRE(p.k_sel >= 0 && p.k_sel <= p.n && (p.k_sel == 0 || p.sel_out), SF_EINVAL, "bad k_sel / sel_out");
  SF_REQUIRE(al(p.h, 16) && al(p.y, 16) && al(p.w, 16) && al(p.a, 16) && al(p.b, 16) && al(p.out, 16), SF_EINVAL,
             "tensors must be 16-byte aligned");
  return SF_OK;
}

}  // namespace

extern "C" sf_status sf_embed(const uint16_t* table_f16, int64_t vocab, int32_t hidden, const int32_t* ids,
                              int32_t batch, float* h_out, sf_stream stream) {
  SF_REQUIRE(table_f16 && ids && h_out, SF_EINVAL, "null argument");
  SF_REQUIRE(vocab > 0 && hidden > 0 && batch > 0, SF_EINVAL, "bad sizes");
  hipLaunchKernelGGL(embed_kernel, dim3(batch), dim3(256), 0, (hipStream_t)stream, table_f16, vocab, hidden, ids, h_out);
  SF_LAUNCH_CHECK();
  return SF_OK;
}

extern "C" sf_status sf_add_rmsnorm(float* h, const float* y, const float* w, int32_t batch, int32_t hidden, float eps,
                                    uint16_t* x_f16, sf_stream stream) {
  SF_REQUIRE(h && w && x_f16, SF_EINVAL, "null argument");
  SF_REQUIRE(batch > 0 && hidden > 0 && eps >= 0.f, SF_EINVAL, "bad sizes");
  const auto al = [](const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; };
  if (hidden % 4 == 0 && hidden <= 4 * NORMV_T * NORMV_N && al(h, 16) && (!y || al(y, 16)) && al(w, 16) &&
      al(x_f16, 8))
    hipLaunchKernelGGL(add_rmsnorm_vec_kernel, dim3(batch), dim3(NORMV_T), 0, (hipStream_t)stream, h, y, w, hidden,
                       eps, x_f16);
  else
    hipLaunchKernelGGL(add_rmsnorm_kernel, dim3(batch), dim3(NORM_T), 0, (hipStream_t)stream, h, y, w, hidden, eps,
                       x_f16);
  SF_LAUNCH_CHECK();
  return SF_OK;
}

extern "C" sf_status sf_qk_rope(const float* q, const float* k, int32_t batch, int32_t n_q, int32_t n_kv,
                                const float* q_norm_w, const float* k_norm_w, float eps, int32_t pos, float theta,
                                uint16_t* q_f16, float* k_out, sf_stream stream) {
  SF_REQUIRE(q && k && q_f16 && k_out, SF_EINVAL, "null argument");
  SF_REQUIRE(batch > 0 && n_q > 0 && n_kv > 0 && pos >= 0 && theta > 1.f, SF_EINVAL, "bad sizes");
  SF_REQUIRE((q_norm_w == nullptr) == (k_norm_w == nullptr), SF_EINVAL, "give both head-norm weights or neither");
  hipLaunchKernelGGL(qk_rope_kernel, dim3(n_q + n_kv, batch), dim3(64), 0, (hipStream_t)stream, q, k, n_q, n_kv,
                     q_norm_w, k_norm_w, eps, pos, (double)theta, q_f16, k_out);
  SF_LAUNCH_CHECK();
  return SF_OK;
}

extern "C" sf_status sf_swiglu(const float* gate, const float* up, int64_t n, uint16_t* act_f16, sf_stream stream) {
  SF_REQUIRE(gate && up && act_f16 && n > 0, SF_EINVAL, "bad arguments");
  hipLaunchKernelGGL(swiglu_kernel, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, gate, up, n, act_f16);
  SF_LAUNCH_CHECK();
  return SF_OK;
}

extern "C" sf_status sf_residual_add(float* h, const float* d, int64_t n, sf_stream stream) {
  SF_REQUIRE(h && d && n > 0, SF_EINVAL, "bad arguments");
  hipLaunchKernelGGL(residual_add_kernel, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, h, d, n);
  SF_LAUNCH_CHECK();
  return SF_OK;
}

extern "C" sf_status sf_to_f16(const float* x, int64_t n, uint16_t* out_f16, sf_stream stream) {
  SF_REQUIRE(x && out_f16 && n > 0, SF_EINVAL, "bad arguments");
  hipLaunchKernelGGL(to_f16_kernel, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, x, n, out_f16);
  SF_LAUNCH_CHECK();
  return SF_OK;
}

extern "C" sf_status sf_argmax(const float* logits, int32_t batch, int64_t vocab, int32_t* ids, sf_stream stream) {
  SF_REQUIRE(logits && ids && batch > 0 && vocab > 0, SF_EINVAL, "bad arguments");
  hipLaunchKernelGGL(argmax_kernel, dim3(batch), dim3(AMAX_T), 0, (hipStream_t)stream, logits, vocab, ids);
  SF_LAUNCH_CHECK();
  return SF_OK;
}

extern "C" sf_status sf_add_rmsnorm_select(float* h, const float* y, const float* w, int32_t batch, int32_t hidden,
                                           float eps, uint16_t* x_f16, int32_t k_sel, int32_t* sel_out,
                                           sf_stream stream) {
  SF_REQUIRE(h && w && eps >= 0.f, SF_EINVAL, "null argument");
  ProdArgs p{h, y, w, nullptr, nullptr, batch, hidden, eps, x_f16, k_sel, sel_out};
  sf_status st = check_produce(p);
  if (st != SF_OK) return st;
  return launch_produce<PROD_NORM>(p, (hipStream_t)stream);
}

extern "C" sf_status sf_swiglu_select(const float* gate, const float* up, int32_t batch, int32_t n, uint16_t* act_f16,
                                      int32_t k_sel, int32_t* sel_out, sf_stream stream) {
  SF_REQUIRE(gate && up, SF_EINVAL, "null argument");
  ProdArgs p{nullptr, nullptr, nullptr, gate, up, batch, n, 0.f, act_f16, k_sel, sel_out};
  sf_status st = check_produce(p);
  if (st != SF_OK) return st;
  return launch_produce<PROD_SWIGLU>(p, (hipStream_t)stream);
}

extern "C" sf_status sf_to_f16_select(const float* x, int32_t batch, int32_t n, uint16_t* out_f16, int32_t k_sel,
                                      int32_t* sel_out, sf_stream stream) {
  SF_REQUIRE(x, SF_EINVAL, "null argument");
  ProdArgs p{nullptr, nullptr, nullptr, x, nullptr, batch, n, 0.f, out_f16, k_sel, sel_out};
  sf_status st = check_produce(p);
  if (st != SF_OK) return st;
  return launch_produce<PROD_CAST>(p, (hipStream_t)stream);
}
