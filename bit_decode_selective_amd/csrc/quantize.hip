// Nested quantisation (resident + refinement codes), KV append, and the test-only
// dequantisation export.
//
// Representation: rag-lover.com StrataFlux summary, explainer dialogue (解説) --
// the fetched refinement bits subdivide the interval between resident low-bit
// levels.  Format fixed by this library: per group of 128 values, one (b+r)-bit
// asymmetric uniform code; fp16 offset z = fp16(min) and step s = fp16((max-min)/Q),
// each one round-to-nearest-even of the fp64 value; c = clamp(rint((x-z)/s), 0, Q)
// in fp64; resident = c >> r, refinement = c & (2^r - 1); LSB-first bit streams.
//
// Every code decision is taken in fp64 with IEEE-exact operations (subtract,
// divide, round-to-nearest-even), so the codes are reproducible bit for bit by any
// IEEE fp64 implementation of the same formula.
#include "group_quant.h"

namespace {

using namespace sfq;

__global__ __launch_bounds__(256) void quantize_rows_kernel(const float* __restrict__ x,
                                                            int64_t rows, int64_t cols, int b,
                                                            int r, uint8_t* __restrict__ resident,
                                                            uint32_t* __restrict__ sz,
                                                            uint8_t* __restrict__ refine_rows) {
  __shared__ uint8_t lds[4][256];
  const int wave = threadIdx.x >> 6;
  const int64_t ngr = cols / 128;
  const int64_t gid = (int64_t)blockIdx.x * 4 + wave;
  if (gid >= rows * ngr) return;  // whole wave leaves together
  const int64_t row = gid / ngr, g = gid - row * ngr;
  uint32_t* res = (uint32_t*)(resident + row * (cols * b / 8) + g * 16 * b);
  uint32_t* ref = refine_rows ? (uint32_t*)(refine_rows + row * (cols * r / 8) + g * 16 * r) : nullptr;
  quantize_group_wave(x + row * cols + g * 128, b, r, lds[wave], lds[wave] + 128, res,
                      sz + row * ngr + g, ref);
}

// Channel-major refinement: unit k = refinement bits of column k over all rows.
// One thread per (column k, 32-bit word w of unit k); the codes are recomputed from
// x and the group's s, z with the same fp64 formula as quantize_rows_kernel.
__global__ __launch_bounds__(256) void refine_channel_major_kernel(
    const float* __restrict__ x, int64_t rows, int64_t cols, int b, int r,
    const uint32_t* __restrict__ sz, uint8_t* __restrict__ refine) {
  const int64_t words_per_unit = rows * r / 32;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t k = idx % cols, w = idx / cols;
  if (w >= words_per_unit) return;
  const int Q = (1 << (b + r)) - 1;
  const int64_t ngr = cols / 128;
  uint32_t word = 0;
  int64_t prev_n = -1;
  uint32_t clo = 0;
  for (int p = 0; p < 32; ++p) {
    const int64_t P = 32 * w + p;
    const int64_t n = P / r;
    const int j = (int)(P - n * r);
    if (n != prev_n) {
      const uint32_t szw = sz[n * ngr + k / 128];
      const uint32_t s16 = szw & 0xFFFFu;
      const uint32_t c = code_of(x[n * cols + k], h2d(szw >> 16), h2d(s16), s16, Q);
      clo = c & ((1u << r) - 1u);
      prev_n = n;
    }
    word |= ((clo >> j) & 1u) << p;
  }
  ((uint32_t*)(refine + k * (rows * r / 8)))[w] = word;
}

// KV append: one wave per (batch, head, token, K|V) group.
__global__ __launch_bounds__(256) void kv_append_kernel(const float* __restrict__ k_new,
                                                        const float* __restrict__ v_new,
                                                        int batch, int n_kv, int n_tok, int t0,
                                                        int t_cap, int b, int r,
                                                        uint8_t* k_res, uint32_t* k_sz,
                                                        uint8_t* v_res, uint32_t* v_sz,
                                                        uint8_t* refine_out, int64_t refine_ld) {
  __shared__ uint8_t lds[4][256];
  const int wave = threadIdx.x >> 6;
  const int64_t gid = (int64_t)blockIdx.x * 4 + wave;
  const int64_t total = (int64_t)batch * n_kv * n_tok * 2;
  if (gid >= total) return;
  const int which = (int)(gid & 1);  // 0 = K, 1 = V
  const int64_t e = gid >> 1;        // (bh, tok)
  const int64_t tok = e % n_tok, bh = e / n_tok;
  const float* src = (which ? v_new : k_new) + e * 128;
  const int64_t pos = bh * t_cap + t0 + tok;
  uint8_t* res_base = which ? v_res : k_res;
  uint32_t* sz_base = which ? v_sz : k_sz;
  const int64_t unit_bytes = 2 * 16 * r;
  uint32_t* ref = (refine_out && r > 0)
                      ? (uint32_t*)(refine_out + (bh * refine_ld + tok) * unit_bytes + which * 16 * r)
                      : nullptr;
  quantize_group_wave(src, b, r, lds[wave], lds[wave] + 128,
                      (uint32_t*)(res_base + pos * 16 * b), sz_base + pos, ref);
}

__device__ __forceinline__ uint32_t read_bits(const uint8_t* base, int64_t bitpos, int width) {
  // width <= 8: the field lies in at most two consecutive bytes
  const int64_t byte = bitpos >> 3;
  const int off = (int)(bitpos & 7);
  uint32_t v = base[byte];
  if (off + width > 8) v |= (uint32_t)base[byte + 1] << 8;
  return (v >> off) & ((1u << width) - 1u);
}

__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ resident,
                                                      const uint32_t* __restrict__ sz,
                                                      const uint8_t* __restrict__ refine,
                                                      int64_t rows, int64_t cols, int b, int r,
                                                      int layout, int which,
                                                      float* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * cols) return;
  const int64_t n = idx / cols, k = idx - n * cols;
  const uint32_t hi = read_bits(resident + n * (cols * b / 8), k * b, b);
  const uint32_t szw = sz[n * (cols / 128) + k / 128];
  const float s = sf_h2f(szw), z = sf_h2f(szw >> 16);
  float v;
  if (which == 0) {
    v = fmaf(s * (float)(1u << r), (float)hi, z);
  } else {
    uint32_t lo = 0;
    if (r > 0) {
      if (layout == SF_REFINE_CHANNEL_MAJOR)
        lo = read_bits(refine + k * (rows * r / 8), n * r, r);
      else
        lo = read_bits(refine + n * (cols * r / 8), k * r, r);
    }
    v = fmaf(s, (float)((hi << r) | lo), z);
  }
  out[idx] = v;
}

bool fmt_ok(const sf_qfmt& f) {
  return f.b >= 1 && f.r >= 0 && f.b + f.r <= 8 && f.group == 128;
}

}  // namespace

extern "C" sf_status sf_quantize_nested(const float* x, int64_t rows, int64_t cols, sf_qfmt fmt,
                                        int32_t refine_layout, uint8_t* resident, uint32_t* sz,
                                        uint8_t* refine, sf_stream stream) {
  SF_REQUIRE(fmt_ok(fmt), SF_EUNSUPPORTED, "need 1<=b, 0<=r, b+r<=8, group 128");
  SF_REQUIRE(x && resident && sz, SF_EINVAL, "null tensor");
  SF_REQUIRE(rows > 0 && cols > 0 && cols % 128 == 0, SF_EINVAL, "cols must be a positive multiple of 128");
  SF_REQUIRE(refine_layout == SF_REFINE_CHANNEL_MAJOR || refine_layout == SF_REFINE_ROW_MAJOR,
             SF_EINVAL, "bad refine_layout");
  const bool want_ref = refine != nullptr && fmt.r > 0;
  if (want_ref && refine_layout == SF_REFINE_CHANNEL_MAJOR)
    SF_REQUIRE((rows * fmt.r) % 32 == 0, SF_EINVAL, "channel-major refinement needs rows*r % 32 == 0");
  hipStream_t s = (hipStream_t)stream;
  const int64_t groups = rows * (cols / 128);
  const int64_t blocks = (groups + 3) / 4;
  uint8_t* row_ref = (want_ref && refine_layout == SF_REFINE_ROW_MAJOR) ? refine : nullptr;
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, rows, cols,
                     fmt.b, fmt.r, resident, sz, row_ref);
  SF_LAUNCH_CHECK();
  if (want_ref && refine_layout == SF_REFINE_CHANNEL_MAJOR) {
    const int64_t threads = cols * (rows * fmt.r / 32);
    hipLaunchKernelGGL(refine_channel_major_kernel, dim3((unsigned)((threads + 255) / 256)),
                       dim3(256), 0, s, x, rows, cols, fmt.b, fmt.r, (const uint32_t*)sz, refine);
    SF_LAUNCH_CHECK();
  }
  return SF_OK;
}

extern "C" sf_status sf_debug_dequantize(const uint8_t* resident, const uint32_t* sz,
                                         const uint8_t* refine, int64_t rows, int64_t cols,
                                         sf_qfmt fmt, int32_t refine_layout, int32_t which,
                                         float* out, sf_stream stream) {
  SF_REQUIRE(fmt_ok(fmt), SF_EUNSUPPORTED, "bad format");
  SF_REQUIRE(resident && sz && out, SF_EINVAL, "null tensor");
  SF_REQUIRE(rows > 0 && cols > 0 && cols % 128 == 0, SF_EINVAL, "bad shape");
  SF_REQUIRE(which == 0 || which == 1, SF_EINVAL, "which must be 0 or 1");
  SF_REQUIRE(which == 0 || fmt.r == 0 || refine, SF_EINVAL, "full value needs refine");
  const int64_t n = rows * cols;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, resident, sz, refine, rows, cols, fmt.b, fmt.r,
                     refine_layout, which, out);
  SF_LAUNCH_CHECK();
  return SF_OK;
}

extern "C" sf_status sf_kv_append(const float* k_new, const float* v_new, int32_t n_tok,
                                  int32_t t0, const sf_qkv* kv, uint8_t* refine_out,
                                  int64_t refine_ld, sf_stream stream) {
  SF_REQUIRE(kv && k_new && v_new, SF_EINVAL, "null argument");
  SF_REQUIRE(fmt_ok(kv->fmt), SF_EUNSUPPORTED, "bad format");
  SF_REQUIRE(kv->head_dim == 128, SF_EUNSUPPORTED, "head_dim must be 128");
  SF_REQUIRE(kv->k_res && kv->k_sz && kv->v_res && kv->v_sz, SF_EINVAL, "null cache tensor");
  SF_REQUIRE(n_tok >= 0 && t0 >= 0 && (int64_t)t0 + n_tok <= kv->t_cap, SF_EINVAL,
             "positions beyond t_cap");
  SF_REQUIRE(kv->batch > 0 && kv->n_kv_heads > 0, SF_EINVAL, "bad shape");
  SF_REQUIRE(refine_out == nullptr || refine_ld >= n_tok, SF_EINVAL, "refine_ld must be >= n_tok");
  if (n_tok == 0) return SF_OK;
  const int64_t waves = (int64_t)kv->batch * kv->n_kv_heads * n_tok * 2;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                     (hipStream_t)stream, k_new, v_new, kv->batch, kv->n_kv_heads, n_tok, t0,
                     kv->t_cap, kv->fmt.b, kv->fmt.r, kv->k_res, kv->k_sz, kv->v_res, kv->v_sz,
                     refine_out, (int64_t)refine_ld);
  SF_LAUNCH_CHECK();
  return SF_OK;
}
