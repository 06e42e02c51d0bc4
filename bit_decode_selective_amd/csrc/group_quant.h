// One group of 128 values quantised by one wave into the nested format: fp16
// offset z = fp16(min) and step s = fp16((max - min) / Q), each one round-to-nearest-
// even of the fp64 value; c = clamp(rint((x - z) / s), 0, Q) in fp64; resident =
// c >> r, refinement = c & (2^r - 1); LSB-first bit streams.  Every code decision
// is an IEEE-exact fp64 operation, so any IEEE fp64 implementation of the formula
// reproduces the codes bit for bit.  Shared by the quantiser and KV append kernels
// and by the attention split pass that appends the new token itself.
#pragma once

#include "sf_internal.h"

namespace sfq {

// Correctly rounded (nearest-even) fp64 -> fp16 conversion, bit pattern result.
// Done with integer arithmetic so there is no intermediate fp32 rounding.
__device__ inline uint32_t f64_to_f16_rne(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t sign = (uint32_t)(u >> 63) << 15;
  const int ex = (int)((u >> 52) & 0x7FF);
  const uint64_t mant = u & 0xFFFFFFFFFFFFFull;
  if (ex == 0x7FF) return sign | 0x7C00u | (mant ? 0x200u : 0u);
  if (ex == 0) return sign;  // zero, or an fp64 subnormal (far below fp16's range)
  const int e = ex - 1023;
  if (e > 15) return sign | 0x7C00u;
  const uint64_t m = mant | (1ull << 52);
  // fp16 quantum is 2^(max(e,-14) - 10); m carries 2^(e - 52).
  const int shift = (e >= -14) ? 42 : 42 + (-14 - e);
  if (shift > 63) return sign;
  uint64_t q = m >> shift;
  const uint64_t rem = m & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  uint32_t bits = (e >= -14) ? (uint32_t)(((e + 14) << 10) + q) : (uint32_t)q;
  if (bits >= 0x7C00u) bits = 0x7C00u;
  return sign | bits;
}

__device__ __forceinline__ double h2d(uint32_t bits16) { return (double)sf_h2f(bits16); }

__device__ __forceinline__ uint32_t code_of(float x, double z, double s, uint32_t s16, int Q) {
  if ((s16 & 0x7FFFu) == 0) return 0;
  double t = __builtin_rint(((double)x - z) / s);
  if (t < 0.0) t = 0.0;
  if (t > (double)Q) t = (double)Q;
  return (uint32_t)t;
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Builds stream word w (0 <= w < 4*W) of a 128-code group of W-bit codes in LDS.
template <int W>
__device__ __forceinline__ uint32_t stream_word_t(const uint8_t* codes, int w) {
  uint32_t word = 0;
#pragma unroll
  for (int p = 0; p < 32; ++p) {
    const int P = 32 * w + p;
    const int i = P / W, j = P % W;
    word |= (uint32_t)((codes[i] >> j) & 1u) << p;
  }
  return word;
}

__device__ __forceinline__ uint32_t stream_word(const uint8_t* codes, int width, int w) {
  switch (width) {
    case 1: return stream_word_t<1>(codes, w);
    case 2: return stream_word_t<2>(codes, w);
    case 3: return stream_word_t<3>(codes, w);
    case 4: return stream_word_t<4>(codes, w);
    case 5: return stream_word_t<5>(codes, w);
    case 6: return stream_word_t<6>(codes, w);
    case 7: return stream_word_t<7>(codes, w);
    default: return stream_word_t<8>(codes, w);
  }
}

// One wave quantises one group of 128 fp32 values at `src`.  Writes the group's
// 4*b resident words, its sz word, and (if ref_dst) its 4*r refinement words.
// res_lds / sz_lds (LDS, may be null): a copy of the resident words and the sz word
// for the workgroup's own use.
__device__ inline void quantize_group_wave(const float* src, int b, int r, uint8_t* lds_hi,
                                           uint8_t* lds_lo, uint32_t* res_dst, uint32_t* sz_dst,
                                           uint32_t* ref_dst, uint32_t* res_lds = nullptr,
                                           uint32_t* sz_lds = nullptr) {
  const int lane = threadIdx.x & 63;
  const float v0 = src[lane], v1 = src[lane + 64];
  const float mn = wave_min(fminf(v0, v1));
  const float mx = wave_max(fmaxf(v0, v1));
  const int Q = (1 << (b + r)) - 1;
  const uint32_t z16 = f64_to_f16_rne((double)mn);
  const uint32_t s16 = f64_to_f16_rne(((double)mx - (double)mn) / (double)Q);
  const double z = h2d(z16), s = h2d(s16);
  const uint32_t c0 = code_of(v0, z, s, s16, Q), c1 = code_of(v1, z, s, s16, Q);
  const uint32_t lo_mask = (1u << r) - 1u;
  lds_hi[lane] = (uint8_t)(c0 >> r);
  lds_hi[lane + 64] = (uint8_t)(c1 >> r);
  lds_lo[lane] = (uint8_t)(c0 & lo_mask);
  lds_lo[lane + 64] = (uint8_t)(c1 & lo_mask);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  if (lane < 4 * b) {
    const uint32_t w = stream_word(lds_hi, b, lane);
    res_dst[lane] = w;
    if (res_lds) res_lds[lane] = w;
  }
  if (ref_dst && r > 0 && lane >= 32 && lane - 32 < 4 * r)
    ref_dst[lane - 32] = stream_word(lds_lo, r, lane - 32);
  if (lane == 0) {
    *sz_dst = s16 | (z16 << 16);
    if (sz_lds) *sz_lds = s16 | (z16 << 16);
  }
  __builtin_amdgcn_wave_barrier();
}

}  // namespace sfq
