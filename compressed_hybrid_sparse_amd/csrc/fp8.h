// FP8 E4M3 storage written by the library: the per-row quantisation shared by chs_quantize_e4m3,
// chs_compress_fp8 and chs_append_fp8.
//
// Source: "DeepSeek-V4 本地部署，SGLang 把活做絕了", V4 到底改了啥 (the checkpoints keep attention in
// FP8) and "SGLang 如何为 DeepSeek V4 打造「Day-0」推理加速", 4.3 部署配置建议 (an fp8 KV cache). The
// pages fix no format, rounding or scale rule. Reading taken: OCP 8-bit E4M3 (bias 7, exponent 0
// subnormal, S.1111.111 NaN, no infinities) with one fp32 scale per row,
//   scale = amax / 448,   inv = min(448 / amax, FLT_MAX),   code_c = E4M3(x_c * inv),
// amax the row's largest magnitude, every operation rounded once to fp32 (IEEE division, which HIP
// compiles fp32 `/` to by default, twice per row; one multiply per element), E4M3() the nearest
// value with ties to the even code, magnitudes above 448 saturating to 448. A row of zeros has scale
// 0 and codes 0x00. Row r then decodes as scale_r * decode(code), which the FP8 readers
// (chs_index_topk_fp8, chs_decode_attn_fp8) take.
#pragma once

#include "common.h"

namespace chs {
namespace {

// E4M3 code of an fp32 value, from its bits: the sign is kept (zeros included); below 2^-6 the
// result is subnormal, round(|y| * 2^9) (exact scaling, then round half to even); above, the
// exponent is rebiased and the 23-bit mantissa rounded to 3 bits, half to even, a carry moving
// into the exponent; from 464 (the tie between 448 and the missing 480) up the magnitude is 448.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x43E80000u) {                              // |y| >= 464
    code = 0x7Eu;
  } else if (a < 0x3C800000u) {                        // |y| < 2^-6
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  } else {
    const uint32_t e = (a >> 23) - 120u;               // E4M3 biased exponent: e32 - 127 + 7
    const uint32_t mant = a & 0x7FFFFFu;
    const uint32_t q = mant >> 20, rem = mant & 0xFFFFFu;
    const uint32_t up = (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ? 1u : 0u;
    code = min((e << 3) + q + up, 0x7Eu);              // [448, 464) rounds to 448
  }
  return sign | code;
}

// Maximum over each group of G adjacent lanes (G a power of two, at most 64, the same in every
// lane); every lane of a group gets it.
__device__ __forceinline__ float group_max(float v, int G) {
  for (int o = 1; o < G; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// The stored row scale, and the factor that maps the row onto the E4M3 range, for a row maximum amax.
__device__ __forceinline__ float e4m3_scale(float amax) { return amax / 448.0f; }
__device__ __forceinline__ float e4m3_inv(float amax) { return fminf(448.0f / amax, 3.40282347e38f); }

// N (4 or 8) values of a row with row maximum amax into N codes, packed little-endian into N / 4
// words.
template <int N>
__device__ __forceinline__ void e4m3_pack(const float* v, float amax, uint32_t* w) {
  const float inv = e4m3_inv(amax);
#pragma unroll
  for (int k = 0; k < N / 4; ++k) {
    uint32_t r = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) r |= (amax == 0.f ? 0u : e4m3_encode(v[4 * k + j] * inv)) << (8 * j);
    w[k] = r;
  }
}

// Stores the N codes of e4m3_pack (N / 4 words) at p, which is N-byte aligned.
template <int N>
__device__ __forceinline__ void e4m3_store(uint8_t* p, const uint32_t* w) {
  if (N == 8) *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
  else *reinterpret_cast<uint32_t*>(p) = w[0];
}

}  // namespace
}  // namespace chs
