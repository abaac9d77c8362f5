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
// words. E4M3() is gfx950's conversion (v_cvt_pk_fp8_f32: OCP E4M3, round to nearest even, the sign
// kept on zeros, two values per instruction). The scaled values never exceed 448 by more than the
// rounding of one product, so no input reaches the overflow point (464) where the instruction's
// result and the saturating rule would part.
template <int N>
__device__ __forceinline__ void e4m3_pack(const float* v, float amax, uint32_t* w) {
  const float inv = e4m3_inv(amax);
#pragma unroll
  for (int k = 0; k < N / 4; ++k) {
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * k] * inv, v[4 * k + 1] * inv, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * k + 2] * inv, v[4 * k + 3] * inv, r, true);
    w[k] = amax == 0.f ? 0u : (uint32_t)r;
  }
}

// Stores the N codes of e4m3_pack (N / 4 words) at p, which is N-byte aligned. NT: non-temporal,
// for a pass that streams its inputs (the compressor: 430 -> 408 us at 1M tokens; the row
// quantiser measured 26.4 us plain against 26.9 us non-temporal, so it stores plainly).
template <int N, bool NT = false>
__device__ __forceinline__ void e4m3_store(uint8_t* p, const uint32_t* w) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  if (N == 8) {
    const u32x2 v{w[0], w[1]};
    if (NT) __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
    else *reinterpret_cast<u32x2*>(p) = v;
  } else {
    if (NT) __builtin_nontemporal_store(w[0], reinterpret_cast<uint32_t*>(p));
    else *reinterpret_cast<uint32_t*>(p) = w[0];
  }
}

}  // namespace
}  // namespace chs
