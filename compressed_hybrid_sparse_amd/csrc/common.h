// Internal helpers shared by the libchs kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "chs.h"

namespace chs {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// bfloat16 <-> fp32. A bf16 value is the high half of an fp32 bit pattern.
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }
// Round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// 2^x on the transcendental unit (v_exp_f32). Results below the normal range flush to zero,
// which only drops weights that are negligible next to the running maximum's weight of 1.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

inline size_t elem_size(chs_dtype dt) { return dt == CHS_BF16 ? 2 : 4; }
inline bool dtype_ok(int dt) { return dt == CHS_F32 || dt == CHS_BF16; }

inline chs_status launch_status() {
  return hipGetLastError() == hipSuccess ? CHS_OK : CHS_ERR_LAUNCH;
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace chs
