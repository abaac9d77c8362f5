// chs_quantize_e4m3: rows the caller holds (bf16 or fp32) into E4M3 codes with one fp32 scale per
// row, the rule of fp8.h. It fills the FP8 cache where the rows do not come out of the compressor:
// the window rows of a prefill, index keys produced elsewhere.
//
// Source: "DeepSeek-V4 本地部署，SGLang 把活做絕了", V4 到底改了啥 (attention kept in FP8);
// "SGLang 如何为 DeepSeek V4 打造「Day-0」推理加速", 4.3 部署配置建议 (an fp8 KV cache).
//
// gfx950 design: a streaming pass (read 2 or 4 bytes, write 1 byte per element, plus 4 bytes per
// row), bound by HBM. Each lane owns chunks of 8 consecutive elements (one 16-byte bf16 load, or
// two fp32 loads); the G lanes of a row (G = the row's chunk count rounded up to a power of two, at
// most 64) are adjacent, so the row maximum is a cross-lane reduction with no LDS and no barrier,
// and a lane keeps its values in registers between the maximum and the encoding (at most 8 chunks,
// d <= 4096).
#include "fp8.h"

namespace chs {
namespace {

constexpr int kQThreads = 256;
constexpr int kQMaxChunks = 8;   // chunks of 8 elements per lane (d <= 4096)

template <typename ET>
__device__ __forceinline__ void load8(const ET* p, float* v);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* v) {
  const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
  for (int j = 0; j < 4; ++j) { v[2 * j] = bf16_lo(r[j]); v[2 * j + 1] = bf16_hi(r[j]); }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
  const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1);
#pragma unroll
  for (int j = 0; j < 4; ++j) { v[j] = a[j]; v[4 + j] = b[j]; }
}

// Grid: (ceil(n / rows per block)). A group of G lanes serves RPG rows (RPG * cpl <= 8 chunks per
// lane, every load issued before the first is used): lane l of wave w serves rows
// ((4 * block + w) * (64 / G) + l / G) * RPG + k (k < RPG) and, in each, its chunks l % G + i * G (i < cpl).
template <typename ET>
__global__ __launch_bounds__(kQThreads) void quantize_kernel(int64_t n, int32_t d, int32_t G, int32_t cpl,
                                                             int32_t rpg, const ET* __restrict__ in,
                                                             uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row0 = (((int64_t)blockIdx.x * (kQThreads / 64) + wave) * (64 / G) + lane / G) * rpg;
  if (row0 >= n) return;                                // the G lanes of a row group leave together
  const int cpr = d / 8, c0 = lane % G;
  // Slot q = k * cpl + i: row row0 + k, chunk c0 + i * G.
  float v[kQMaxChunks][8];
#pragma unroll
  for (int q = 0; q < kQMaxChunks; ++q) {
    const int k = q / cpl, i = q - k * cpl, c = c0 + i * G;
    if (k < rpg && row0 + k < n && c < cpr) load8<ET>(in + (row0 + k) * d + c * 8, v[q]);
  }
  float am[kQMaxChunks];
#pragma unroll
  for (int k = 0; k < kQMaxChunks; ++k) am[k] = 0.f;
#pragma unroll
  for (int q = 0; q < kQMaxChunks; ++q) {
    const int k = q / cpl, i = q - k * cpl, c = c0 + i * G;
    if (k < rpg && row0 + k < n && c < cpr)
#pragma unroll
      for (int j = 0; j < 8; ++j) am[k] = fmaxf(am[k], fabsf(v[q][j]));
  }
#pragma unroll
  for (int k = 0; k < kQMaxChunks; ++k)
    if (k < rpg) am[k] = group_max(am[k], G);
#pragma unroll
  for (int q = 0; q < kQMaxChunks; ++q) {
    const int k = q / cpl, i = q - k * cpl, c = c0 + i * G;
    if (k < rpg && row0 + k < n && c < cpr) {
      uint32_t w[2];
      e4m3_pack<8>(v[q], am[k], w);
      e4m3_store<8>(codes + (row0 + k) * d + c * 8, w);
    }
  }
#pragma unroll
  for (int k = 0; k < kQMaxChunks; ++k)                // row k's scale from lane k mod G of the group
    if (k < rpg && (k & (G - 1)) == c0 && row0 + k < n) scales[row0 + k] = e4m3_scale(am[k]);
}

}  // namespace
}  // namespace chs

extern "C" chs_status chs_quantize_e4m3(chs_dtype dtype, int64_t n_rows, int32_t d, const void* in, uint8_t* codes,
                                        float* scales, void* stream) {
  using namespace chs;
  if (!dtype_ok(dtype)) return CHS_ERR_DTYPE;
  if (n_rows < 0 || n_rows > ((int64_t)1 << 40) || d < 8 || d > 4096 || d % 8 != 0) return CHS_ERR_SHAPE;
  if (n_rows == 0) return CHS_OK;
  if (!in || !codes || !scales) return CHS_ERR_NULL;
  const int cpr = d / 8;
  int G = 1;
  while (G < cpr && G < 64) G *= 2;
  const int cpl = (cpr + G - 1) / G;
  const int rpg = kQMaxChunks / cpl;                    // rows per lane group
  const int64_t rows_per_block = (int64_t)(kQThreads / 64) * (64 / G) * rpg;
  const int64_t blocks = (n_rows + rows_per_block - 1) / rows_per_block;
  if (blocks > 0x7FFFFFFF) return CHS_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == CHS_BF16)
    hipLaunchKernelGGL(quantize_kernel<uint16_t>, dim3((unsigned)blocks), dim3(kQThreads), 0, s, n_rows, d, G, cpl,
                       rpg, static_cast<const uint16_t*>(in), codes, scales);
  else
    hipLaunchKernelGGL(quantize_kernel<float>, dim3((unsigned)blocks), dim3(kQThreads), 0, s, n_rows, d, G, cpl,
                       rpg, static_cast<const float*>(in), codes, scales);
  return launch_status();
}
