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
// Rows (one chunk each) a lane loads at once in quantize_rows_kernel: on 262,144 x 128 bf16 rows 8
// measured 26.4 us per call, 4 26.6 us, 2 28.3 us.
constexpr int kQRows = 8;

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

// d = 8 G exactly (G = 8, 16, 32 or 64: d = 64, 128, 256, 512), the common case, with compile-time
// shapes: a row is G adjacent lanes, one 16-byte chunk each; wave w of block b serves the 8 (64 / G)
// consecutive rows from ((4 b + w) 8 (64 / G)), load k of lane l reading row k (64 / G) + l / G, so
// every load instruction covers 64 / G whole consecutive rows (1 KiB of bf16). All 8 loads are issued
// unconditionally (rows past n read row n - 1) before the first is used; stores are guarded. The
// arithmetic is the general kernel's, so the codes and scales are the same.
template <typename ET, int G>
__global__ __launch_bounds__(kQThreads) void quantize_rows_kernel(int64_t n, const ET* __restrict__ in,
                                                                  uint8_t* __restrict__ codes,
                                                                  float* __restrict__ scales) {
  constexpr int RPI = 64 / G;                           // rows per load instruction
  constexpr int D = 8 * G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane % G, rl = lane / G;
  const int64_t base = ((int64_t)blockIdx.x * (kQThreads / 64) + wave) * (kQRows * RPI);
  if (base >= n) return;
  float v[kQRows][8];
#pragma unroll
  for (int k = 0; k < kQRows; ++k) {
    const int64_t row = min(base + k * RPI + rl, n - 1);
    load8<ET>(in + row * D + c * 8, v[k]);
  }
  float am[kQRows];
#pragma unroll
  for (int k = 0; k < kQRows; ++k) {
    am[k] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) am[k] = fmaxf(am[k], fabsf(v[k][j]));
    am[k] = group_max(am[k], G);
  }
#pragma unroll
  for (int k = 0; k < kQRows; ++k) {
    const int64_t row = base + k * RPI + rl;
    uint32_t w[2];
    e4m3_pack<8>(v[k], am[k], w);
    if (row < n) e4m3_store<8>(codes + row * D + c * 8, w);
  }
  // Row k * RPI + rl's scale from lane c == k of its row (G >= 8).
  float sc = 0.f;
#pragma unroll
  for (int k = 0; k < kQRows; ++k) sc = c == k ? e4m3_scale(am[k]) : sc;
  const int64_t srow = base + (int64_t)c * RPI + rl;
  if (c < kQRows && srow < n) scales[srow] = sc;
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
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (cpr == 8 || cpr == 16 || cpr == 32 || cpr == 64) {
    const int64_t rows_per_block = (int64_t)(kQThreads / 64) * kQRows * (64 / cpr);
    const int64_t blocks = (n_rows + rows_per_block - 1) / rows_per_block;
    if (blocks > 0x7FFFFFFF) return CHS_ERR_SHAPE;
    auto go = [&](auto kern, const auto* src) {
      hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kQThreads), 0, s, n_rows, src, codes, scales);
    };
    const uint16_t* hb = static_cast<const uint16_t*>(in);
    const float* hf = static_cast<const float*>(in);
    switch (cpr) {
      case 8: dtype == CHS_BF16 ? go(quantize_rows_kernel<uint16_t, 8>, hb) : go(quantize_rows_kernel<float, 8>, hf); break;
      case 16: dtype == CHS_BF16 ? go(quantize_rows_kernel<uint16_t, 16>, hb) : go(quantize_rows_kernel<float, 16>, hf); break;
      case 32: dtype == CHS_BF16 ? go(quantize_rows_kernel<uint16_t, 32>, hb) : go(quantize_rows_kernel<float, 32>, hf); break;
      default: dtype == CHS_BF16 ? go(quantize_rows_kernel<uint16_t, 64>, hb) : go(quantize_rows_kernel<float, 64>, hf); break;
    }
    return launch_status();
  }
  int G = 1;
  while (G < cpr && G < 64) G *= 2;
  const int cpl = (cpr + G - 1) / G;
  const int rpg = kQMaxChunks / cpl;                    // rows per lane group
  const int64_t rows_per_block = (int64_t)(kQThreads / 64) * (64 / G) * rpg;
  const int64_t blocks = (n_rows + rows_per_block - 1) / rows_per_block;
  if (blocks > 0x7FFFFFFF) return CHS_ERR_SHAPE;
  if (dtype == CHS_BF16)
    hipLaunchKernelGGL(quantize_kernel<uint16_t>, dim3((unsigned)blocks), dim3(kQThreads), 0, s, n_rows, d, G, cpl,
                       rpg, static_cast<const uint16_t*>(in), codes, scales);
  else
    hipLaunchKernelGGL(quantize_kernel<float>, dim3((unsigned)blocks), dim3(kQThreads), 0, s, n_rows, d, G, cpl,
                       rpg, static_cast<const float*>(in), codes, scales);
  return launch_status();
}
