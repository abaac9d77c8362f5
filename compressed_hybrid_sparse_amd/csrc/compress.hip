// chs_compress: the fused group softmax-pool, one HBM pass.
//
// Source: "SGLang 如何为 DeepSeek V4 打造「Day-0」推理加速", 创新 2 (Flash Compressor): the
// naive pipeline makes a round trip to HBM per stage (load tokens, score, softmax, weighted
// sum, store); fusing the stages leaves one read of the tokens and gates and one write of the
// compressed entry. "DeepSeek-V4 本地部署，SGLang 把活做絕了", V4 到底改了啥: C4 pools 4 tokens,
// C128 pools 128.
//
// gfx950 design. The work is a streaming reduction (about 4 flop per byte), so it is bound by
// HBM, not by MFMA. Each thread owns one 16-byte column chunk (8 bf16 or 4 fp32 channels) of
// one group and walks the group's rows, so the per-channel softmax needs no cross-lane
// reduction at all; adjacent threads own adjacent chunks of the same row, so every row load of
// a wave is one contiguous, fully coalesced 1 KiB (d = 512, bf16). Tokens and gates are read
// once with non-temporal loads (they are not reused); the bias rows stay in cache. Small groups
// (m <= 8) keep every row in registers and take the max, the exponentials and the weighted sum
// in one shot; larger groups (C128) stream 8 rows at a time with a running maximum
// (online softmax), so registers stay bounded for any m.
#include "common.h"

namespace chs {
namespace {

template <typename ET>
struct Vec16;

template <>
struct Vec16<uint16_t> {  // 8 bf16 channels
  static constexpr int N = 8;
  __device__ static void load(const uint16_t* p, float* v) {
    u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
    for (int j = 0; j < 4; ++j) { v[2 * j] = bf16_lo(r[j]); v[2 * j + 1] = bf16_hi(r[j]); }
  }
  __device__ static void store(uint16_t* p, const float* v) {
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
    *reinterpret_cast<u32x4*>(p) = r;
  }
};

template <>
struct Vec16<float> {  // 4 fp32 channels
  static constexpr int N = 4;
  __device__ static void load(const float* p, float* v) {
    f32x4 r = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = r[j];
  }
  __device__ static void store(float* p, const float* v) {
    f32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = v[j];
    *reinterpret_cast<f32x4*>(p) = r;
  }
};

__device__ __forceinline__ void load_bias(const float* p, float* v, int n) {
#pragma unroll
  for (int j = 0; j < 8; j += 4) {
    if (j < n) {
      f32x4 r = *reinterpret_cast<const f32x4*>(p + j);
      v[j] = r[0]; v[j + 1] = r[1]; v[j + 2] = r[2]; v[j + 3] = r[3];
    }
  }
}

// One (group, 16-byte channel chunk) item: M > 0 is a compile-time group size (<= 8); M == 0
// takes any m, streamed in chunks of 8 rows with a running maximum.
template <typename ET, int M>
__device__ __forceinline__ void compress_item(int32_t d, int32_t m, const ET* __restrict__ xp,
                                              const ET* __restrict__ zp, const float* __restrict__ bp,
                                              ET* __restrict__ op) {
  using V = Vec16<ET>;
  constexpr int N = V::N;
  constexpr int R = M > 0 ? M : 8;
  float mx[N], sum[N], acc[N];
#pragma unroll
  for (int j = 0; j < N; ++j) { mx[j] = -INFINITY; sum[j] = 0.f; acc[j] = 0.f; }

  for (int r0 = 0; r0 < m; r0 += R) {
    const int nr = (M > 0) ? R : min(R, m - r0);
    float xv[R][N], av[R][N];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r < nr) {
        V::load(xp + (int64_t)(r0 + r) * d, xv[r]);
        V::load(zp + (int64_t)(r0 + r) * d, av[r]);
      }
    }
    float cmax[N];
#pragma unroll
    for (int j = 0; j < N; ++j) cmax[j] = -INFINITY;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r < nr) {
        float bv[8];
        load_bias(bp + (int64_t)(r0 + r) * d, bv, N);
#pragma unroll
        for (int j = 0; j < N; ++j) {
          av[r][j] = (av[r][j] + bv[j]) * kLog2e;   // logit in base-2 units
          cmax[j] = fmaxf(cmax[j], av[r][j]);
        }
      }
    }
    if (M == 0) {
      // Online softmax: rescale what was accumulated under the previous maximum.
#pragma unroll
      for (int j = 0; j < N; ++j) {
        const float nm = fmaxf(mx[j], cmax[j]);
        const float sc = fast_exp2(mx[j] - nm);
        sum[j] *= sc;
        acc[j] *= sc;
        mx[j] = nm;
      }
    } else {
#pragma unroll
      for (int j = 0; j < N; ++j) mx[j] = cmax[j];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r < nr) {
#pragma unroll
        for (int j = 0; j < N; ++j) {
          const float e = fast_exp2(av[r][j] - mx[j]);
          sum[j] += e;
          acc[j] = fmaf(e, xv[r][j], acc[j]);
        }
      }
    }
  }
  float o[N];
#pragma unroll
  for (int j = 0; j < N; ++j) o[j] = acc[j] / sum[j];
  V::store(op, o);
}

// Grid: (x: items of the longest sequence, y: sequence). A launch holds fewer than 2^32
// work-items per grid dimension, so the x dimension strides over the sequence's items.
template <typename ET, int M>
__global__ __launch_bounds__(256) void compress_kernel(int32_t d, int32_t m, const ET* __restrict__ x,
                                                       const ET* __restrict__ gate,
                                                       const float* __restrict__ bias,
                                                       const int64_t* __restrict__ cu_tokens,
                                                       const int64_t* __restrict__ cu_groups,
                                                       int64_t max_groups, ET* __restrict__ out) {
  constexpr int N = Vec16<ET>::N;
  const int cpr = d / N;
  const int b = blockIdx.y;
  const int64_t t0 = cu_tokens[b];
  int64_t n_groups = (cu_tokens[b + 1] - t0) / m;
  const int64_t o0 = cu_groups[b];
  const int64_t room = cu_groups[b + 1] - o0;
  if (room < n_groups) n_groups = room;
  if (n_groups > max_groups) n_groups = max_groups;
  for (int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; item < n_groups * cpr;
       item += (int64_t)gridDim.x * blockDim.x) {
    const int64_t g = item / cpr;
    const int64_t col = (item - g * cpr) * N;
    const int64_t row = t0 + g * m;
    compress_item<ET, M>(d, m, x + row * d + col, gate + row * d + col, bias + col,
                         out + (o0 + g) * d + col);
  }
}

template <typename ET>
chs_status launch(int32_t batch, int32_t d, int32_t m, const void* x, const void* gate,
                  const float* bias, const int64_t* cu_tokens, const int64_t* cu_groups,
                  int64_t max_groups, void* out, hipStream_t stream) {
  const int cpr = d / Vec16<ET>::N;
  const int64_t items = max_groups * cpr;
  int64_t blocks = (items + 255) / 256;
  if (blocks > (1 << 22)) blocks = 1 << 22;   // grid-stride beyond 2^30 work-items
  dim3 grid((unsigned)blocks, (unsigned)batch), block(256);
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, stream, d, m, static_cast<const ET*>(x),
                       static_cast<const ET*>(gate), bias, cu_tokens, cu_groups, max_groups,
                       static_cast<ET*>(out));
  };
  switch (m) {
    case 1: args(compress_kernel<ET, 1>); break;
    case 2: args(compress_kernel<ET, 2>); break;
    case 4: args(compress_kernel<ET, 4>); break;
    case 8: args(compress_kernel<ET, 8>); break;
    default: args(compress_kernel<ET, 0>); break;
  }
  return launch_status();
}

}  // namespace
}  // namespace chs

extern "C" chs_status chs_compress(chs_dtype dtype, int32_t batch, int32_t d, int32_t m,
                                   const void* x, const void* gate, const float* bias,
                                   const int64_t* cu_tokens, const int64_t* cu_groups,
                                   int64_t max_groups, void* out, void* stream) {
  using namespace chs;
  if (!dtype_ok(dtype)) return CHS_ERR_DTYPE;
  if (batch < 1 || batch > 65535 || m < 1 || m > 1024 || d < 1 || d > 4096 || max_groups < 0)
    return CHS_ERR_SHAPE;
  if ((d * elem_size(dtype)) % 16 != 0) return CHS_ERR_SHAPE;
  if (!x || !gate || !bias || !cu_tokens || !cu_groups || !out) return CHS_ERR_NULL;
  if (max_groups == 0) return CHS_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return dtype == CHS_BF16
             ? launch<uint16_t>(batch, d, m, x, gate, bias, cu_tokens, cu_groups, max_groups, out, s)
             : launch<float>(batch, d, m, x, gate, bias, cu_tokens, cu_groups, max_groups, out, s);
}
