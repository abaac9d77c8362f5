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
// in one shot; larger groups (C128) stream 4 rows at a time with a running maximum
// (online softmax), so registers stay bounded for any m, with the next 4 rows in flight; up to
// d = 512 a workgroup stages each block's bias rows once in LDS for all its groups.
//
// chs_compress_fp8 is the same pass with E4M3 output: the pooled fp32 values of a group's row are
// quantised in registers (the row maximum over the row's chunks by cross-lane moves, the threads of
// a row being adjacent lanes of one wave), and the row is stored as 1-byte codes plus one fp32
// scale, so the pass still reads the tokens and gates once and writes each entry once.
#include "fp8.h"
#include "pool.h"

namespace chs {
namespace {

// Output of one entry chunk: the storage type (FP8 false) or E4M3 codes plus the row's scale (FP8
// true; the cpr threads of a row, cpr a power of two <= 64, are adjacent lanes and all call it).
template <typename ET, bool FP8>
__device__ __forceinline__ void store_entry(const float* o, int cpr, int64_t row, int64_t col, int32_t d, ET* out,
                                            uint8_t* codes, float* scales, bool store) {
  constexpr int N = Vec16<ET>::N;
  if (FP8) {
    float am = 0.f;
#pragma unroll
    for (int j = 0; j < N; ++j) am = fmaxf(am, fabsf(o[j]));
    am = group_max(am, cpr);
    const float sc = e4m3_scale(am);
    uint32_t w[N / 4];
    e4m3_pack<N>(o, am, w);
    if (store) {
      e4m3_store<N, true>(codes + row * d + col, w);
      if (col == 0) scales[row] = sc;
    }
  } else if (store) {
    Vec16<ET>::store(out + row * d + col, o);
  }
}

// Grid: (x: items of the longest sequence, y: sequence). A launch holds fewer than 2^32
// work-items per grid dimension, so the x dimension strides over the sequence's items.
template <typename ET, int M, bool FP8>
__global__ __launch_bounds__(256) void compress_kernel(int32_t d, int32_t m, const ET* __restrict__ x,
                                                       const ET* __restrict__ gate,
                                                       const float* __restrict__ bias,
                                                       const int64_t* __restrict__ cu_tokens,
                                                       const int64_t* __restrict__ cu_groups,
                                                       int64_t max_groups, ET* __restrict__ out,
                                                       uint8_t* __restrict__ codes, float* __restrict__ scales) {
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
    const ET* xp = x + row * d + col;
    const ET* zp = gate + row * d + col;
    const float* bp = bias + col;
    float o[N];
    pool_group_values<ET, M>(
        m, [&](int r) { return xp + (int64_t)r * d; }, [&](int r) { return zp + (int64_t)r * d; },
        [&](int r) { return bp + (int64_t)r * d; }, o);
    store_entry<ET, FP8>(o, cpr, o0 + g, col, d, out, codes, scales, true);
  }
}


// Groups of any m for d <= kStageMaxD: the same online softmax as pool_stream (blocks of 4 rows,
// the next block's rows in flight during the arithmetic), but the bias rows of a block are
// staged once per workgroup in LDS (two stages, the next block's bias requested with its rows)
// instead of being read by every thread from the cache: a bias row is the same for every group.
// The workgroup walks its items in lock step (every thread takes every barrier; a thread past
// the last item computes a clamped item and stores nothing).
constexpr int kStageRows = 4;
constexpr int kStageMaxD = 512;
constexpr int kStageVec = kStageRows * kStageMaxD / 4 / 256;   // bias f32x4 per thread and stage

template <typename ET, bool FP8>
__global__ __launch_bounds__(256) void compress_staged_kernel(int32_t d, int32_t m, const ET* __restrict__ x,
                                                              const ET* __restrict__ gate,
                                                              const float* __restrict__ bias,
                                                              const int64_t* __restrict__ cu_tokens,
                                                              const int64_t* __restrict__ cu_groups,
                                                              int64_t max_groups, ET* __restrict__ out,
                                                              uint8_t* __restrict__ codes, float* __restrict__ scales) {
  using V = Vec16<ET>;
  constexpr int N = V::N;
  constexpr int R = kStageRows;
  extern __shared__ f32x4 stage_lds[];   // [2][R * d / 4]
  const int tid = threadIdx.x;
  const int cpr = d / N;
  const int q4 = d / 4;                  // f32x4 per bias row
  const int nv = R * q4;                 // f32x4 per stage
  const int b = blockIdx.y;
  const int64_t t0 = cu_tokens[b];
  int64_t n_groups = (cu_tokens[b + 1] - t0) / m;
  const int64_t o0 = cu_groups[b];
  const int64_t room = cu_groups[b + 1] - o0;
  if (room < n_groups) n_groups = room;
  if (n_groups > max_groups) n_groups = max_groups;
  const int64_t total = n_groups * cpr;
  const f32x4* bias4 = reinterpret_cast<const f32x4*>(bias);
  // Stage slot i of block r0 holds bias row min(r0 + i / q4, m - 1), column quad i % q4.
  auto bias_src = [&](int r0, int i) { return bias4 + (int64_t)min(r0 + i / q4, m - 1) * q4 + i % q4; };
  for (int64_t base = (int64_t)blockIdx.x * 256; base < total; base += (int64_t)gridDim.x * 256) {
    const bool live = base + tid < total;
    const int64_t item = live ? base + tid : total - 1;
    const int64_t g = item / cpr;
    const int64_t col = (item - g * cpr) * N;
    const ET* xp = x + (t0 + g * m) * d + col;
    const ET* zp = gate + (t0 + g * m) * d + col;
    __syncthreads();   // the previous item's readers are done with both stages
#pragma unroll
    for (int k = 0; k < kStageVec; ++k) {
      const int i = tid + 256 * k;
      if (i < nv) stage_lds[i] = *bias_src(0, i);
    }
    u32x4 xc[R], zc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int rr = min(r, m - 1);
      xc[r] = V::load_raw(xp + (int64_t)rr * d);
      zc[r] = V::load_raw(zp + (int64_t)rr * d);
    }
    PoolState<N> st;
    st.init();
    int cur = 0;
    for (int r0 = 0; r0 < m; r0 += R) {
      const int nr = min(R, m - r0);
      u32x4 xn[R], zn[R];
      f32x4 bn[kStageVec];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int rr = min(r0 + R + r, m - 1);
        xn[r] = V::load_raw(xp + (int64_t)rr * d);
        zn[r] = V::load_raw(zp + (int64_t)rr * d);
      }
#pragma unroll
      for (int k = 0; k < kStageVec; ++k) {
        const int i = min(tid + 256 * k, nv - 1);
        bn[k] = *bias_src(r0 + R, i);
      }
      __syncthreads();   // stage cur is written
      const float* bl = reinterpret_cast<const float*>(stage_lds + cur * nv);
      float xv[R][N], av[R][N], cmax[N];
#pragma unroll
      for (int j = 0; j < N; ++j) cmax[j] = -INFINITY;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        V::unpack(xc[r], xv[r]);
        V::unpack(zc[r], av[r]);
        float bv[8];
        const float* brow = bl + r * d + col;
#pragma unroll
        for (int j = 0; j < N; j += 4) {
          const f32x4 t = *reinterpret_cast<const f32x4*>(brow + j);
          bv[j] = t[0]; bv[j + 1] = t[1]; bv[j + 2] = t[2]; bv[j + 3] = t[3];
        }
#pragma unroll
        for (int j = 0; j < N; ++j) {
          av[r][j] = r < nr ? (av[r][j] + bv[j]) * kLog2e : -INFINITY;
          cmax[j] = fmaxf(cmax[j], av[r][j]);
        }
      }
#pragma unroll
      for (int j = 0; j < N; ++j) {
        const float nm = fmaxf(st.mx[j], cmax[j]);
        const float sc = fast_exp2(st.mx[j] - nm);
        st.sum[j] *= sc;
        st.acc[j] *= sc;
        st.mx[j] = nm;
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (r < nr) {
#pragma unroll
          for (int j = 0; j < N; ++j) {
            const float e = fast_exp2(av[r][j] - st.mx[j]);
            st.sum[j] += e;
            st.acc[j] = fmaf(e, xv[r][j], st.acc[j]);
          }
        }
      }
      // The other stage was last read before this block's barrier: safe to overwrite.
#pragma unroll
      for (int k = 0; k < kStageVec; ++k) {
        const int i = tid + 256 * k;
        if (i < nv) stage_lds[(cur ^ 1) * nv + i] = bn[k];
      }
      cur ^= 1;
#pragma unroll
      for (int r = 0; r < R; ++r) { xc[r] = xn[r]; zc[r] = zn[r]; }
    }
    float o[N];
    pool_values<N>(st, o);
    store_entry<ET, FP8>(o, cpr, o0 + g, col, d, out, codes, scales, live);
  }
}

template <typename ET, bool FP8>
chs_status launch(int32_t batch, int32_t d, int32_t m, const void* x, const void* gate,
                  const float* bias, const int64_t* cu_tokens, const int64_t* cu_groups,
                  int64_t max_groups, void* out, uint8_t* codes, float* scales, hipStream_t stream) {
  const int cpr = d / Vec16<ET>::N;
  const int64_t items = max_groups * cpr;
  int64_t blocks = (items + 255) / 256;
  if (blocks > (1 << 22)) blocks = 1 << 22;   // grid-stride beyond 2^30 work-items
  dim3 grid((unsigned)blocks, (unsigned)batch), block(256);
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, stream, d, m, static_cast<const ET*>(x),
                       static_cast<const ET*>(gate), bias, cu_tokens, cu_groups, max_groups,
                       static_cast<ET*>(out), codes, scales);
  };
  switch (m) {
    case 1: args(compress_kernel<ET, 1, FP8>); break;
    case 2: args(compress_kernel<ET, 2, FP8>); break;
    case 4: args(compress_kernel<ET, 4, FP8>); break;
    case 8: args(compress_kernel<ET, 8, FP8>); break;
    default:
      if (d <= kStageMaxD) {
        const size_t lds = 2 * (size_t)kStageRows * d * sizeof(float);
        hipLaunchKernelGGL((compress_staged_kernel<ET, FP8>), grid, block, lds, stream, d, m,
                           static_cast<const ET*>(x), static_cast<const ET*>(gate), bias, cu_tokens, cu_groups,
                           max_groups, static_cast<ET*>(out), codes, scales);
      } else {
        args(compress_kernel<ET, 0, FP8>);
      }
      break;
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
             ? launch<uint16_t, false>(batch, d, m, x, gate, bias, cu_tokens, cu_groups, max_groups, out, nullptr,
                                       nullptr, s)
             : launch<float, false>(batch, d, m, x, gate, bias, cu_tokens, cu_groups, max_groups, out, nullptr,
                                    nullptr, s);
}

extern "C" chs_status chs_compress_fp8(chs_dtype dtype, int32_t batch, int32_t d, int32_t m, const void* x,
                                       const void* gate, const float* bias, const int64_t* cu_tokens,
                                       const int64_t* cu_groups, int64_t max_groups, uint8_t* out_codes,
                                       float* out_scales, void* stream) {
  using namespace chs;
  if (!dtype_ok(dtype)) return CHS_ERR_DTYPE;
  if (batch < 1 || batch > 65535 || m < 1 || m > 1024 || d < 1 || d > 4096 || max_groups < 0)
    return CHS_ERR_SHAPE;
  if ((d * elem_size(dtype)) % 16 != 0) return CHS_ERR_SHAPE;
  // A row's chunks must be adjacent lanes of one wave: d / (elements per 16 bytes) a power of two
  // of at most 64 (bf16: d in {8, 16, ..., 512}; fp32: d in {4, ..., 256}).
  const int cpr = (int)(d * elem_size(dtype) / 16);
  if (cpr > 64 || (cpr & (cpr - 1)) != 0) return CHS_ERR_UNSUPPORTED;
  if (!x || !gate || !bias || !cu_tokens || !cu_groups || !out_codes || !out_scales) return CHS_ERR_NULL;
  if (max_groups == 0) return CHS_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return dtype == CHS_BF16
             ? launch<uint16_t, true>(batch, d, m, x, gate, bias, cu_tokens, cu_groups, max_groups, nullptr,
                                      out_codes, out_scales, s)
             : launch<float, true>(batch, d, m, x, gate, bias, cu_tokens, cu_groups, max_groups, nullptr, out_codes,
                                   out_scales, s);
}
