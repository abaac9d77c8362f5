// chs_decode_attn: one softmax over the sliding window plus the selected (C4) or all (C128)
// compressed entries, keys doubling as values.
//
// Source: "DeepSeek-V4 本地部署，SGLang 把活做絕了", Kernel 層一堆狠活 (FlashMLA's new interface
// runs the window attention and the extra C4/C128 attention in one call) and V4 到底改了啥
// (window of 128; C4 top-512; C128 dense). "SGLang 如何为 DeepSeek V4 打造「Day-0」推理加速",
// 3.2 (MLA decode is memory-bound; FlashMLA wants the head count padded to 64 or 128) and
// 创新 3 (C128 reads every entry each step).
//
// gfx950 design (bf16). All query heads of a sequence share one latent KV row, so the heads
// form the M dimension of the MFMA contraction (16 per tile, unused heads masked in-kernel, so
// callers never pad). The key list (window rows, then the selected or all compressed rows) is
// split across workgroups (split-KV); a workgroup of 4 waves covers one 16-head tile and walks
// its slice of the key list 32 rows at a time:
//   1. the chunk's top-k entries are read first (scalar loads, ahead of the Q loads), then the
//      32 rows are gathered with coalesced 16-byte loads, 8 rows per wave, into one row-major
//      LDS tile, so K = V is staged once;
//   2. S = Q K^T with v_mfma_f32_16x16x32_bf16, each wave contracting a quarter of the
//      channels; the four partial tiles are summed through LDS in a fixed order;
//   3. online softmax in fp32 (base-2 logits, running max and sum per head, DPP row
//      reductions), the same in every wave;
//   4. P (rounded to bf16, and the running sum is taken over the rounded values so the weights
//      sum to one exactly) goes through LDS into the A-operand layout, and each wave computes
//      O += P V for its quarter of the channels, the B operand read with transposing LDS loads.
// Each workgroup writes its unnormalised O with its running max and sum; a combine kernel
// merges the splits with the log-sum-exp identity and writes out and lse. fp32 storage takes a
// plain VALU kernel with the same split and merge (it has to meet an fp32 tolerance that bf16
// MFMA operands cannot).
#include "attn_core.h"

namespace chs {
namespace {

using namespace attn;
constexpr int kThreads = kAttnThreads;

// ---------------------------------------------------------------- bf16 MFMA split kernel
// One workgroup of 4 waves per (split, sequence, 16-head tile).
// PAGED: the window and the compressed entries come from paged pools (AttnArgs::pg).
template <int D, bool PAGED = false>
__global__ __launch_bounds__(kThreads) void attn_bf16_kernel(AttnArgs a) {
  __shared__ AttnShared<D, 1> sh;
  NoHook none;
  attn_split<D, 1, NoHook, false, PAGED>(a, blockIdx.y, blockIdx.x, blockIdx.z, threadIdx.x, sh, none);
}

// The same with FP8 E4M3 storage and per-row scales (PAGED: rows and scales from paged pools).
template <int D, bool PAGED = false>
__global__ __launch_bounds__(kThreads) void attn_fp8_kernel(AttnArgs a) {
  __shared__ AttnShared<D, 1> sh;
  NoHook none;
  attn_split<D, 1, NoHook, true, PAGED>(a, blockIdx.y, blockIdx.x, blockIdx.z, threadIdx.x, sh, none);
}

// The dense form (every compressed entry attended, more than 48 heads): one workgroup of 16
// waves per (split, sequence, 64 heads), so each gathered row is read from HBM once for all
// of them, and the split's chunks stream with the rows of the next chunks requested while the
// current one is computed. FP8 / PAGED as above.
template <int D, bool FP8, bool PAGED>
__global__ __launch_bounds__(kDenseThreads) void attn_dense_kernel(AttnArgs a) {
  __shared__ AttnShared<D, 4> sh;
  NoHook none;
  attn_split<D, 4, NoHook, FP8, PAGED, 1>(a, blockIdx.y, blockIdx.x, 4 * blockIdx.z, threadIdx.x, sh, none);
}

template <bool FP8, bool PAGED>
void launch_dense(int d, dim3 grid, hipStream_t s, const AttnArgs& a) {
  switch (d) {
    case 64: hipLaunchKernelGGL((attn_dense_kernel<64, FP8, PAGED>), grid, dim3(kDenseThreads), 0, s, a); break;
    case 128: hipLaunchKernelGGL((attn_dense_kernel<128, FP8, PAGED>), grid, dim3(kDenseThreads), 0, s, a); break;
    case 256: hipLaunchKernelGGL((attn_dense_kernel<256, FP8, PAGED>), grid, dim3(kDenseThreads), 0, s, a); break;
    default: hipLaunchKernelGGL((attn_dense_kernel<512, FP8, PAGED>), grid, dim3(kDenseThreads), 0, s, a); break;
  }
}

// ---------------------------------------------------------------- fp32 VALU split kernel
// One workgroup per (split, sequence, head). Chunks of 256 key slots: one thread per key for
// the logits, then one thread per channel for the weighted sum.
__global__ __launch_bounds__(kThreads) void attn_f32_kernel(AttnArgs a) {
  __shared__ float qs[1024];
  __shared__ float ps[kThreads];
  __shared__ int64_t offs[kThreads];
  __shared__ int32_t isw[kThreads];
  __shared__ float red[kThreads / 64];
  const int b = blockIdx.y, split = blockIdx.x, h = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int D = a.D;
  const SlotMap sm(a, b);
  const int32_t s_begin = split * a.kps, s_end = min(s_begin + a.kps, sm.nslots());
  const float* qp = static_cast<const float*>(a.q) + ((int64_t)b * a.H + h) * D;
  for (int i = tid; i < D; i += kThreads) qs[i] = qp[i];
  const float* swa = static_cast<const float*>(a.swa);
  const float* comp = static_cast<const float*>(a.comp);
  float acc[4] = {0, 0, 0, 0};
  float m_run = -INFINITY, l_run = 0.f;
  for (int32_t s0 = s_begin; s0 < s_end; s0 += kThreads) {
    __syncthreads();
    const int32_t s = s0 + tid;
    bool is_swa = false;
    const int64_t off = (s < s_end) ? sm.row(a, b, s, &is_swa) : -1;
    offs[tid] = off;
    isw[tid] = is_swa;
    __syncthreads();
    float x = -INFINITY;
    if (off >= 0) {
      const float* kr = (is_swa ? swa : comp) + off;
      float dot = 0.f;
      for (int i = 0; i < D; ++i) dot = fmaf(qs[i], kr[i], dot);
      x = dot * a.scale_log2;
    }
    float cm = x;
    for (int o = 32; o > 0; o >>= 1) cm = fmaxf(cm, __shfl_xor(cm, o, 64));
    if (lane == 0) red[wave] = cm;
    __syncthreads();
    cm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float mn = fmaxf(m_run, cm);
    const bool none = (mn == -INFINITY);
    const float alpha = none ? 1.f : exp2f(m_run - mn);
    const float p = (none || off < 0) ? 0.f : exp2f(x - mn);
    ps[tid] = p;
    float sum = p;
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
    __syncthreads();
    if (lane == 0) red[wave] = sum;
    __syncthreads();
    sum = red[0] + red[1] + red[2] + red[3];
    l_run = l_run * alpha + sum;
    m_run = mn;
    const int nk = min(kThreads, s_end - s0);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] *= alpha;
    for (int i = 0; i < nk; ++i) {
      const int64_t ro = offs[i];
      if (ro < 0) continue;
      const float* kr = (isw[i] ? swa : comp) + ro;
      const float pi = ps[i];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cc = tid + q * kThreads;
        if (cc < D) acc[q] = fmaf(pi, kr[cc], acc[q]);
      }
    }
  }
  const int64_t pslot = (int64_t)b * a.n_splits + split;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int cc = tid + q * kThreads;
    if (cc < D) a.part_o[(pslot * a.H + h) * D + cc] = acc[q];
  }
  if (tid == 0) { a.part_ml[(pslot * a.H + h) * 2] = m_run; a.part_ml[(pslot * a.H + h) * 2 + 1] = l_run; }
}

// ---------------------------------------------------------------- merge of the splits
// out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s and lse = (M + log2 L) * ln 2, per head.
// bf16 partials (MFMA layout): one workgroup per (group of 16 heads, 1024 accumulator words
// of their tile, sequence); each thread reads one 16-byte accumulator (4 heads x 1 channel)
// per split, so every load is a whole, coalesced vector. Split weights are computed once per
// head in LDS.
// Four lanes of a quad share one accumulator word, each summing a strided quarter of the
// splits, so a launch has four times as many workgroups as words / 256.
// bf16 partials: one block per (64 output words of a 16-head tile, head group, sequence).
template <int KB>
__global__ __launch_bounds__(kThreads) void combine_mfma_kernel(AttnArgs a, float* out, float* lse) {
  __shared__ CombineShared<kCombineSplits> sh;
  combine_tile<kCombineSplits, KB>(a, out, lse, blockIdx.x, blockIdx.y, blockIdx.z, threadIdx.x, sh);
}

// fp32 partials ([H][D] per split): one workgroup per (sequence, head).
__global__ __launch_bounds__(kThreads) void combine_rows_kernel(AttnArgs a, float* out, float* lse) {
  __shared__ float wts[kCombineSplits];
  __shared__ float red[2][kThreads / 64];
  const int b = blockIdx.y, h = blockIdx.x, D = a.D;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ns = a.n_splits;
  const float* ml = a.part_ml + ((int64_t)b * ns * a.H + h) * 2;
  float mloc = -INFINITY;
  for (int s = tid; s < ns; s += kThreads) mloc = fmaxf(mloc, ml[(int64_t)s * a.H * 2]);
  for (int o = 32; o > 0; o >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o, 64));
  if (lane == 0) red[0][wave] = mloc;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  float lloc = 0.f;
  for (int s = tid; s < ns; s += kThreads) {
    const float ms = ml[(int64_t)s * a.H * 2];
    const float wgt = (ms == -INFINITY) ? 0.f : exp2f(ms - M);
    wts[s] = wgt;
    lloc += wgt * ml[(int64_t)s * a.H * 2 + 1];
  }
  for (int o = 32; o > 0; o >>= 1) lloc += __shfl_xor(lloc, o, 64);
  if (lane == 0) red[1][wave] = lloc;
  __syncthreads();
  const float L = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  const bool empty = !(L > 0.f);
  const float invL = empty ? 0.f : 1.f / L;
  for (int cc = tid; cc < D; cc += kThreads) {
    float acc = 0.f;
#pragma unroll 8
    for (int s = 0; s < ns; ++s) acc = fmaf(wts[s], a.part_o[(((int64_t)b * ns + s) * a.H + h) * D + cc], acc);
    out[((int64_t)b * a.H + h) * D + cc] = acc * invL;
  }
  if (lse && tid == 0)
    lse[(int64_t)b * a.H + h] = empty ? -INFINITY : (M + log2f(L)) * 0.69314718055994531f;
}

}  // namespace
}  // namespace chs

extern "C" size_t chs_decode_attn_workspace_size(chs_dtype dtype, int32_t batch, int32_t n_heads, int32_t d,
                                                 int32_t window, int32_t k, int64_t max_comp) {
  using namespace chs;
  if (batch < 1 || n_heads < 1 || d < 1 || window < 0 || k < 0 || max_comp < 0) return 0;
  SplitPlan p = plan_splits(dtype, batch, n_heads, window, k, max_comp);
  return ws_bytes(dtype, batch, n_heads, d, p, nullptr, nullptr, nullptr);
}

namespace chs {
namespace {

// Split kernel + combine for bf16 / fp32 storage, contiguous or paged (pg zeroed: contiguous).
chs_status launch_attn(chs_dtype dtype, int32_t batch, int32_t n_heads, int32_t d, int32_t window, int32_t k,
                       float scale, const void* q, const void* swa_kv, const int32_t* swa_len, const void* comp_kv,
                       const int64_t* cu_comp, const attn::Paging& pg, const int32_t* topk, int64_t max_comp,
                       float* out, float* lse, void* workspace, size_t workspace_bytes, hipStream_t s) {
  const int kk = topk ? k : 0;
  SplitPlan p = plan_splits(dtype, batch, n_heads, window, kk, max_comp);
  AttnArgs a;
  a.q = q; a.swa = swa_kv; a.swa_len = swa_len; a.comp = comp_kv; a.cu_comp = cu_comp; a.topk = topk;
  a.swa_scale = nullptr; a.comp_scale = nullptr;
  a.pg = pg;
  a.H = n_heads; a.D = d; a.W = window; a.k = kk; a.max_comp = max_comp;
  a.scale_log2 = scale * kLog2e;
  a.n_splits = p.n_splits; a.kps = p.kps;
  a.head_tiles = dtype == CHS_BF16 ? (n_heads + 63) / 64 : n_heads;
  const size_t need = ws_bytes(dtype, batch, n_heads, d, p, &a.part_o, &a.part_ml, static_cast<char*>(workspace));
  if (workspace_bytes < need) return CHS_ERR_WORKSPACE;
  const bool paged = pg.pt != nullptr;
  if (dense_split(dtype, kk, n_heads)) {
    const dim3 grid(p.n_splits, batch, (n_heads + 63) / 64);
    paged ? launch_dense<false, true>(d, grid, s, a) : launch_dense<false, false>(d, grid, s, a);
  } else if (dtype == CHS_BF16) {
    dim3 grid(p.n_splits, batch, (n_heads + 15) / 16);
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, s, a); };
    switch (d) {
      case 64: paged ? go(attn_bf16_kernel<64, true>) : go(attn_bf16_kernel<64>); break;
      case 128: paged ? go(attn_bf16_kernel<128, true>) : go(attn_bf16_kernel<128>); break;
      case 256: paged ? go(attn_bf16_kernel<256, true>) : go(attn_bf16_kernel<256>); break;
      default: paged ? go(attn_bf16_kernel<512, true>) : go(attn_bf16_kernel<512>); break;
    }
  } else {
    dim3 grid(p.n_splits, batch, n_heads);
    hipLaunchKernelGGL(attn_f32_kernel, grid, dim3(kThreads), 0, s, a);
  }
  if (launch_status() != CHS_OK) return CHS_ERR_LAUNCH;
  if (dtype == CHS_BF16) {
    const int words_per_block = kThreads / kCombineLanes;
    const dim3 cgrid((unsigned)((d / 16 * 64 + words_per_block - 1) / words_per_block), (unsigned)((n_heads + 15) / 16),
                     (unsigned)batch);
    if (combine_batch(p.n_splits) == 16)
      hipLaunchKernelGGL(combine_mfma_kernel<16>, cgrid, dim3(kThreads), 0, s, a, out, lse);
    else
      hipLaunchKernelGGL(combine_mfma_kernel<8>, cgrid, dim3(kThreads), 0, s, a, out, lse);
  } else {
    hipLaunchKernelGGL(combine_rows_kernel, dim3(n_heads, batch), dim3(kThreads), 0, s, a, out, lse);
  }
  return launch_status();
}

}  // namespace
}  // namespace chs

extern "C" chs_status chs_decode_attn(chs_dtype dtype, int32_t batch, int32_t n_heads, int32_t d,
                                      int32_t window, int32_t k, float scale, const void* q,
                                      const void* swa_kv, const int32_t* swa_len, const void* comp_kv,
                                      const int64_t* cu_comp, const int32_t* topk, int64_t max_comp,
                                      float* out, float* lse, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  using namespace chs;
  const chs_status st = attn::check_args(dtype, batch, n_heads, d, window, k, scale, q, swa_kv, swa_len, comp_kv,
                                         cu_comp, topk, max_comp, out);
  if (st != CHS_OK) return st;
  if (!workspace) return CHS_ERR_NULL;
  const attn::Paging none{};
  return launch_attn(dtype, batch, n_heads, d, window, k, scale, q, swa_kv, swa_len, comp_kv, cu_comp, none, topk,
                     max_comp, out, lse, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

extern "C" chs_status chs_decode_attn_paged(chs_dtype dtype, int32_t batch, int32_t n_heads, int32_t d,
                                            int32_t window, int32_t k, float scale, const void* q,
                                            const void* swa_pool, const int32_t* swa_page, int64_t swa_pages,
                                            const int32_t* swa_len, const void* comp_pool, int64_t pool_pages,
                                            int32_t page_size, const int32_t* page_table, int32_t pt_stride,
                                            const int64_t* comp_len, const int32_t* topk, int64_t max_comp,
                                            float* out, float* lse, void* workspace, size_t workspace_bytes,
                                            void* stream) {
  using namespace chs;
  // The shared checks null-test their cu argument; here the per-sequence counts take its place.
  const chs_status st = attn::check_args(dtype, batch, n_heads, d, window, k, scale, q, swa_pool, swa_len, comp_pool,
                                         comp_len, topk, max_comp, out);
  if (st != CHS_OK) return st;
  if (!workspace || !page_table || (window > 0 && !swa_page)) return CHS_ERR_NULL;
  if (page_size < 1 || page_size > 65536 || (page_size & (page_size - 1)) != 0 || pt_stride < 1 ||
      pool_pages < 1 || (window > 0 && swa_pages < 1))
    return CHS_ERR_SHAPE;
  attn::Paging pg{};
  pg.swa_page = window > 0 ? swa_page : nullptr;
  pg.swa_pages = swa_pages;
  pg.pt = page_table;
  pg.comp_len = comp_len;
  pg.pt_stride = pt_stride;
  pg.shift = __builtin_ctz((unsigned)page_size);
  pg.pool_pages = pool_pages;
  return launch_attn(dtype, batch, n_heads, d, window, k, scale, q, swa_pool, swa_len, comp_pool, nullptr, pg, topk,
                     max_comp, out, lse, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

namespace chs {
namespace {

chs_status launch_attn_fp8(int32_t batch, int32_t n_heads, int32_t d, int32_t window, int32_t k, float scale,
                           const void* q, const void* swa_kv, const float* swa_scale, const int32_t* swa_len,
                           const void* comp_kv, const float* comp_scale, const int64_t* cu_comp,
                           const attn::Paging& pg, const int32_t* topk, int64_t max_comp, float* out, float* lse,
                           void* workspace, size_t workspace_bytes, hipStream_t s) {
  const int kk = topk ? k : 0;
  SplitPlan p = plan_splits(CHS_BF16, batch, n_heads, window, kk, max_comp);
  AttnArgs a;
  a.q = q; a.swa = swa_kv; a.swa_len = swa_len; a.comp = comp_kv; a.cu_comp = cu_comp; a.topk = topk;
  a.swa_scale = swa_scale; a.comp_scale = comp_scale;
  a.pg = pg;
  a.H = n_heads; a.D = d; a.W = window; a.k = kk; a.max_comp = max_comp;
  a.scale_log2 = scale * kLog2e;
  a.n_splits = p.n_splits; a.kps = p.kps;
  a.head_tiles = (n_heads + 63) / 64;
  const size_t need = ws_bytes(CHS_BF16, batch, n_heads, d, p, &a.part_o, &a.part_ml, static_cast<char*>(workspace));
  if (workspace_bytes < need) return CHS_ERR_WORKSPACE;
  dim3 grid(p.n_splits, batch, (n_heads + 15) / 16);
  const bool paged = pg.pt != nullptr;
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, s, a); };
  if (dense_split(CHS_BF16, kk, n_heads)) {
    const dim3 dgrid(p.n_splits, batch, (n_heads + 63) / 64);
    paged ? launch_dense<true, true>(d, dgrid, s, a) : launch_dense<true, false>(d, dgrid, s, a);
  } else {
    switch (d) {
      case 64: paged ? go(attn_fp8_kernel<64, true>) : go(attn_fp8_kernel<64>); break;
      case 128: paged ? go(attn_fp8_kernel<128, true>) : go(attn_fp8_kernel<128>); break;
      case 256: paged ? go(attn_fp8_kernel<256, true>) : go(attn_fp8_kernel<256>); break;
      default: paged ? go(attn_fp8_kernel<512, true>) : go(attn_fp8_kernel<512>); break;
    }
  }
  if (launch_status() != CHS_OK) return CHS_ERR_LAUNCH;
  const int words_per_block = kThreads / kCombineLanes;
  const dim3 cgrid((unsigned)((d / 16 * 64 + words_per_block - 1) / words_per_block), (unsigned)((n_heads + 15) / 16),
                   (unsigned)batch);
  if (combine_batch(p.n_splits) == 16)
    hipLaunchKernelGGL(combine_mfma_kernel<16>, cgrid, dim3(kThreads), 0, s, a, out, lse);
  else
    hipLaunchKernelGGL(combine_mfma_kernel<8>, cgrid, dim3(kThreads), 0, s, a, out, lse);
  return launch_status();
}

}  // namespace
}  // namespace chs

extern "C" chs_status chs_decode_attn_fp8(int32_t batch, int32_t n_heads, int32_t d, int32_t window, int32_t k,
                                          float scale, const void* q, const void* swa_kv, const float* swa_scale,
                                          const int32_t* swa_len, const void* comp_kv, const float* comp_scale,
                                          const int64_t* cu_comp, const int32_t* topk, int64_t max_comp,
                                          float* out, float* lse, void* workspace, size_t workspace_bytes,
                                          void* stream) {
  using namespace chs;
  const chs_status st = attn::check_args(CHS_BF16, batch, n_heads, d, window, k, scale, q, swa_kv, swa_len, comp_kv,
                                         cu_comp, topk, max_comp, out);
  if (st != CHS_OK) return st;
  if (!workspace) return CHS_ERR_NULL;
  if (window > 0 && !swa_scale) return CHS_ERR_NULL;
  if (!comp_scale && (topk ? k > 0 : max_comp > 0)) return CHS_ERR_NULL;
  const attn::Paging none{};
  return launch_attn_fp8(batch, n_heads, d, window, k, scale, q, swa_kv, swa_scale, swa_len, comp_kv, comp_scale,
                         cu_comp, none, topk, max_comp, out, lse, workspace, workspace_bytes,
                         static_cast<hipStream_t>(stream));
}

extern "C" chs_status chs_decode_attn_fp8_paged(int32_t batch, int32_t n_heads, int32_t d, int32_t window, int32_t k,
                                                float scale, const void* q, const void* swa_pool,
                                                const float* swa_scale_pool, const int32_t* swa_page,
                                                int64_t swa_pages, const int32_t* swa_len, const void* comp_pool,
                                                const float* comp_scale_pool, int64_t pool_pages, int32_t page_size,
                                                const int32_t* page_table, int32_t pt_stride, const int64_t* comp_len,
                                                const int32_t* topk, int64_t max_comp, float* out, float* lse,
                                                void* workspace, size_t workspace_bytes, void* stream) {
  using namespace chs;
  // The shared checks null-test their cu argument; here the per-sequence counts take its place.
  const chs_status st = attn::check_args(CHS_BF16, batch, n_heads, d, window, k, scale, q, swa_pool, swa_len,
                                         comp_pool, comp_len, topk, max_comp, out);
  if (st != CHS_OK) return st;
  if (!workspace || !page_table || (window > 0 && (!swa_page || !swa_scale_pool))) return CHS_ERR_NULL;
  if (!comp_scale_pool && (topk ? k > 0 : max_comp > 0)) return CHS_ERR_NULL;
  if (page_size < 1 || page_size > 65536 || (page_size & (page_size - 1)) != 0 || pt_stride < 1 ||
      pool_pages < 1 || (window > 0 && swa_pages < 1))
    return CHS_ERR_SHAPE;
  attn::Paging pg{};
  pg.swa_page = window > 0 ? swa_page : nullptr;
  pg.swa_pages = swa_pages;
  pg.pt = page_table;
  pg.comp_len = comp_len;
  pg.pt_stride = pt_stride;
  pg.shift = __builtin_ctz((unsigned)page_size);
  pg.pool_pages = pool_pages;
  return launch_attn_fp8(batch, n_heads, d, window, k, scale, q, swa_pool, swa_scale_pool, swa_len, comp_pool,
                         comp_scale_pool, nullptr, pg, topk, max_comp, out, lse, workspace, workspace_bytes,
                         static_cast<hipStream_t>(stream));
}
