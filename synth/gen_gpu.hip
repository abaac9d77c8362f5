// Device filler for the counter-based synthetic inputs (test and benchmark infrastructure,
// not part of the attention library). Each thread writes one element; the value is the same
// pure function of (seed, tensor, index) that the host filler computes, so both produce
// identical bits. Built with -ffp-contract=off (see gen_core.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gen_core.h"

namespace {

// The grid of a launch holds fewer than 2^32 work-items, so every kernel strides over its range.
#define SYN_FOR_EACH(j, n) \
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < (n); j += (int64_t)gridDim.x * blockDim.x)

__global__ void fill_normal_kernel(uint64_t stream, uint64_t start, int64_t count, double mean,
                                   double stdv, int bf16, void* out) {
  SYN_FOR_EACH(j, count) {
    float v = syn_normal_f32(stream, start + (uint64_t)j, mean, stdv);
    if (bf16) static_cast<uint16_t*>(out)[j] = syn_f32_to_bf16(v);
    else static_cast<float*>(out)[j] = v;
  }
}

__global__ void fill_uniform_kernel(uint64_t stream, uint64_t start, int64_t count, double lo,
                                    double hi, float* out) {
  SYN_FOR_EACH(j, count) out[j] = syn_uniform_f32(stream, start + (uint64_t)j, lo, hi);
}

__global__ void fill_index_keys_kernel(uint64_t s_noise, uint64_t s_load, int64_t row_start,
                                       int64_t nrows, int32_t dim, int32_t nspike,
                                       const double* U, double alpha, int bf16, void* out) {
  SYN_FOR_EACH(j, nrows * dim) {
    int64_t r = j / dim;
    int32_t t = (int32_t)(j - r * dim);
    float v = syn_index_key(s_noise, s_load, (uint64_t)(row_start + r), (uint32_t)t,
                            (uint32_t)dim, (uint32_t)nspike, U, alpha);
    if (bf16) static_cast<uint16_t*>(out)[j] = syn_f32_to_bf16(v);
    else static_cast<float*>(out)[j] = v;
  }
}

unsigned grid_for(int64_t n) {
  int64_t b = (n + 255) / 256;
  return (unsigned)(b < 65536 * 8 ? b : 65536 * 8);
}

}  // namespace

extern "C" {

// All pointers are device pointers; `stream` is a hipStream_t (NULL = default stream).
// Returns 0 on success, otherwise the hipError_t of the launch.
int syn_gpu_fill_normal(uint64_t seed, uint64_t tensor, uint64_t start, int64_t count,
                        double mean, double stdv, int bf16, void* out, void* stream) {
  if (count <= 0) return 0;
  hipLaunchKernelGGL(fill_normal_kernel, dim3(grid_for(count)), dim3(256), 0,
                     (hipStream_t)stream, syn_stream(seed, tensor), start, count, mean, stdv,
                     bf16, out);
  return (int)hipGetLastError();
}

int syn_gpu_fill_uniform(uint64_t seed, uint64_t tensor, uint64_t start, int64_t count, double lo,
                         double hi, float* out, void* stream) {
  if (count <= 0) return 0;
  hipLaunchKernelGGL(fill_uniform_kernel, dim3(grid_for(count)), dim3(256), 0,
                     (hipStream_t)stream, syn_stream(seed, tensor), start, count, lo, hi, out);
  return (int)hipGetLastError();
}

// U: device pointer to nspike*dim doubles (the basis the host built with syn_spike_basis).
int syn_gpu_fill_index_keys(uint64_t seed, uint64_t t_noise, uint64_t t_load, int64_t row_start,
                            int64_t nrows, int32_t dim, int32_t nspike, const double* U,
                            double alpha, int bf16, void* out, void* stream) {
  if (nrows <= 0) return 0;
  hipLaunchKernelGGL(fill_index_keys_kernel, dim3(grid_for(nrows * dim)), dim3(256), 0,
                     (hipStream_t)stream, syn_stream(seed, t_noise), syn_stream(seed, t_load),
                     row_start, nrows, dim, nspike, U, alpha, bf16, out);
  return (int)hipGetLastError();
}

}  // extern "C"
