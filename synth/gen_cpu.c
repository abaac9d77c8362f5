/* Host filler for the counter-based synthetic inputs (test and benchmark infrastructure).
 * Every function fills out[j] with element (start + j) of a logical tensor; elements are
 * independent, so the loops run in parallel with OpenMP without changing any bit.
 * Built with -ffp-contract=off (see gen_core.h). */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "gen_core.h"

uint64_t syn_stream_of(uint64_t seed, uint64_t tensor) { return syn_stream(seed, tensor); }

void syn_fill_bits(uint64_t seed, uint64_t tensor, uint64_t start, int64_t count, uint64_t* out) {
  uint64_t st = syn_stream(seed, tensor);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < count; ++j) out[j] = syn_bits(st, start + (uint64_t)j);
}

/* N(mean, std^2) as fp32; if round_bf16, each value is further rounded to bfloat16 (RNE) and
 * stored back as the fp32 value of that bfloat16. */
void syn_fill_normal_f32(uint64_t seed, uint64_t tensor, uint64_t start, int64_t count,
                         double mean, double stdv, int round_bf16, float* out) {
  uint64_t st = syn_stream(seed, tensor);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < count; ++j) {
    float v = syn_normal_f32(st, start + (uint64_t)j, mean, stdv);
    out[j] = round_bf16 ? syn_bf16_to_f32(syn_f32_to_bf16(v)) : v;
  }
}

/* N(mean, std^2) rounded to bfloat16, as raw bf16 bits. */
void syn_fill_normal_bf16(uint64_t seed, uint64_t tensor, uint64_t start, int64_t count,
                          double mean, double stdv, uint16_t* out) {
  uint64_t st = syn_stream(seed, tensor);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < count; ++j)
    out[j] = syn_f32_to_bf16(syn_normal_f32(st, start + (uint64_t)j, mean, stdv));
}

void syn_fill_uniform_f32(uint64_t seed, uint64_t tensor, uint64_t start, int64_t count,
                          double lo, double hi, float* out) {
  uint64_t st = syn_stream(seed, tensor);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < count; ++j) out[j] = syn_uniform_f32(st, start + (uint64_t)j, lo, hi);
}

/* Standard normals in double (no rounding), used only to build the spike basis. */
void syn_fill_normal_f64(uint64_t seed, uint64_t tensor, uint64_t start, int64_t count, double* out) {
  uint64_t st = syn_stream(seed, tensor);
  for (int64_t j = 0; j < count; ++j) out[j] = syn_normal(st, start + (uint64_t)j);
}

/* nspike orthonormal rows of length dim: seeded Gaussian rows, then modified Gram-Schmidt.
 * Host only; the result is handed to both fillers so they use the same basis bits. */
void syn_spike_basis(uint64_t seed, uint64_t tensor, int32_t nspike, int32_t dim, double* U) {
  syn_fill_normal_f64(seed, tensor, 0, (int64_t)nspike * dim, U);
  for (int32_t r = 0; r < nspike; ++r) {
    double* u = U + (int64_t)r * dim;
    for (int32_t q = 0; q < r; ++q) {
      const double* v = U + (int64_t)q * dim;
      double dot = 0.0;
      for (int32_t t = 0; t < dim; ++t) dot += u[t] * v[t];
      for (int32_t t = 0; t < dim; ++t) u[t] -= dot * v[t];
    }
    double nn = 0.0;
    for (int32_t t = 0; t < dim; ++t) nn += u[t] * u[t];
    double inv = 1.0 / sqrt(nn);
    for (int32_t t = 0; t < dim; ++t) u[t] *= inv;
  }
}

/* Rows [row_start, row_start + nrows) of the spiked index-key tensor [*, dim] (see gen_core.h).
 * round_bf16 as in syn_fill_normal_f32. */
void syn_fill_index_keys(uint64_t seed, uint64_t t_noise, uint64_t t_load, int64_t row_start,
                         int64_t nrows, int32_t dim, int32_t nspike, const double* U, double alpha,
                         int round_bf16, float* out) {
  uint64_t sn = syn_stream(seed, t_noise), sl = syn_stream(seed, t_load);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nrows; ++r)
    for (int32_t t = 0; t < dim; ++t) {
      float v = syn_index_key(sn, sl, (uint64_t)(row_start + r), (uint32_t)t, (uint32_t)dim,
                              (uint32_t)nspike, U, alpha);
      out[r * dim + t] = round_bf16 ? syn_bf16_to_f32(syn_f32_to_bf16(v)) : v;
    }
}
