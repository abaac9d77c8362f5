// The group softmax-pool of one 16-byte channel chunk, shared by chs_compress (a whole prefill)
// and chs_append (the group that one decode-time token completes).
//
// Source: "SGLang 如何为 DeepSeek V4 打造「Day-0」推理加速", 创新 2 (Flash Compressor: load the
// tokens and gates, score, softmax, weighted sum and store in one on-chip pass).
//
// A chunk is 8 bf16 or 4 fp32 channels. Rows are reached through accessors (row index -> chunk
// pointer), so the rows of a group need not be contiguous: a prefill walks x + r*d, an append
// reads a ring. Logits are carried in base-2 units (times log2 e) so the exponentials are
// single v_exp_f32 instructions.
#pragma once

#include "common.h"

namespace chs {
namespace {

template <typename ET>
struct Vec16;

template <>
struct Vec16<uint16_t> {  // 8 bf16 channels
  static constexpr int N = 8;
  // The 16 raw bytes, non-temporal (rows are read once), and their widening to fp32.
  __device__ static u32x4 load_raw(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
  __device__ static void unpack(const u32x4& r, float* v) {
#pragma unroll
    for (int j = 0; j < 4; ++j) { v[2 * j] = bf16_lo(r[j]); v[2 * j + 1] = bf16_hi(r[j]); }
  }
  __device__ static void load(const uint16_t* p, float* v) { unpack(load_raw(p), v); }
  __device__ static void store(uint16_t* p, const float* v) {
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
    __builtin_nontemporal_store(r, reinterpret_cast<u32x4*>(p));   // not re-read soon
  }
  __device__ static void copy(uint16_t* dst, const uint16_t* src) {
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
  }
};

template <>
struct Vec16<float> {  // 4 fp32 channels
  static constexpr int N = 4;
  __device__ static u32x4 load_raw(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
  __device__ static void unpack(const u32x4& r, float* v) {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = __uint_as_float(r[j]);
  }
  __device__ static void load(const float* p, float* v) { unpack(load_raw(p), v); }
  __device__ static void store(float* p, const float* v) {
    f32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = v[j];
    __builtin_nontemporal_store(r, reinterpret_cast<f32x4*>(p));
  }
  __device__ static void copy(float* dst, const float* src) {
    *reinterpret_cast<f32x4*>(dst) = *reinterpret_cast<const f32x4*>(src);
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

// Running state of one chunk's softmax-pool: maximum logit (base 2), sum of exponentials and
// the weighted sum of rows, all relative to the maximum.
template <int N>
struct PoolState {
  float mx[N], sum[N], acc[N];
  __device__ void init() {
#pragma unroll
    for (int j = 0; j < N; ++j) { mx[j] = -INFINITY; sum[j] = 0.f; acc[j] = 0.f; }
  }
  // Folds in another state (the same chunk over other rows). Symmetric: merging a into b and b
  // into a give the same bits. Two empty states (maximum -inf) merge into an empty state.
  __device__ void merge(const float* omx, const float* osum, const float* oacc) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const float nm = fmaxf(mx[j], omx[j]);
      const float a = mx[j] == nm ? 1.f : fast_exp2(mx[j] - nm);
      const float b = omx[j] == nm ? 1.f : fast_exp2(omx[j] - nm);
      sum[j] = sum[j] * a + osum[j] * b;
      acc[j] = acc[j] * a + oacc[j] * b;
      mx[j] = nm;
    }
  }
};

// Folds rows r0 .. r0 + nr - 1 (1 <= nr <= R) into the state: the block's maximum first, then
// the previous sums rescaled to it (skipped when FIRST: the state is fresh), then each row's
// exponential and weighted contribution in row order. bias(r) is row r's bias chunk.
// All R loads are issued unconditionally, so they are in flight together: a load under a
// runtime guard gets its own wait for completion. Slots r >= nr re-read the block's last row
// and take the logit -inf, so they add exactly zero (a weight of 0 times a finite row).
// ALL_LOADS_FIRST keeps the compiler from interleaving the loads with the arithmetic (which it
// does to save registers, leaving a few loads in flight at a time): for a launch with one
// group per workgroup, where the round trips are the whole cost.
template <typename ET, int R, bool FIRST, bool ALL_LOADS_FIRST = false, typename XRow, typename ZRow, typename BRow>
__device__ __forceinline__ void pool_block(PoolState<Vec16<ET>::N>& st, int r0, int nr, XRow xrow, ZRow zrow,
                                           BRow brow) {
  using V = Vec16<ET>;
  constexpr int N = V::N;
  float xv[R][N], av[R][N], bv[R][8];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int rr = r0 + (r < nr ? r : nr - 1);
    V::load(xrow(rr), xv[r]);
    V::load(zrow(rr), av[r]);
    load_bias(brow(rr), bv[r], N);
  }
  if (ALL_LOADS_FIRST) __builtin_amdgcn_sched_barrier(0);
  float cmax[N];
#pragma unroll
  for (int j = 0; j < N; ++j) cmax[j] = -INFINITY;
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      av[r][j] = r < nr ? (av[r][j] + bv[r][j]) * kLog2e : -INFINITY;   // logit in base-2 units
      cmax[j] = fmaxf(cmax[j], av[r][j]);
    }
  }
  if (FIRST) {
#pragma unroll
    for (int j = 0; j < N; ++j) st.mx[j] = cmax[j];
  } else {
    // Online softmax: rescale what was accumulated under the previous maximum.
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const float nm = fmaxf(st.mx[j], cmax[j]);
      const float sc = fast_exp2(st.mx[j] - nm);
      st.sum[j] *= sc;
      st.acc[j] *= sc;
      st.mx[j] = nm;
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r < nr) {   // a uniform branch (nr is the same for every lane); no loads inside
#pragma unroll
      for (int j = 0; j < N; ++j) {
        const float e = fast_exp2(av[r][j] - st.mx[j]);
        st.sum[j] += e;
        st.acc[j] = fmaf(e, xv[r][j], st.acc[j]);
      }
    }
  }
}

// The pooled fp32 values of the chunk.
template <int N>
__device__ __forceinline__ void pool_values(const PoolState<N>& st, float* o) {
#pragma unroll
  for (int j = 0; j < N; ++j) o[j] = st.acc[j] / st.sum[j];
}

template <typename ET>
__device__ __forceinline__ void pool_store(const PoolState<Vec16<ET>::N>& st, ET* op) {
  constexpr int N = Vec16<ET>::N;
  float o[N];
  pool_values<N>(st, o);
  Vec16<ET>::store(op, o);
}

// Any m, in blocks of R rows with a running maximum (online softmax), so registers stay bounded.
// The rows of the next block are requested before the current block is computed, so a wave
// always has a block of HBM reads in flight while it does the arithmetic. The current block's
// bias (a cache hit: one [m, d] table for every group) is requested before them, because a
// wave's loads complete in issue order for its wait counter: waiting for the bias then leaves
// the next block's reads outstanding. Slots past row m - 1 re-read the last row and are
// masked as in pool_block.
template <typename ET, int R, typename XRow, typename ZRow, typename BRow>
__device__ __forceinline__ void pool_stream(PoolState<Vec16<ET>::N>& st, int m, XRow xrow, ZRow zrow,
                                            BRow brow) {
  using V = Vec16<ET>;
  constexpr int N = V::N;
  u32x4 xc[R], zc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int rr = min(r, m - 1);
    xc[r] = V::load_raw(xrow(rr));
    zc[r] = V::load_raw(zrow(rr));
  }
  for (int r0 = 0; r0 < m; r0 += R) {
    const int nr = min(R, m - r0);
    float bv[R][8];
#pragma unroll
    for (int r = 0; r < R; ++r) load_bias(brow(r0 + (r < nr ? r : nr - 1)), bv[r], N);
    __builtin_amdgcn_sched_barrier(0);   // keep the bias requests ahead of the next block's
    u32x4 xn[R], zn[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int rr = min(r0 + R + r, m - 1);
      xn[r] = V::load_raw(xrow(rr));
      zn[r] = V::load_raw(zrow(rr));
    }
    __builtin_amdgcn_sched_barrier(0);
    float xv[R][N], av[R][N], cmax[N];
#pragma unroll
    for (int j = 0; j < N; ++j) cmax[j] = -INFINITY;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      V::unpack(xc[r], xv[r]);
      V::unpack(zc[r], av[r]);
#pragma unroll
      for (int j = 0; j < N; ++j) {
        av[r][j] = r < nr ? (av[r][j] + bv[r][j]) * kLog2e : -INFINITY;   // logit in base-2 units
        cmax[j] = fmaxf(cmax[j], av[r][j]);
      }
    }
#pragma unroll
    for (int j = 0; j < N; ++j) {   // rescale to the new maximum (the first block: 0 * 0)
      const float nm = fmaxf(st.mx[j], cmax[j]);
      const float sc = fast_exp2(st.mx[j] - nm);
      st.sum[j] *= sc;
      st.acc[j] *= sc;
      st.mx[j] = nm;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r < nr) {   // uniform: nr is the same for every lane
#pragma unroll
        for (int j = 0; j < N; ++j) {
          const float e = fast_exp2(av[r][j] - st.mx[j]);
          st.sum[j] += e;
          st.acc[j] = fmaf(e, xv[r][j], st.acc[j]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) { xc[r] = xn[r]; zc[r] = zn[r]; }
  }
}

// A whole group of m rows into its pooled fp32 values o: M > 0 is a compile-time group size
// (<= 8, one block); M == 0 takes any m through pool_stream.
template <typename ET, int M, bool ALL_LOADS_FIRST = false, typename XRow, typename ZRow, typename BRow>
__device__ __forceinline__ void pool_group_values(int m, XRow xrow, ZRow zrow, BRow brow, float* o) {
  PoolState<Vec16<ET>::N> st;
  st.init();
  if (M > 0) {
    pool_block<ET, (M > 0 ? M : 1), true, ALL_LOADS_FIRST>(st, 0, M, xrow, zrow, brow);
  } else {
    pool_stream<ET, 4>(st, m, xrow, zrow, brow);
  }
  pool_values<Vec16<ET>::N>(st, o);
}

// The same, stored in the storage type at op.
template <typename ET, int M, bool ALL_LOADS_FIRST = false, typename XRow, typename ZRow, typename BRow>
__device__ __forceinline__ void pool_group(int m, XRow xrow, ZRow zrow, BRow brow, ET* op) {
  float o[Vec16<ET>::N];
  pool_group_values<ET, M, ALL_LOADS_FIRST>(m, xrow, zrow, brow, o);
  Vec16<ET>::store(op, o);
}

}  // namespace
}  // namespace chs
