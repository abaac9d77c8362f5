// chs_index_topk: indexer scores, then the exact top-k by radix selection, with no global sort.
//
// Source: "SGLang 如何为 DeepSeek V4 打造「Day-0」推理加速", 创新 2 (Lightning TopK): a global
// sort of 256K candidates costs over 100 us at batch 1; instead, blocks build radix histograms
// of their scores, a threshold is found, and each block writes out only its own entries above
// it. Same page, 创新 5: the indexer scores every compressed candidate before the top-k.
// "DeepSeek-V4 本地部署，SGLang 把活做絕了", Kernel 層一堆狠活: top-512 of 256K at 1M context.
//
// The pages' design reduces per-CTA histograms inside a thread-block cluster through
// distributed shared memory, which gfx950 does not have; on MI355X a device-scope fence costs
// tens of nanoseconds per workgroup, serialised, and same-address atomics about ten. So no
// kernel here synchronises workgroups with each other: every cross-workgroup step is a kernel
// boundary, and the data crossing it is written with plain stores.
//
//   K1 score_kernel (one workgroup per 128 candidates, many resident per CU): streams the
//      index keys once (non-temporal 16-byte loads, v_dot2_f32_bf16 or fp32 FMAs, DPP lane
//      reductions), writes the fp32 scores, and writes the maximum order-preserving key of
//      every sub-chunk of SC consecutive candidates. max_kernel does only the maxima, for
//      caller-provided scores.
//   K2 bound_kernel (one workgroup per sequence): L = the k-th largest sub-chunk maximum
//      (radix select in LDS over at most 16384 maxima, rounded down to 22 key bits). L never
//      exceeds the k-th largest score: k disjoint sub-chunks each hold a score >= L. So every
//      top-k candidate, and every tie at the threshold, has key >= L. Also the largest key.
//   K3 select_kernel (one workgroup per 1024 candidates): writes the chunk's candidates with
//      key >= L, in index order, to the chunk's own region, and their count.
//   K4 final_kernel (one workgroup per sequence): gathers the regions in chunk order (so in
//      index order), finds the exact k-th largest key tau by 8-bit radix passes over the bits
//      below the prefix that L and the largest key share, takes every key above tau and the
//      first ties at tau in index order, and writes the selection ascending by a prefix count:
//      no sort is needed. If the superset exceeds the LDS capacity (heavy ties, adversarial
//      inputs), the same passes stream from a global copy instead.
// The composite order (key descending, then index ascending) is total, so the selected set is
// unique and bit-identical to a full sort of the same scores.
#include "common.h"

namespace chs {
namespace {

constexpr int kThreads = 256;        // K1, K3
constexpr int kBoundThreads = 1024;  // K2
constexpr int kFinalThreads = 512;   // K4
constexpr int kScoreChunk = 128;     // candidates per K1 workgroup
constexpr int kMaxChunk = 2048;      // scores per max_kernel workgroup (256 threads x 8)
constexpr int kSelChunk = 1024;      // candidates per K3 workgroup (256 threads x 4)
constexpr int kMaxMaxima = 16384;    // sub-chunk maxima K2 ranks (LDS)
constexpr int kLdsCand = 8192;       // superset size K4 keeps in LDS
constexpr int kMaxSelChunks = 4096;  // K3 chunks per sequence (max_cand <= 4M)
constexpr int kMaxK = 2048;
constexpr int64_t kMaxCand = (int64_t)kMaxSelChunks * kSelChunk;

struct Workspace {
  uint32_t* maxima;   // [batch][rc]: sub-chunk maximum keys, sub-chunk j at index j
  uint32_t* bound;    // [batch][2]: L, largest key
  uint32_t* counts;   // [batch][rc / kSelChunk]
  uint32_t* region;   // [batch][rc][2]: per K3 chunk, (key, index) in index order
  uint32_t* gather;   // [batch][rc][2]: K4's global superset copy (large supersets only)
  float* scores;      // [batch][rc] when the caller passes no score array
};

// Candidate capacity per sequence, rounded up to whole K3 chunks.
__host__ __device__ inline int64_t round_cand(int64_t max_cand) {
  return (max_cand + kSelChunk - 1) / kSelChunk * kSelChunk;
}

size_t ws_layout(int32_t batch, int64_t max_cand, Workspace* w, char* base) {
  const size_t nb = (size_t)batch;
  const size_t rc = (size_t)round_cand(max_cand > 0 ? max_cand : 0);
  size_t off = 0;
  const size_t o_max = off; off = align_up(off + nb * rc * 4, 256);
  const size_t o_bnd = off; off = align_up(off + nb * 2 * 4, 256);
  const size_t o_cnt = off; off = align_up(off + nb * (rc / kSelChunk + 1) * 4, 256);
  const size_t o_reg = off; off = align_up(off + nb * rc * 8, 256);
  const size_t o_gat = off; off = align_up(off + nb * rc * 8, 256);
  const size_t o_sc = off; off = align_up(off + nb * rc * 4, 256);
  if (w) {
    w->maxima = reinterpret_cast<uint32_t*>(base + o_max);
    w->bound = reinterpret_cast<uint32_t*>(base + o_bnd);
    w->counts = reinterpret_cast<uint32_t*>(base + o_cnt);
    w->region = reinterpret_cast<uint32_t*>(base + o_reg);
    w->gather = reinterpret_cast<uint32_t*>(base + o_gat);
    w->scores = reinterpret_cast<float*>(base + o_sc);
  }
  return off;
}

// Order-preserving key: a larger float gives a larger unsigned key; -0.0 maps like +0.0.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct Args {
  const void* q;        // [batch][nh][dim] (NULL: scores are input)
  const float* w;       // [batch][nh]
  const void* keys;     // [cu[batch]][dim]
  const int64_t* cu;    // [batch+1]
  int64_t max_cand;
  int32_t nh, nvec, lpc;
  int32_t sc;           // sub-chunk size (power of two, at most kScoreChunk)
  int32_t k;
  float* scores;        // caller's packed array, or NULL -> workspace
  Workspace ws;
};

__device__ __forceinline__ int64_t cand_count(const Args& a, int b, int64_t* base) {
  const int64_t c0 = a.cu[b];
  int64_t n = a.cu[b + 1] - c0;
  if (n > a.max_cand) n = a.max_cand;
  if (n < 0) n = 0;
  *base = c0;
  return n;
}
__device__ __forceinline__ float* score_ptr(const Args& a, int b, int64_t c0) {
  return a.scores ? a.scores + c0 : a.ws.scores + (int64_t)b * round_cand(a.max_cand);
}
__device__ __forceinline__ uint32_t* maxima_ptr(const Args& a, int b) {
  return a.ws.maxima + (size_t)b * round_cand(a.max_cand);
}
__device__ __forceinline__ size_t sel_chunk_base(const Args& a, int b) {
  return (size_t)b * (size_t)(round_cand(a.max_cand) / kSelChunk);
}

// ---------------------------------------------------------------- block scans
// Exclusive prefix sum over blockDim.x (a multiple of 64, at most 1024) threads.
// scratch: at least blockDim.x / 64 words. Returns the exclusive prefix; *total gets the sum.
__device__ uint32_t block_exclusive_sum(uint32_t v, uint32_t* total, uint32_t* scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  if (lane == 63) scratch[wave] = inc;
  __syncthreads();
  uint32_t before = 0, all = 0;
  for (int w = 0; w < nw; ++w) {
    const uint32_t t = scratch[w];
    before += (w < wave) ? t : 0u;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + inc - v;
}

// Block-wide maximum (blockDim.x a multiple of 64); scratch as above.
__device__ uint32_t block_max(uint32_t v, uint32_t* scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  uint32_t all = 0;
  for (int w = 0; w < nw; ++w) all = max(all, scratch[w]);
  __syncthreads();
  return all;
}

// Given a 256-bin histogram and a rank r >= 1 counted from the top, wave 0 finds the bin that
// holds the r-th largest element and the count strictly above it; results in out[0], out[1].
__device__ void top_rank_bin256(const uint32_t* hist, uint32_t r, uint32_t* out) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    // Lane l owns bins 255-4l .. 252-4l (descending scan order).
    uint32_t c[4], local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) { c[i] = hist[255 - 4 * lane - i]; local += c[i]; }
    uint32_t inc = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t t = __shfl_up(inc, o, 64);
      if (lane >= o) inc += t;
    }
    uint32_t run = inc - local;
    if (run < r && inc >= r) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (run + c[i] >= r) { out[0] = 255 - 4 * lane - i; out[1] = run; break; }
        run += c[i];
      }
    }
  }
}

// ---------------------------------------------------------------- K1: scores + sub-chunk maxima
template <typename ET>
struct Dot16;

template <>
struct Dot16<uint16_t> {   // 8 bf16 per 16 bytes: four v_dot2_f32_bf16
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  // Element j is copied to a scalar before the bit cast: clang lowers a bit cast applied
  // directly to an ext-vector element access as a cast of element 0.
  __device__ static bf16x2 pair(uint32_t x) { return __builtin_bit_cast(bf16x2, x); }
  __device__ static float dot(const u32x4& a, const u32x4& b, float acc) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t x = a[j], y = b[j];
      acc = __builtin_amdgcn_fdot2_f32_bf16(pair(x), pair(y), acc, false);
    }
    return acc;
  }
};

template <>
struct Dot16<float> {      // 4 fp32 per 16 bytes
  __device__ static float dot(const u32x4& a, const u32x4& b, float acc) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t x = a[j], y = b[j];
      acc = fmaf(__uint_as_float(x), __uint_as_float(y), acc);
    }
    return acc;
  }
};

// Sum over groups of `lpc` adjacent lanes (lpc a power of two <= 64); every lane of a group
// ends with the group total. Within a row of 16 lanes this uses DPP lane swizzles.
__device__ __forceinline__ float group_sum(float v, int lpc) {
  if (lpc >= 2) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));  // xor 1
  if (lpc >= 4) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));  // xor 2
  if (lpc >= 8) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)); // half-row mirror
  if (lpc >= 16) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)); // row mirror
  if (lpc >= 32) v += __shfl_xor(v, 16, 64);
  if (lpc >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// Write the maxima of the sub-chunks that [j0, j1) covers (j0 a multiple of sc; LDS holds them
// from index 0).
__device__ __forceinline__ void store_maxima(const Args& a, int b, int64_t j0, int64_t j1, const uint32_t* smax) {
  const int cnt = (int)((j1 - j0 + a.sc - 1) / a.sc);
  uint32_t* g = maxima_ptr(a, b) + j0 / a.sc;
  for (int i = threadIdx.x; i < cnt; i += blockDim.x) g[i] = smax[i];
}

template <typename ET, int NH, int MAXV>
__global__ __launch_bounds__(kThreads) void score_kernel(Args a) {
  __shared__ uint32_t smax[kScoreChunk];
  const int b = blockIdx.y;
  int64_t c0;
  const int64_t n = cand_count(a, b, &c0);
  const int64_t chunk0 = (int64_t)blockIdx.x * kScoreChunk;
  if (chunk0 >= n) return;
  const int64_t chunk_end = min<int64_t>(chunk0 + kScoreChunk, n);
  if (threadIdx.x < kScoreChunk) smax[threadIdx.x] = 0u;   // 0: below every key

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lpc = a.lpc;
  const int sub = lane & (lpc - 1);
  const int slot = (wave * 64 + lane) / lpc;          // candidate slot within a pass
  const int per_pass = kThreads / lpc;
  const u32x4* kb = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.keys) + (size_t)c0 * a.nvec * 16);
  // Issue the chunk's key loads first (U passes of per_pass candidates), then the query slices.
  constexpr int U = 4;
  u32x4 kv[U][MAXV];
  int64_t j[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    j[u] = chunk0 + u * per_pass + slot;
#pragma unroll
    for (int v = 0; v < MAXV; ++v) {
      const int vi = sub + v * lpc;
      kv[u][v] = (j[u] < chunk_end && vi < a.nvec) ? __builtin_nontemporal_load(kb + j[u] * a.nvec + vi)
                                                   : u32x4{0, 0, 0, 0};
    }
  }
  u32x4 qv[NH][MAXV];                                 // this lane's slice of every query
  float wv[NH];
  const u32x4* qb = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.q) +
                                                   (size_t)b * a.nh * a.nvec * 16);
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    wv[h] = h < a.nh ? a.w[(size_t)b * a.nh + h] : 0.f;
#pragma unroll
    for (int v = 0; v < MAXV; ++v) {
      const int vi = sub + v * lpc;
      qv[h][v] = (h < a.nh && vi < a.nvec) ? qb[h * a.nvec + vi] : u32x4{0, 0, 0, 0};
    }
  }
  __syncthreads();
  float* sp = score_ptr(a, b, c0);
  // per_pass * U >= kScoreChunk whenever lpc <= 8; wider rows take more rounds.
  for (int64_t base = chunk0; base < chunk_end; base += per_pass * U) {
    if (base != chunk0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        j[u] = base + u * per_pass + slot;
#pragma unroll
        for (int v = 0; v < MAXV; ++v) {
          const int vi = sub + v * lpc;
          kv[u][v] = (j[u] < chunk_end && vi < a.nvec) ? __builtin_nontemporal_load(kb + j[u] * a.nvec + vi)
                                                       : u32x4{0, 0, 0, 0};
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float s = 0.f;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        float dot = 0.f;
#pragma unroll
        for (int v = 0; v < MAXV; ++v) dot = Dot16<ET>::dot(qv[h][v], kv[u][v], dot);
        dot = group_sum(dot, lpc);
        s = fmaf(wv[h], fmaxf(dot, 0.f), s);
      }
      if (sub == 0 && j[u] < chunk_end) {
        sp[j[u]] = s;
        atomicMax(&smax[(int)(j[u] - chunk0) / a.sc], score_key(s));
      }
    }
  }
  __syncthreads();
  store_maxima(a, b, chunk0, chunk_end, smax);
}

// K1 for caller-provided scores: sub-chunk maxima only (8 scores per thread, 16-byte loads
// when the row is 16-byte aligned).
__global__ __launch_bounds__(kThreads) void max_kernel(Args a) {
  __shared__ uint32_t smax[kMaxChunk];
  const int b = blockIdx.y;
  int64_t c0;
  const int64_t n = cand_count(a, b, &c0);
  const int64_t chunk0 = (int64_t)blockIdx.x * kMaxChunk;
  if (chunk0 >= n) return;
  const int64_t chunk_end = min<int64_t>(chunk0 + kMaxChunk, n);
  for (int i = threadIdx.x; i < kMaxChunk; i += kThreads) smax[i] = 0u;
  const float* sp = score_ptr(a, b, c0);
  float v[8];
  const int64_t j = chunk0 + 4 * threadIdx.x;   // this thread: j..j+3 and j+1024..j+1027
  const bool vec = ((reinterpret_cast<uintptr_t>(sp) & 15) == 0);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t jj = j + h * 1024;
    if (vec && jj + 3 < chunk_end) {
      const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sp + jj));
      v[4 * h] = x[0]; v[4 * h + 1] = x[1]; v[4 * h + 2] = x[2]; v[4 * h + 3] = x[3];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * h + e] = (jj + e < chunk_end) ? sp[jj + e] : 0.f;
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t jj = j + h * 1024 + e;
      if (jj < chunk_end) atomicMax(&smax[(int)(jj - chunk0) / a.sc], score_key(v[4 * h + e]));
    }
  __syncthreads();
  store_maxima(a, b, chunk0, chunk_end, smax);
}

// ---------------------------------------------------------------- K2: the bound L
// L = the k-th largest of the sequence's sub-chunk maxima (the first kMaxMaxima of them when
// there are more: any k disjoint sub-chunks give a valid bound), rounded down to its top 22
// bits; 0 (no pruning) when there are fewer than k maxima. Also the largest maximum, which is
// the largest key of the sequence.
__global__ __launch_bounds__(kBoundThreads) void bound_kernel(Args a) {
  __shared__ uint32_t vals[kMaxMaxima];
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t scratch[40];
  const int b = blockIdx.x;
  int64_t c0;
  const int64_t n = cand_count(a, b, &c0);
  const uint32_t keff = (uint32_t)min<int64_t>(a.k, n);
  const int64_t m_all = (n + a.sc - 1) / a.sc;
  const int m = (int)min<int64_t>(m_all, kMaxMaxima);
  const uint32_t* g = maxima_ptr(a, b);
  uint32_t vmax = 0;
  for (int i = threadIdx.x; i < m; i += kBoundThreads) { vals[i] = g[i]; vmax = max(vmax, vals[i]); }
  vmax = block_max(vmax, scratch);   // (the maxima beyond kMaxMaxima only matter for pruning)
  if (m_all > m) {
    for (int64_t i = m + threadIdx.x; i < m_all; i += kBoundThreads) vmax = max(vmax, g[i]);
    vmax = block_max(vmax, scratch);
  }
  uint32_t L = 0;
  if (n > (int64_t)keff && m_all >= (int64_t)keff && keff > 0) {
    uint32_t prefix = 0, r = keff;
    for (int p = 0; p < 2; ++p) {
      const int shift = p == 0 ? 21 : 10;
      for (int i = threadIdx.x; i < 2048; i += kBoundThreads) hist[i] = 0u;
      __syncthreads();
      for (int i = threadIdx.x; i < m; i += kBoundThreads) {
        const uint32_t v = vals[i];
        if (p == 0 || (v >> 21) == prefix) atomicAdd(&hist[(v >> shift) & 2047u], 1u);
      }
      __syncthreads();
      // The bin of the r-th largest: each thread owns 2 bins in descending order.
      const uint32_t c1 = hist[2047 - 2 * threadIdx.x], c2 = hist[2046 - 2 * threadIdx.x];
      uint32_t total;
      const uint32_t run = block_exclusive_sum(c1 + c2, &total, scratch);
      if (run < r && run + c1 >= r) { scratch[32] = 2047 - 2 * threadIdx.x; scratch[33] = run; }
      else if (run + c1 < r && run + c1 + c2 >= r) { scratch[32] = 2046 - 2 * threadIdx.x; scratch[33] = run + c1; }
      __syncthreads();
      const uint32_t bin = scratch[32];
      r -= scratch[33];
      prefix = (p == 0) ? bin : ((prefix << 11) | bin);
      __syncthreads();
    }
    L = prefix << 10;
  }
  if (threadIdx.x == 0) { a.ws.bound[2 * b] = L; a.ws.bound[2 * b + 1] = vmax; }
}

// ---------------------------------------------------------------- K3: the superset
__global__ __launch_bounds__(kThreads) void select_kernel(Args a) {
  __shared__ uint32_t scratch[8];
  const int b = blockIdx.y;
  int64_t c0;
  const int64_t n = cand_count(a, b, &c0);
  const int64_t chunk0 = (int64_t)blockIdx.x * kSelChunk;
  if (chunk0 >= n) return;
  const int64_t chunk_end = min<int64_t>(chunk0 + kSelChunk, n);
  const uint32_t L = a.ws.bound[2 * b];
  const float* sp = score_ptr(a, b, c0);
  // Thread t owns candidates chunk0 + 4t .. 4t+3 (consecutive, so index order is kept).
  const int64_t j = chunk0 + 4 * threadIdx.x;
  float v[4];
  if (((reinterpret_cast<uintptr_t>(sp) & 15) == 0) && j + 3 < chunk_end) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(sp + j);
    v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (j + e < chunk_end) ? sp[j + e] : 0.f;
  }
  uint32_t key[4], cnt = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    key[e] = score_key(v[e]);
    cnt += (j + e < chunk_end && key[e] >= L) ? 1u : 0u;
  }
  uint32_t total;
  uint32_t pos = block_exclusive_sum(cnt, &total, scratch);
  const size_t cidx = sel_chunk_base(a, b) + blockIdx.x;
  uint32_t* reg = a.ws.region + cidx * kSelChunk * 2;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (j + e < chunk_end && key[e] >= L) {
      reg[2 * pos] = key[e];
      reg[2 * pos + 1] = (uint32_t)(j + e);
      ++pos;
    }
  }
  if (threadIdx.x == 0) a.ws.counts[cidx] = total;
}

// ---------------------------------------------------------------- K4: exact selection
struct FinalShared {
  uint32_t key[kLdsCand];
  uint32_t idx[kLdsCand];
  uint32_t off[kMaxSelChunks + 1];
  uint32_t hist[256];
  uint32_t scratch[40];
};

// Superset accessors: LDS (small supersets) or the workspace's global copy.
struct LdsSet {
  FinalShared* sh;
  __device__ uint32_t key(uint32_t i) const { return sh->key[i]; }
  __device__ uint32_t idx(uint32_t i) const { return sh->idx[i]; }
};
struct GlobalSet {
  const uint32_t* g;
  __device__ uint32_t key(uint32_t i) const { return g[2 * (size_t)i]; }
  __device__ uint32_t idx(uint32_t i) const { return g[2 * (size_t)i + 1]; }
};

// Exact selection of the keff largest (key desc, then position asc) of T candidates held in
// index order, all with keys in [lo, hi]; writes their indices ascending to out[0..keff) and
// -1 to out[keff..k).
template <typename S>
__device__ void select_exact(const S& set, uint32_t T, uint32_t keff, uint32_t lo, uint32_t hi, int32_t* out,
                             int32_t k, FinalShared& sh) {
  uint32_t tau = 0, ties_take = 0xFFFFFFFFu;
  if (T > keff) {
    // Bits above `start` are shared by every key in [lo, hi]: skip those radix passes.
    const int diff_bits = (lo == hi) ? 0 : 32 - __clz(lo ^ hi);
    const int npass = (diff_bits + 7) / 8;
    uint32_t r = keff;
    uint32_t prefix = (npass >= 4) ? 0u : (hi >> (8 * npass));   // the shared high bits
    for (int p = npass - 1; p >= 0; --p) {
      const int shift = 8 * p;
      for (int i = threadIdx.x; i < 256; i += blockDim.x) sh.hist[i] = 0u;
      __syncthreads();
      for (uint32_t i = threadIdx.x; i < T; i += blockDim.x) {
        const uint32_t kk = set.key(i);
        const bool match = (p == 3) || ((kk >> (shift + 8)) == prefix);
        if (match) atomicAdd(&sh.hist[(kk >> shift) & 255u], 1u);
      }
      __syncthreads();
      top_rank_bin256(sh.hist, r, sh.scratch + 32);
      __syncthreads();
      r -= sh.scratch[33];
      prefix = (prefix << 8) | sh.scratch[32];
      __syncthreads();
    }
    tau = prefix;
    ties_take = r;   // the first r candidates (in index order) with key == tau are taken
  }
  // Ordered pass: tiles of blockDim.x consecutive candidates, one per thread, with carries.
  uint32_t ties_before = 0, sel_before = 0;
  for (uint32_t t0 = 0; t0 < T; t0 += blockDim.x) {
    const uint32_t i = t0 + threadIdx.x;
    uint32_t kk = 0, ix = 0;
    if (i < T) { kk = set.key(i); ix = set.idx(i); }
    const bool is_tie = i < T && T > keff && kk == tau;
    uint32_t tie_total;
    const uint32_t tie_rank = ties_before + block_exclusive_sum(is_tie ? 1u : 0u, &tie_total, sh.scratch);
    const bool sel = i < T && (T <= keff || kk > tau || (is_tie && tie_rank < ties_take));
    uint32_t sel_total;
    const uint32_t pos = sel_before + block_exclusive_sum(sel ? 1u : 0u, &sel_total, sh.scratch);
    if (sel && pos < keff) out[pos] = (int32_t)ix;
    ties_before += tie_total;
    sel_before += sel_total;
  }
  for (int i = (int)keff + threadIdx.x; i < k; i += blockDim.x) out[i] = -1;
}

__global__ __launch_bounds__(kFinalThreads) void final_kernel(Args a, int32_t* topk) {
  __shared__ FinalShared sh;
  const int b = blockIdx.x;
  int64_t c0;
  const int64_t n = cand_count(a, b, &c0);
  int32_t* out = topk + (size_t)b * a.k;
  const uint32_t keff = (uint32_t)min<int64_t>(a.k, n);
  if (keff == 0) {
    for (int i = threadIdx.x; i < a.k; i += blockDim.x) out[i] = -1;
    return;
  }
  const int nch = (int)((n + kSelChunk - 1) / kSelChunk);
  const size_t cb = sel_chunk_base(a, b);
  // Offsets of the chunk regions in the ordered superset.
  uint32_t carry = 0;
  for (int first = 0; first < nch; first += blockDim.x) {
    const int c = first + threadIdx.x;
    const uint32_t v = c < nch ? min(a.ws.counts[cb + c], (uint32_t)kSelChunk) : 0u;
    uint32_t total;
    const uint32_t ex = block_exclusive_sum(v, &total, sh.scratch);
    if (c < nch) sh.off[c] = carry + ex;
    carry += total;
  }
  if (threadIdx.x == 0) sh.off[nch] = carry;
  __syncthreads();
  const uint32_t T = carry;
  const uint32_t* reg = a.ws.region + cb * kSelChunk * 2;
  // Gather: entry e lives in the chunk c with off[c] <= e < off[c+1] (binary search).
  const bool in_lds = T <= (uint32_t)kLdsCand;
  uint32_t* gdst = a.ws.gather + (size_t)b * round_cand(a.max_cand) * 2;
  for (uint32_t e = threadIdx.x; e < T; e += blockDim.x) {
    int lo = 0, hi = nch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sh.off[mid] <= e) lo = mid; else hi = mid - 1;
    }
    const size_t src = ((size_t)lo * kSelChunk + (e - sh.off[lo])) * 2;
    const uint32_t kk = reg[src], ix = reg[src + 1];
    if (in_lds) { sh.key[e] = kk; sh.idx[e] = ix; }
    else { gdst[2 * (size_t)e] = kk; gdst[2 * (size_t)e + 1] = ix; }
  }
  __syncthreads();
  const uint32_t lo_key = a.ws.bound[2 * b], hi_key = a.ws.bound[2 * b + 1];
  if (in_lds) select_exact(LdsSet{&sh}, T, keff, lo_key, hi_key, out, a.k, sh);
  else select_exact(GlobalSet{gdst}, T, keff, lo_key, hi_key, out, a.k, sh);
}

template <typename ET, int NH>
void launch_scores_nh(dim3 grid, hipStream_t s, const Args& a, int maxv) {
  switch (maxv) {
    case 1: hipLaunchKernelGGL((score_kernel<ET, NH, 1>), grid, dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((score_kernel<ET, NH, 2>), grid, dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL((score_kernel<ET, NH, 4>), grid, dim3(kThreads), 0, s, a); break;
  }
}

template <typename ET>
void launch_scores(dim3 grid, hipStream_t s, const Args& a, int maxv) {
  if (a.nh <= 1) launch_scores_nh<ET, 1>(grid, s, a, maxv);
  else if (a.nh <= 2) launch_scores_nh<ET, 2>(grid, s, a, maxv);
  else if (a.nh <= 4) launch_scores_nh<ET, 4>(grid, s, a, maxv);
  else if (a.nh <= 8) launch_scores_nh<ET, 8>(grid, s, a, maxv);
  else launch_scores_nh<ET, 16>(grid, s, a, maxv);
}

// Sub-chunk size: up to 64 candidates, smaller when the longest sequence would otherwise give
// fewer than 2k maxima, larger (up to a score chunk) when it would give more than kMaxMaxima.
int pick_subchunk(int64_t max_cand, int32_t k) {
  int sc = 64;
  while (sc > 1 && max_cand / sc < 2LL * k) sc >>= 1;
  while (sc < kScoreChunk && max_cand / sc > kMaxMaxima) sc <<= 1;
  return sc;
}

}  // namespace
}  // namespace chs

extern "C" size_t chs_index_topk_workspace_size(int32_t batch, int64_t max_cand, int32_t k) {
  (void)k;
  if (batch < 1 || max_cand < 0) return 0;
  return chs::ws_layout(batch, max_cand, nullptr, nullptr);
}

extern "C" chs_status chs_index_topk(chs_dtype dtype, int32_t batch, int32_t n_heads,
                                     int32_t head_dim, int32_t k, const void* q_idx,
                                     const float* w, const void* k_idx, const int64_t* cu_cand,
                                     int64_t max_cand, float* scores, int32_t* topk,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  using namespace chs;
  if (!dtype_ok(dtype)) return CHS_ERR_DTYPE;
  if (batch < 1 || batch > 65535 || k < 1 || k > kMaxK || max_cand < 0 || max_cand >= (1LL << 31))
    return CHS_ERR_SHAPE;
  if (max_cand > kMaxCand) return CHS_ERR_UNSUPPORTED;
  const size_t es = elem_size(dtype);
  int nvec = 0, lpc = 1, maxv = 1;
  if (q_idx) {
    if (n_heads < 1 || n_heads > 16 || head_dim < 8 || head_dim > 512 || (head_dim * es) % 16 != 0)
      return CHS_ERR_SHAPE;
    if (!w || !k_idx) return CHS_ERR_NULL;
    nvec = (int)(head_dim * es / 16);
    // Lanes per candidate: the largest power of two <= nvec/2 (at most 64); each lane then
    // covers at most 4 of the row's 16-byte vectors.
    while (lpc * 2 <= nvec / 2 && lpc < 64) lpc *= 2;
    maxv = (nvec + lpc - 1) / lpc;
    if (maxv > 4) return CHS_ERR_UNSUPPORTED;
    maxv = maxv == 3 ? 4 : maxv;
  } else if (!scores) {
    return CHS_ERR_NULL;
  }
  if (!cu_cand || !topk || !workspace) return CHS_ERR_NULL;
  Workspace ws;
  const size_t need = ws_layout(batch, max_cand, &ws, static_cast<char*>(workspace));
  if (workspace_bytes < need) return CHS_ERR_WORKSPACE;
  Args a;
  a.q = q_idx; a.w = w; a.keys = k_idx; a.cu = cu_cand; a.max_cand = max_cand;
  a.nh = n_heads; a.nvec = nvec; a.lpc = lpc; a.k = k; a.scores = scores; a.ws = ws;
  a.sc = pick_subchunk(max_cand, k);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (max_cand > 0) {
    if (q_idx) {
      const dim3 grid((unsigned)((max_cand + kScoreChunk - 1) / kScoreChunk), (unsigned)batch);
      if (dtype == CHS_BF16) launch_scores<uint16_t>(grid, s, a, maxv);
      else launch_scores<float>(grid, s, a, maxv);
    } else {
      const dim3 grid((unsigned)((max_cand + kMaxChunk - 1) / kMaxChunk), (unsigned)batch);
      hipLaunchKernelGGL(max_kernel, grid, dim3(kThreads), 0, s, a);
    }
    if (launch_status() != CHS_OK) return CHS_ERR_LAUNCH;
    hipLaunchKernelGGL(bound_kernel, dim3((unsigned)batch), dim3(kBoundThreads), 0, s, a);
    if (launch_status() != CHS_OK) return CHS_ERR_LAUNCH;
    const dim3 sgrid((unsigned)((max_cand + kSelChunk - 1) / kSelChunk), (unsigned)batch);
    hipLaunchKernelGGL(select_kernel, sgrid, dim3(kThreads), 0, s, a);
    if (launch_status() != CHS_OK) return CHS_ERR_LAUNCH;
  }
  hipLaunchKernelGGL(final_kernel, dim3((unsigned)batch), dim3(kFinalThreads), 0, s, a, topk);
  return launch_status();
}
