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
// kernel here synchronises workgroups with each other; kernel boundaries order the phases:
//   K1 score_kernel (persistent grid, query slices in registers, next chunk's loads issued
//      before the current chunk is scored) streams the index keys once and writes the fp32
//      scores plus a maximum order-preserving key per group of candidates; max_kernel does
//      the same for caller-provided scores.
//   K2 bound_kernel (one workgroup per sequence): L = k-th largest group maximum, a lower
//      bound on the k-th largest score (k disjoint groups each hold a score >= L).
//   K3 select_kernel: every chunk of 1024 candidates keeps the ones with key >= L in index
//      order and writes them, with their count, to its own region.
//   K4 final_kernel (one workgroup per sequence): gathers the regions and selects exactly,
//      by one-at-a-time removal when the superset exceeds k by at most 64, else by radix
//      steps to the k-th largest key tau and an ordered pass (keys above tau, then the first
//      ties at tau), written ascending by a prefix count.
// The composite order (key descending, then index ascending) is total, so the selected set is
// unique and bit-identical to a full sort of the same scores.
#include <algorithm>

#include "common.h"

namespace chs {
namespace {

constexpr int kThreads = 256;        // every kernel here
constexpr int kPasses = 8;           // K1 passes per chunk (one 16-byte load each per lane)
constexpr int kScoreGrid = 1024;     // K1 workgroups per launch (all sequences together)
constexpr int kMaxChunk = 2048;      // scores per max_kernel chunk (256 threads x 8)
constexpr int kSelChunk = 1024;      // candidates per K3 workgroup (256 threads x 4)
constexpr int kMaxMaxima = 8192;     // group maxima K2 ranks (the first ones if more)
constexpr int kLdsCand = 8192;       // superset size K4 keeps in LDS
constexpr int kMaxSelChunks = 4096;  // K3 chunks per sequence (max_cand <= 4M)
constexpr int kPeekChunks = 512;     // K4 fetches region heads with the counts up to this many chunks
constexpr int kPeek = 8;             // entries per region head
constexpr int kRemoveMax = 64;       // K4 removes one by one when T - k <= this
constexpr int kMaxK = 2048;
constexpr int kRegMax = (kMaxK + kRemoveMax + 63) / 64;   // superset entries per lane (removal path)
constexpr int64_t kMaxCand = (int64_t)kMaxSelChunks * kSelChunk;

struct Workspace {
  uint32_t* maxima;   // [batch][rc]: group maximum keys
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
  int32_t chunk;        // K1 candidates per chunk
  int32_t gpc;          // group maxima per K1 chunk: score 1, 4 or 32; max 1, 4 or 16
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

// ---------------------------------------------------------------- reductions and scans
// Exclusive prefix sum over blockDim.x (a multiple of 64) threads; scratch: blockDim.x / 64
// words. Returns the exclusive prefix; *total gets the sum.
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

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}

__device__ uint32_t block_max(uint32_t v, uint32_t* scratch) {
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) scratch[wave] = v;
  __syncthreads();
  uint32_t all = 0;
  for (int w = 0; w < nw; ++w) all = max(all, scratch[w]);
  __syncthreads();
  return all;
}

__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Radix digits below the bits shared by every key in [lo, hi]: the first digit covers the
// top `width` differing bits. Returns the number of differing bits.
__device__ __forceinline__ int differing_bits(uint32_t lo, uint32_t hi) {
  return lo == hi ? 0 : 32 - __clz(lo ^ hi);
}

// One radix step over `m` keys (from `get`) that all share their bits above `shift + width`:
// histogram (nb >= 2^width bins, nb = 8 * blockDim.x... see callers) of the `width`-bit digit
// at `shift` over keys whose bits from `shift + width` up equal `prefix`, then the digit
// holding the r-th largest. Returns the digit; *above gets the count with larger digits.
template <typename Get>
__device__ uint32_t radix_step(Get get, uint32_t m, int shift, int width, uint32_t prefix, uint32_t r,
                               uint32_t* hist, uint32_t* scratch, uint32_t* above) {
  const int nb = 1 << width;                       // width <= 11: at most 2048 bins
  for (int i = threadIdx.x; i < 2048; i += blockDim.x) hist[i] = 0u;
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < m; i += blockDim.x) {
    const uint32_t v = get(i);
    if ((uint32_t)((uint64_t)v >> (shift + width)) == prefix) atomicAdd(&hist[(v >> shift) & (nb - 1)], 1u);
  }
  __syncthreads();
  // Thread t owns digits 2047-8t .. 2040-8t (descending).
  uint32_t c[8], local = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) { c[i] = hist[2047 - 8 * threadIdx.x - i]; local += c[i]; }
  uint32_t total;
  uint32_t run = block_exclusive_sum(local, &total, scratch);
  if (run < r && run + local >= r) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (run + c[i] >= r) { scratch[32] = 2047 - 8 * threadIdx.x - i; scratch[33] = run; break; }
      run += c[i];
    }
  }
  __syncthreads();
  const uint32_t digit = scratch[32];
  *above = scratch[33];
  __syncthreads();
  return digit;
}

// The r-th largest of m keys in [lo, hi] (1 <= r <= m), by 11-bit radix steps below the bits
// lo and hi share; `steps` caps the number of steps (lower bits are then returned as 0, so the
// result is rounded down). *rank_left gets r minus the number of keys above the result's
// last-resolved digit (the rank among keys equal to the result when all bits are resolved).
template <typename Get>
__device__ uint32_t radix_select_desc(Get get, uint32_t m, uint32_t r, uint32_t lo, uint32_t hi, int steps,
                                      uint32_t* hist, uint32_t* scratch, uint32_t* rank_left) {
  int rem = differing_bits(lo, hi);
  uint32_t prefix = rem == 32 ? 0u : (uint32_t)((uint64_t)hi >> rem);
  for (int s = 0; s < steps && rem > 0; ++s) {
    const int width = rem < 11 ? rem : 11;
    rem -= width;
    uint32_t above;
    const uint32_t d = radix_step(get, m, rem, width, prefix, r, hist, scratch, &above);
    r -= above;
    prefix = (prefix << width) | d;
  }
  *rank_left = r;
  return (uint32_t)((uint64_t)prefix << rem);
}

// ---------------------------------------------------------------- K1: scores + group maxima
template <typename ET>
struct Dot16;

template <>
struct Dot16<uint16_t> {   // 8 bf16 per 16 bytes: four v_dot2_f32_bf16
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  // Element j is copied to a scalar before the bit cast: clang lowers a bit cast applied
  // directly to an ext-vector element access as a cast of element 0.
  __device__ static bf16x2 pair(uint32_t x) { return __builtin_bit_cast(bf16x2, x); }
  __device__ static float dot(const u32x4& a, const u32x4& b) {
    float acc = 0.f;
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
  __device__ static float dot(const u32x4& a, const u32x4& b) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t x = a[j], y = b[j];
      acc = fmaf(__uint_as_float(x), __uint_as_float(y), acc);
    }
    return acc;
  }
};

// Sum over groups of LPC adjacent lanes (a power of two <= 64); every lane of a group ends
// with the group total. Within a row of 16 lanes this uses DPP lane swizzles.
template <int LPC>
__device__ __forceinline__ float group_sum(float v) {
  if (LPC >= 2) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));  // xor 1
  if (LPC >= 4) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));  // xor 2
  if (LPC >= 8) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)); // half-row mirror
  if (LPC >= 16) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)); // row mirror
  if (LPC >= 32) v += __shfl_xor(v, 16, 64);
  if (LPC >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

template <int LPC>
__device__ __forceinline__ void load_chunk(const u32x4* kb, int nvec, int64_t chunk0, int64_t n, int slot, int sub,
                                           u32x4 (&kv)[kPasses]) {
  constexpr int PER = kThreads / LPC;
#pragma unroll
  for (int u = 0; u < kPasses; ++u) {
    const int64_t j = chunk0 + u * PER + slot;
    kv[u] = (j < n && sub < nvec) ? __builtin_nontemporal_load(kb + j * nvec + sub) : u32x4{0, 0, 0, 0};
  }
}

// Score one chunk from registers; write scores and the chunk's group maxima.
template <typename ET, int NH, int LPC>
__device__ __forceinline__ void score_chunk(const Args& a, int64_t chunk, int64_t n, int slot, int sub,
                                            const u32x4 (&qv)[NH], const float (&wv)[NH], const u32x4 (&kv)[kPasses],
                                            float* sp, uint32_t* gmax, uint32_t* smax) {
  constexpr int PER = kThreads / LPC;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t mx = 0;
#pragma unroll
  for (int u = 0; u < kPasses; ++u) {
    const int64_t j = chunk * a.chunk + u * PER + slot;
    float s = 0.f;
#pragma unroll
    for (int h = 0; h < NH; ++h) s = fmaf(wv[h], fmaxf(group_sum<LPC>(Dot16<ET>::dot(qv[h], kv[u])), 0.f), s);
    const bool valid = j < n;
    if (sub == 0 && valid) sp[j] = s;
    const uint32_t key = valid ? score_key(s) : 0u;   // 0: below every key
    if (a.gpc == 32) {                                 // group = this wave's candidates of pass u
      const uint32_t m = wave_max(key);
      if (lane == 0) gmax[(chunk * 4 + wave) * kPasses + u] = m;
    }
    mx = max(mx, key);
  }
  if (a.gpc == 4) {                                    // group = this wave's candidates of the chunk
    const uint32_t m = wave_max(mx);
    if (lane == 0) gmax[chunk * 4 + wave] = m;
  } else if (a.gpc == 1) {                             // group = the chunk
    const uint32_t m = wave_max(mx);
    if (lane == 0) smax[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) gmax[chunk] = max(max(smax[0], smax[1]), max(smax[2], smax[3]));
    __syncthreads();
  }
}

template <typename ET, int NH, int LPC>
__global__ __launch_bounds__(kThreads) void score_kernel(Args a) {
  constexpr int PER = kThreads / LPC;
  __shared__ uint32_t smax[4];
  const int b = blockIdx.y;
  int64_t c0;
  const int64_t n = cand_count(a, b, &c0);
  const int64_t nch = (n + a.chunk - 1) / a.chunk;
  int64_t chunk = blockIdx.x;
  if (chunk >= nch) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & (LPC - 1);
  const int slot = (wave * 64 + lane) / LPC;          // candidate slot within a pass
  const u32x4* kb = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.keys) + (size_t)c0 * a.nvec * 16);
  u32x4 ka[kPasses], kc[kPasses];
  load_chunk<LPC>(kb, a.nvec, chunk * a.chunk, n, slot, sub, ka);
  u32x4 qv[NH];                                       // this lane's 16 bytes of every query
  float wv[NH];
  const u32x4* qb = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.q) + (size_t)b * a.nh * a.nvec * 16);
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    wv[h] = h < a.nh ? a.w[(size_t)b * a.nh + h] : 0.f;
    qv[h] = (h < a.nh && sub < a.nvec) ? qb[h * a.nvec + sub] : u32x4{0, 0, 0, 0};
  }
  float* sp = score_ptr(a, b, c0);
  uint32_t* gmax = maxima_ptr(a, b);
  (void)PER;
  // Two register buffers: the next chunk's loads are in flight while the current one is scored.
  for (;;) {
    const int64_t next = chunk + gridDim.x;
    if (next < nch) load_chunk<LPC>(kb, a.nvec, next * a.chunk, n, slot, sub, kc);
    score_chunk<ET, NH, LPC>(a, chunk, n, slot, sub, qv, wv, ka, sp, gmax, smax);
    if (next >= nch) break;
    chunk = next;
    const int64_t next2 = chunk + gridDim.x;
    if (next2 < nch) load_chunk<LPC>(kb, a.nvec, next2 * a.chunk, n, slot, sub, ka);
    score_chunk<ET, NH, LPC>(a, chunk, n, slot, sub, qv, wv, kc, sp, gmax, smax);
    if (next2 >= nch) break;
    chunk = next2;
  }
}

// K1 for caller-provided scores: group maxima only. Chunks of 2048 scores (8 per thread, two
// 16-byte loads); a group is a chunk, a wave's 512 scores, or a 16-lane row's 128 scores.
__global__ __launch_bounds__(kThreads) void max_kernel(Args a) {
  __shared__ uint32_t smax[4];
  const int b = blockIdx.y;
  int64_t c0;
  const int64_t n = cand_count(a, b, &c0);
  const int64_t nch = (n + kMaxChunk - 1) / kMaxChunk;
  const float* sp = score_ptr(a, b, c0);
  uint32_t* gmax = maxima_ptr(a, b);
  const bool vec = ((reinterpret_cast<uintptr_t>(sp) & 15) == 0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int64_t chunk = blockIdx.x; chunk < nch; chunk += gridDim.x) {
    const int64_t chunk0 = chunk * kMaxChunk;
    uint32_t m = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t j = chunk0 + h * 1024 + 4 * threadIdx.x;
      float v[4];
      if (vec && j + 3 < n) {
        const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sp + j));
        v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (j + e < n) ? sp[j + e] : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) m = max(m, (j + e < n) ? score_key(v[e]) : 0u);
    }
    if (a.gpc == 16) {
      m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false));
      m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false));
      m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x141, 0xF, 0xF, false));
      m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x140, 0xF, 0xF, false));
      if ((lane & 15) == 0) gmax[chunk * 16 + wave * 4 + (lane >> 4)] = m;
    } else {
      m = wave_max(m);
      if (a.gpc == 4) {
        if (lane == 0) gmax[chunk * 4 + wave] = m;
      } else {
        if (lane == 0) smax[wave] = m;
        __syncthreads();
        if (threadIdx.x == 0) gmax[chunk] = max(max(smax[0], smax[1]), max(smax[2], smax[3]));
        __syncthreads();
      }
    }
  }
}

// ---------------------------------------------------------------- K2: the bound L
__global__ __launch_bounds__(kThreads) void bound_kernel(Args a) {
  constexpr int PER = kMaxMaxima / kThreads;   // 32 maxima per thread, in registers
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t scratch[40];
  const int b = blockIdx.x;
  int64_t c0;
  const int64_t n = cand_count(a, b, &c0);
  const uint32_t keff = (uint32_t)min<int64_t>(a.k, n);
  const int64_t m_all = (n + a.chunk - 1) / a.chunk * a.gpc;
  const int m = (int)min<int64_t>(m_all, kMaxMaxima);   // any k disjoint groups give a bound
  const uint32_t* g = maxima_ptr(a, b);
  uint32_t v[PER];
  uint32_t vmax = 0, vmin = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = i * kThreads + threadIdx.x;
    v[i] = e < m ? g[e] : 0u;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (i * kThreads + (int)threadIdx.x < m) { vmax = max(vmax, v[i]); vmin = min(vmin, v[i]); }
  }
  for (int64_t e = kMaxMaxima + threadIdx.x; e < m_all; e += kThreads) vmax = max(vmax, g[e]);
  vmax = block_max(vmax, scratch);
  vmin = ~block_max(~vmin, scratch);
  uint32_t L = 0;
  if (n > (int64_t)keff && m >= (int)keff && keff > 0) {
    // The maxima go through LDS once for the two radix steps.
    __shared__ uint32_t vals[kMaxMaxima];
#pragma unroll
    for (int i = 0; i < PER; ++i) vals[i * kThreads + threadIdx.x] = v[i];
    __syncthreads();
    uint32_t rank_left;
    L = radix_select_desc([&](uint32_t i) { return vals[i]; }, (uint32_t)m, keff, vmin, vmax, 2, hist, scratch,
                          &rank_left);
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
  uint32_t hist[2048];
  uint32_t scratch[40];
};

// Keep the first `keff` of T candidates (index order) in the composite order (key desc, then
// position asc); write their indices ascending. Case T - keff <= kRemoveMax, by wave 0 alone:
// remove the smallest candidate T - keff times.
__device__ void select_by_removal(const FinalShared& sh, uint32_t T, uint32_t keff, int32_t* out) {
  const int lane = threadIdx.x & 63;
  const uint32_t E = (T + 63) / 64;   // <= kRegMax
  const uint32_t i0 = min(T, lane * E);
  uint64_t comp[kRegMax];             // (key, position from the end): the minimum goes first
#pragma unroll
  for (int i = 0; i < kRegMax; ++i) {
    const uint32_t e = i0 + i;
    comp[i] = (i < (int)E && e < T) ? (((uint64_t)sh.key[e] << 32) | (uint64_t)(0xFFFFFFFFu - e)) : ~0ull;
  }
  for (uint32_t rnd = keff; rnd < T; ++rnd) {
    uint64_t mn = ~0ull;
    int at = -1;
#pragma unroll
    for (int i = 0; i < kRegMax; ++i) if (comp[i] < mn) { mn = comp[i]; at = i; }
    uint64_t w = mn;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint64_t t = ((uint64_t)(uint32_t)__shfl_xor((int)(w >> 32), o, 64) << 32) |
                         (uint32_t)__shfl_xor((int)(uint32_t)w, o, 64);
      w = t < w ? t : w;
    }
    if (mn == w && at >= 0) {
#pragma unroll
      for (int i = 0; i < kRegMax; ++i) if (i == at) comp[i] = ~0ull;
    }
  }
  uint32_t kept = 0;
#pragma unroll
  for (int i = 0; i < kRegMax; ++i) kept += comp[i] != ~0ull ? 1u : 0u;
  uint32_t pos = wave_inclusive_sum(kept) - kept;
#pragma unroll
  for (int i = 0; i < kRegMax; ++i) {
    if (comp[i] != ~0ull) {
      if (pos < keff) out[pos] = (int32_t)sh.idx[i0 + i];
      ++pos;
    }
  }
}

// General case: exact k-th largest key tau by radix steps, then an ordered pass that keeps
// keys above tau and the first ties at tau. The whole workgroup; candidates from `get_key`,
// `get_idx` (LDS or the workspace's global copy).
template <typename GK, typename GI>
__device__ void select_by_radix(GK get_key, GI get_idx, uint32_t T, uint32_t keff, uint32_t lo, uint32_t hi,
                                int32_t* out, FinalShared& sh) {
  uint32_t ties_take;
  const uint32_t tau = radix_select_desc(get_key, T, keff, lo, hi, 3, sh.hist, sh.scratch, &ties_take);
  uint32_t ties_before = 0, sel_before = 0;
  for (uint32_t t0 = 0; t0 < T; t0 += blockDim.x) {
    const uint32_t i = t0 + threadIdx.x;
    uint32_t kk = 0, ix = 0;
    if (i < T) { kk = get_key(i); ix = get_idx(i); }
    const bool is_tie = i < T && kk == tau;
    uint32_t tie_total;
    const uint32_t tie_rank = ties_before + block_exclusive_sum(is_tie ? 1u : 0u, &tie_total, sh.scratch);
    const bool sel = i < T && (kk > tau || (is_tie && tie_rank < ties_take));
    uint32_t sel_total;
    const uint32_t pos = sel_before + block_exclusive_sum(sel ? 1u : 0u, &sel_total, sh.scratch);
    if (sel && pos < keff) out[pos] = (int32_t)ix;
    ties_before += tie_total;
    sel_before += sel_total;
  }
}

__global__ __launch_bounds__(kThreads) void final_kernel(Args a, int32_t* topk) {
  __shared__ FinalShared sh;
  const int b = blockIdx.x;
  int64_t c0;
  const int64_t n = cand_count(a, b, &c0);
  int32_t* out = topk + (size_t)b * a.k;
  const uint32_t keff = (uint32_t)min<int64_t>(a.k, n);
  for (int i = (int)keff + threadIdx.x; i < a.k; i += blockDim.x) out[i] = -1;
  if (keff == 0) return;
  const int nch = (int)((n + kSelChunk - 1) / kSelChunk);
  const size_t cb = sel_chunk_base(a, b);
  const uint32_t* reg = a.ws.region + cb * kSelChunk * 2;
  const bool peek = nch <= kPeekChunks;
  // Round trip 1: every region's count and (small sequences) its first kPeek entries.
  u32x4 head[kPeek / 2 * ((kPeekChunks + kThreads - 1) / kThreads)];
  uint32_t carry = 0;
  for (int first = 0, it = 0; first < nch; first += kThreads, ++it) {
    const int c = first + threadIdx.x;
    uint32_t v = 0;
    if (c < nch) {
      v = min(a.ws.counts[cb + c], (uint32_t)kSelChunk);
      if (peek) {
        const u32x4* hp = reinterpret_cast<const u32x4*>(reg + (size_t)c * kSelChunk * 2);
#pragma unroll
        for (int q = 0; q < kPeek / 2; ++q) head[it * (kPeek / 2) + q] = hp[q];
      }
    }
    uint32_t total;
    const uint32_t ex = block_exclusive_sum(v, &total, sh.scratch);
    if (c < nch) sh.off[c] = carry + ex;
    carry += total;
  }
  if (threadIdx.x == 0) sh.off[nch] = carry;
  __syncthreads();
  const uint32_t T = carry;
  const bool in_lds = T <= (uint32_t)kLdsCand;
  uint32_t* gdst = a.ws.gather + (size_t)b * round_cand(a.max_cand) * 2;
  if (peek && in_lds) {
    // Place the region heads, then fetch whatever did not fit in a head.
    for (int first = 0, it = 0; first < nch; first += kThreads, ++it) {
      const int c = first + threadIdx.x;
      if (c < nch) {
        const uint32_t o = sh.off[c], cnt = sh.off[c + 1] - o;
#pragma unroll
        for (int q = 0; q < kPeek / 2; ++q) {
          const u32x4 hv = head[it * (kPeek / 2) + q];
          if (2 * q < (int)cnt) { sh.key[o + 2 * q] = hv[0]; sh.idx[o + 2 * q] = hv[1]; }
          if (2 * q + 1 < (int)cnt) { sh.key[o + 2 * q + 1] = hv[2]; sh.idx[o + 2 * q + 1] = hv[3]; }
        }
        for (uint32_t e = kPeek; e < cnt; ++e) {
          sh.key[o + e] = reg[((size_t)c * kSelChunk + e) * 2];
          sh.idx[o + e] = reg[((size_t)c * kSelChunk + e) * 2 + 1];
        }
      }
    }
  } else {
    // Entry e lives in the chunk c with off[c] <= e < off[c+1] (binary search).
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
  }
  __syncthreads();
  if (T <= keff) {                         // every candidate is selected, in index order
    for (uint32_t e = threadIdx.x; e < T; e += blockDim.x)
      out[e] = (int32_t)(in_lds ? sh.idx[e] : gdst[2 * (size_t)e + 1]);
    return;
  }
  const uint32_t lo_key = a.ws.bound[2 * b], hi_key = a.ws.bound[2 * b + 1];
  if (in_lds && T - keff <= (uint32_t)kRemoveMax) {
    if (threadIdx.x < 64) select_by_removal(sh, T, keff, out);
  } else if (in_lds) {
    select_by_radix([&](uint32_t i) { return sh.key[i]; }, [&](uint32_t i) { return sh.idx[i]; }, T, keff, lo_key,
                    hi_key, out, sh);
  } else {
    select_by_radix([&](uint32_t i) { return gdst[2 * (size_t)i]; },
                    [&](uint32_t i) { return gdst[2 * (size_t)i + 1]; }, T, keff, lo_key, hi_key, out, sh);
  }
}

template <typename ET, int NH>
void launch_scores_nh(dim3 grid, hipStream_t s, const Args& a) {
  switch (a.lpc) {
    case 1: hipLaunchKernelGGL((score_kernel<ET, NH, 1>), grid, dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((score_kernel<ET, NH, 2>), grid, dim3(kThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((score_kernel<ET, NH, 4>), grid, dim3(kThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL((score_kernel<ET, NH, 8>), grid, dim3(kThreads), 0, s, a); break;
    case 16: hipLaunchKernelGGL((score_kernel<ET, NH, 16>), grid, dim3(kThreads), 0, s, a); break;
    case 32: hipLaunchKernelGGL((score_kernel<ET, NH, 32>), grid, dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL((score_kernel<ET, NH, 64>), grid, dim3(kThreads), 0, s, a); break;
  }
}

template <typename ET>
void launch_scores(dim3 grid, hipStream_t s, const Args& a) {
  if (a.nh <= 1) launch_scores_nh<ET, 1>(grid, s, a);
  else if (a.nh <= 2) launch_scores_nh<ET, 2>(grid, s, a);
  else if (a.nh <= 4) launch_scores_nh<ET, 4>(grid, s, a);
  else if (a.nh <= 8) launch_scores_nh<ET, 8>(grid, s, a);
  else launch_scores_nh<ET, 16>(grid, s, a);
}

// Groups per K1 chunk: the coarsest choice that still gives the longest sequence at least 2k
// group maxima (finer groups give a weaker bound, coarser ones too few groups).
int pick_groups(int64_t max_cand, int32_t chunk, int32_t k, const int* choices, int nchoices) {
  const int64_t nch = (max_cand + chunk - 1) / chunk;
  for (int i = 0; i < nchoices; ++i)
    if (nch * choices[i] >= 2LL * k) return choices[i];
  return choices[nchoices - 1];
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
  int nvec = 0, lpc = 1;
  if (q_idx) {
    if (n_heads < 1 || n_heads > 16 || head_dim < 8 || head_dim > 512 || (head_dim * es) % 16 != 0)
      return CHS_ERR_SHAPE;
    if (!w || !k_idx) return CHS_ERR_NULL;
    nvec = (int)(head_dim * es / 16);   // 16-byte vectors per key row (<= 64)
    while (lpc < nvec) lpc *= 2;        // one vector per lane
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
  if (q_idx) {
    static const int score_groups[3] = {1, 4, 32};
    a.chunk = (kThreads / lpc) * kPasses;
    a.gpc = pick_groups(max_cand, a.chunk, k, score_groups, 3);
  } else {
    static const int max_groups[3] = {1, 4, 16};
    a.chunk = kMaxChunk;
    a.gpc = pick_groups(max_cand, a.chunk, k, max_groups, 3);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (max_cand > 0) {
    // Persistent grid: about kScoreGrid workgroups over all sequences.
    const int64_t chunks = (max_cand + a.chunk - 1) / a.chunk;
    const int64_t per_seq = std::max<int64_t>(1, kScoreGrid / batch);
    const dim3 grid((unsigned)std::min<int64_t>(chunks, per_seq), (unsigned)batch);
    if (q_idx) {
      if (dtype == CHS_BF16) launch_scores<uint16_t>(grid, s, a);
      else launch_scores<float>(grid, s, a);
    } else {
      hipLaunchKernelGGL(max_kernel, grid, dim3(kThreads), 0, s, a);
    }
    if (launch_status() != CHS_OK) return CHS_ERR_LAUNCH;
    hipLaunchKernelGGL(bound_kernel, dim3((unsigned)batch), dim3(kThreads), 0, s, a);
    if (launch_status() != CHS_OK) return CHS_ERR_LAUNCH;
    const dim3 sgrid((unsigned)((max_cand + kSelChunk - 1) / kSelChunk), (unsigned)batch);
    hipLaunchKernelGGL(select_kernel, sgrid, dim3(kThreads), 0, s, a);
    if (launch_status() != CHS_OK) return CHS_ERR_LAUNCH;
  }
  hipLaunchKernelGGL(final_kernel, dim3((unsigned)batch), dim3(kThreads), 0, s, a, topk);
  return launch_status();
}
