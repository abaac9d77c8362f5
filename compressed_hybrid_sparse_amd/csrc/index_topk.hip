// chs_index_topk: indexer scores, then the exact top-k by an LDS-histogram radix select.
//
// Source: "SGLang 如何为 DeepSeek V4 打造「Day-0」推理加速", 创新 2 (Lightning TopK): a global
// sort of 256K candidates costs over 100 us at batch 1; instead each block builds a local
// radix histogram, the histograms are reduced, a threshold is found, and each block writes out
// its own entries above it. "DeepSeek-V4 本地部署，SGLang 把活做絕了", Kernel 層一堆狠活: top-512
// of 256K candidates at 1M context. The same first page, 创新 5: the indexer scores every
// candidate before the top-k selects.
//
// The pages' design uses clusters of 8 CTAs with distributed shared memory, which gfx950 does
// not have. Here the cross-workgroup steps use the "last workgroup done" pattern instead: every
// workgroup flushes its partial result with device-scope atomics, bumps a per-sequence counter,
// and the workgroup that brings the counter to its final value does the sequential step. No
// workgroup ever waits on another, so the kernels need no co-residency and cannot deadlock.
//
// Kernel A (score_hist): one workgroup per chunk of CH candidates of one sequence. It streams
//   the chunk's index keys once (non-temporal 16-byte loads), computes the scores with
//   v_dot2_f32_bf16 (or fp32 FMAs), writes them, and counts them in an LDS histogram over the
//   top 11 bits of an order-preserving 32-bit key. The last workgroup of a sequence reduces
//   the global histogram and finds the bin that holds the k-th largest key.
// Kernel B (select): each workgroup re-reads its chunk's scores (1 MiB for 256K candidates,
//   from cache) and appends every candidate in or above the threshold bin to a per-sequence
//   list. The last workgroup refines the threshold exactly with more radix passes over that
//   short list (in LDS when it fits), breaks ties at the threshold by lower index, and writes
//   the ascending index set.
// The composite order (key descending, index ascending) is a total order, so the selected set
// is unique and the result is bit-identical to a full sort of the same scores.
#include "common.h"

namespace chs {
namespace {

constexpr int kThreads = 256;
constexpr int kBins1 = 2048;     // first pass: key bits [31:21]
constexpr int kChunk = 512;      // candidates per workgroup
constexpr int kListLds = 4096;   // final selection runs from LDS up to this many list entries
constexpr int kMaxK = 2048;
constexpr int kCtrlWords = 8;    // per sequence: see Ctrl

// Per-sequence control words in the workspace. All of them return to zero when a call ends.
enum Ctrl { kDoneA = 0, kBin1 = 1, kAbove = 2, kListCount = 3, kDoneB = 4 };

struct Workspace {
  uint32_t* hist;   // [batch][kBins1]
  uint32_t* ctrl;   // [batch][kCtrlWords]
  uint32_t* list;   // [batch][max_cand][2]: (key, index)
  float* scores;    // [batch][max_cand] (used when the caller passes no score array)
};

size_t ws_layout(int32_t batch, int64_t max_cand, Workspace* w, char* base) {
  size_t off = 0;
  const size_t nb = (size_t)batch;
  const size_t mc = (size_t)(max_cand > 0 ? max_cand : 0);
  size_t o_hist = off; off = align_up(off + nb * kBins1 * 4, 256);
  size_t o_ctrl = off; off = align_up(off + nb * kCtrlWords * 4, 256);
  size_t o_list = off; off = align_up(off + nb * mc * 8, 256);
  size_t o_scores = off; off = align_up(off + nb * mc * 4, 256);
  if (w) {
    w->hist = reinterpret_cast<uint32_t*>(base + o_hist);
    w->ctrl = reinterpret_cast<uint32_t*>(base + o_ctrl);
    w->list = reinterpret_cast<uint32_t*>(base + o_list);
    w->scores = reinterpret_cast<float*>(base + o_scores);
  }
  return off;
}

// Order-preserving key: a larger float gives a larger unsigned key; -0.0 maps like +0.0.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t atomic_load_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_store_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Block-wide exclusive prefix sum over kThreads threads; returns the block total in *total.
__device__ uint32_t block_exclusive_sum(uint32_t v, uint32_t* total, uint32_t* scratch /*[kThreads/64 + 1]*/) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  if (lane == 63) scratch[wave] = inc;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    uint32_t t = scratch[w];
    if (w < wave) before += t;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + inc - v;
}

// In a histogram of `nbins` counts (nbins % kThreads == 0), find for rank r >= 1 counted from
// the top (descending=true) or from the bottom: the bin holding the r-th element, and the
// number of elements strictly before that bin in the scan order. Result in out[0..1].
__device__ void find_rank_bin(const uint32_t* hist, int nbins, uint32_t r, bool descending,
                              uint32_t* scratch, uint32_t* out) {
  const int per = nbins / kThreads;
  // Thread t owns scan positions [t*per, (t+1)*per); position p maps to bin p (ascending) or
  // nbins-1-p (descending).
  uint32_t local = 0;
  for (int i = 0; i < per; ++i) {
    int p = threadIdx.x * per + i;
    local += hist[descending ? nbins - 1 - p : p];
  }
  uint32_t total;
  uint32_t before = block_exclusive_sum(local, &total, scratch);
  if (before < r && before + local >= r) {
    uint32_t run = before;
    for (int i = 0; i < per; ++i) {
      int p = threadIdx.x * per + i;
      int bin = descending ? nbins - 1 - p : p;
      uint32_t c = hist[bin];
      if (run + c >= r) { out[0] = (uint32_t)bin; out[1] = run; break; }
      run += c;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------- kernel A: score + histogram
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
    for (int j = 0; j < 4; ++j) acc = fmaf(__uint_as_float(a[j]), __uint_as_float(b[j]), acc);
    return acc;
  }
};

// Sum a float over groups of `lpc` adjacent lanes (lpc a power of two <= 64); every lane of a
// group ends with the group total. Within rows of 16 lanes this uses DPP lane swizzles.
__device__ __forceinline__ float group_sum(float v, int lpc) {
  if (lpc >= 2) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));  // xor 1
  if (lpc >= 4) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));  // xor 2
  if (lpc >= 8) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)); // half-row mirror
  if (lpc >= 16) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)); // row mirror
  if (lpc >= 32) v += __shfl_xor(v, 16, 64);
  if (lpc >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

struct ScoreArgs {
  const void* q;        // [batch][nh][dim] (NULL: scores are input)
  const float* w;       // [batch][nh]
  const void* keys;     // [cu_cand[batch]][dim]
  const int64_t* cu;    // [batch+1]
  int64_t max_cand;
  int32_t nh, dim;
  int32_t nvec;         // 16-byte vectors per key row
  int32_t lpc;          // lanes per candidate
  float* scores;        // caller's packed array, or NULL -> workspace [b][max_cand]
  Workspace ws;
  int32_t k;
};

__device__ __forceinline__ int64_t cand_count(const ScoreArgs& a, int b, int64_t* base) {
  const int64_t c0 = a.cu[b];
  int64_t n = a.cu[b + 1] - c0;
  if (n > a.max_cand) n = a.max_cand;
  if (n < 0) n = 0;
  *base = c0;
  return n;
}

__device__ __forceinline__ float* score_ptr(const ScoreArgs& a, int b, int64_t c0) {
  return a.scores ? a.scores + c0 : a.ws.scores + (int64_t)b * a.max_cand;
}

// Tail of kernel A, run by every workgroup: flush the LDS histogram, count the workgroup done,
// and in the sequence's last workgroup locate the threshold bin.
__device__ void flush_and_find_bin1(const ScoreArgs& a, int b, int64_t n, uint32_t* lhist,
                                    uint32_t* scratch) {
  __syncthreads();
  uint32_t* gh = a.ws.hist + (size_t)b * kBins1;
  for (int i = threadIdx.x; i < kBins1; i += kThreads) {
    uint32_t c = lhist[i];
    if (c) atomicAdd(gh + i, c);
  }
  __threadfence();
  __syncthreads();
  const int nchunks = n > 0 ? (int)((n + kChunk - 1) / kChunk) : 1;
  uint32_t* ctrl = a.ws.ctrl + (size_t)b * kCtrlWords;
  if (threadIdx.x == 0) scratch[8] = atomicAdd(ctrl + kDoneA, 1u);
  __syncthreads();
  if (scratch[8] != (uint32_t)(nchunks - 1)) return;
  // Last workgroup of sequence b.
  __threadfence();
  for (int i = threadIdx.x; i < kBins1; i += kThreads) lhist[i] = atomicExch(gh + i, 0u);
  __syncthreads();
  const uint32_t keff = (uint32_t)min<int64_t>(a.k, n);
  if (keff > 0) {
    find_rank_bin(lhist, kBins1, keff, true, scratch, scratch + 12);
    if (threadIdx.x == 0) {
      atomic_store_agent(ctrl + kBin1, scratch[12]);
      atomic_store_agent(ctrl + kAbove, scratch[13]);
    }
  }
  if (threadIdx.x == 0) atomic_store_agent(ctrl + kDoneA, 0u);
}

template <typename ET, int NH, int MAXV>
__global__ __launch_bounds__(kThreads) void score_hist_kernel(ScoreArgs a) {
  __shared__ uint32_t lhist[kBins1];
  __shared__ uint32_t scratch[16];
  const int b = blockIdx.y;
  int64_t c0;
  const int64_t n = cand_count(a, b, &c0);
  const int64_t chunk0 = (int64_t)blockIdx.x * kChunk;
  const int nchunks = n > 0 ? (int)((n + kChunk - 1) / kChunk) : 1;
  if ((int)blockIdx.x >= nchunks) return;
  for (int i = threadIdx.x; i < kBins1; i += kThreads) lhist[i] = 0;
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lpc = a.lpc;
  const int sub = lane & (lpc - 1);
  const int slot = (wave * 64 + lane) / lpc;          // candidate slot within a pass
  const int per_pass = kThreads / lpc;
  // This lane's slice of every indexer query: vectors sub, sub + lpc, ...
  u32x4 qv[NH][MAXV];
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
  const u32x4* kb = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.keys) + (size_t)c0 * a.nvec * 16);
  float* sp = score_ptr(a, b, c0);
  const int64_t chunk_end = min<int64_t>(chunk0 + kChunk, n);
  constexpr int U = 4;   // passes in flight per lane: U * MAXV 16-byte loads
  for (int64_t base = chunk0; base < chunk_end; base += per_pass * U) {
    u32x4 kv[U][MAXV];
    int64_t j[U];
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
        atomicAdd(&lhist[score_key(s) >> 21], 1u);
      }
    }
  }
  flush_and_find_bin1(a, b, n, lhist, scratch);
}

// Kernel A for caller-provided scores: histogram only.
__global__ __launch_bounds__(kThreads) void hist_kernel(ScoreArgs a) {
  __shared__ uint32_t lhist[kBins1];
  __shared__ uint32_t scratch[16];
  const int b = blockIdx.y;
  int64_t c0;
  const int64_t n = cand_count(a, b, &c0);
  const int nchunks = n > 0 ? (int)((n + kChunk - 1) / kChunk) : 1;
  if ((int)blockIdx.x >= nchunks) return;
  for (int i = threadIdx.x; i < kBins1; i += kThreads) lhist[i] = 0;
  __syncthreads();
  const float* sp = score_ptr(a, b, c0);
  const int64_t chunk0 = (int64_t)blockIdx.x * kChunk, chunk_end = min<int64_t>(chunk0 + kChunk, n);
  for (int64_t j = chunk0 + threadIdx.x; j < chunk_end; j += kThreads)
    atomicAdd(&lhist[score_key(sp[j]) >> 21], 1u);
  flush_and_find_bin1(a, b, n, lhist, scratch);
}

// ---------------------------------------------------------------- kernel B: select
struct SelectShared {
  uint32_t key[kListLds];
  uint32_t idx[kListLds];
  uint32_t hist[kBins1];
  uint32_t sorted[kMaxK];
  uint32_t scratch[16];
};

// Threshold refinement and output, run by the last workgroup of sequence b. The list holds
// every candidate whose key is in the threshold bin b1 or above: `above` of them above b1.
template <bool IN_LDS>
__device__ void final_select(SelectShared& sh, const uint32_t* glist, uint32_t nlist, uint32_t keff,
                             uint32_t b1, uint32_t above, int32_t* out, int32_t k) {
  auto KEY = [&](uint32_t i) { return IN_LDS ? sh.key[i] : glist[2 * (size_t)i]; };
  auto IDX = [&](uint32_t i) { return IN_LDS ? sh.idx[i] : glist[2 * (size_t)i + 1]; };
  uint32_t tau = 0, idx_thr = 0xFFFFFFFFu;
  if (nlist > keff) {
    // Rank of the k-th largest inside bin b1 (1-based, descending).
    uint32_t r = keff - above;
    uint32_t prefix = b1;   // known high bits of the threshold key
    // Passes over key bits [20:10] and [9:0] among candidates sharing the known prefix.
    const int shifts[2] = {10, 0};
    const int widths[2] = {11, 10};
    int known = 11;
    for (int p = 0; p < 2; ++p) {
      const int nb = 1 << widths[p];
      for (int i = threadIdx.x; i < nb; i += kThreads) sh.hist[i] = 0;
      __syncthreads();
      for (uint32_t i = threadIdx.x; i < nlist; i += kThreads) {
        uint32_t kk = KEY(i);
        if ((kk >> (32 - known)) == prefix) atomicAdd(&sh.hist[(kk >> shifts[p]) & (nb - 1)], 1u);
      }
      __syncthreads();
      find_rank_bin(sh.hist, nb, r, true, sh.scratch, sh.scratch + 12);
      const uint32_t bin = sh.scratch[12], before = sh.scratch[13];
      __syncthreads();
      r -= before;
      prefix = (prefix << widths[p]) | bin;
      known += widths[p];
    }
    tau = prefix;
    // r is now the number of candidates with key == tau to take (1..ties), lowest index first.
    for (int i = threadIdx.x; i < kBins1; i += kThreads) sh.hist[i] = 0;
    if (threadIdx.x == 0) sh.scratch[14] = 0;
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < nlist; i += kThreads)
      if (KEY(i) == tau) atomicAdd(&sh.scratch[14], 1u);
    __syncthreads();
    const uint32_t ties = sh.scratch[14];
    if (r < ties) {
      // r-th smallest index among the ties: radix passes over index bits [30:20], [19:10], [9:0].
      const int ish[3] = {20, 10, 0};
      const int iw[3] = {11, 10, 10};
      uint32_t ipre = 0;
      int iknown = 1;   // bit 31 of an index is always 0
      for (int p = 0; p < 3; ++p) {
        const int nb = 1 << iw[p];
        for (int i = threadIdx.x; i < kBins1; i += kThreads) sh.hist[i] = 0;
        __syncthreads();
        for (uint32_t i = threadIdx.x; i < nlist; i += kThreads) {
          if (KEY(i) != tau) continue;
          uint32_t ix = IDX(i);
          if ((ix >> (32 - iknown)) == ipre) atomicAdd(&sh.hist[(ix >> ish[p]) & (nb - 1)], 1u);
        }
        __syncthreads();
        find_rank_bin(sh.hist, nb, r, false, sh.scratch, sh.scratch + 12);
        const uint32_t bin = sh.scratch[12], before = sh.scratch[13];
        __syncthreads();
        r -= before;
        ipre = (ipre << iw[p]) | bin;
        iknown += iw[p];
      }
      idx_thr = ipre;
    }
  }
  // Gather the selection (exactly keff entries), sort ascending, write with -1 padding.
  if (threadIdx.x == 0) sh.scratch[15] = 0;
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < nlist; i += kThreads) {
    const uint32_t kk = KEY(i), ix = IDX(i);
    const bool take = (nlist <= keff) || kk > tau || (kk == tau && ix <= idx_thr);
    if (take) {
      uint32_t pos = atomicAdd(&sh.scratch[15], 1u);
      if (pos < (uint32_t)kMaxK) sh.sorted[pos] = ix;
    }
  }
  __syncthreads();
  const uint32_t cnt = min(sh.scratch[15], (uint32_t)kMaxK);
  uint32_t P = 1;
  while (P < cnt) P <<= 1;
  for (uint32_t i = cnt + threadIdx.x; i < P; i += kThreads) sh.sorted[i] = 0xFFFFFFFFu;
  __syncthreads();
  // Bitonic sort of P entries, ascending.
  for (uint32_t size = 2; size <= P; size <<= 1) {
    for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
      for (uint32_t t = threadIdx.x; t < P / 2; t += kThreads) {
        const uint32_t i = 2 * t - (t & (stride - 1));
        const uint32_t jx = i + stride;
        const bool up = ((i & size) == 0);
        const uint32_t x = sh.sorted[i], y = sh.sorted[jx];
        if ((x > y) == up) { sh.sorted[i] = y; sh.sorted[jx] = x; }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < k; i += kThreads) out[i] = (uint32_t)i < cnt ? (int32_t)sh.sorted[i] : -1;
}

__global__ __launch_bounds__(kThreads) void select_kernel(ScoreArgs a, int32_t* topk) {
  __shared__ SelectShared sh;
  const int b = blockIdx.y;
  int64_t c0;
  const int64_t n = cand_count(a, b, &c0);
  const int nchunks = n > 0 ? (int)((n + kChunk - 1) / kChunk) : 1;
  if ((int)blockIdx.x >= nchunks) return;
  uint32_t* ctrl = a.ws.ctrl + (size_t)b * kCtrlWords;
  uint32_t* glist = a.ws.list + (size_t)b * a.max_cand * 2;
  const uint32_t keff = (uint32_t)min<int64_t>(a.k, n);
  const uint32_t b1 = atomic_load_agent(ctrl + kBin1);
  // Append this chunk's candidates in or above bin b1 to the sequence's list.
  const float* sp = score_ptr(a, b, c0);
  const int64_t chunk0 = (int64_t)blockIdx.x * kChunk, chunk_end = min<int64_t>(chunk0 + kChunk, n);
  for (int64_t j0 = chunk0; j0 < chunk_end; j0 += kThreads) {
    const int64_t j = j0 + threadIdx.x;
    uint32_t kk = 0;
    bool take = false;
    if (j < chunk_end && keff > 0) {
      kk = score_key(sp[j]);
      take = (kk >> 21) >= b1;
    }
    uint32_t total;
    const uint32_t off = block_exclusive_sum(take ? 1u : 0u, &total, sh.scratch);
    if (total) {
      if (threadIdx.x == 0) sh.scratch[8] = atomicAdd(ctrl + kListCount, total);
      __syncthreads();
      const uint32_t pos = sh.scratch[8] + off;
      // pos < n <= max_cand whenever the workspace started zeroed; the bound keeps even a
      // dirty workspace from addressing memory outside the list.
      if (take && pos < (uint64_t)a.max_cand) {
        glist[2 * (size_t)pos] = kk;
        glist[2 * (size_t)pos + 1] = (uint32_t)j;
      }
      __syncthreads();
    }
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) sh.scratch[9] = atomicAdd(ctrl + kDoneB, 1u);
  __syncthreads();
  if (sh.scratch[9] != (uint32_t)(nchunks - 1)) return;
  // Last workgroup of sequence b.
  __threadfence();
  const uint32_t nlist = (uint32_t)min<int64_t>(atomic_load_agent(ctrl + kListCount), n);
  const uint32_t above = atomic_load_agent(ctrl + kAbove);
  int32_t* out = topk + (size_t)b * a.k;
  if (nlist <= (uint32_t)kListLds) {
    for (uint32_t i = threadIdx.x; i < nlist; i += kThreads) {
      sh.key[i] = __hip_atomic_load(glist + 2 * (size_t)i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sh.idx[i] = __hip_atomic_load(glist + 2 * (size_t)i + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    final_select<true>(sh, glist, nlist, keff, b1, above, out, a.k);
  } else {
    final_select<false>(sh, glist, nlist, keff, b1, above, out, a.k);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    atomic_store_agent(ctrl + kListCount, 0u);
    atomic_store_agent(ctrl + kDoneB, 0u);
    atomic_store_agent(ctrl + kBin1, 0u);
    atomic_store_agent(ctrl + kAbove, 0u);
  }
}

template <typename ET, int NH>
void launch_scores_nh(dim3 grid, hipStream_t s, const ScoreArgs& a, int maxv) {
  switch (maxv) {
    case 1: hipLaunchKernelGGL((score_hist_kernel<ET, NH, 1>), grid, dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((score_hist_kernel<ET, NH, 2>), grid, dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL((score_hist_kernel<ET, NH, 4>), grid, dim3(kThreads), 0, s, a); break;
  }
}

template <typename ET>
void launch_scores(dim3 grid, hipStream_t s, const ScoreArgs& a, int maxv) {
  if (a.nh <= 1) launch_scores_nh<ET, 1>(grid, s, a, maxv);
  else if (a.nh <= 2) launch_scores_nh<ET, 2>(grid, s, a, maxv);
  else if (a.nh <= 4) launch_scores_nh<ET, 4>(grid, s, a, maxv);
  else if (a.nh <= 8) launch_scores_nh<ET, 8>(grid, s, a, maxv);
  else launch_scores_nh<ET, 16>(grid, s, a, maxv);
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
  ScoreArgs a;
  a.q = q_idx; a.w = w; a.keys = k_idx; a.cu = cu_cand; a.max_cand = max_cand;
  a.nh = n_heads; a.dim = head_dim; a.nvec = nvec; a.lpc = lpc; a.scores = scores; a.ws = ws; a.k = k;
  const int64_t chunks = max_cand > 0 ? (max_cand + kChunk - 1) / kChunk : 1;
  dim3 grid((unsigned)chunks, (unsigned)batch);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (q_idx) {
    if (dtype == CHS_BF16) launch_scores<uint16_t>(grid, s, a, maxv);
    else launch_scores<float>(grid, s, a, maxv);
  } else {
    hipLaunchKernelGGL(hist_kernel, grid, dim3(kThreads), 0, s, a);
  }
  if (launch_status() != CHS_OK) return CHS_ERR_LAUNCH;
  hipLaunchKernelGGL(select_kernel, grid, dim3(kThreads), 0, s, a, topk);
  return launch_status();
}
