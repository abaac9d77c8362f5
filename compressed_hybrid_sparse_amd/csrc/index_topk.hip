// chs_index_topk: indexer scores, then the exact top-k by radix selection, with no global sort.
//
// Source: "SGLang 如何为 DeepSeek V4 打造「Day-0」推理加速", 创新 2 (Lightning TopK): a global
// sort of 256K candidates costs over 100 us at batch 1; instead, blocks build radix histograms
// of their scores, a threshold is found, and each block writes out only its own entries above
// it. Same page, 创新 5: the indexer scores every compressed candidate before the top-k.
// "DeepSeek-V4 本地部署，SGLang 把活做絕了", Kernel 層一堆狠活: top-512 of 256K at 1M context.
//
// The pages' design reduces per-CTA histograms inside a thread-block cluster through
// distributed shared memory, which gfx950 does not have; on MI355X the L2s of the 8 XCDs are
// not coherent, so a handoff between workgroups inside a kernel needs an agent-scope release
// and acquire (an L2 write-back and invalidate, microseconds when data is in flight), while
// back-to-back kernels in a graph hand off for free. So no kernel here synchronises
// workgroups with each other, and a call is two kernels:
//
//   K1 streams the index keys once, every load instruction reading 1 KiB of whole rows (16
//      bytes per lane, non-temporal), all of a wave's loads issued before the first use
//      (unconditional, with clamped addresses, so the compiler can count them). For up to 16
//      heads and head_dim 64, 128 or 256 (bf16 keys, or FP8 E4M3 keys with per-row scales,
//      converted to bf16 exactly) score_mfma_kernel computes the head dots as 16x16x32 bf16
//      MFMAs over 16-key tiles, each tile passing through the wave's LDS tile into the MFMA
//      layout; other shapes take score_kernel, where LPC lanes (16 for 128 bf16 channels)
//      share a key row and v_dot2_f32_bf16 (or fp32 FMAs) and DPP sums form the dots. Both
//      write the fp32 scores and, for every group of GS consecutive candidates (GS = 32; 16 or
//      8 for very wide keys in score_kernel), the group's largest key, the position of that
//      maximum and its second-largest key. max_kernel does the same for caller-provided scores.
//   K2 collect_kernel, one 1024-thread workgroup per sequence (one CU, 4 waves per SIMD, so
//      the instructions it issues per candidate are what costs: it touches group statistics,
//      not scores, wherever it can):
//      (A) bins the maxima of runs of 4 groups (or of single groups when there are few; past
//          8192 groups a "group" is the set of groups congruent modulo 8192), (key - smallest)
//          >> shift, into 2048 monotone bins; L = the lower edge of the bin holding the k-th
//          largest. L never exceeds the k-th largest score, because k disjoint runs each hold
//          a score >= L; so every top-k candidate, and every tie at the threshold, has key >= L
//          and sits in a group whose maximum is >= L;
//      (B) builds the superset of keys >= L in index order in LDS with one block scan: a group
//          whose maximum is >= L but whose second key is below L holds exactly one such key,
//          its maximum, known from the statistics; the others ("full", typically a few
//          percent) are read whole, two per wave; kept keys are binned into 2048 monotone
//          bins over [L, max];
//      (C) the bin holding the k-th largest kept key gives tau after comparing only the few
//          keys inside it (a crowded bin, from heavy ties, falls back to radix steps); an
//          ordered pass then writes the keys above tau and the first ties at tau, ascending
//          by index (no sort).
//      Inputs that defeat the bound (a superset too large for LDS: heavy ties, many equal
//      zeros) are selected by the whole workgroup straight from the score array instead.
//      Gathers go through buffer loads (32-bit offsets, reads beyond the array return 0).
// The composite order (key descending, then index ascending) is total, so the selected set is
// unique and bit-identical to a full sort of the same scores.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "common.h"
#include "attn_core.h"

namespace chs {
namespace {

constexpr int kThreads = 256;          // K1 workgroup
constexpr int kPasses = 8;             // K1 loads per lane (16 bytes each)
constexpr int kGroup = 32;             // candidates per group (K1 uses 16 or 8 for keys > 512 B)
constexpr int kMinGroup = 8;
constexpr int kCThreads = 1024;        // K2 workgroup: sixteen waves, four per SIMD
constexpr int kCWaves = kCThreads / 64;
constexpr int kMaxPerThread = 8;       // group maxima per K2 thread per tile (contiguous)
constexpr int kTile = kCThreads * kMaxPerThread;   // 8192 groups: one pass of the K2 block
constexpr int kBins = 2048;            // bound and superset histograms; global radix bins
constexpr int kLdsCand = 4096;         // superset entries LDS holds
constexpr int kFullCap = 256;          // groups whose second key may reach L (read whole)
constexpr int kBinCap = 64;            // threshold-bin entries resolved directly
constexpr int kGlobalRounds = 16;      // global path: scores per thread per batch
constexpr int kScanRounds = 16;        // the most rounds one ordered scan covers
constexpr int kMaxK = 2048;
constexpr int64_t kMaxCand = 1 << 22;

struct Workspace {
  uint32_t* maxima;   // [batch][mcap]: group maximum keys
  uint32_t* second;   // [batch][mcap]: group statistics words (see pack_second)
  float* scores;      // [batch][rc] when the caller passes no score array
};

// Candidate capacity per sequence, rounded up to 1024; group maxima capacity per sequence.
__host__ __device__ inline int64_t round_cand(int64_t max_cand) { return (max_cand + 1023) / 1024 * 1024; }
__host__ __device__ inline int64_t maxima_cap(int64_t max_cand) { return round_cand(max_cand) / kMinGroup; }

size_t ws_layout(int32_t batch, int64_t max_cand, Workspace* w, char* base) {
  const size_t nb = (size_t)batch;
  const int64_t mc = max_cand > 0 ? max_cand : 0;
  size_t off = 0;
  const size_t o_max = off; off = align_up(off + nb * (size_t)maxima_cap(mc) * 4, 256);
  const size_t o_sec = off; off = align_up(off + nb * (size_t)maxima_cap(mc) * 4, 256);
  const size_t o_sc = off;  off = align_up(off + nb * (size_t)round_cand(mc) * 4, 256);
  if (w) {
    w->maxima = reinterpret_cast<uint32_t*>(base + o_max);
    w->second = reinterpret_cast<uint32_t*>(base + o_sec);
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

// A raw buffer resource over `bytes` bytes at p: loads through it take a 32-bit byte offset
// (one VGPR per address instead of two) and return 0 beyond the end.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint32_t buffer_u32(__amdgpu_buffer_rsrc_t r, uint32_t index) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, index * 4u, 0, 0);
}
__device__ __forceinline__ u32x4 buffer_u32x4(__amdgpu_buffer_rsrc_t r, uint32_t index) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, index * 4u, 0, 0);
}

struct Args {
  const void* q;        // [batch][nh][dim] (NULL: scores are input)
  const float* w;       // [batch][nh]
  const void* keys;     // [cu[batch]][dim]
  const int64_t* cu;    // [batch+1]
  int64_t max_cand;
  int32_t nh, nvec;     // heads; 16-byte vectors per key row
  int32_t gs;           // group size (a power of two)
  int32_t k;
  float* scores;        // caller's packed array, or NULL -> workspace
  const float* kscale;  // [cu[batch]] per-row scales of FP8 keys (NULL otherwise)
  Workspace ws;
  // Paged key pool (NULL: keys packed by cu). Candidate j of sequence b is pool row
  // pt[b * pt_stride + j / 2^shift] * 2^shift + j mod 2^shift; cand_len[b] candidates; scores at
  // b * max_cand + j of the caller's array.
  const int32_t* pt;
  const int64_t* cand_len;
  int32_t pt_stride, shift;
  int64_t pool_pages;
};

__device__ __forceinline__ int64_t cand_count(const Args& a, int b, int64_t* base) {
  if (a.cand_len) {
    int64_t n = a.cand_len[b];
    const int64_t cap = (int64_t)a.pt_stride << a.shift;
    if (n > cap) n = cap;
    if (n > a.max_cand) n = a.max_cand;
    if (n < 0) n = 0;
    *base = (int64_t)b * a.max_cand;
    return n;
  }
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
  return a.ws.maxima + (size_t)b * maxima_cap(a.max_cand);
}
__device__ __forceinline__ uint32_t* second_ptr(const Args& a, int b) {
  return a.ws.second + (size_t)b * maxima_cap(a.max_cand);
}

// Group statistics: the maximum key, the lowest position (< 32) holding it, and the largest
// key at any other position. Stored as the maximum plus one word, (second & ~31) | position:
// (word | 31) is never below the second key, so a test against it can only be conservative.
struct Top2 {
  uint32_t m1, p1, m2;
};
__device__ __forceinline__ uint32_t pack_second(const Top2& s) { return (s.m2 & ~31u) | s.p1; }
// Adds key k at position p; a lane's positions grow from call to call, so ties keep the first.
__device__ __forceinline__ void top2_add(Top2& s, uint32_t k, uint32_t p) {
  const bool gt = k > s.m1;
  s.m2 = gt ? s.m1 : max(s.m2, k);
  s.p1 = gt ? p : s.p1;
  s.m1 = gt ? k : s.m1;
}
__device__ __forceinline__ Top2 top2_merge(const Top2& a, const Top2& b) {
  Top2 r;
  r.m1 = max(a.m1, b.m1);
  r.p1 = a.m1 > b.m1 ? a.p1 : (b.m1 > a.m1 ? b.p1 : min(a.p1, b.p1));
  r.m2 = max(max(a.m2, b.m2), min(a.m1, b.m1));
  return r;
}
__device__ __forceinline__ Top2 top2_xor(const Top2& s, int o) {
  return Top2{(uint32_t)__shfl_xor((int)s.m1, o, 64), (uint32_t)__shfl_xor((int)s.p1, o, 64),
              (uint32_t)__shfl_xor((int)s.m2, o, 64)};
}

// ---------------------------------------------------------------- wave and block helpers
// DPP move with zero fill: lanes whose source is outside the row (or whose row is not in
// ROW_MASK) read 0, the identity of the sums and unsigned maxima below.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp0(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive prefix sum over the wave: shifts by 1, 2, 4, 8 within each row of 16 lanes, then
// row_bcast:15 (rows 1 and 3 add the last lane of the row before) and row_bcast:31 (rows 2
// and 3 add lane 31).
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  v += dpp0<0x111>(v);
  v += dpp0<0x112>(v);
  v += dpp0<0x114>(v);
  v += dpp0<0x118>(v);
  v += dpp0<0x142, 0xA>(v);
  v += dpp0<0x143, 0xC>(v);
  return v;
}

// Maximum over the wave, returned wave-uniform (the same DPP pattern leaves it in lane 63).
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = max(v, dpp0<0x111>(v));
  v = max(v, dpp0<0x112>(v));
  v = max(v, dpp0<0x114>(v));
  v = max(v, dpp0<0x118>(v));
  v = max(v, dpp0<0x142, 0xA>(v));
  v = max(v, dpp0<0x143, 0xC>(v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Number of set bits of a wave mask in the lanes below this one.
__device__ __forceinline__ uint32_t mask_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Block-wide helpers for the K2 block (kCWaves waves, declared below). The wave partials go
// through LDS and every thread reads all of them with 16-byte loads, so no dependent chain of
// LDS reads forms. `scratch` is 16-byte aligned; each call ends with a barrier.
// TRAIL = false leaves out the closing barrier where the caller reaches another barrier before
// `scratch` is written again.
template <int NW, bool TRAIL = true>
__device__ uint32_t block_exclusive_sum_t(uint32_t v, uint32_t* total, uint32_t* scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_inclusive_sum(v);
  if (lane == 63) scratch[wave] = inc;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; w += 4) {
    const u32x4 p = *reinterpret_cast<const u32x4*>(&scratch[w]);
#pragma unroll
    for (int j = 0; j < 4; ++j) { before += (w + j < wave) ? p[j] : 0u; all += p[j]; }
  }
  if (TRAIL) __syncthreads();
  *total = all;
  return before + inc - v;
}

template <int NW, bool TRAIL = true>
__device__ void block_minmax_t(uint32_t* vmin, uint32_t* vmax, uint32_t* scratch) {
  const int wave = threadIdx.x >> 6;
  const uint32_t lo = ~wave_max(~*vmin), hi = wave_max(*vmax);
  if ((threadIdx.x & 63) == 0) { scratch[wave] = lo; scratch[NW + wave] = hi; }
  __syncthreads();
  uint32_t l = 0xFFFFFFFFu, h = 0;
#pragma unroll
  for (int w = 0; w < NW; w += 4) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(&scratch[w]);
    const u32x4 y = *reinterpret_cast<const u32x4*>(&scratch[NW + w]);
    l = min(min(l, min(x[0], x[1])), min(x[2], x[3]));
    h = max(max(h, max(y[0], y[1])), max(y[2], y[3]));
  }
  if (TRAIL) __syncthreads();
  *vmin = l; *vmax = h;
}

// Radix digits below the bits shared by every key in [lo, hi]: returns how many bits differ.
__device__ __forceinline__ int differing_bits(uint32_t lo, uint32_t hi) {
  return lo == hi ? 0 : 32 - __clz(lo ^ hi);
}

// ---------------------------------------------------------------- K1: scores + group maxima
template <typename ET>
struct Dot16;

// Dot product of one lane's 16 bytes of a key row with the matching query elements, which
// take QV 16-byte vectors.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// Element j is copied to a scalar before the bit cast: clang lowers a bit cast applied
// directly to an ext-vector element access as a cast of element 0.
__device__ __forceinline__ bf16x2 bf16_pair(uint32_t x) { return __builtin_bit_cast(bf16x2, x); }

template <>
struct Dot16<uint16_t> {   // 8 bf16 per 16 bytes: four v_dot2_f32_bf16
  static constexpr int QV = 1;
  __device__ static float dot(const u32x4* q, const u32x4& k) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t x = q[0][j], y = k[j];
      acc = __builtin_amdgcn_fdot2_f32_bf16(bf16_pair(x), bf16_pair(y), acc, false);
    }
    return acc;
  }
};

template <>
struct Dot16<float> {      // 4 fp32 per 16 bytes
  static constexpr int QV = 1;
  __device__ static float dot(const u32x4* q, const u32x4& k) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t x = q[0][j], y = k[j];
      acc = fmaf(__uint_as_float(x), __uint_as_float(y), acc);
    }
    return acc;
  }
};

template <>
struct Dot16<uint8_t> {    // 16 FP8 E4M3 per 16 bytes against 16 bf16 query values (2 vectors)
  static constexpr int QV = 2;
  // Every E4M3 value is a bf16 value, so the conversion (scale 1) is exact and the products
  // go through v_dot2_f32_bf16 like bf16 keys.
  __device__ static float dot(const u32x4* q, const u32x4& k) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t x = k[j];
      const uint32_t q0 = q[j >> 1][2 * (j & 1)], q1 = q[j >> 1][2 * (j & 1) + 1];
      acc = __builtin_amdgcn_fdot2_f32_bf16(bf16_pair(q0), __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false),
                                            acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(bf16_pair(q1), __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true),
                                            acc, false);
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

// Four heads over a 16-lane row: s = sum_h w_h * ReLU(sum over the row of p[h]), in every
// lane of the row. Reduce-scatter: two exchanges leave lane l with head 2*(l&1) + ((l>>1)&1)
// summed over its quad, row rotations by 4 and 8 finish that head's sum over the row, and a
// quad sum adds the weighted heads; wl is this lane's head weight.
__device__ __forceinline__ float head4_row_score(const float (&p)[4], float wl, int lane) {
  const bool b0 = lane & 1, b1 = (lane >> 1) & 1;
  auto dpp = [](float v, int ctrl) {
    switch (ctrl) {
      case 0xB1: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
      case 0x4E: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
      case 0x124: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xF, 0xF, false));
      default: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false));
    }
  };
  const float s0 = b0 ? p[0] : p[2], s1 = b0 ? p[1] : p[3];        // sent to lane ^ 1
  const float a0 = (b0 ? p[2] : p[0]) + dpp(s0, 0xB1);             // heads (0,1) or (2,3)
  const float a1 = (b0 ? p[3] : p[1]) + dpp(s1, 0xB1);
  float h = (b1 ? a1 : a0) + dpp(b1 ? a0 : a1, 0x4E);              // one head per lane
  h += dpp(h, 0x124);                                              // row_ror:4
  h += dpp(h, 0x128);                                              // row_ror:8
  float r = fmaxf(h, 0.f) * wl;
  r += dpp(r, 0xB1);
  r += dpp(r, 0x4E);
  return r;
}

// Row geometry of K1 for LPC lanes per key row.
template <int LPC>
struct ScoreGeom {
  static constexpr int RP = 64 / LPC;                  // rows per wave per pass
  static constexpr int RW = kPasses * RP;              // rows per wave
  static constexpr int GS = RW < kGroup ? RW : kGroup; // group size
  static constexpr int NG = RW / GS;                   // groups per wave
  static constexpr int PG = kPasses / NG;              // passes per group
};

// Grid (x: runs of 4 * RW rows, y: sequence). Wave w of block x scores rows
// [(4x + w) * RW, +RW); pass u covers rows u * RP .. u * RP + RP - 1 of that run.
template <typename ET, int NH, int LPC>
__global__ __launch_bounds__(kThreads) void score_kernel(Args a) {
  using G = ScoreGeom<LPC>;
  const int b = blockIdx.y;
  int64_t c0;
  const int64_t n = cand_count(a, b, &c0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row0 = ((int64_t)blockIdx.x * (kThreads / 64) + wave) * G::RW;
  if (row0 >= n) return;                               // no barriers follow
  const int sub = lane & (LPC - 1), slot = lane / LPC;
  const int nvec = a.nvec;
  const int subc = sub < nvec ? sub : nvec - 1;
  // Queries and weights first (their loads complete first), then every key load.
  constexpr int QV = Dot16<ET>::QV;                     // query vectors per key vector
  constexpr bool kScaled = std::is_same<ET, uint8_t>::value;
  const u32x4* qb = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.q) + (size_t)b * a.nh * nvec * QV * 16);
  u32x4 qv[NH][QV];
  float wv[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int hc = h < a.nh ? h : a.nh - 1;
#pragma unroll
    for (int i = 0; i < QV; ++i) qv[h][i] = qb[(hc * nvec + subc) * QV + i];
    wv[h] = a.w[(size_t)b * a.nh + hc];
  }
  __builtin_amdgcn_sched_barrier(0);                   // query loads go out (and return) first
  const u32x4* kb = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.keys) + (size_t)c0 * nvec * 16);
  u32x4 kv[kPasses];
  float ks[kPasses];
#pragma unroll
  for (int u = 0; u < kPasses; ++u) {
    int64_t row = row0 + u * G::RP + slot;
    if (row > n - 1) row = n - 1;
    kv[u] = __builtin_nontemporal_load(kb + row * nvec + subc);
    if (kScaled) ks[u] = a.kscale[c0 + row];
  }
  __builtin_amdgcn_sched_barrier(0);
  const bool sub_on = sub < nvec;
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const bool on = sub_on && h < a.nh;
#pragma unroll
    for (int i = 0; i < QV; ++i) qv[h][i] = on ? qv[h][i] : u32x4{0, 0, 0, 0};
    wv[h] = h < a.nh ? wv[h] : 0.f;
  }
  float* sp = score_ptr(a, b, c0);
  uint32_t* gmax = maxima_ptr(a, b);
  // The four-head row reduction applies when a row is exactly one 16-lane DPP row.
  constexpr bool kHead4 = (NH == 4 && LPC == 16);
  float wl = 0.f;
  if (kHead4) {
    const bool b0 = lane & 1, b1 = (lane >> 1) & 1;
    wl = b0 ? (b1 ? wv[3] : wv[2]) : (b1 ? wv[1] : wv[0]);
  }
  uint32_t* gsec = second_ptr(a, b);
  Top2 st[G::NG];
#pragma unroll
  for (int g = 0; g < G::NG; ++g) st[g] = Top2{0u, 255u, 0u};
  // With LPC >= 8, lane (slot * LPC + u) keeps pass u's score, so one store per wave writes the
  // wave's RW consecutive scores.
  constexpr bool kGather = LPC >= kPasses;
  float mine = 0.f;
#pragma unroll
  for (int u = 0; u < kPasses; ++u) {
    const int64_t row = row0 + u * G::RP + slot;
    float s;
    if (kHead4) {
      float pd[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) pd[h] = Dot16<ET>::dot(qv[h], kv[u]);
      s = head4_row_score(pd, wl, lane);
    } else {
      s = 0.f;
#pragma unroll
      for (int h = 0; h < NH; ++h) s = fmaf(wv[h], fmaxf(group_sum<LPC>(Dot16<ET>::dot(qv[h], kv[u])), 0.f), s);
    }
    // A key row scale c >= 0 leaves the ReLUs alone: sum_h w_h ReLU(c x_h) = c sum_h w_h ReLU(x_h).
    if (kScaled) s *= ks[u];
    const bool valid = row < n;
    if (kGather) mine = (sub == u) ? s : mine;
    else if (sub == 0 && valid) sp[row] = s;
    const uint32_t key = valid ? score_key(s) : 0u;   // 0: below every key
    // Position of this row within its group: (u mod PG) * RP + slot.
    top2_add(st[u / G::PG], key, (uint32_t)((u % G::PG) * G::RP + slot));
  }
  if (kGather) {
    const int64_t row = row0 + sub * G::RP + slot;
    if (sub < kPasses && row < n) sp[row] = mine;
  }
  // The lanes of one key row agree; merge the statistics of the wave's rows.
#pragma unroll
  for (int g = 0; g < G::NG; ++g) {
#pragma unroll
    for (int o = LPC; o < 64; o <<= 1) st[g] = top2_merge(st[g], top2_xor(st[g], o));
    if (lane == 0) {
      const int64_t gi = (row0 + g * G::GS) / G::GS;
      gmax[gi] = st[g].m1;
      gsec[gi] = pack_second(st[g]);
    }
  }
}

template <int CTRL>
__device__ __forceinline__ Top2 top2_dpp(const Top2& s) {
  return Top2{(uint32_t)__builtin_amdgcn_mov_dpp((int)s.m1, CTRL, 0xF, 0xF, false),
              (uint32_t)__builtin_amdgcn_mov_dpp((int)s.p1, CTRL, 0xF, 0xF, false),
              (uint32_t)__builtin_amdgcn_mov_dpp((int)s.m2, CTRL, 0xF, 0xF, false)};
}
// Merged over each group of 8 lanes (xor 1, xor 2, half-row mirror), every lane of the 8 gets it.
__device__ __forceinline__ Top2 top2_merge8(Top2 s) {
  s = top2_merge(s, top2_dpp<0xB1>(s));
  s = top2_merge(s, top2_dpp<0x4E>(s));
  return top2_merge(s, top2_dpp<0x141>(s));
}

// One level of the composite reduction: merges (maximum, top composite, second composite)
// with the lane that DPP control CTRL names (all lanes of a row are valid sources).
template <int CTRL>
__device__ __forceinline__ void top2c_step(uint32_t& m, uint32_t& c1, uint32_t& c2) {
  // A zero `old` lets the compiler fold the moves of m and c1 into DPP forms of max and min.
  const uint32_t om = dpp0<CTRL>(m);
  const uint32_t o1 = dpp0<CTRL>(c1);
  const uint32_t o2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)c2, CTRL, 0xF, 0xF, false);
  m = max(m, om);
  c2 = max(max(c2, o2), min(c1, o1));
  c1 = max(c1, o1);
}

// Tiles of 16 keys per wave in score_mfma_kernel: 8 KiB of keys, and at least one group.
constexpr int mfma_tiles(int d, int es) { return 8192 / (16 * d * es) > 2 ? 8192 / (16 * d * es) : 2; }

// K1 as a matrix product, for head_dim D in {64, 128, 256} and up to 16 heads. A wave scores
// tiles of 16 consecutive keys with v_mfma_f32_16x16x32_bf16: A = the queries (row = head),
// B = the keys (column = key), one MFMA per 32 channels.
//   Loads: as in score_kernel, every instruction reads 1 KiB of whole consecutive rows (16
//   bytes per lane, non-temporal), all issued before the first use.
//   Each tile then goes through the wave's own LDS tile (rows padded by 16 bytes, so the 16
//   keys of a fragment read fall in distinct banks) into the B layout: lane (g, c) = (lane / 16,
//   lane % 16) supplies key c's channels for k-slots 8g .. 8g + 7. The channel order inside
//   the contraction is free as long as A and B agree:
//     bf16: MFMA t takes channels 32t + 8g .. + 8;
//     fp8:  a 16-byte fragment read holds channels 64i + 16g .. + 16, MFMA 2i + h its half h
//           (converted to bf16, exactly).
// The result leaves lane (g, c) with the dots of heads 4g .. 4g + 3 against key c; ReLU,
// weights and (fp8) the row scale follow, summed over the 4 lane rows when there are more
// than 4 heads. A wave covers TILES tiles (8 KiB of keys; 2 tiles = one group at least).
// PAGED: the keys (and FP8 row scales) come from paged pools; a wave's keys lie in one page (pages
// of at least as many rows as a wave scores), so one page-table read, issued with the query
// loads, places them.
template <typename ET, int D, int NH4, bool PAGED = false>
__global__ __launch_bounds__(kThreads) void score_mfma_kernel(Args a) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  constexpr int ES = (int)sizeof(ET);                  // 2: bf16 keys, 1: E4M3 keys
  constexpr int ROWB = D * ES;                         // bytes per key row
  constexpr int PITCH = ROWB + 16;                     // LDS row pitch
  constexpr int T = D / 32;                            // MFMAs per tile
  constexpr int TILES = mfma_tiles(D, ES);
  constexpr int LPR = ROWB / 16;                       // lanes per row in a load
  constexpr int RPI = 64 / LPR;                        // rows per load instruction
  constexpr int LOADS = TILES * 16 / RPI;              // load instructions per wave
  constexpr int LPT = 16 / RPI;                        // of them per tile
  constexpr bool kScaled = ES == 1;
  static_assert(D % 64 == 0 && TILES % 2 == 0 && RPI >= 1 && 16 % RPI == 0, "shape");
  __shared__ __attribute__((aligned(16))) unsigned char tile_lds[kThreads / 64][16 * PITCH];
  const int b = blockIdx.y;
  int64_t c0;
  const int64_t n = cand_count(a, b, &c0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
  const int64_t key0 = ((int64_t)blockIdx.x * (kThreads / 64) + wave) * TILES * 16;
  if (key0 >= n) return;                               // no barriers follow
  static_assert(TILES * 16 <= 128, "a wave scores at most 128 keys (the paged calls' smallest page)");
  int64_t krow0 = c0 + key0;                           // storage row of key0; rows follow it
  if (PAGED) {
    const int64_t p = a.pt[(int64_t)b * a.pt_stride + (key0 >> a.shift)];
    const int64_t pc = p < 0 || p >= a.pool_pages ? 0 : p;   // out of the pool: page 0 is read
    krow0 = (pc << a.shift) | (key0 & (((int64_t)1 << a.shift) - 1));
  }
  // Queries (A): MFMA t, lane (g, c): head c, the 8 channels this lane supplies.
  const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((size_t)b * a.nh + min(c, a.nh - 1)) * D;
  u32x4 qv[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int ch = ES == 2 ? 32 * t + 8 * g : 64 * (t >> 1) + 16 * g + 8 * (t & 1);
    qv[t] = *reinterpret_cast<const u32x4*>(qp + ch);
  }
  float wv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * g + r;
    wv[r] = a.w[(size_t)b * a.nh + min(h, a.nh - 1)];
  }
  __builtin_amdgcn_sched_barrier(0);                   // query loads go out (and return) first
  const char* kb = static_cast<const char*>(a.keys) + (size_t)krow0 * ROWB;
  const int rr = lane / LPR, sc = lane % LPR;          // this lane's row and 16-byte chunk in a load
  u32x4 kv[LOADS];
#pragma unroll
  for (int u = 0; u < LOADS; ++u) {
    int64_t row = key0 + u * RPI + rr;
    if (row > n - 1) row = n - 1;
    kv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + (row - key0) * ROWB + 16 * sc));
  }
  float ks[TILES];
  if (kScaled) {
#pragma unroll
    for (int j = 0; j < TILES; ++j) ks[j] = a.kscale[krow0 + (min(key0 + 16 * j + c, n - 1) - key0)];
  }
  __builtin_amdgcn_sched_barrier(0);
  const bool qon = c < a.nh;
#pragma unroll
  for (int t = 0; t < T; ++t) qv[t] = qon ? qv[t] : u32x4{0, 0, 0, 0};
#pragma unroll
  for (int r = 0; r < 4; ++r) wv[r] = 4 * g + r < a.nh ? wv[r] : 0.f;

  float* sp = score_ptr(a, b, c0);
  uint32_t* gmax = maxima_ptr(a, b);
  uint32_t* gsec = second_ptr(a, b);
  unsigned char* lt = tile_lds[wave];
  uint32_t kk[TILES];                                  // the score keys of key c of each tile
#pragma unroll
  for (int j = 0; j < TILES; ++j) {
    // The tile's rows into LDS, then this lane's fragments back out (one wave: LDS operations
    // stay in program order, so no barrier is needed between them).
#pragma unroll
    for (int v = 0; v < LPT; ++v)
      *reinterpret_cast<u32x4*>(lt + (v * RPI + rr) * PITCH + 16 * sc) = kv[j * LPT + v];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < T; ++t) {
      u32x4 kf;
      if (ES == 2) {
        kf = *reinterpret_cast<const u32x4*>(lt + c * PITCH + 64 * t + 16 * g);
      } else {
        const uint2 x = *reinterpret_cast<const uint2*>(lt + c * PITCH + 64 * (t >> 1) + 16 * g + 8 * (t & 1));
        kf[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.x, 1.0f, false));
        kf[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.x, 1.0f, true));
        kf[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.y, 1.0f, false));
        kf[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.y, 1.0f, true));
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qv[t]), __builtin_bit_cast(bf16x8, kf),
                                                    acc, 0, 0, 0);
    }
    float p = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) p = fmaf(wv[r], fmaxf(acc[r], 0.f), p);
    if (NH4 > 1) {                                     // heads 4g .. 4g + 3 live in lane row g
      p += __shfl_xor(p, 16, 64);
      p += __shfl_xor(p, 32, 64);
    }
    // A key row scale >= 0 leaves the ReLUs alone: sum_h w_h ReLU(c x_h) = c sum_h w_h ReLU(x_h).
    if (kScaled) p *= ks[j];
    const int64_t key = key0 + 16 * j + c;
    const bool valid = key < n;
    if (g == 0 && valid) sp[key] = p;
    kk[j] = valid ? score_key(p) : 0u;                 // 0: below every key
  }
  // Group statistics: tiles 2q and 2q + 1 form the group; key c of tile 2q + e sits at
  // position 16e + c. Composite words (key & ~31) | position rank the candidates as in
  // group_stats4, over the 16 lanes of row 0.
#pragma unroll
  for (int q = 0; q < TILES / 2; ++q) {
    const uint32_t k0 = kk[2 * q], k1 = kk[2 * q + 1];
    const uint32_t w0 = (k0 & ~31u) | (uint32_t)c, w1 = (k1 & ~31u) | (uint32_t)(16 + c);
    uint32_t m = max(k0, k1), c1 = max(w0, w1), c2 = min(w0, w1);
    top2c_step<0xB1>(m, c1, c2);     // xor 1
    top2c_step<0x4E>(m, c1, c2);     // xor 2
    top2c_step<0x141>(m, c1, c2);    // half-row mirror
    top2c_step<0x140>(m, c1, c2);    // row mirror: all 16 lanes of the row
    if (lane == 0) {
      const int64_t gi = (key0 + 32 * q) / kGroup;
      gmax[gi] = m;
      gsec[gi] = (c2 & ~31u) | (c1 & 31u);
    }
  }
}

// Statistics of the groups of 32 held by a wave as 8 lanes x 4 consecutive scores. Beside
// the exact maximum it ranks composite words (key & ~31) | position: their largest gives a
// position of the maximum and their second largest the second key with its low five bits
// cleared. When two keys share the maximum's upper 27 bits the position may be either of
// them, but the word then satisfies (word | 31) >= maximum, so a group is only ever read
// through its position when its maximum is the one key that large. Keys are taken raw here
// (-0 one below +0) and mended on the results: the maximum maps key(-0) to key(+0), and a
// second word in the 32 keys below key(+0) is raised to key(+0), which can only mark more
// groups full. Lanes with lane % 8 == 0 store the group's two words; scores whose bit in
// `valid` is clear count as key 0, below every score.
__device__ __forceinline__ void group_stats4(const f32x4& x, const uint32_t (&pos)[4], int lane,
                                             uint32_t* gm, uint32_t* gs, uint32_t valid = 0xFu) {
  uint32_t k[4], c[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t u = __float_as_uint(x[e]);
    k[e] = (valid >> e) & 1u ? u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u) : 0u;
    c[e] = (k[e] & ~31u) | pos[e];
  }
  uint32_t m = max(max(k[0], k[1]), max(k[2], k[3]));
  const uint32_t hi01 = max(c[0], c[1]), lo01 = min(c[0], c[1]);
  const uint32_t hi23 = max(c[2], c[3]), lo23 = min(c[2], c[3]);
  uint32_t c1 = max(hi01, hi23);
  uint32_t c2 = max(max(lo01, lo23), min(hi01, hi23));
  top2c_step<0xB1>(m, c1, c2);     // xor 1
  top2c_step<0x4E>(m, c1, c2);     // xor 2
  top2c_step<0x141>(m, c1, c2);    // half-row mirror: lanes 0-3 with 4-7
  if ((lane & 7) == 0) {
    uint32_t s2 = c2 & ~31u;
    s2 = s2 == 0x7FFFFFE0u ? 0x80000000u : s2;
    *gm = m == 0x7FFFFFFFu ? 0x80000000u : m;
    *gs = s2 | (c1 & 31u);
  }
}

// K1 for caller-provided scores: group statistics only. Wave w of block x covers 256 * P
// consecutive scores starting at (4x + w) * 256 * P: P 16-byte loads per lane when the
// sequence's scores are 16-byte aligned (a group of 32 is then 8 lanes of one load), else
// 4P 4-byte loads (a group is half a wave of one load).
// The statistics of one wave's 256 * P scores from `base` (the body of max_kernel).
template <int P>
__device__ __forceinline__ void max_wave(const Args& a, int b, int64_t n, int64_t c0, int64_t base, int lane) {
  const float* sp = score_ptr(a, b, c0);
  uint32_t* gmax = maxima_ptr(a, b);
  uint32_t* gsec = second_ptr(a, b);
  const int64_t nfull = n / 4;                         // whole 16-byte vectors in the sequence
  if ((reinterpret_cast<uintptr_t>(sp) & 15) == 0 && nfull > 0) {
    f32x4 v[P];
#pragma unroll
    for (int u = 0; u < P; ++u) {
      int64_t j = base / 4 + u * 64 + lane;
      if (j > nfull - 1) j = nfull - 1;
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sp) + j);
    }
    uint32_t pos[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pos[e] = (uint32_t)(lane & 7) * 4 + e;
    // Only the wave that reaches the end of the sequence masks (and reads the last n % 4
    // scores, which no whole vector holds); every other wave takes the unmasked path.
    if (base + 256 * P <= 4 * nfull) {
#pragma unroll
      for (int u = 0; u < P; ++u) {
        const int64_t j0 = base + (u * 64 + lane) * 4;
        group_stats4(v[u], pos, lane, gmax + j0 / kGroup, gsec + j0 / kGroup);
      }
    } else {
      f32x4 t;
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = sp[min(4 * nfull + e, n - 1)];
#pragma unroll
      for (int u = 0; u < P; ++u) {
        const int64_t j0 = base + (u * 64 + lane) * 4;
        f32x4 x = j0 < 4 * nfull ? v[u] : t;
        uint32_t valid = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) valid |= (j0 + e < n ? 1u : 0u) << e;
        group_stats4(x, pos, lane, gmax + j0 / kGroup, gsec + j0 / kGroup, valid);
      }
    }
  } else {
    float v[4 * P];
#pragma unroll
    for (int u = 0; u < 4 * P; ++u) {
      int64_t j = base + u * 64 + lane;
      if (j > n - 1) j = n - 1;
      v[u] = sp[j];
    }
#pragma unroll
    for (int u = 0; u < 4 * P; ++u) {
      const int64_t j = base + u * 64 + lane;
      Top2 st{j < n ? score_key(v[u]) : 0u, (uint32_t)(lane & 31), 0u};
      st = top2_merge8(st);
      st = top2_merge(st, top2_dpp<0x140>(st));        // row mirror: the 16 lanes of a row
      st = top2_merge(st, top2_xor(st, 16));           // rows 0+1, 2+3: a half-wave
      const int64_t g = (base + u * 64) / kGroup;
      if (lane == 0) { gmax[g] = st.m1; gsec[g] = pack_second(st); }
      if (lane == 32) { gmax[g + 1] = st.m1; gsec[g + 1] = pack_second(st); }
    }
  }
}

template <int P>
__global__ __launch_bounds__(kThreads) void max_kernel(Args a) {
  const int b = blockIdx.y;
  int64_t c0;
  const int64_t n = cand_count(a, b, &c0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t base = ((int64_t)blockIdx.x * (kThreads / 64) + wave) * 256 * P;
  if (base >= n) return;
  max_wave<P>(a, b, n, c0, base, lane);
}

// max_kernel for 8 loads per lane with one group per lane. A wave's 2048 scores are 64 groups:
// they are loaded coalesced (1 KiB per instruction), transposed through the wave's LDS tile so that
// lane L holds group L's 32 scores in order, and each lane then walks its own group: the maximum
// by max3, the top two composite words by max3 / med3 (c1' = max3(c1, x, y), c2' = max(c2,
// med3(c1, x, y)) keeps the two largest of c1 >= c2, x, y). About a third of the VALU work of the
// cross-lane reduction, and no cross-lane steps. The results are the same words group_stats4
// writes. Waves that are not whole and aligned take max_wave<8>.
constexpr int kLaneThreads = 256;
constexpr int kLaneTilePitch = 9;   // 16-byte vectors per lane in the tile: 8 plus one of padding

// The median of three (v_med3_u32).
__device__ __forceinline__ uint32_t med3u(uint32_t a, uint32_t b, uint32_t c) {
  return max(min(a, b), min(max(a, b), c));
}

__global__ __launch_bounds__(kLaneThreads) void max_lane_kernel(Args a) {
  __shared__ f32x4 tile[kLaneThreads / 64][64 * kLaneTilePitch];
  const int b = blockIdx.y;
  int64_t c0;
  const int64_t n = cand_count(a, b, &c0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t base = ((int64_t)blockIdx.x * (kLaneThreads / 64) + wave) * 2048;
  if (base >= n) return;
  const float* sp = score_ptr(a, b, c0);
  const int64_t nfull = n / 4;
  if ((reinterpret_cast<uintptr_t>(sp) & 15) != 0 || base + 2048 > 4 * nfull) {
    max_wave<8>(a, b, n, c0, base, lane);
    return;
  }
  const f32x4* sp4 = reinterpret_cast<const f32x4*>(sp) + base / 4;
  f32x4 v[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(sp4 + u * 64 + lane);
  // Vector u * 64 + lane belongs to lane (u * 64 + lane) / 8, at slot lane % 8 of its group.
  f32x4* t = tile[wave];
#pragma unroll
  for (int u = 0; u < 8; ++u) t[(u * 8 + lane / 8) * kLaneTilePitch + (lane & 7)] = v[u];
  // The wave's LDS operations execute in order, so its own writes are visible to these reads.
  __asm__ volatile("" ::: "memory");
#pragma unroll
  for (int u = 0; u < 8; ++u) v[u] = t[lane * kLaneTilePitch + u];
  uint32_t m = 0, c1 = 0, c2 = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      const uint32_t ux = __float_as_uint(v[u][e]), uy = __float_as_uint(v[u][e + 1]);
      const uint32_t kx = ux ^ ((uint32_t)((int32_t)ux >> 31) | 0x80000000u);
      const uint32_t ky = uy ^ ((uint32_t)((int32_t)uy >> 31) | 0x80000000u);
      const uint32_t cx = (kx & ~31u) | (uint32_t)(4 * u + e);
      const uint32_t cy = (ky & ~31u) | (uint32_t)(4 * u + e + 1);
      m = max(m, max(kx, ky));
      c2 = max(c2, med3u(c1, cx, cy));
      c1 = max(c1, max(cx, cy));
    }
  }
  // Mend the raw keys as group_stats4 does: -0 counts as +0.
  uint32_t s2 = c2 & ~31u;
  s2 = s2 == 0x7FFFFFE0u ? 0x80000000u : s2;
  const int64_t g = base / kGroup + lane;
  maxima_ptr(a, b)[g] = m == 0x7FFFFFFFu ? 0x80000000u : m;
  second_ptr(a, b)[g] = s2 | (c1 & 31u);
}

// ---------------------------------------------------------------- K2: collect and select
struct alignas(16) CollectShared {
  uint32_t key[kLdsCand];       // superset keys, index order
  uint32_t idx[kLdsCand];       // superset candidate indices
  uint32_t fkey[kFullCap][kGroup];   // kept keys of the full groups, by slot
  uint32_t fmask[kFullCap];     // their candidates with key >= L
  uint32_t fgroup[kFullCap];    // the group in each slot
  uint32_t fbase[kFullCap];     // superset position of each slot's first kept key
  uint32_t hist[kBins];         // bound bins (A), then superset bins (B, C)
  uint32_t red[2 * kCWaves];
  uint32_t tot[kScanRounds * kCWaves + 4];
  uint32_t binv[kBinCap];       // keys in the bin that holds the k-th largest
  uint32_t misc[8];             // 0, 1: bin and rank; 2: bin fill; 3, 4: tau, ties; 5: full slots
};

// Ordered scan over items (round r, thread t), taken in that order, for the K2 block: given
// this thread's count for each round, returns the total and sets off[r] to the sum of the
// counts before item (r, t). Wave sums use DPP; wave 0 scans the per-(round, wave) totals.
// Ends with a barrier, so LDS written before the call is visible after it.
template <int R>
__device__ uint32_t ordered_scan(const uint32_t (&cnt)[R], uint32_t (&off)[R], CollectShared& sh) {
  static_assert(R <= kScanRounds, "too many rounds");
  constexpr int N = R * kCWaves;
  constexpr int PL = (N + 63) / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t wtot[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t inc = wave_inclusive_sum(cnt[r]);
    off[r] = inc - cnt[r];
    wtot[r] = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) sh.tot[wave * R + r] = wtot[r];
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    uint32_t v[PL], sum = 0;
#pragma unroll
    for (int p = 0; p < PL; ++p) {
      const int i = lane * PL + p;      // position in (round, wave) order
      v[p] = i < N ? sh.tot[(i % kCWaves) * R + i / kCWaves] : 0u;
      sum += v[p];
    }
    const uint32_t inc = wave_inclusive_sum(sum);
    uint32_t run = inc - sum;
#pragma unroll
    for (int p = 0; p < PL; ++p) {
      const int i = lane * PL + p;
      if (i < N) sh.tot[(i % kCWaves) * R + i / kCWaves] = run;
      run += v[p];
    }
    if (lane == 63) sh.tot[N] = inc;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) off[r] += sh.tot[wave * R + r];
  const uint32_t total = sh.tot[N];
  __syncthreads();
  return total;
}

// The r-th largest (1 <= r <= m) of m keys from `get`, all in [lo, hi], by 11-bit radix
// steps below the bits lo and hi share (2048 bins, two per thread); *ties_take gets how many
// keys equal to the result rank within the top r.
template <typename Get>
__device__ uint32_t block_radix_select(Get get, uint32_t m, uint32_t r, uint32_t lo, uint32_t hi,
                                       CollectShared& sh, uint32_t* ties_take) {
  int rem = differing_bits(lo, hi);
  uint32_t prefix = rem == 32 ? 0u : (uint32_t)((uint64_t)hi >> rem);
  while (rem > 0) {
    const int width = rem < 11 ? rem : 11;
    rem -= width;
    const uint32_t nb = 1u << width;
    for (int i = threadIdx.x; i < kBins; i += kCThreads) sh.hist[i] = 0u;
    __syncthreads();
    for (uint32_t x0 = 0; x0 < m; x0 += kGlobalRounds * kCThreads) {
      uint32_t kk[kGlobalRounds];
#pragma unroll
      for (int q = 0; q < kGlobalRounds; ++q) kk[q] = get(min(x0 + q * kCThreads + threadIdx.x, m - 1));
#pragma unroll
      for (int q = 0; q < kGlobalRounds; ++q) {
        const uint32_t v = kk[q];
        if (x0 + q * kCThreads + threadIdx.x < m && (uint32_t)((uint64_t)v >> (rem + width)) == prefix)
          atomicAdd(&sh.hist[(v >> rem) & (nb - 1)], 1u);
      }
    }
    __syncthreads();
    const uint32_t t = threadIdx.x;
    const uint32_t c0 = sh.hist[kBins - 1 - 2 * t], c1 = sh.hist[kBins - 2 - 2 * t];
    uint32_t total;
    const uint32_t run = block_exclusive_sum_t<kCWaves>(c0 + c1, &total, sh.red);
    if (run < r && run + c0 + c1 >= r) {
      if (run + c0 >= r) { sh.misc[0] = kBins - 1 - 2 * t; sh.misc[1] = run; }
      else { sh.misc[0] = kBins - 2 - 2 * t; sh.misc[1] = run + c0; }
    }
    __syncthreads();
    r -= sh.misc[1];
    prefix = (prefix << width) | sh.misc[0];
    __syncthreads();
  }
  *ties_take = r;
  return prefix;
}

// Writes, ascending, the indices of the m candidates (key from `key`, index from `idx`, in
// index order) that are above tau or among the first ties_take equal to it. R rounds of the
// block per batch (R * 1024 candidates). One ordered scan per batch counts, for every
// candidate, the keys above tau (low 16 bits) and the ties (high 16 bits) before it: a
// candidate is taken if it is above tau or is a tie with fewer than ties_take ties before it,
// and its place is (keys above tau before it) + min(ties before it, ties_take).
template <int R, typename GK, typename GI>
__device__ void ordered_select(GK key, GI idx, uint32_t m, uint32_t tau, uint32_t ties_take, uint32_t keff,
                               int32_t* out, CollectShared& sh) {
  static_assert(R * kCThreads < 65536, "per-batch counts must fit 16 bits");
  uint32_t gt_before = 0, ties_before = 0;
  for (uint32_t x0 = 0; x0 < m; x0 += R * kCThreads) {
    uint32_t kk[R], c[R], off[R];
#pragma unroll
    for (int q = 0; q < R; ++q) kk[q] = key(min(x0 + q * kCThreads + threadIdx.x, m - 1));
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const bool in = x0 + q * kCThreads + threadIdx.x < m;
      c[q] = !in ? 0u : kk[q] > tau ? 1u : kk[q] == tau ? 0x10000u : 0u;
    }
    const uint32_t total = ordered_scan(c, off, sh);
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const bool in = x0 + q * kCThreads + threadIdx.x < m;
      const uint32_t gt = gt_before + (off[q] & 0xFFFFu), eq = ties_before + (off[q] >> 16);
      const bool take = in && (kk[q] > tau || (kk[q] == tau && eq < ties_take));
      const uint32_t pos = gt + min(eq, ties_take);
      if (take && pos < keff) out[pos] = (int32_t)idx(x0 + q * kCThreads + threadIdx.x);
    }
    gt_before += total & 0xFFFFu;
    ties_before += total >> 16;
  }
}

// The rare paths live out of line so the common path's code stays compact: a single
// workgroup runs it once, so its size, not its instruction count, sets how long instruction
// fetch takes.
// Global path: exact selection over all n candidates, read from the score array.
__device__ __attribute__((noinline)) void select_global(__amdgpu_buffer_rsrc_t srs, uint32_t n, uint32_t keff,
                                                        int32_t* out, CollectShared& sh) {
  uint32_t ties_take;
  auto key = [&](uint32_t i) { return score_key(__uint_as_float(buffer_u32(srs, i))); };
  const uint32_t tau = block_radix_select(key, n, keff, 0u, 0xFFFFFFFFu, sh, &ties_take);
  ordered_select<kGlobalRounds>(key, [&](uint32_t i) { return i; }, n, tau, ties_take, keff, out, sh);
}

// A crowded threshold bin (heavy ties): tau and the ties to take by radix steps over the LDS
// superset, keys in [L, their maximum].
// Returned by value (in registers): an out-parameter would put the caller's variable in
// scratch memory on the common path too.
struct TauTies {
  uint32_t tau, ties_take;
};
__device__ __attribute__((noinline)) TauTies tau_by_radix(CollectShared& sh, uint32_t T, uint32_t keff, uint32_t L) {
  uint32_t hi = 0;
  for (uint32_t i = threadIdx.x; i < T; i += kCThreads) hi = max(hi, sh.key[i]);
  uint32_t unused = 0xFFFFFFFFu;
  block_minmax_t<kCWaves>(&unused, &hi, sh.red);
  TauTies r;
  r.tau = block_radix_select([&](uint32_t i) { return sh.key[i]; }, T, keff, L, hi, sh, &r.ties_take);
  return r;
}

// The bound of the collect step: over the workgroup's nonzero values u (NU per thread, at
// least keff of them), the lower edge of the bin holding the keff-th largest, with 2048
// monotone bins (u - umin) >> shift: every value in that bin or above is at least the edge,
// and there are at least keff of them. Also returns the largest value in *umax.
template <int NU>
__device__ uint32_t block_bound(const uint32_t (&u)[NU], uint32_t keff, uint32_t* umax, CollectShared& sh) {
  const uint32_t t = threadIdx.x;
  uint32_t lo = 0xFFFFFFFFu, hi = 0;
#pragma unroll
  for (int j = 0; j < NU; ++j) {
    lo = min(lo, u[j] - 1u);                            // key 0 wraps to the top: ignored
    hi = max(hi, u[j]);
  }
  block_minmax_t<kCWaves, false>(&lo, &hi, sh.red);     // its barrier also orders the clears
  const uint32_t vmin = lo + 1u;
  *umax = hi;
  const int span_bits = differing_bits(0u, hi - vmin);
  const int shift = span_bits > 11 ? span_bits - 11 : 0;
#pragma unroll
  for (int j = 0; j < NU; ++j)
    if (u[j] != 0u) atomicAdd(&sh.hist[(u[j] - vmin) >> shift], 1u);
  __syncthreads();
  const uint32_t h0 = sh.hist[kBins - 1 - 2 * t], h1 = sh.hist[kBins - 2 - 2 * t];
  uint32_t total;
  const uint32_t run = block_exclusive_sum_t<kCWaves, false>(h0 + h1, &total, sh.red);
  if (run < keff && run + h0 + h1 >= keff) sh.misc[0] = run + h0 >= keff ? kBins - 1 - 2 * t : kBins - 2 - 2 * t;
  __syncthreads();
  return vmin + (sh.misc[0] << shift);
}

// The exact top-k of sequence b into out[0 .. k) (global or LDS), run by a whole workgroup of
// kCThreads threads (t = threadIdx.x) on LDS `sh`, from the first statistics tile ft that
// collect_prefetch requested. Every early return below is uniform over the workgroup.
// The first tile of sequence b's group statistics (thread t: groups 8t .. 8t+7), requested before
// anything else is known: its address depends on the sequence only, and the buffer bound covers
// the sequence's whole statistics area. collect_seq clears the entries past the sequence's groups
// once the candidate count has arrived.
struct FirstTile {
  uint32_t mv[kMaxPerThread], sv[kMaxPerThread];
};
__device__ __forceinline__ void collect_prefetch(const Args& a, int b, FirstTile& ft) {
  const uint32_t t = threadIdx.x;
  const uint32_t cap = (uint32_t)maxima_cap(a.max_cand);
  const __amdgpu_buffer_rsrc_t mrs = buffer_rsrc(maxima_ptr(a, b), cap * 4u);
  const __amdgpu_buffer_rsrc_t qrs = buffer_rsrc(second_ptr(a, b), cap * 4u);
  const u32x4 m0 = buffer_u32x4(mrs, kMaxPerThread * t), m1 = buffer_u32x4(mrs, kMaxPerThread * t + 4);
  const u32x4 q0 = buffer_u32x4(qrs, kMaxPerThread * t), q1 = buffer_u32x4(qrs, kMaxPerThread * t + 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ft.mv[j] = m0[j]; ft.mv[4 + j] = m1[j]; ft.sv[j] = q0[j]; ft.sv[4 + j] = q1[j];
  }
}

__device__ __forceinline__ void collect_seq(const Args& a, int b, int32_t* out, CollectShared& sh, FirstTile& ft) {
  const uint32_t t = threadIdx.x;
  uint32_t (&mv)[kMaxPerThread] = ft.mv;                 // thread t: groups t0 + 8t .. 8t+7
  uint32_t (&sv)[kMaxPerThread] = ft.sv;
  int64_t c0;
  const uint32_t n = (uint32_t)cand_count(a, b, &c0);   // <= 2^22: 32-bit index math below
  const uint32_t keff = min((uint32_t)a.k, n);
  for (uint32_t i = keff + t; i < (uint32_t)a.k; i += kCThreads) out[i] = -1;
  if (keff == 0) return;
  if (n <= keff) {                                      // every candidate is selected
    for (uint32_t i = t; i < n; i += kCThreads) out[i] = (int32_t)i;
    return;
  }
  const float* sp = score_ptr(a, b, c0);
  const __amdgpu_buffer_rsrc_t srs = buffer_rsrc(sp, n * 4u);
  const int gs = a.gs;
  const int gshift = __ffs(gs) - 1;
  const uint32_t ng = (n + gs - 1) >> gshift;
  const uint32_t nt = min(ng, (uint32_t)kTile);
  const __amdgpu_buffer_rsrc_t mrs = buffer_rsrc(maxima_ptr(a, b), ng * 4u);
  const __amdgpu_buffer_rsrc_t qrs = buffer_rsrc(second_ptr(a, b), ng * 4u);
#pragma unroll
  for (int j = 0; j < kMaxPerThread; ++j)
    if (kMaxPerThread * t + j >= ng) { mv[j] = 0u; sv[j] = 0u; }
  auto load_tile = [&](uint32_t t0) {
    const uint32_t e0 = t0 + kMaxPerThread * t;
    const u32x4 m0 = buffer_u32x4(mrs, e0), m1 = buffer_u32x4(mrs, e0 + 4);
    const u32x4 s0 = buffer_u32x4(qrs, e0), s1 = buffer_u32x4(qrs, e0 + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) { mv[j] = m0[j]; mv[4 + j] = m1[j]; sv[j] = s0[j]; sv[4 + j] = s1[j]; }
  };

  // (A) The bound L: at least keff disjoint sets of groups have a maximum >= L, so L never
  // exceeds the k-th largest score. The sets are the tile slots: slot e (< 8192) holds groups
  // e, e + 8192, e + 2 * 8192, ... (one group when the sequence fits one tile), and its
  // maximum is the largest over the tiles. L is the lower edge of the bin holding the
  // keff-th largest of the maxima of runs of 4 consecutive slots when there are at least
  // 4 keff slots (a run at or above L holds a slot at or above L), else of the slot maxima.
  // Bins: (u - umin) >> shift, 2048 of them, monotone. Groups past the sequence read as key 0,
  // below every score, and take no part. Every tile's maxima are ranked, so the bound and the
  // largest key (the superset's bin range) cover the whole sequence.
  uint32_t rm[kMaxPerThread];                           // slot maxima over the tiles (tile 0 is in mv)
#pragma unroll
  for (int j = 0; j < kMaxPerThread; ++j) rm[j] = mv[j];
  for (uint32_t t0 = kTile; t0 < ng; t0 += 4u * kTile) {
    // Up to four further tiles per round: their loads are issued before any is used.
    u32x4 x[4][2];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t e0 = min(t0 + (uint32_t)r * kTile, ng) + kMaxPerThread * t;   // past ng: reads 0
      x[r][0] = buffer_u32x4(mrs, e0);
      x[r][1] = buffer_u32x4(mrs, e0 + 4);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) { rm[j] = max(rm[j], x[r][0][j]); rm[4 + j] = max(rm[4 + j], x[r][1][j]); }
  }
  for (uint32_t i = t; i < kBins; i += kCThreads) sh.hist[i] = 0u;
  if (t == 0) { sh.misc[2] = 0; sh.misc[5] = 0; }
  uint32_t L = 0, vmax = 0;
  if (nt >= 4u * keff) {
    const uint32_t u[2] = {max(max(rm[0], rm[1]), max(rm[2], rm[3])), max(max(rm[4], rm[5]), max(rm[6], rm[7]))};
    L = block_bound<2>(u, keff, &vmax, sh);
  } else if (nt >= keff) {
    L = block_bound<kMaxPerThread>(rm, keff, &vmax, sh);
  } else {                                              // fewer than k groups: every candidate
    __syncthreads();
  }
  for (uint32_t i = t; i < kBins; i += kCThreads) sh.hist[i] = 0u;   // reused for the superset

  // (B) The superset: every candidate with key >= L, in index order, binned by key over
  // [L, max] as it is kept. A group whose maximum is below L holds none. A group whose
  // statistics word shows no second key that could reach L ((word | 31) < L) holds exactly
  // one, its maximum at the stored position. The others ("full", typically a few percent of
  // the listed ones) are read whole by the thread that owns them, their kept keys staged in
  // LDS. One ordered scan per tile places everything.
  uint32_t T = 0, fdone = 0;                            // superset size; full slots read so far
  bool fits = true;
  const uint32_t top = max(vmax, L);
  const float scale2 = top > L ? (float)(kBins - 1) / (float)(top - L) : 0.f;
  auto bin2 = [&](uint32_t v) { return min((uint32_t)(kBins - 1), (uint32_t)((float)(v - L) * scale2)); };
  for (uint32_t t0 = 0; t0 < ng; t0 += kTile) {
    if (t0 > 0) load_tile(t0);
    const uint32_t g0 = t0 + kMaxPerThread * t;          // this thread's first group
    uint32_t lm = 0, fm = 0;
#pragma unroll
    for (int j = 0; j < kMaxPerThread; ++j) {
      const bool listed = g0 + j < ng && mv[j] >= L;
      lm |= (listed ? 1u : 0u) << j;
      fm |= ((listed && (sv[j] | 31u) >= L) ? 1u : 0u) << j;
    }
    // Full groups get LDS slots (in no particular order) and are read whole, two per wave,
    // one score per lane; then each thread counts what its groups keep.
    uint32_t slot0 = 0;
    if (fm) {
      slot0 = atomicAdd(&sh.misc[5], (uint32_t)__popc(fm));
      uint32_t slot = slot0;
#pragma unroll
      for (int j = 0; j < kMaxPerThread; ++j)
        if ((fm >> j) & 1u) {
          if (slot < (uint32_t)kFullCap) sh.fgroup[slot] = g0 + j;
          ++slot;
        }
    }
    __syncthreads();
    const uint32_t nfull = min(sh.misc[5], (uint32_t)kFullCap);   // this tile's slots: fdone ..
    {
      const int lane = t & 63, half = lane >> 5, li = lane & 31;
      for (uint32_t j0 = fdone + 2 * (t >> 6); j0 < nfull; j0 += 2 * kCWaves) {
        const uint32_t j = j0 + half;
        const bool on = j < nfull;
        const uint32_t c = on ? (sh.fgroup[j] << gshift) + li : 0u;
        const uint32_t v = score_key(__uint_as_float(buffer_u32(srs, c)));
        const bool keep = on && li < gs && c < n && v >= L;
        const uint32_t m = (uint32_t)(__ballot(keep) >> (32 * half));
        if (on) {
          sh.fkey[j][li] = v;
          if (li == 0) sh.fmask[j] = m;
        }
      }
    }
    __syncthreads();
    const uint32_t fstart = fdone;
    fdone = nfull;
    uint32_t cnt[1] = {(uint32_t)__popc(lm & ~fm)}, off[1];
    for (uint32_t i = 0, nf = (uint32_t)__popc(fm); i < nf; ++i)
      if (slot0 + i < (uint32_t)kFullCap) cnt[0] += (uint32_t)__popc(sh.fmask[slot0 + i]);
    const uint32_t total = ordered_scan(cnt, off, sh);
    if (sh.misc[5] > (uint32_t)kFullCap || T + total > (uint32_t)kLdsCand) { fits = false; break; }
    // A group with one key at or above L is placed by its owner; a full group's place is
    // recorded and its kept keys are placed afterwards by the lanes that read them.
    uint32_t pos = T + off[0];
#pragma unroll
    for (int j = 0; j < kMaxPerThread; ++j) {
      if ((lm >> j) & 1u) {
        if (!((fm >> j) & 1u)) {
          sh.key[pos] = mv[j];
          sh.idx[pos] = ((g0 + j) << gshift) + (sv[j] & 31u);
          atomicAdd(&sh.hist[bin2(mv[j])], 1u);
          ++pos;
        } else {
          const uint32_t slot = slot0 + (uint32_t)__popc(fm & ((1u << j) - 1u));
          sh.fbase[slot] = pos;
          pos += (uint32_t)__popc(sh.fmask[slot]);
        }
      }
    }
    if (nfull > fstart) {                               // uniform: this tile has full groups
      __syncthreads();
      const int lane = t & 63, half = lane >> 5, li = lane & 31;
      for (uint32_t j0 = fstart + 2 * (t >> 6); j0 < nfull; j0 += 2 * kCWaves) {
        const uint32_t j = j0 + half;
        if (j < nfull) {
          const uint32_t m = sh.fmask[j];
          if ((m >> li) & 1u) {
            const uint32_t p = sh.fbase[j] + (uint32_t)__popc(m & ((1u << li) - 1u)), v = sh.fkey[j][li];
            sh.key[p] = v;
            sh.idx[p] = (sh.fgroup[j] << gshift) + li;
            atomicAdd(&sh.hist[bin2(v)], 1u);
          }
        }
      }
    }
    T += total;
  }
  __syncthreads();

  // (C) Exact selection.
  if (!fits) {                                          // global path
    select_global(srs, n, keff, out, sh);
    return;
  }
  if (T <= keff) {                                      // (only when the bound is not binding)
    for (uint32_t i = t; i < keff; i += kCThreads) out[i] = i < T ? (int32_t)sh.idx[i] : -1;
    return;
  }
  // The bin holding the keff-th largest superset key, and the rank still to place inside it.
  {
    const uint32_t h0 = sh.hist[kBins - 1 - 2 * t], h1 = sh.hist[kBins - 2 - 2 * t];
    uint32_t total;
    const uint32_t run = block_exclusive_sum_t<kCWaves, false>(h0 + h1, &total, sh.red);
    if (run < keff && run + h0 + h1 >= keff) {
      if (run + h0 >= keff) { sh.misc[0] = kBins - 1 - 2 * t; sh.misc[1] = run; }
      else { sh.misc[0] = kBins - 2 - 2 * t; sh.misc[1] = run + h0; }
    }
    __syncthreads();
  }
  const uint32_t bstar2 = sh.misc[0], rank = keff - sh.misc[1];
  for (uint32_t i = t; i < T; i += kCThreads) {
    const uint32_t v = sh.key[i];
    if (bin2(v) == bstar2) {
      const uint32_t slot = atomicAdd(&sh.misc[2], 1u);
      if (slot < (uint32_t)kBinCap) sh.binv[slot] = v;
    }
  }
  __syncthreads();
  const uint32_t nbin = sh.misc[2];
  uint32_t tau, ties_take;
  if (nbin <= (uint32_t)kBinCap) {
    // tau is the key kappa of the bin with #{> kappa} < rank <= #{>= kappa}.
    if (t < nbin) {
      const uint32_t kappa = sh.binv[t];
      uint32_t gt = 0, ge = 0;
      for (uint32_t j = 0; j < nbin; ++j) {
        const uint32_t v = sh.binv[j];
        gt += v > kappa ? 1u : 0u;
        ge += v >= kappa ? 1u : 0u;
      }
      if (gt < rank && rank <= ge) { sh.misc[3] = kappa; sh.misc[4] = rank - gt; }
    }
    __syncthreads();
    tau = sh.misc[3];
    ties_take = sh.misc[4];
  } else {                                              // a crowded bin (heavy ties)
    const TauTies r = tau_by_radix(sh, T, keff, L);
    tau = r.tau;
    ties_take = r.ties_take;
  }
  auto lk = [&](uint32_t i) { return sh.key[i]; };
  auto li = [&](uint32_t i) { return sh.idx[i]; };
  ordered_select<1>(lk, li, T, tau, ties_take, keff, out, sh);
}

__global__ __launch_bounds__(kCThreads) void collect_kernel(Args a, int32_t* topk) {
  __shared__ CollectShared sh;
  FirstTile ft;
  collect_prefetch(a, blockIdx.x, ft);
  collect_seq(a, blockIdx.x, topk + (size_t)blockIdx.x * a.k, sh, ft);
}

// The MFMA form of K1 when it applies (up to 16 heads, head_dim 64, 128 or 256): sets a->gs
// and launches; returns false otherwise.
template <typename ET>
bool launch_scores_mfma(int32_t batch, int32_t head_dim, Args* a, hipStream_t s) {
  if (a->nh > 16 || (head_dim != 64 && head_dim != 128 && head_dim != 256)) return false;
  const int64_t per_block = 4 * 16 * (int64_t)mfma_tiles(head_dim, (int)sizeof(ET));
  const dim3 grid((unsigned)((a->max_cand + per_block - 1) / per_block), (unsigned)batch);
  a->gs = kGroup;
  const bool wide = a->nh > 4;
  const bool paged = a->pt != nullptr;
#define CHS_MFMA(DD)                                                                                    \
  if (paged && wide) hipLaunchKernelGGL((score_mfma_kernel<ET, DD, 4, true>), grid, dim3(kThreads), 0, s, *a);  \
  else if (paged) hipLaunchKernelGGL((score_mfma_kernel<ET, DD, 1, true>), grid, dim3(kThreads), 0, s, *a);    \
  else if (wide) hipLaunchKernelGGL((score_mfma_kernel<ET, DD, 4>), grid, dim3(kThreads), 0, s, *a);           \
  else hipLaunchKernelGGL((score_mfma_kernel<ET, DD, 1>), grid, dim3(kThreads), 0, s, *a);
  switch (head_dim) {
    case 64: CHS_MFMA(64) break;
    case 128: CHS_MFMA(128) break;
    default: CHS_MFMA(256) break;
  }
#undef CHS_MFMA
  return true;
}

template <typename ET, int NH>
void launch_scores_nh(dim3 grid, hipStream_t s, const Args& a, int lpc) {
  switch (lpc) {
    case 2: hipLaunchKernelGGL((score_kernel<ET, NH, 2>), grid, dim3(kThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((score_kernel<ET, NH, 4>), grid, dim3(kThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL((score_kernel<ET, NH, 8>), grid, dim3(kThreads), 0, s, a); break;
    case 16: hipLaunchKernelGGL((score_kernel<ET, NH, 16>), grid, dim3(kThreads), 0, s, a); break;
    case 32: hipLaunchKernelGGL((score_kernel<ET, NH, 32>), grid, dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL((score_kernel<ET, NH, 64>), grid, dim3(kThreads), 0, s, a); break;
  }
}

template <typename ET>
void launch_scores(dim3 grid, hipStream_t s, const Args& a, int lpc) {
  if (a.nh <= 1) launch_scores_nh<ET, 1>(grid, s, a, lpc);
  else if (a.nh <= 2) launch_scores_nh<ET, 2>(grid, s, a, lpc);
  else if (a.nh <= 4) launch_scores_nh<ET, 4>(grid, s, a, lpc);
  else if (a.nh <= 8) launch_scores_nh<ET, 8>(grid, s, a, lpc);
  else launch_scores_nh<ET, 16>(grid, s, a, lpc);
}

}  // namespace
}  // namespace chs

extern "C" size_t chs_index_topk_workspace_size(int32_t batch, int64_t max_cand, int32_t k) {
  (void)k;
  if (batch < 1 || max_cand < 0) return 0;
  return chs::ws_layout(batch, max_cand, nullptr, nullptr);
}

namespace chs {
namespace {

// Validates chs_index_topk's arguments, lays out its workspace and fills *a and *lpc (lanes per
// key row of the score kernel).
chs_status topk_setup(chs_dtype dtype, int32_t batch, int32_t n_heads, int32_t head_dim, int32_t k,
                      const void* q_idx, const float* w, const void* k_idx, const int64_t* cu_cand,
                      int64_t max_cand, float* scores, int32_t* topk, void* workspace, size_t workspace_bytes,
                      Args* a, int* lpc) {
  if (!dtype_ok(dtype)) return CHS_ERR_DTYPE;
  if (batch < 1 || batch > 65535 || k < 1 || k > kMaxK || max_cand < 0 || max_cand >= (1LL << 31))
    return CHS_ERR_SHAPE;
  if (max_cand > kMaxCand) return CHS_ERR_UNSUPPORTED;
  const size_t es = elem_size(dtype);
  int nvec = 0;
  *lpc = 2;
  if (q_idx) {
    if (n_heads < 1 || n_heads > 16 || head_dim < 8 || head_dim * es > 1024 || (head_dim * es) % 16 != 0)
      return CHS_ERR_SHAPE;
    if (!w || !k_idx) return CHS_ERR_NULL;
    nvec = (int)(head_dim * es / 16);   // 16-byte vectors per key row (<= 64)
    while (*lpc < nvec) *lpc *= 2;      // one vector per lane, at least two lanes per row
  } else if (!scores) {
    return CHS_ERR_NULL;
  }
  if (!cu_cand || !topk || !workspace) return CHS_ERR_NULL;
  Workspace ws;
  const size_t need = ws_layout(batch, max_cand, &ws, static_cast<char*>(workspace));
  if (workspace_bytes < need) return CHS_ERR_WORKSPACE;
  a->q = q_idx; a->w = w; a->keys = k_idx; a->cu = cu_cand; a->max_cand = max_cand;
  a->nh = n_heads; a->nvec = nvec; a->k = k; a->scores = scores; a->ws = ws; a->kscale = nullptr;
  a->gs = kGroup;
  a->pt = nullptr; a->cand_len = nullptr; a->pt_stride = 0; a->shift = 0; a->pool_pages = 0;
  return CHS_OK;
}

// The first kernel of the selection: scores and group statistics (q_idx given), or group
// statistics of the caller's scores. Sets a->gs. Launches nothing when max_cand is 0.
chs_status topk_first(chs_dtype dtype, int32_t batch, Args* a, int lpc, hipStream_t s) {
  const int64_t max_cand = a->max_cand;
  if (max_cand == 0) return CHS_OK;
  if (a->q) {
    if (dtype == CHS_BF16 && launch_scores_mfma<uint16_t>(batch, a->nvec * 8, a, s)) return launch_status();
    const int rw = kPasses * (64 / lpc);              // rows per wave
    a->gs = std::min(rw, kGroup);
    const dim3 grid((unsigned)((max_cand + 4 * rw - 1) / (4 * rw)), (unsigned)batch);
    if (dtype == CHS_BF16) launch_scores<uint16_t>(grid, s, *a, lpc);
    else launch_scores<float>(grid, s, *a, lpc);
  } else {
    // Loads per lane: the most (up to kPasses) that still give about 1024 workgroups
    // (a workgroup covers 1024 * p scores).
    int p = kPasses;
    while (p > 1 && (int64_t)batch * ((max_cand + 1024 * p - 1) / (1024 * p)) < 1024) p /= 2;
    const dim3 grid((unsigned)((max_cand + 1024 * p - 1) / (1024 * p)), (unsigned)batch);
    switch (p) {
      case 1: hipLaunchKernelGGL(max_kernel<1>, grid, dim3(kThreads), 0, s, *a); break;
      case 2: hipLaunchKernelGGL(max_kernel<2>, grid, dim3(kThreads), 0, s, *a); break;
      case 4: hipLaunchKernelGGL(max_kernel<4>, grid, dim3(kThreads), 0, s, *a); break;
      default: {
        // 8 loads per lane: the lane-per-group kernel (workgroups of 2048 * 4 scores).
        static_assert(kPasses == 8, "max_lane_kernel covers 8 vectors per lane");
        const dim3 g8((unsigned)((max_cand + 4 * 2048 - 1) / (4 * 2048)), (unsigned)batch);
        hipLaunchKernelGGL(max_lane_kernel, g8, dim3(kLaneThreads), 0, s, *a);
        break;
      }
    }
  }
  return launch_status();
}

}  // namespace
}  // namespace chs

extern "C" chs_status chs_index_topk(chs_dtype dtype, int32_t batch, int32_t n_heads,
                                     int32_t head_dim, int32_t k, const void* q_idx,
                                     const float* w, const void* k_idx, const int64_t* cu_cand,
                                     int64_t max_cand, float* scores, int32_t* topk,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  using namespace chs;
  Args a;
  int lpc = 2;
  chs_status st = topk_setup(dtype, batch, n_heads, head_dim, k, q_idx, w, k_idx, cu_cand, max_cand, scores, topk,
                             workspace, workspace_bytes, &a, &lpc);
  if (st != CHS_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (topk_first(dtype, batch, &a, lpc, s) != CHS_OK) return CHS_ERR_LAUNCH;
  hipLaunchKernelGGL(collect_kernel, dim3((unsigned)batch), dim3(kCThreads), 0, s, a, topk);
  return launch_status();
}

extern "C" chs_status chs_index_scores(chs_dtype dtype, int32_t batch, int32_t n_heads, int32_t head_dim,
                                       const void* q_idx, const float* w, const void* k_idx, const int64_t* cu_cand,
                                       int64_t max_cand, float* scores, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  using namespace chs;
  if (!q_idx || !scores) return CHS_ERR_NULL;
  Args a;
  int lpc = 2;
  int32_t unused_topk = 0;                              // the selection's output is never written here
  chs_status st = topk_setup(dtype, batch, n_heads, head_dim, 1, q_idx, w, k_idx, cu_cand, max_cand, scores,
                             &unused_topk, workspace, workspace_bytes, &a, &lpc);
  if (st != CHS_OK) return st;
  return topk_first(dtype, batch, &a, lpc, static_cast<hipStream_t>(stream)) == CHS_OK ? CHS_OK : CHS_ERR_LAUNCH;
}

namespace chs {
namespace {

// Validates chs_index_topk_fp8's arguments, lays out the selection's workspace and fills *a.
chs_status topk_fp8_setup(int32_t batch, int32_t n_heads, int32_t head_dim, int32_t k, const void* q_idx,
                          const float* w, const void* k_idx, const float* k_scale, const int64_t* cu_cand,
                          int64_t max_cand, float* scores, int32_t* topk, void* workspace, size_t workspace_bytes,
                          Args* a) {
  if (batch < 1 || batch > 65535 || k < 1 || k > kMaxK || max_cand < 0 || max_cand >= (1LL << 31) ||
      n_heads < 1 || n_heads > 16 || head_dim < 16 || head_dim > 512 || head_dim % 16 != 0)
    return CHS_ERR_SHAPE;
  if (max_cand > kMaxCand) return CHS_ERR_UNSUPPORTED;
  if (!q_idx || !w || !k_idx || !k_scale || !cu_cand || !topk || !workspace) return CHS_ERR_NULL;
  Workspace ws;
  const size_t need = ws_layout(batch, max_cand, &ws, static_cast<char*>(workspace));
  if (workspace_bytes < need) return CHS_ERR_WORKSPACE;
  a->q = q_idx; a->w = w; a->keys = k_idx; a->cu = cu_cand; a->max_cand = max_cand;
  a->nh = n_heads; a->nvec = head_dim / 16; a->k = k; a->scores = scores; a->ws = ws; a->kscale = k_scale;
  a->gs = kGroup;
  a->pt = nullptr; a->cand_len = nullptr; a->pt_stride = 0; a->shift = 0; a->pool_pages = 0;
  return CHS_OK;
}

// The first kernel of the FP8 selection: scores and group statistics over E4M3 keys. Sets a->gs.
chs_status topk_fp8_first(int32_t batch, int32_t head_dim, Args* a, hipStream_t s) {
  if (a->max_cand == 0) return CHS_OK;
  int lpc = 2;
  while (lpc < a->nvec) lpc *= 2;                       // one 16-byte key vector per lane
  if (!launch_scores_mfma<uint8_t>(batch, head_dim, a, s)) {
    const int rw = kPasses * (64 / lpc);
    a->gs = std::min(rw, kGroup);
    const dim3 grid((unsigned)((a->max_cand + 4 * rw - 1) / (4 * rw)), (unsigned)batch);
    launch_scores<uint8_t>(grid, s, *a, lpc);
  }
  return launch_status();
}

}  // namespace
}  // namespace chs

extern "C" chs_status chs_index_topk_fp8(int32_t batch, int32_t n_heads, int32_t head_dim, int32_t k,
                                         const void* q_idx, const float* w, const void* k_idx,
                                         const float* k_scale, const int64_t* cu_cand, int64_t max_cand,
                                         float* scores, int32_t* topk, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  using namespace chs;
  Args a;
  const chs_status st = topk_fp8_setup(batch, n_heads, head_dim, k, q_idx, w, k_idx, k_scale, cu_cand, max_cand,
                                       scores, topk, workspace, workspace_bytes, &a);
  if (st != CHS_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (topk_fp8_first(batch, head_dim, &a, s) != CHS_OK) return CHS_ERR_LAUNCH;
  hipLaunchKernelGGL(collect_kernel, dim3((unsigned)batch), dim3(kCThreads), 0, s, a, topk);
  return launch_status();
}

namespace chs {
namespace {

// Validates chs_index_topk_paged's arguments, lays out the selection's workspace and fills *a.
chs_status topk_paged_setup(chs_dtype dtype, int32_t batch, int32_t n_heads, int32_t head_dim, int32_t k,
                            const void* q_idx, const float* w, const void* key_pool, int64_t pool_pages,
                            int32_t page_size, const int32_t* page_table, int32_t pt_stride, const int64_t* cand_len,
                            int64_t max_cand, float* scores, int32_t* topk, void* workspace, size_t workspace_bytes,
                            Args* a) {
  if (!dtype_ok(dtype)) return CHS_ERR_DTYPE;
  if (batch < 1 || batch > 65535 || k < 1 || k > kMaxK || max_cand < 0 || max_cand >= (1LL << 31) ||
      n_heads < 1 || n_heads > 16 || head_dim < 8 || head_dim > 512 || page_size < 64 || page_size > 65536 ||
      (page_size & (page_size - 1)) != 0 || pt_stride < 1 || pool_pages < 1)
    return CHS_ERR_SHAPE;
  if (max_cand > kMaxCand) return CHS_ERR_UNSUPPORTED;
  if (dtype != CHS_BF16 || (head_dim != 64 && head_dim != 128 && head_dim != 256)) return CHS_ERR_UNSUPPORTED;
  if (!q_idx || !w || !key_pool || !page_table || !cand_len || !topk || !workspace) return CHS_ERR_NULL;
  Workspace ws;
  const size_t need = ws_layout(batch, max_cand, &ws, static_cast<char*>(workspace));
  if (workspace_bytes < need) return CHS_ERR_WORKSPACE;
  a->q = q_idx; a->w = w; a->keys = key_pool; a->cu = nullptr; a->max_cand = max_cand;
  a->nh = n_heads; a->nvec = head_dim / 8; a->k = k; a->scores = scores; a->ws = ws; a->kscale = nullptr;
  a->gs = kGroup;
  a->pt = page_table; a->cand_len = cand_len; a->pt_stride = pt_stride; a->shift = __builtin_ctz((unsigned)page_size);
  a->pool_pages = pool_pages;
  return CHS_OK;
}

}  // namespace
}  // namespace chs

extern "C" chs_status chs_index_topk_paged(chs_dtype dtype, int32_t batch, int32_t n_heads, int32_t head_dim,
                                           int32_t k, const void* q_idx, const float* w, const void* key_pool,
                                           int64_t pool_pages, int32_t page_size, const int32_t* page_table,
                                           int32_t pt_stride, const int64_t* cand_len, int64_t max_cand,
                                           float* scores, int32_t* topk, void* workspace, size_t workspace_bytes,
                                           void* stream) {
  using namespace chs;
  Args a;
  const chs_status st = topk_paged_setup(dtype, batch, n_heads, head_dim, k, q_idx, w, key_pool, pool_pages,
                                         page_size, page_table, pt_stride, cand_len, max_cand, scores, topk,
                                         workspace, workspace_bytes, &a);
  if (st != CHS_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (max_cand > 0) {
    launch_scores_mfma<uint16_t>(batch, head_dim, &a, s);
    if (launch_status() != CHS_OK) return CHS_ERR_LAUNCH;
  }
  hipLaunchKernelGGL(collect_kernel, dim3((unsigned)batch), dim3(kCThreads), 0, s, a, topk);
  return launch_status();
}

extern "C" chs_status chs_index_topk_fp8_paged(int32_t batch, int32_t n_heads, int32_t head_dim, int32_t k,
                                               const void* q_idx, const float* w, const void* key_pool,
                                               const float* scale_pool, int64_t pool_pages, int32_t page_size,
                                               const int32_t* page_table, int32_t pt_stride, const int64_t* cand_len,
                                               int64_t max_cand, float* scores, int32_t* topk, void* workspace,
                                               size_t workspace_bytes, void* stream) {
  using namespace chs;
  if (batch < 1 || batch > 65535 || k < 1 || k > kMaxK || max_cand < 0 || max_cand >= (1LL << 31) ||
      n_heads < 1 || n_heads > 16 || head_dim < 16 || head_dim > 512 || page_size < 1 || page_size > 65536 ||
      (page_size & (page_size - 1)) != 0 || pt_stride < 1 || pool_pages < 1)
    return CHS_ERR_SHAPE;
  if (max_cand > kMaxCand) return CHS_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return CHS_ERR_UNSUPPORTED;
  if (page_size < 16 * mfma_tiles(head_dim, 1)) return CHS_ERR_SHAPE;   // a wave's keys in one page
  if (!q_idx || !w || !key_pool || !scale_pool || !page_table || !cand_len || !topk || !workspace)
    return CHS_ERR_NULL;
  Workspace ws;
  const size_t need = ws_layout(batch, max_cand, &ws, static_cast<char*>(workspace));
  if (workspace_bytes < need) return CHS_ERR_WORKSPACE;
  Args a;
  a.q = q_idx; a.w = w; a.keys = key_pool; a.cu = nullptr; a.max_cand = max_cand;
  a.nh = n_heads; a.nvec = head_dim / 16; a.k = k; a.scores = scores; a.ws = ws; a.kscale = scale_pool;
  a.gs = kGroup;
  a.pt = page_table; a.cand_len = cand_len; a.pt_stride = pt_stride; a.shift = __builtin_ctz((unsigned)page_size);
  a.pool_pages = pool_pages;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (max_cand > 0) {
    launch_scores_mfma<uint8_t>(batch, head_dim, &a, s);
    if (launch_status() != CHS_OK) return CHS_ERR_LAUNCH;
  }
  hipLaunchKernelGGL(collect_kernel, dim3((unsigned)batch), dim3(kCThreads), 0, s, a, topk);
  return launch_status();
}

// ---------------------------------------------------------------- the C4 decode step, fused
// chs_decode_step: the selection's second kernel and the attention's split kernel are one
// launch. Every attention split whose key slots reach past the window runs the exact top-k of
// its sequence itself (the same collect body, into LDS) and reads its entries from there, so
// the selection is done redundantly by those workgroups and no workgroup waits for another;
// window-only splits start attending at once. The split of the first selected slot (head tile
// 0) also stores the top-k row, from waves 4 .. 15, which then end; the attention body is the
// four-wave one of chs_decode_attn, reading the selection from LDS. Scores, top-k, out and lse are bit-identical
// to chs_index_topk followed by chs_decode_attn.
namespace chs {
namespace {

// TILES 16-head tiles per workgroup: 1 (four waves attend, the others store the top-k row and end)
// or 4 (all sixteen waves attend 64 heads, so a split's selection runs once, not once per head
// tile). The split plan and the arithmetic are the same either way, so the results are too.
// FP8: the entries and window rows are E4M3 codes with per-row scales (the FP8 split body).
// PAGED: the window and the entries come through the page tables of aa.pg (the paged split body).
template <int D, int TILES, bool FP8 = false, bool PAGED = false>
__global__ __launch_bounds__(kCThreads) void collect_attn_kernel(Args ia, attn::AttnArgs aa, int32_t* topk) {
  union alignas(16) StepShared {
    CollectShared c;
    attn::AttnShared<D, TILES> at;
  };
  __shared__ StepShared sh;
  __shared__ int32_t sel[kMaxK];
  const int b = blockIdx.y, split = blockIdx.x, z = blockIdx.z;
  FirstTile ft;                                         // before the slot map's reads are waited on
  collect_prefetch(ia, b, ft);
  const attn::SlotMap sm(aa, b);
  const int32_t s_begin = split * aa.kps, s_end = min(s_begin + aa.kps, sm.nslots());
  const bool selects = s_begin < s_end && s_end > sm.nswa;   // uniform over the workgroup
  if (selects) {
    collect_seq(ia, b, sel, sh.c, ft);
    __syncthreads();                                    // sel is complete; the LDS is the attention's
  }
  if constexpr (TILES == 4) {
    // All 16 waves attend the split for 64 heads; the top-k row is stored afterwards (a store before
    // the gathers would hold the wait counter they use).
    attn::NoHook none;
    attn::attn_split_sm<D, 4, attn::NoHook, FP8, PAGED>(aa, sm, b, split, 4 * z, threadIdx.x, sh.at, none, sel);
    if (selects && z == 0 && s_begin <= sm.nswa)
      for (int i = threadIdx.x; i < aa.k; i += kCThreads) topk[(int64_t)b * aa.k + i] = sel[i];
  } else {
    if (threadIdx.x >= attn::kAttnThreads) {            // whole waves
      // The attention's waves issue no global store before their gathers; the top-k row is
      // stored by these ones.
      if (selects && z == 0 && s_begin <= sm.nswa)
        for (int i = threadIdx.x - attn::kAttnThreads; i < aa.k; i += kCThreads - attn::kAttnThreads)
          topk[(int64_t)b * aa.k + i] = sel[i];
      return;
    }
    attn::NoHook none;
    attn::attn_split_sm<D, 1, attn::NoHook, FP8, PAGED>(aa, sm, b, split, z, threadIdx.x, sh.at, none, sel);
  }
}

// Workspace of chs_decode_step: the selection's, then the attention's partials.
size_t step_ws(int32_t batch, int32_t n_heads, int32_t d, int32_t window, int32_t k, int64_t max_comp,
               size_t* attn_off) {
  const size_t sel = align_up(ws_layout(batch, max_comp, nullptr, nullptr), 256);
  const attn::SplitPlan p = attn::plan_splits(CHS_BF16, batch, n_heads, d, window, k, max_comp);
  if (attn_off) *attn_off = sel;
  return sel + attn::ws_bytes(CHS_BF16, batch, n_heads, d, p, nullptr, nullptr, nullptr);
}

}  // namespace
}  // namespace chs

extern "C" size_t chs_decode_step_workspace_size(int32_t batch, int32_t n_heads, int32_t d, int32_t window,
                                                 int32_t k, int64_t max_comp) {
  if (batch < 1 || n_heads < 1 || d < 1 || window < 0 || k < 1 || max_comp < 0) return 0;
  return chs::step_ws(batch, n_heads, d, window, k, max_comp, nullptr);
}

namespace chs {
namespace {

// The row scales of an FP8 step (chs_decode_step_fp8); all NULL for bf16 storage.
struct Fp8Scales {
  const float* keys;   // [cu_comp[batch]] index-key row scales
  const float* swa;    // [batch, window] window row scales
  const float* comp;   // [cu_comp[batch]] entry row scales
  bool on() const { return keys != nullptr; }
};

chs_status decode_step_impl(int32_t batch, int32_t n_heads, int32_t d, int32_t window, int32_t k, float scale,
                            int32_t idx_heads, int32_t idx_dim, const void* q_idx, const float* w, const void* k_idx,
                            const void* q, const void* swa_kv, const int32_t* swa_len, const void* comp_kv,
                            const int64_t* cu_comp, int64_t max_comp, float* scores, int32_t* topk, float* out,
                            float* lse, void* workspace, size_t workspace_bytes, void* stream,
                            const Fp8Scales& f8 = Fp8Scales{nullptr, nullptr, nullptr}) {
  chs_status st = attn::check_args(CHS_BF16, batch, n_heads, d, window, k, scale, q, swa_kv, swa_len, comp_kv,
                                   cu_comp, topk, max_comp, out);
  if (st != CHS_OK) return st;
  if (k < 1) return CHS_ERR_SHAPE;
  if (!q_idx || !topk || !workspace) return CHS_ERR_NULL;
  if (f8.on() && ((window > 0 && !f8.swa) || !f8.comp)) return CHS_ERR_NULL;
  size_t attn_off = 0;
  const size_t need = step_ws(batch, n_heads, d, window, k, max_comp, &attn_off);
  if (workspace_bytes < need) return CHS_ERR_WORKSPACE;
  Args ia;
  int lpc = 2;
  st = f8.on() ? topk_fp8_setup(batch, idx_heads, idx_dim, k, q_idx, w, k_idx, f8.keys, cu_comp, max_comp, scores,
                                topk, workspace, attn_off, &ia)
               : topk_setup(CHS_BF16, batch, idx_heads, idx_dim, k, q_idx, w, k_idx, cu_comp, max_comp, scores, topk,
                            workspace, attn_off, &ia, &lpc);
  if (st != CHS_OK) return st;
  const attn::SplitPlan p = attn::plan_splits(CHS_BF16, batch, n_heads, d, window, k, max_comp);
  attn::AttnArgs a;
  a.q = q; a.swa = swa_kv; a.swa_len = swa_len; a.comp = comp_kv; a.cu_comp = cu_comp; a.topk = topk;
  a.swa_scale = f8.swa; a.comp_scale = f8.comp;
  a.pg = attn::Paging{nullptr, 0, nullptr, nullptr, 0, 0, 0};
  a.H = n_heads; a.D = d; a.W = window; a.k = k; a.max_comp = max_comp;
  a.scale_log2 = scale * kLog2e;
  a.n_splits = p.n_splits; a.kps = p.kps;
  a.head_tiles = (n_heads + 63) / 64;
  attn::ws_bytes(CHS_BF16, batch, n_heads, d, p, &a.part_o, &a.part_ml, static_cast<char*>(workspace) + attn_off);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((f8.on() ? topk_fp8_first(batch, idx_dim, &ia, s) : topk_first(CHS_BF16, batch, &ia, lpc, s)) != CHS_OK)
    return CHS_ERR_LAUNCH;
  if (p.wide && !f8.on()) {
    // Many sequences at d = 512: the attention's splits run in the 64-head kernel, which stages each
    // split's entries from the top-k list, so the selection runs once per sequence into that list
    // and the attention is chs_decode_attn's own launch (the results are the two calls', trivially).
    hipLaunchKernelGGL(collect_kernel, dim3((unsigned)batch), dim3(kCThreads), 0, s, ia, topk);
    if (launch_status() != CHS_OK) return CHS_ERR_LAUNCH;
    return chs_decode_attn(CHS_BF16, batch, n_heads, d, window, k, scale, q, swa_kv, swa_len, comp_kv, cu_comp, topk,
                           max_comp, out, lse, static_cast<char*>(workspace) + attn_off, workspace_bytes - attn_off,
                           stream);
  }
  // One workgroup per 16-head tile while the selecting workgroups fit the GPU at once (each selection
  // then runs on its own CU and the copies cost nothing); past that, one per 64 heads, so each split
  // selects once: at 64 sequences the step took 196 us against 227 us.
  const bool wide = (int64_t)p.n_splits * batch * ((n_heads + 15) / 16) > 256;
  const dim3 grid(p.n_splits, batch, wide ? (n_heads + 63) / 64 : (n_heads + 15) / 16);
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(kCThreads), 0, s, ia, a, topk); };
  if (f8.on()) {
    // FP8 storage: the split body of chs_decode_attn_fp8 (16-head tiles also at many sequences, where the
    // wide plan's longer splits take several chunks), so the results are that call's.
    switch (d) {
      case 64: wide ? go(collect_attn_kernel<64, 4, true>) : go(collect_attn_kernel<64, 1, true>); break;
      case 128: wide ? go(collect_attn_kernel<128, 4, true>) : go(collect_attn_kernel<128, 1, true>); break;
      case 256: wide ? go(collect_attn_kernel<256, 4, true>) : go(collect_attn_kernel<256, 1, true>); break;
      default: wide ? go(collect_attn_kernel<512, 4, true>) : go(collect_attn_kernel<512, 1, true>); break;
    }
  } else {
    switch (d) {
      case 64: wide ? go(collect_attn_kernel<64, 4>) : go(collect_attn_kernel<64, 1>); break;
      case 128: wide ? go(collect_attn_kernel<128, 4>) : go(collect_attn_kernel<128, 1>); break;
      case 256: wide ? go(collect_attn_kernel<256, 4>) : go(collect_attn_kernel<256, 1>); break;
      default: wide ? go(collect_attn_kernel<512, 4>) : go(collect_attn_kernel<512, 1>); break;
    }
  }
  if (launch_status() != CHS_OK) return CHS_ERR_LAUNCH;
  attn::launch_combine(a, batch, n_heads, d, out, lse, s);
  return launch_status();
}

// Scratch of chs_decode_step_noalloc: one array per GPU, part of the code object, so the call itself
// allocates nothing. Host code uses the device address hipGetSymbolAddress returns for the current
// device (the array's name is not a device address on the host).
constexpr size_t kNoAllocScratch = CHS_NOALLOC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) unsigned char scratch[kNoAllocScratch];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

// The scratch array's device address on the current device, looked up once per device.
chs_status scratch_for_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CHS_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CHS_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return CHS_OK;
}

}  // namespace
}  // namespace chs

extern "C" chs_status chs_decode_step(int32_t batch, int32_t n_heads, int32_t d, int32_t window, int32_t k,
                                      float scale, int32_t idx_heads, int32_t idx_dim, const void* q_idx,
                                      const float* w, const void* k_idx, const void* q, const void* swa_kv,
                                      const int32_t* swa_len, const void* comp_kv, const int64_t* cu_comp,
                                      int64_t max_comp, float* scores, int32_t* topk, float* out, float* lse,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  return chs::decode_step_impl(batch, n_heads, d, window, k, scale, idx_heads, idx_dim, q_idx, w, k_idx, q, swa_kv,
                               swa_len, comp_kv, cu_comp, max_comp, scores, topk, out, lse, workspace,
                               workspace_bytes, stream);
}

namespace chs {
namespace {

chs_status decode_step_paged_impl(int32_t batch, int32_t n_heads, int32_t d, int32_t window, int32_t k, float scale,
                                  int32_t idx_heads, int32_t idx_dim, const void* q_idx, const float* w,
                                  const void* key_pool, const void* q, const void* swa_pool, const int32_t* swa_page,
                                  int64_t swa_pages, const int32_t* swa_len, const void* comp_pool,
                                  int64_t pool_pages, int32_t page_size, const int32_t* page_table, int32_t pt_stride,
                                  const int64_t* comp_len, int64_t max_comp, float* scores, int32_t* topk, float* out,
                                  float* lse, void* workspace, size_t workspace_bytes, hipStream_t s) {
  // The shared checks null-test their cu argument; here the per-sequence counts take its place.
  chs_status st = attn::check_args(CHS_BF16, batch, n_heads, d, window, k, scale, q, swa_pool, swa_len, comp_pool,
                                   comp_len, topk, max_comp, out);
  if (st != CHS_OK) return st;
  if (k < 1) return CHS_ERR_SHAPE;
  if (!q_idx || !workspace || (window > 0 && !swa_page)) return CHS_ERR_NULL;
  if (window > 0 && swa_pages < 1) return CHS_ERR_SHAPE;
  size_t attn_off = 0;
  const size_t need = step_ws(batch, n_heads, d, window, k, max_comp, &attn_off);
  if (workspace_bytes < need) return CHS_ERR_WORKSPACE;
  Args ia;
  st = topk_paged_setup(CHS_BF16, batch, idx_heads, idx_dim, k, q_idx, w, key_pool, pool_pages, page_size,
                        page_table, pt_stride, comp_len, max_comp, scores, topk, workspace, attn_off, &ia);
  if (st != CHS_OK) return st;
  const attn::SplitPlan p = attn::plan_splits(CHS_BF16, batch, n_heads, d, window, k, max_comp);
  attn::AttnArgs a;
  a.q = q; a.swa = swa_pool; a.swa_len = swa_len; a.comp = comp_pool; a.cu_comp = nullptr; a.topk = topk;
  a.swa_scale = nullptr; a.comp_scale = nullptr;
  a.pg = attn::Paging{};
  a.pg.swa_page = window > 0 ? swa_page : nullptr;
  a.pg.swa_pages = swa_pages;
  a.pg.pt = page_table;
  a.pg.comp_len = comp_len;
  a.pg.pt_stride = pt_stride;
  a.pg.shift = __builtin_ctz((unsigned)page_size);
  a.pg.pool_pages = pool_pages;
  a.H = n_heads; a.D = d; a.W = window; a.k = k; a.max_comp = max_comp;
  a.scale_log2 = scale * kLog2e;
  a.n_splits = p.n_splits; a.kps = p.kps;
  a.head_tiles = (n_heads + 63) / 64;
  attn::ws_bytes(CHS_BF16, batch, n_heads, d, p, &a.part_o, &a.part_ml, static_cast<char*>(workspace) + attn_off);
  if (max_comp > 0) {
    launch_scores_mfma<uint16_t>(batch, idx_dim, &ia, s);
    if (launch_status() != CHS_OK) return CHS_ERR_LAUNCH;
  }
  if (p.wide) {
    // Many sequences at d = 512: as chs_decode_step, the selection once per sequence, then the paged
    // attention call's own 64-head launch.
    hipLaunchKernelGGL(collect_kernel, dim3((unsigned)batch), dim3(kCThreads), 0, s, ia, topk);
    if (launch_status() != CHS_OK) return CHS_ERR_LAUNCH;
    return chs_decode_attn_paged(CHS_BF16, batch, n_heads, d, window, k, scale, q, swa_pool, swa_page, swa_pages,
                                 swa_len, comp_pool, pool_pages, page_size, page_table, pt_stride, comp_len, topk,
                                 max_comp, out, lse, static_cast<char*>(workspace) + attn_off,
                                 workspace_bytes - attn_off, s);
  }
  const bool wide = (int64_t)p.n_splits * batch * ((n_heads + 15) / 16) > 256;
  const dim3 grid(p.n_splits, batch, wide ? (n_heads + 63) / 64 : (n_heads + 15) / 16);
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(kCThreads), 0, s, ia, a, topk); };
  switch (d) {
    case 64: wide ? go(collect_attn_kernel<64, 4, false, true>) : go(collect_attn_kernel<64, 1, false, true>); break;
    case 128: wide ? go(collect_attn_kernel<128, 4, false, true>) : go(collect_attn_kernel<128, 1, false, true>); break;
    case 256: wide ? go(collect_attn_kernel<256, 4, false, true>) : go(collect_attn_kernel<256, 1, false, true>); break;
    default: wide ? go(collect_attn_kernel<512, 4, false, true>) : go(collect_attn_kernel<512, 1, false, true>); break;
  }
  if (launch_status() != CHS_OK) return CHS_ERR_LAUNCH;
  attn::launch_combine(a, batch, n_heads, d, out, lse, s);
  return launch_status();
}

}  // namespace
}  // namespace chs

extern "C" chs_status chs_decode_step_paged(int32_t batch, int32_t n_heads, int32_t d, int32_t window, int32_t k,
                                            float scale, int32_t idx_heads, int32_t idx_dim, const void* q_idx,
                                            const float* w, const void* key_pool, const void* q,
                                            const void* swa_pool, const int32_t* swa_page, int64_t swa_pages,
                                            const int32_t* swa_len, const void* comp_pool, int64_t pool_pages,
                                            int32_t page_size, const int32_t* page_table, int32_t pt_stride,
                                            const int64_t* comp_len, int64_t max_comp, float* scores, int32_t* topk,
                                            float* out, float* lse, void* workspace, size_t workspace_bytes,
                                            void* stream) {
  return chs::decode_step_paged_impl(batch, n_heads, d, window, k, scale, idx_heads, idx_dim, q_idx, w, key_pool, q,
                                     swa_pool, swa_page, swa_pages, swa_len, comp_pool, pool_pages, page_size,
                                     page_table, pt_stride, comp_len, max_comp, scores, topk, out, lse, workspace,
                                     workspace_bytes, static_cast<hipStream_t>(stream));
}

extern "C" chs_status chs_decode_step_fp8(int32_t batch, int32_t n_heads, int32_t d, int32_t window, int32_t k,
                                          float scale, int32_t idx_heads, int32_t idx_dim, const void* q_idx,
                                          const float* w, const void* k_codes, const float* k_scale, const void* q,
                                          const void* swa_codes, const float* swa_scale, const int32_t* swa_len,
                                          const void* comp_codes, const float* comp_scale, const int64_t* cu_comp,
                                          int64_t max_comp, float* scores, int32_t* topk, float* out, float* lse,
                                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!k_scale) return CHS_ERR_NULL;
  return chs::decode_step_impl(batch, n_heads, d, window, k, scale, idx_heads, idx_dim, q_idx, w, k_codes, q,
                               swa_codes, swa_len, comp_codes, cu_comp, max_comp, scores, topk, out, lse, workspace,
                               workspace_bytes, stream, chs::Fp8Scales{k_scale, swa_scale, comp_scale});
}

extern "C" chs_status chs_decode_step_noalloc(int32_t batch, int32_t n_heads, int32_t d, int32_t window, int32_t k,
                                              float scale, int32_t idx_heads, int32_t idx_dim, const void* q_idx,
                                              const float* w, const void* k_idx, const void* q, const void* swa_kv,
                                              const int32_t* swa_len, const void* comp_kv, const int64_t* cu_comp,
                                              int64_t max_comp, float* scores, int32_t* topk, float* out, float* lse,
                                              void* stream) {
  using namespace chs;
  // The size check comes first, so an oversized call is refused before the device is touched.
  const size_t need = chs_decode_step_workspace_size(batch, n_heads, d, window, k, max_comp);
  if (need == 0) return CHS_ERR_SHAPE;
  if (need > kNoAllocScratch) return CHS_ERR_WORKSPACE;
  void* ws = nullptr;
  const chs_status st = scratch_for_current_device(&ws);
  if (st != CHS_OK) return st;
  return decode_step_impl(batch, n_heads, d, window, k, scale, idx_heads, idx_dim, q_idx, w, k_idx, q, swa_kv,
                          swa_len, comp_kv, cu_comp, max_comp, scores, topk, out, lse, ws, kNoAllocScratch, stream);
}
