// chs_append: one decode-time token per sequence into the window and the compression state.
//
// Source: "DeepSeek-V4 本地部署，SGLang 把活做絕了", ShadowRadix: besides the window pool, each
// layer keeps a compression state ring for the group still being formed, addressed inside the
// sequence's SWA page as page * ring size + position mod ring size; the ring is 8 slots for C4
// and 128 for C128 (doubled under speculative decoding). Same page, V4 到底改了啥: a 128-token
// window beside C4 (groups of 4) and C128 (groups of 128). "SGLang 如何为 DeepSeek V4 打造
// 「Day-0」推理加速", 创新 2: the compressor's stages fused into one pass.
//
// Per sequence b with n_b tokens before the call, the new token t = n_b:
//   1. its row x goes to window slot t mod W (the window is a ring; attention over it is a set);
//   2. its gate logits z go to state-ring slot ring_page[b] * R + t mod R;
//   3. if t completes a group (t + 1 divisible by m), the group g = t / m is pooled exactly as
//      chs_compress pools it and stored at compressed row comp_start[b] + g;
//   4. n_b advances by one; swa_len[b] = min(n_b, W) and comp_count[b] = floor(n_b / m).
// The group's token rows are read from the window ring: with m <= W a completed group still lies
// there in full, so the state ring holds gates only, and a token's row is written once.
//
// gfx950 design. The launch is latency-bound (a few KiB per sequence, plus one group's rows when
// it completes), so the aim is one round of loads and little serial work per group.
//   m in {1, 2, 4, 8}: one workgroup per sequence; one thread per 16-byte channel chunk pools the
//   whole group in registers (the same function and order as chs_compress, so the entries are
//   bit-identical to a prefill's). Thread 0 reads and advances the counters: no other workgroup
//   reads them.
//   other m (C128): a group of 128 rows x 512 channels is about 0.7 M lane operations and 65 K
//   exponentials, several microseconds for one CU, so a sequence's chunks are spread over
//   several workgroups. A thread pools 8 (16 for m > 512) rows of one chunk; the nb blocks of a
//   chunk (a power of two, at most 64) are adjacent lanes of one wave, merged by a butterfly of
//   cross-lane moves, with no LDS and no barrier. Since several workgroups read a sequence's
//   count, a second, one-thread-per-sequence kernel advances the counters after them.
// The new token's row and gate are read from the inputs, not from the rings being written in the
// same launch, so no thread depends on another's store.
//
// chs_append_fp8 keeps an FP8 cache (E4M3 codes plus one fp32 scale per row, the rule of fp8.h):
// the window gets the quantised row, which is lossy, so the state ring keeps the group's token rows
// beside its gates in the storage type (the pages' ring keeps both), and a completed group is pooled
// from the ring and quantised. The row scale is a maximum over the whole row, so one workgroup of 512
// threads serves a sequence: a chunk's rows are split over adjacent lanes (merged by the butterfly
// below; for m in {1, 2, 4, 8} one lane pools the whole group, bit-identical to chs_compress_fp8), and the row
// maxima of the new token and of the pooled entry meet in LDS.
#include <algorithm>

#include "fp8.h"
#include "pool.h"

namespace chs {
namespace {

struct AppendArgs {
  int32_t d, m, window, ring;
  int64_t ring_pages, comp_rows;
  const void* x_new;
  const void* z_new;
  const float* bias;
  int64_t* n_tokens;
  void* swa;
  int32_t* swa_len;
  void* gate_ring;
  const int32_t* ring_page;
  void* comp;
  const int64_t* comp_start;
  int64_t* comp_count;
  // Paged pools (NULL: contiguous). The window is page swa_page[b] of the window pool and the gate
  // ring sits at the same page (the ring nested in the SWA page); entry g goes to pool row
  // pt[b * pt_stride + g / 2^shift] * 2^shift + g mod 2^shift.
  const int32_t* swa_page;
  int64_t swa_pages;
  const int32_t* pt;
  int32_t pt_stride, shift;
};

constexpr int kSplitThreads = 256;
constexpr int kMaxStreams = 4;

// The compressor streams of one launch (grid dimension y or z): streams share dtype, batch and m
// and have their own rows, rings, pools and counters.
struct AppendSet {
  AppendArgs s[kMaxStreams];
};

// The counters after a token: n + 1, min(n + 1, W), floor((n + 1) / m).
__device__ __forceinline__ void advance_counters(const AppendArgs& a, int b, int64_t n) {
  a.n_tokens[b] = n + 1;
  if (a.swa_len) a.swa_len[b] = (int32_t)(n + 1 < a.window ? n + 1 : a.window);
  if (a.comp_count) a.comp_count[b] = (n + 1) / a.m;
}

__device__ __forceinline__ int64_t read_count(const AppendArgs& a, int b) {
  const int64_t n = a.n_tokens[b];
  return n < 0 ? 0 : n;                                 // a negative count is taken as empty
}

// Where sequence b's rings live, and whether its ring page is valid (else the gate write and
// the group are skipped).
template <typename ET>
struct SeqRings {
  ET* swa;
  ET* ring;
  bool page_ok;      // the gate ring's page is valid (else the gate write and the group are skipped)
  bool swa_ok;       // the window's page is valid (else the window write is skipped too)
  __device__ SeqRings(const AppendArgs& a, int b) {
    int64_t wpage = b;
    swa_ok = true;
    int64_t page;
    if (a.swa_page) {
      wpage = a.swa_page[b];
      swa_ok = wpage >= 0 && wpage < a.swa_pages;
      if (!swa_ok) wpage = 0;
      page = a.swa_page[b];
    } else {
      page = a.ring_page[b];
    }
    swa = static_cast<ET*>(a.swa) + wpage * a.window * a.d;
    page_ok = swa_ok && page >= 0 && page < a.ring_pages;
    ring = static_cast<ET*>(a.gate_ring) + (page_ok ? page : 0) * a.ring * a.d;
  }
};

// Pool row of entry g of sequence b, or -1 when it falls outside the caller's pool.
__device__ __forceinline__ int64_t entry_row(const AppendArgs& a, int b, int64_t g) {
  if (a.pt) {
    const int64_t idx = g >> a.shift;
    if (idx >= a.pt_stride) return -1;
    const int64_t p = a.pt[(int64_t)b * a.pt_stride + idx];
    const int64_t row = (p << a.shift) | (g & ((1 << a.shift) - 1));
    return p < 0 || row >= a.comp_rows ? -1 : row;
  }
  const int64_t row = a.comp_start[b] + g;
  return row < 0 || row >= a.comp_rows ? -1 : row;
}

// m in {1, 2, 4, 8}: one workgroup per (sequence, stream) (grid.x = batch, grid.y = stream).
template <typename ET, int M>
__global__ __launch_bounds__(256) void append_small_kernel(AppendSet set) {
  const AppendArgs& a = set.s[blockIdx.y];
  using V = Vec16<ET>;
  constexpr int N = V::N;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int d = a.d;
  const int cpr = d / N;
  const ET* xn = static_cast<const ET*>(a.x_new) + (int64_t)b * d;
  const ET* zn = static_cast<const ET*>(a.z_new) + (int64_t)b * d;
  // The new token's first chunk per thread is loaded before the count is known, so its round
  // trip overlaps the count's.
  u32x4 x0 = {0, 0, 0, 0}, z0 = {0, 0, 0, 0};
  if (tid < cpr) {
    x0 = *reinterpret_cast<const u32x4*>(xn + tid * N);
    z0 = *reinterpret_cast<const u32x4*>(zn + tid * N);
  }
  __shared__ int64_t s_t;
  if (tid == 0) {
    const int64_t n = read_count(a, b);
    s_t = n;
    advance_counters(a, b, n);
  }
  __syncthreads();
  const int64_t t = s_t;
  const SeqRings<ET> sr(a, b);
  const int64_t wslot = t % a.window, rslot = t % a.ring;
  if (tid < cpr && sr.swa_ok) {
    *reinterpret_cast<u32x4*>(sr.swa + wslot * d + tid * N) = x0;
    if (sr.page_ok) *reinterpret_cast<u32x4*>(sr.ring + rslot * d + tid * N) = z0;
  }
  for (int c = tid + 256; c < cpr && sr.swa_ok; c += 256) {
    V::copy(sr.swa + wslot * d + c * N, xn + c * N);
    if (sr.page_ok) V::copy(sr.ring + rslot * d + c * N, zn + c * N);
  }
  if ((t + 1) % M != 0 || !sr.page_ok) return;
  // The completed group: tokens t + 1 - M .. t. Row r < M - 1 sits at window slot
  // (t0 + r) mod W and ring slot (t0 + r) mod R; row M - 1 is the new token.
  const int64_t row = entry_row(a, b, t / M);
  if (row < 0) return;                                  // outside the caller's pool: skipped
  ET* out = static_cast<ET*>(a.comp) + row * d;
  const int64_t t0 = t + 1 - M;
  const int w0 = (int)(t0 % a.window), q0 = (int)(t0 % a.ring);
  const int W = a.window, R = a.ring;
  for (int c = tid; c < cpr; c += 256) {
    const int col = c * N;
    pool_group<ET, M, true>(
        M,
        [&](int r) -> const ET* {
          if (r == M - 1) return xn + col;
          const int s = w0 + r;
          return sr.swa + (int64_t)(s < W ? s : s - W) * d + col;
        },
        [&](int r) -> const ET* {
          if (r == M - 1) return zn + col;
          const int s = q0 + r;
          return sr.ring + (int64_t)(s < R ? s : s - R) * d + col;
        },
        [&](int r) { return a.bias + (int64_t)r * d + col; }, out + col);
  }
}

// Blocks per chunk for any m: rows per thread 8 (16 when m > 512), nb a power of two <= 64.
__host__ __device__ inline int split_rows_per_thread(int m) { return m > 512 ? 16 : 8; }
__host__ __device__ inline int split_blocks(int m) {
  const int rpt = split_rows_per_thread(m);
  int nb = 1;
  while (nb * rpt < m) nb *= 2;
  return nb;
}

// Merges a float across lanes lane ^ (1 << level) within groups of 2^(level+1) lanes (DPP for
// the first four levels, a cross-lane permute beyond). The mirrors pair disjoint halves, which
// is all a symmetric merge needs.
template <int LEVEL>
__device__ __forceinline__ float partner(float v) {
  if (LEVEL == 0) return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
  if (LEVEL == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
  if (LEVEL == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
  if (LEVEL == 3) return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));
  return __shfl_xor(v, 1 << LEVEL, 64);
}

template <int LEVEL, int N>
__device__ __forceinline__ void merge_level(PoolState<N>& st) {
  float omx[N], osum[N], oacc[N];
#pragma unroll
  for (int j = 0; j < N; ++j) {
    omx[j] = partner<LEVEL>(st.mx[j]);
    osum[j] = partner<LEVEL>(st.sum[j]);
    oacc[j] = partner<LEVEL>(st.acc[j]);
  }
  st.merge(omx, osum, oacc);
}

// Any m: grid (ceil(max cpr * nb / 256), batch, stream). Thread (chunk, block) with block =
// lane % nb. Workgroups past the stream's last chunk exit at once (streams differ in width).
template <typename ET>
__global__ __launch_bounds__(kSplitThreads) void append_split_kernel(AppendSet set) {
  const AppendArgs& a = set.s[blockIdx.z];
  using V = Vec16<ET>;
  constexpr int N = V::N;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int d = a.d;
  const int cpr = d / N;
  const int m = a.m;
  const int nb = split_blocks(m);
  const int rpt = split_rows_per_thread(m);
  if ((int64_t)blockIdx.x * kSplitThreads / nb >= cpr) return;   // uniform: the whole workgroup
  const int blk = tid & (nb - 1);
  const int c = (blockIdx.x * kSplitThreads + tid) / nb;
  const int64_t t = read_count(a, b);
  const ET* xn = static_cast<const ET*>(a.x_new) + (int64_t)b * d;
  const ET* zn = static_cast<const ET*>(a.z_new) + (int64_t)b * d;
  const SeqRings<ET> sr(a, b);
  if (blk == 0 && c < cpr && sr.swa_ok) {
    V::copy(sr.swa + (t % a.window) * d + c * N, xn + c * N);
    if (sr.page_ok) V::copy(sr.ring + (t % a.ring) * d + c * N, zn + c * N);
  }
  if ((t + 1) % m != 0 || !sr.page_ok) return;
  const int64_t row = entry_row(a, b, t / m);
  if (row < 0) return;                                  // outside the caller's pool: skipped
  const int64_t t0 = t + 1 - m;
  const int w0 = (int)(t0 % a.window), q0 = (int)(t0 % a.ring);
  const int W = a.window, R = a.ring;
  const int col = (c < cpr ? c : cpr - 1) * N;          // lanes past the last chunk read a valid one
  auto xrow = [&](int r) -> const ET* {
    if (r == m - 1) return xn + col;
    const int s = w0 + r;
    return sr.swa + (int64_t)(s < W ? s : s - W) * d + col;
  };
  auto zrow = [&](int r) -> const ET* {
    if (r == m - 1) return zn + col;
    const int s = q0 + r;
    return sr.ring + (int64_t)(s < R ? s : s - R) * d + col;
  };
  auto brow = [&](int r) { return a.bias + (int64_t)r * d + col; };
  PoolState<N> st;
  st.init();
  const int r0 = blk * rpt;
  if (r0 < m) {
    pool_block<ET, 8, true, true>(st, r0, min(8, m - r0), xrow, zrow, brow);
    if (rpt == 16 && r0 + 8 < m) pool_block<ET, 8, false, true>(st, r0 + 8, min(8, m - r0 - 8), xrow, zrow, brow);
  }
  // Butterfly over the nb lanes of the chunk (nb is uniform: every lane takes the same levels).
  if (nb > 1) merge_level<0>(st);
  if (nb > 2) merge_level<1>(st);
  if (nb > 4) merge_level<2>(st);
  if (nb > 8) merge_level<3>(st);
  if (nb > 16) merge_level<4>(st);
  if (nb > 32) merge_level<5>(st);
  if (blk == 0 && c < cpr) pool_store<ET>(st, static_cast<ET*>(a.comp) + row * d + col);
}

// ---------------------------------------------------------------- FP8 cache
struct AppendFp8Args {
  int32_t d, m, window, ring;
  int64_t ring_pages, comp_rows;
  const void* x_new;
  const void* z_new;
  const float* bias;
  int64_t* n_tokens;
  uint8_t* swa_codes;         // [batch][window][d]
  float* swa_scale;           // [batch][window]
  int32_t* swa_len;
  void* x_ring;               // [ring_pages * ring][d], storage type
  void* gate_ring;            // [ring_pages * ring][d], storage type
  const int32_t* ring_page;   // [batch]
  uint8_t* comp_codes;        // [comp_rows][d]
  float* comp_scale;          // [comp_rows]
  const int64_t* comp_start;  // [batch]
  int64_t* comp_count;
};

constexpr int kFp8Threads = 512;

// One workgroup per sequence. Thread (chunk c, block blk) = (tid / nb, tid % nb): nb lanes per
// chunk (a power of two, at most 64), so a chunk's lanes are adjacent in one wave. M in {1, 2, 4, 8}:
// lane blk = 0 pools the whole group with the prefill's instantiation (so the bits match); M = 0: any
// m, the rows split over the chunk's lanes.
template <typename ET, int M>
__global__ __launch_bounds__(kFp8Threads) void append_fp8_kernel(AppendFp8Args a) {
  using V = Vec16<ET>;
  constexpr int N = V::N;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int d = a.d, m = a.m, W = a.window, R = a.ring;
  const int cpr = d / N;                                // a power of two <= 64 (checked on the host)
  const int nb = min(kFp8Threads / cpr, 64);
  const int c = tid / nb, blk = tid & (nb - 1);
  const bool on = c < cpr;                              // whole groups of nb lanes
  const int col = (on ? c : cpr - 1) * N;
  const ET* xn = static_cast<const ET*>(a.x_new) + (int64_t)b * d;
  const ET* zn = static_cast<const ET*>(a.z_new) + (int64_t)b * d;
  u32x4 x0 = {0, 0, 0, 0}, z0 = {0, 0, 0, 0};
  if (on && blk == 0) {                                 // requested before the count is known
    x0 = *reinterpret_cast<const u32x4*>(xn + col);
    z0 = *reinterpret_cast<const u32x4*>(zn + col);
  }
  __shared__ int64_t s_t;
  __shared__ float s_am[2][64];
  if (tid == 0) {
    int64_t n = a.n_tokens[b];
    n = n < 0 ? 0 : n;
    s_t = n;
    a.n_tokens[b] = n + 1;
    if (a.swa_len) a.swa_len[b] = (int32_t)(n + 1 < W ? n + 1 : W);
    if (a.comp_count) a.comp_count[b] = (n + 1) / m;
  }
  __syncthreads();
  const int64_t t = s_t;
  const int64_t page = a.ring_page[b];
  const bool page_ok = page >= 0 && page < a.ring_pages;
  ET* xr = static_cast<ET*>(a.x_ring) + (page_ok ? page : 0) * R * d;
  ET* zr = static_cast<ET*>(a.gate_ring) + (page_ok ? page : 0) * R * d;
  if (on && blk == 0 && page_ok) {
    *reinterpret_cast<u32x4*>(xr + (t % R) * d + col) = x0;
    *reinterpret_cast<u32x4*>(zr + (t % R) * d + col) = z0;
  }
  int64_t row = -1;
  if (page_ok && (t + 1) % m == 0) {
    row = a.comp_start[b] + t / m;
    if (row < 0 || row >= a.comp_rows) row = -1;        // outside the caller's pool: skipped
  }
  float o[N];
#pragma unroll
  for (int j = 0; j < N; ++j) o[j] = 0.f;
  if (row >= 0 && on) {                                 // uniform over each chunk's lanes
    const int64_t t0 = t + 1 - m;
    const int q0 = (int)(t0 % R);
    auto xrow = [&](int r) -> const ET* {
      if (r == m - 1) return xn + col;
      const int sl = q0 + r;
      return xr + (int64_t)(sl < R ? sl : sl - R) * d + col;
    };
    auto zrow = [&](int r) -> const ET* {
      if (r == m - 1) return zn + col;
      const int sl = q0 + r;
      return zr + (int64_t)(sl < R ? sl : sl - R) * d + col;
    };
    auto brow = [&](int r) { return a.bias + (int64_t)r * d + col; };
    PoolState<N> st;
    st.init();
    if (M > 0) {
      if (blk == 0) pool_block<ET, (M > 0 ? M : 1), true>(st, 0, M, xrow, zrow, brow);
    } else {
      const int rpt = (m + nb - 1) / nb;
      const int r0 = blk * rpt, r1 = min(r0 + rpt, m);
      for (int rr = r0; rr < r1; rr += 4) {
        if (rr == r0) pool_block<ET, 4, true, true>(st, rr, min(4, r1 - rr), xrow, zrow, brow);
        else pool_block<ET, 4, false, true>(st, rr, min(4, r1 - rr), xrow, zrow, brow);
      }
      if (nb > 1) merge_level<0>(st);
      if (nb > 2) merge_level<1>(st);
      if (nb > 4) merge_level<2>(st);
      if (nb > 8) merge_level<3>(st);
      if (nb > 16) merge_level<4>(st);
      if (nb > 32) merge_level<5>(st);
    }
    pool_values<N>(st, o);
  }
  // The row maxima of the new token's row and of the pooled entry, one chunk per lane blk == 0.
  float xv[N];
  V::unpack(x0, xv);
  if (on && blk == 0) {
    float ax = 0.f, ao = 0.f;
#pragma unroll
    for (int j = 0; j < N; ++j) { ax = fmaxf(ax, fabsf(xv[j])); ao = fmaxf(ao, fabsf(o[j])); }
    s_am[0][c] = ax;
    s_am[1][c] = ao;
  }
  __syncthreads();
  if (!(on && blk == 0)) return;
  float ax = 0.f, ao = 0.f;
  for (int i = 0; i < cpr; ++i) { ax = fmaxf(ax, s_am[0][i]); ao = fmaxf(ao, s_am[1][i]); }
  uint32_t w[N / 4];
  const int64_t wrow = (int64_t)b * W + t % W;
  const float sx = e4m3_scale(ax);
  e4m3_pack<N>(xv, ax, w);
  e4m3_store<N>(a.swa_codes + wrow * d + col, w);
  if (c == 0) a.swa_scale[wrow] = sx;
  if (row >= 0) {
    const float so = e4m3_scale(ao);
    e4m3_pack<N>(o, ao, w);
    e4m3_store<N>(a.comp_codes + row * d + col, w);
    if (c == 0) a.comp_scale[row] = so;
  }
}

__global__ __launch_bounds__(256) void append_advance_kernel(AppendSet set, int32_t batch) {
  const AppendArgs& a = set.s[blockIdx.y];
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b < batch) advance_counters(a, b, read_count(a, b));
}

// One launch for all the streams (plus the counter kernel for the split path).
template <typename ET>
chs_status launch_append(const AppendSet& set, int n, int32_t batch, hipStream_t s) {
  const int m = set.s[0].m;
  dim3 grid((unsigned)batch, (unsigned)n);
  switch (m) {
    case 1: hipLaunchKernelGGL((append_small_kernel<ET, 1>), grid, dim3(256), 0, s, set); break;
    case 2: hipLaunchKernelGGL((append_small_kernel<ET, 2>), grid, dim3(256), 0, s, set); break;
    case 4: hipLaunchKernelGGL((append_small_kernel<ET, 4>), grid, dim3(256), 0, s, set); break;
    case 8: hipLaunchKernelGGL((append_small_kernel<ET, 8>), grid, dim3(256), 0, s, set); break;
    default: {
      int64_t threads = 0;
      for (int i = 0; i < n; ++i) threads = std::max<int64_t>(threads, (int64_t)(set.s[i].d / Vec16<ET>::N) * split_blocks(m));
      dim3 g2((unsigned)((threads + kSplitThreads - 1) / kSplitThreads), (unsigned)batch, (unsigned)n);
      hipLaunchKernelGGL(append_split_kernel<ET>, g2, dim3(kSplitThreads), 0, s, set);
      if (hipGetLastError() != hipSuccess) return CHS_ERR_LAUNCH;
      hipLaunchKernelGGL(append_advance_kernel, dim3((unsigned)((batch + 255) / 256), (unsigned)n), dim3(256), 0, s,
                         set, batch);
      break;
    }
  }
  return launch_status();
}

}  // namespace
}  // namespace chs

namespace chs {
namespace {

chs_status check_append(chs_dtype dtype, int32_t batch, int32_t d, int32_t m, int32_t window, int32_t ring_size,
                        const void* x_new, const void* z_new, const float* bias, const int64_t* n_tokens,
                        const void* swa_kv, const void* gate_ring, const void* comp_kv, int64_t comp_rows) {
  if (!dtype_ok(dtype)) return CHS_ERR_DTYPE;
  if (batch < 1 || batch > 65535 || d < 1 || d > 4096 || m < 1 || m > 1024 || window < m ||
      window > (1 << 20) || ring_size < m || ring_size > (1 << 20) || comp_rows < 0)
    return CHS_ERR_SHAPE;
  if ((d * elem_size(dtype)) % 16 != 0) return CHS_ERR_SHAPE;
  if (!x_new || !z_new || !bias || !n_tokens || !swa_kv || !gate_ring || !comp_kv) return CHS_ERR_NULL;
  return CHS_OK;
}

}  // namespace
}  // namespace chs

extern "C" chs_status chs_append(chs_dtype dtype, int32_t batch, int32_t d, int32_t m, int32_t window,
                                 int32_t ring_size, const void* x_new, const void* z_new, const float* bias,
                                 int64_t* n_tokens, void* swa_kv, int32_t* swa_len, void* gate_ring,
                                 const int32_t* ring_page, int64_t ring_pages, void* comp_kv,
                                 const int64_t* comp_start, int64_t comp_rows, int64_t* comp_count,
                                 void* stream) {
  using namespace chs;
  const chs_status st = check_append(dtype, batch, d, m, window, ring_size, x_new, z_new, bias, n_tokens, swa_kv,
                                     gate_ring, comp_kv, comp_rows);
  if (st != CHS_OK) return st;
  if (ring_pages < 1) return CHS_ERR_SHAPE;
  if (!ring_page || !comp_start) return CHS_ERR_NULL;
  AppendSet set{};
  set.s[0] = AppendArgs{d, m, window, ring_size, ring_pages, comp_rows, x_new, z_new, bias, n_tokens, swa_kv, swa_len,
                        gate_ring, ring_page, comp_kv, comp_start, comp_count, nullptr, 0, nullptr, 0, 0};
  hipStream_t s = static_cast<hipStream_t>(stream);
  return dtype == CHS_BF16 ? launch_append<uint16_t>(set, 1, batch, s) : launch_append<float>(set, 1, batch, s);
}

extern "C" chs_status chs_append_paged(chs_dtype dtype, int32_t batch, int32_t d, int32_t m, int32_t window,
                                       int32_t ring_size, const void* x_new, const void* z_new, const float* bias,
                                       int64_t* n_tokens, void* swa_pool, const int32_t* swa_page, int64_t swa_pages,
                                       int32_t* swa_len, void* gate_ring, void* comp_pool, int64_t pool_pages,
                                       int32_t page_size, const int32_t* page_table, int32_t pt_stride,
                                       int64_t* comp_count, void* stream) {
  using namespace chs;
  if (pool_pages < 0 || pool_pages > ((int64_t)1 << 40) / (page_size > 0 ? page_size : 1)) return CHS_ERR_SHAPE;
  const chs_status st = check_append(dtype, batch, d, m, window, ring_size, x_new, z_new, bias, n_tokens, swa_pool,
                                     gate_ring, comp_pool, pool_pages * (int64_t)page_size);
  if (st != CHS_OK) return st;
  if (swa_pages < 1 || page_size < 1 || page_size > 65536 || (page_size & (page_size - 1)) != 0 || pt_stride < 1)
    return CHS_ERR_SHAPE;
  if (!swa_page || !page_table) return CHS_ERR_NULL;
  AppendSet set{};
  set.s[0] = AppendArgs{d, m, window, ring_size, swa_pages, pool_pages * (int64_t)page_size, x_new, z_new, bias,
                        n_tokens, swa_pool, swa_len, gate_ring, nullptr, comp_pool, nullptr, comp_count, swa_page,
                        swa_pages, page_table, pt_stride, __builtin_ctz((unsigned)page_size)};
  hipStream_t s = static_cast<hipStream_t>(stream);
  return dtype == CHS_BF16 ? launch_append<uint16_t>(set, 1, batch, s) : launch_append<float>(set, 1, batch, s);
}

extern "C" chs_status chs_append_multi(chs_dtype dtype, int32_t batch, int32_t m, int32_t n_streams,
                                       const chs_append_stream* streams, void* stream) {
  using namespace chs;
  if (n_streams < 1 || n_streams > kMaxStreams) return CHS_ERR_SHAPE;
  if (!streams) return CHS_ERR_NULL;
  AppendSet set{};
  for (int i = 0; i < n_streams; ++i) {
    const chs_append_stream& t = streams[i];
    const bool paged = t.page_table != nullptr;
    const int64_t page_size = paged ? t.page_size : 1;
    if (paged && (t.page_size < 1 || t.page_size > 65536 || (t.page_size & (t.page_size - 1)) != 0 ||
                  t.pt_stride < 1 || t.pool_pages < 0 || t.pool_pages > ((int64_t)1 << 40) / page_size))
      return CHS_ERR_SHAPE;
    const int64_t rows = paged ? t.pool_pages * page_size : t.comp_rows;
    const chs_status st = check_append(dtype, batch, t.d, m, t.window, t.ring_size, t.x_new, t.z_new, t.bias,
                                       t.n_tokens, t.swa_kv, t.gate_ring, t.comp_kv, rows);
    if (st != CHS_OK) return st;
    if (paged) {
      if (t.swa_pages < 1) return CHS_ERR_SHAPE;
      if (!t.swa_page) return CHS_ERR_NULL;
      set.s[i] = AppendArgs{t.d, m, t.window, t.ring_size, t.swa_pages, rows, t.x_new, t.z_new, t.bias, t.n_tokens,
                            t.swa_kv, t.swa_len, t.gate_ring, nullptr, t.comp_kv, nullptr, t.comp_count, t.swa_page,
                            t.swa_pages, t.page_table, t.pt_stride, __builtin_ctz((unsigned)t.page_size)};
    } else {
      if (t.ring_pages < 1) return CHS_ERR_SHAPE;
      if (!t.ring_page || !t.comp_start) return CHS_ERR_NULL;
      set.s[i] = AppendArgs{t.d, m, t.window, t.ring_size, t.ring_pages, rows, t.x_new, t.z_new, t.bias, t.n_tokens,
                            t.swa_kv, t.swa_len, t.gate_ring, t.ring_page, t.comp_kv, t.comp_start, t.comp_count,
                            nullptr, 0, nullptr, 0, 0};
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  return dtype == CHS_BF16 ? launch_append<uint16_t>(set, n_streams, batch, s)
                           : launch_append<float>(set, n_streams, batch, s);
}

extern "C" chs_status chs_append_fp8(chs_dtype dtype, int32_t batch, int32_t d, int32_t m, int32_t window,
                                     int32_t ring_size, const void* x_new, const void* z_new, const float* bias,
                                     int64_t* n_tokens, uint8_t* swa_codes, float* swa_scale, int32_t* swa_len,
                                     void* x_ring, void* gate_ring, const int32_t* ring_page, int64_t ring_pages,
                                     uint8_t* comp_codes, float* comp_scale, const int64_t* comp_start,
                                     int64_t comp_rows, int64_t* comp_count, void* stream) {
  using namespace chs;
  const chs_status st = check_append(dtype, batch, d, m, window, ring_size, x_new, z_new, bias, n_tokens, swa_codes,
                                     gate_ring, comp_codes, comp_rows);
  if (st != CHS_OK) return st;
  if (ring_pages < 1) return CHS_ERR_SHAPE;
  const int cpr = (int)(d * elem_size(dtype) / 16);
  if (cpr > 64 || (cpr & (cpr - 1)) != 0) return CHS_ERR_UNSUPPORTED;
  if (!swa_scale || !x_ring || !ring_page || !comp_scale || !comp_start) return CHS_ERR_NULL;
  AppendFp8Args a{d, m, window, ring_size, ring_pages, comp_rows, x_new, z_new, bias, n_tokens, swa_codes, swa_scale,
                  swa_len, x_ring, gate_ring, ring_page, comp_codes, comp_scale, comp_start, comp_count};
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, dim3((unsigned)batch), dim3(kFp8Threads), 0, s, a); };
  const bool bf = dtype == CHS_BF16;
  switch (m) {
    case 1: bf ? go(append_fp8_kernel<uint16_t, 1>) : go(append_fp8_kernel<float, 1>); break;
    case 2: bf ? go(append_fp8_kernel<uint16_t, 2>) : go(append_fp8_kernel<float, 2>); break;
    case 4: bf ? go(append_fp8_kernel<uint16_t, 4>) : go(append_fp8_kernel<float, 4>); break;
    case 8: bf ? go(append_fp8_kernel<uint16_t, 8>) : go(append_fp8_kernel<float, 8>); break;
    default: bf ? go(append_fp8_kernel<uint16_t, 0>) : go(append_fp8_kernel<float, 0>); break;
  }
  return launch_status();
}
