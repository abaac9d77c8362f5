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
// gfx950 design. One workgroup per sequence, so the counters are read and advanced by one
// thread with no cross-workgroup ordering. The work is a few KiB per sequence, so the launch
// is latency-bound: the aim is one round of loads per group.
//   m <= 8: one thread per 16-byte channel chunk pools the whole group in registers (the same
//   function and order as chs_compress, so the entries are bit-identical to a prefill's).
//   m > 8: a thread pools one block of 8 rows of one chunk; the blocks of a chunk (a power-of-two
//   count, at most 128) are adjacent threads of one pass, and their states are merged through LDS
//   in block order. A pass covers 512 / blocks chunks.
// The new token's row and gate are read from the inputs, not from the rings being written in the
// same launch, so no thread depends on another's store.
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
};

constexpr int kSplitThreads = 512;

template <typename ET, int M, int THREADS>
__global__ __launch_bounds__(THREADS) void append_kernel(AppendArgs a) {
  using V = Vec16<ET>;
  constexpr int N = V::N;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int d = a.d;
  const int cpr = d / N;
  __shared__ int64_t s_t;
  if (tid == 0) {
    int64_t n = a.n_tokens[b];
    if (n < 0) n = 0;                                   // a negative count is taken as empty
    s_t = n;
    a.n_tokens[b] = n + 1;
    if (a.swa_len) a.swa_len[b] = (int32_t)(n + 1 < a.window ? n + 1 : a.window);
    if (a.comp_count) a.comp_count[b] = (n + 1) / a.m;
  }
  __syncthreads();
  const int64_t t = s_t;
  const ET* xn = static_cast<const ET*>(a.x_new) + (int64_t)b * d;
  const ET* zn = static_cast<const ET*>(a.z_new) + (int64_t)b * d;
  ET* swa_b = static_cast<ET*>(a.swa) + (int64_t)b * a.window * d;
  const int64_t page = a.ring_page[b];
  const bool page_ok = page >= 0 && page < a.ring_pages;  // an out-of-range page is skipped
  ET* ring_b = static_cast<ET*>(a.gate_ring) + (page_ok ? page : 0) * a.ring * d;

  // 1 + 2: the new token's row and gate.
  const int64_t wslot = t % a.window, rslot = t % a.ring;
  for (int c = tid; c < cpr; c += THREADS) {
    V::copy(swa_b + wslot * d + c * N, xn + c * N);
    if (page_ok) V::copy(ring_b + rslot * d + c * N, zn + c * N);
  }
  const int m = a.m;
  if ((t + 1) % m != 0 || !page_ok) return;

  // 3: the completed group, tokens t0 .. t. Row r < m - 1 sits at window slot (t0 + r) mod W
  // and ring slot (t0 + r) mod R; row m - 1 is the new token.
  const int64_t t0 = t + 1 - m;
  const int64_t row = a.comp_start[b] + t / m;
  if (row < 0 || row >= a.comp_rows) return;            // outside the caller's pool: skipped
  ET* out = static_cast<ET*>(a.comp) + row * d;
  const int w0 = (int)(t0 % a.window), q0 = (int)(t0 % a.ring);
  const int W = a.window, R = a.ring;
  if (M > 0) {
    for (int c = tid; c < cpr; c += THREADS) {
      const int col = c * N;
      pool_group<ET, M>(
          m,
          [&](int r) -> const ET* {
            if (r == M - 1) return xn + col;
            const int s = w0 + r;
            return swa_b + (int64_t)(s < W ? s : s - W) * d + col;
          },
          [&](int r) -> const ET* {
            if (r == M - 1) return zn + col;
            const int s = q0 + r;
            return ring_b + (int64_t)(s < R ? s : s - R) * d + col;
          },
          [&](int r) { return a.bias + (int64_t)r * d + col; }, out + col);
    }
  } else {
    __shared__ float part[3][N][THREADS];
    int nb = 1;
    while (nb * 8 < m) nb *= 2;                          // blocks per chunk (power of two)
    const int chunks_per_pass = THREADS / nb;
    const int blk = tid & (nb - 1);
    for (int c0 = 0; c0 < cpr; c0 += chunks_per_pass) {
      const int c = c0 + tid / nb;
      const int r0 = blk * 8;
      PoolState<N> st;
      st.init();
      if (c < cpr && r0 < m) {
        const int col = c * N;
        pool_block<ET, 8, true>(
            st, r0, min(8, m - r0),
            [&](int r) -> const ET* {
              if (r == m - 1) return xn + col;
              const int s = w0 + r;
              return swa_b + (int64_t)(s < W ? s : s - W) * d + col;
            },
            [&](int r) -> const ET* {
              if (r == m - 1) return zn + col;
              const int s = q0 + r;
              return ring_b + (int64_t)(s < R ? s : s - R) * d + col;
            },
            [&](int r) { return a.bias + (int64_t)r * d + col; });
      }
#pragma unroll
      for (int j = 0; j < N; ++j) {
        part[0][j][tid] = st.mx[j];
        part[1][j][tid] = st.sum[j];
        part[2][j][tid] = st.acc[j];
      }
      __syncthreads();
      if (blk == 0 && c < cpr) {
        const int nblk = (m + 7) / 8;
        for (int k = 1; k < nblk; ++k) {
          float omx[N], osum[N], oacc[N];
#pragma unroll
          for (int j = 0; j < N; ++j) {
            omx[j] = part[0][j][tid + k];
            osum[j] = part[1][j][tid + k];
            oacc[j] = part[2][j][tid + k];
          }
          st.merge(omx, osum, oacc);
        }
        pool_store<ET>(st, out + c * N);
      }
      __syncthreads();
    }
  }
}

template <typename ET>
chs_status launch_append(const AppendArgs& a, int32_t batch, hipStream_t s) {
  dim3 grid((unsigned)batch);
  switch (a.m) {
    case 1: hipLaunchKernelGGL((append_kernel<ET, 1, 256>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((append_kernel<ET, 2, 256>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((append_kernel<ET, 4, 256>), grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL((append_kernel<ET, 8, 256>), grid, dim3(256), 0, s, a); break;
    default:   // any other m (3, 5, 6, 7 are one block of rows), through the block-split path
      hipLaunchKernelGGL((append_kernel<ET, 0, kSplitThreads>), grid, dim3(kSplitThreads), 0, s, a);
      break;
  }
  return launch_status();
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
  if (!dtype_ok(dtype)) return CHS_ERR_DTYPE;
  if (batch < 1 || batch > (1 << 20) || d < 1 || d > 4096 || m < 1 || m > 1024 || window < m ||
      window > (1 << 20) || ring_size < m || ring_size > (1 << 20) || ring_pages < 1 || comp_rows < 0)
    return CHS_ERR_SHAPE;
  if ((d * elem_size(dtype)) % 16 != 0) return CHS_ERR_SHAPE;
  if (!x_new || !z_new || !bias || !n_tokens || !swa_kv || !gate_ring || !ring_page || !comp_kv || !comp_start)
    return CHS_ERR_NULL;
  AppendArgs a{d, m, window, ring_size, ring_pages, comp_rows, x_new, z_new, bias, n_tokens, swa_kv, swa_len,
               gate_ring, ring_page, comp_kv, comp_start, comp_count};
  hipStream_t s = static_cast<hipStream_t>(stream);
  return dtype == CHS_BF16 ? launch_append<uint16_t>(a, batch, s) : launch_append<float>(a, batch, s);
}
