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
#include <type_traits>

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

// ---------------------------------------------------------------- dense bf16, d = 512
// Every compressed entry attended by many heads is a skinny GEMM pair per sequence (64 heads x
// 512 channels against thousands of keys). One workgroup of 12 waves (three per SIMD) runs one
// split for 64 heads as a two-stage pipeline over chunks of 32 keys:
//   - waves 0-3 (producers) compute S^T = K Q^T for their 16 heads over the whole chunk
//     (v_mfma_f32_16x16x32_bf16, K from LDS as the A operand, Q^T held in registers), then the
//     online softmax: each producer holds all of its heads' keys, so no other wave takes part; P
//     (rounded to bf16) and the per-head rescale factor go to LDS, and the producers request the
//     rows of the chunk two ahead, one every two MFMA steps (in the selected form the consumers do);
//   - waves 4-11 (consumers) hold O for all 64 heads, 64 channels each, and in the next phase
//     rescale it and add P V for the chunk (v_mfma_f32_32x32x16_bf16, V = K read back with the
//     transposing LDS load), every fragment requested before the first MFMA.
// In phase t the producers work on chunk t while the consumers work on chunk t - 1, so each SIMD
// has a wave in Q K^T or the softmax beside two in P V, and the softmax's VALU work overlaps the
// consumers' MFMAs. One barrier per phase, against three per 64-key chunk when every wave did both
// stages (C128 at 4 x 8,320 keys 26.9 -> 24.9 us, at 64 sequences 48 -> 43-45 us). The reference
// maximum of a head moves only when a chunk exceeds it by more than kD512Slack (base 2), so most
// phases leave every rescale factor exactly 1 and the consumers skip the rescale (P stays below
// 2^8, well inside bf16 and the fp32 sums). Key rows go from HBM straight into LDS
// (global_load_lds_dwordx4, one 1 KB row per instruction, the row pitch padded by 32 bytes) into
// four buffers: a chunk is read in two phases and requested two phases ahead.
// Per 32-key chunk (32 KB of keys) the LDS sees 32 KB of row writes, 128 KB of K reads (each
// producer reads the chunk for its 16 heads), 32 KB of transposing V reads and 32 KB of P reads;
// per SIMD the producer and the two consumers issue 512 cycles of MFMA each way. The partial
// results use the layout of the 16-head-tile kernels, so the same merge applies. Measured and not
// kept: 8 waves (four consumers of 128 channels; 0.4 us slower at 4 x 8,320 keys), K fragments
// requested 7 or 15 steps ahead instead of 3, row pitches padded by 16, 48 or 64 bytes.
constexpr int kD512Threads = 768;             // 12 waves
constexpr int kD512Chunk = 32;                // keys per phase
constexpr int kD512Bufs = 4;                  // key row buffers
constexpr int kD512Pitch = 512 + 16;          // bf16 elements per LDS key row
constexpr int kD512PPitch = kD512Chunk + 8;   // bf16 elements per LDS row of P
constexpr float kD512Slack = 8.f;             // base-2 logits a chunk may exceed the reference maximum by

typedef float f32x16 __attribute__((ext_vector_type(16)));

// One row by DMA into LDS: lane l's 16 bytes at src (its own address) land at dst + 16 l, dst the
// same in every lane (it goes into M0). Written as an instruction of its own rather than through the
// compiler builtin: the builtin lets the compiler track the LDS write, and it then waits for every
// DMA in flight before LDS reads it cannot tell apart from the destination, which would empty the
// prefetch each phase. The instruction writes no register; the kernel waits for it (vmcnt) before
// the rows are read, and never reads or writes the destination rows meanwhile.
__device__ __forceinline__ void lds_row_dma(const uint16_t* src, uint16_t* dst) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)dst);
  __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds));
}

// Waits until at most N of this wave's vector memory operations are outstanding (they complete in
// order, so the older row DMAs have landed).
template <int N>
__device__ __forceinline__ void wait_vm() { __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// v combined with lane l ^ 16's (lane l ^ 32's) value by op: gfx950's row swaps (v_permlane16_swap,
// v_permlane32_swap) in place of an LDS-pipe lane permute. With both operands v, the swap leaves each
// lane its own value in one result and its partner's in the other (in an order that depends on the
// row), so a commutative op gives the same bits as the permute.
template <typename Op>
__device__ __forceinline__ float xor16(float v, Op op) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <typename Op>
__device__ __forceinline__ float xor32(float v, Op op) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// A workgroup barrier for LDS data only: this wave's LDS operations are complete, then every wave
// meets. __syncthreads() would also wait for the row DMAs still in flight (they write LDS), which
// must stay in flight across phases.
__device__ __forceinline__ void lds_barrier() { __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// A page-table entry at an index that is the same in every lane, read through the scalar unit: the
// wait for it is on the scalar/LDS counter, not behind the row DMAs in flight.
__device__ __forceinline__ int64_t page_entry(const int32_t* pt, int64_t idx) {
  const __attribute__((address_space(4))) int32_t* p = (const __attribute__((address_space(4))) int32_t*)pt;
  return p[idx];
}

// PAGED: entries through the page table (an entry whose page is outside the pool is skipped) and
// the window through the sequence's window page, as in the other split kernels.
// TOPK: the split's slots past the window are the selected entries a.topk lists (C4 at many
// sequences); the split's slice of the list is staged in LDS first, and an entry outside [0, G) is
// skipped.
template <bool PAGED, bool TOPK>
__global__ __launch_bounds__(kD512Threads) void attn_dense512_kernel(AttnArgs a) {
  constexpr int D = 512, KC = kD512Chunk, NB = kD512Bufs, KP = kD512Pitch, PP = kD512PPitch;
  __shared__ __attribute__((aligned(16))) uint16_t kt[NB][KC * KP];
  __shared__ __attribute__((aligned(16))) uint16_t pb[2][64 * PP];
  __shared__ __attribute__((aligned(16))) float alph[2][64];   // [chunk & 1][head]: rescale factor
  __shared__ uint8_t rowok[NB][KC];                            // PAGED, TOPK: which rows of each buffer hold a key
  __shared__ int32_t selrow[TOPK ? kWideMaxSelected : 1];      // TOPK: the split's selected entries

  const int b = blockIdx.y, split = blockIdx.x, zg = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wl = wave & 3;                        // producer: head tile
  const int l32 = lane & 31, lh = lane >> 5;      // 32 x 32 operand layout (P V)
  const int c16 = lane & 15, g4 = lane >> 4;      // 16 x 16 operand layout (Q K^T)
  const int hq = 16 * wl + c16;                   // producer: this lane's head
  const SlotMap sm(a, b);
  const int32_t s_begin = split * a.kps;
  const int32_t s_end = min(s_begin + a.kps, sm.nslots());
  const int nchunks = s_end > s_begin ? (s_end - s_begin + KC - 1) / KC : 0;
  const uint16_t* swa = static_cast<const uint16_t*>(a.swa);
  const uint16_t* comp = static_cast<const uint16_t*>(a.comp);

  // Row r of chunk c into buffer c % NB, by DMA (lane l brings bytes 16 l .. + 15): requesting wave
  // iw (below) takes rows kRowsPerWave iw .. + kRowsPerWave - 1. Every value that picks a row is the
  // same in all lanes. Slots that hold no key read the query buffer instead (the row is then masked).
  const uint64_t swa_a = (uint64_t)(uintptr_t)(swa + sm.swa_row0 * D);
  const uint64_t comp_a = (uint64_t)(uintptr_t)(comp + (sm.comp0 - sm.nswa) * D);
  const uint64_t safe_a = (uint64_t)(uintptr_t)a.q;
  // TOPK: selected positions j0 .. j0 + nsel - 1 belong to this split.
  const int32_t j0 = max(s_begin - sm.nswa, 0);
  const int32_t nsel = TOPK ? max(s_end - sm.nswa - j0, 0) : 0;
  if (TOPK) {
    const int32_t* tk = a.topk + (int64_t)b * a.k;
    for (int i = threadIdx.x; i < nsel; i += kD512Threads) selrow[i] = tk[j0 + i];
    __syncthreads();
  }
  // Who requests the rows: the producers, 8 rows each, spread over their Q K^T steps; in the
  // selected form the consumers, 4 each, between their P V MFMAs. A selected row costs its wave an
  // LDS round trip for the entry and the request (at 64 sequences of 50,000 entries a producer that
  // requested 8 per phase took 2.1 us instead of 0.8, whether the entries were scattered or
  // consecutive); spread over the eight consumers, with one LDS read for a wave's entries, the
  // kernel went from 24.1 to 21.6 us.
  constexpr bool kConsumerRows = TOPK;
  constexpr int kRowsPerWave = kConsumerRows ? 4 : 8;
  const bool issuer = kConsumerRows ? wave >= 4 : wave < 4;
  const int iw = kConsumerRows ? wave - 4 : wave;
  // TOPK: the selected entries of this wave's rows of chunk c, lane i holding row i's, from one LDS
  // read (each row then takes its own with a lane read, instead of an LDS round trip per row).
  auto sel_entries = [&](int c) -> int32_t {
    if (!TOPK) return 0;
    const int32_t s = s_begin + c * KC + kRowsPerWave * iw + (lane < kRowsPerWave ? lane : 0);
    return selrow[min(max(s - sm.nswa - j0, 0), max(nsel - 1, 0))];
  };
  auto row_src = [&](int c, int i, int32_t sel) -> uint64_t {
    const int bi = c & (NB - 1);
    const int r = kRowsPerWave * iw + i;
    const int32_t s = s_begin + c * KC + r;
    const uint64_t in_w = 0ull - (uint64_t)(s < sm.nswa);
    bool ok = s < s_end;
    uint64_t comp_row = comp_a + (uint64_t)(int64_t)s * (D * 2);
    if (PAGED || TOPK) {
      // The entry (read at a clamped position, so also for window rows and past the end), then,
      // paged, its page.
      int64_t j = (int64_t)s - sm.nswa;
      if (TOPK) {
        const int32_t e = __builtin_amdgcn_readlane(sel, i);
        ok = ok && (s < sm.nswa || (e >= 0 && e < sm.G));
        j = e;
      }
      j = min(max(j, (int64_t)0), sm.G > 0 ? sm.G - 1 : (int64_t)0);
      if (PAGED) {
        const int64_t pg = page_entry(a.pg.pt, (int64_t)b * a.pg.pt_stride + (j >> a.pg.shift));
        const bool pok = pg >= 0 && pg < a.pg.pool_pages;
        ok = ok && (s < sm.nswa || pok);
        comp_row = (uint64_t)(uintptr_t)(comp + (((pok ? pg : 0) << a.pg.shift) | (j & ((1 << a.pg.shift) - 1))) * D);
      } else {
        comp_row = (uint64_t)(uintptr_t)(comp + (sm.comp0 + j) * D);
      }
      if (lane == 0) rowok[bi][r] = ok ? 1 : 0;
    }
    const uint64_t past = 0ull - (uint64_t)(!ok);
    const uint64_t row = (PAGED || TOPK) ? (((swa_a + (uint64_t)(int64_t)s * (D * 2)) & in_w) | (comp_row & ~in_w))
                                         : ((swa_a & in_w) | (comp_a & ~in_w)) + (uint64_t)(int64_t)s * (D * 2);
    return (safe_a & past) | (row & ~past);
  };
  auto row_dma = [&](int c, int i, uint64_t src) {
    lds_row_dma(reinterpret_cast<const uint16_t*>(src) + 8 * lane, &kt[c & (NB - 1)][(kRowsPerWave * iw + i) * KP]);
  };
  auto issue_rows = [&](int c) {
    const int32_t sel = sel_entries(c);
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) row_dma(c, i, row_src(c, i, sel));
  };

  // The 64 query rows by DMA (waves 0-7, 8 rows each) into buffers 2 and 3, free until chunk 2 is
  // requested in phase 0; then the requesting waves request chunks 0 and 1. Heads past H read head
  // H - 1; their rows are never combined.
  if (wave < 8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int hl = 8 * wave + i;
      const int h = min(64 * zg + hl, a.H - 1);
      lds_row_dma(static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.H + h) * D + 8 * lane, &kt[2 + (hl >> 5)][(hl & 31) * KP]);
    }
  }
  if (issuer) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      if (c < nchunks) issue_rows(c);
    }
    if (nchunks > 1) wait_vm<2 * kRowsPerWave>(); else if (nchunks > 0) wait_vm<kRowsPerWave>(); else wait_vm<0>();
  } else {
    wait_vm<0>();
  }
  lds_barrier();                         // every wave's query rows landed

  // The top of phase t: a requesting wave's rows of chunk t have landed (chunk t + 1's may still be
  // in flight), and every wave is done with phase t - 1, so chunk t + 2 may be requested into the
  // buffer chunk t - 2 used.
  auto phase_top = [&](int t) {
    if (issuer) {
      if (t + 1 < nchunks) wait_vm<kRowsPerWave>(); else wait_vm<0>();
    }
    lds_barrier();
  };
  const int64_t pslot = (int64_t)b * a.n_splits + split;

  if (wave < 4) {
    // ---- producer: Q K^T and the online softmax for heads 16 wl .. +15 (this lane: head hq).
    // Q^T (B operand): lane (head hq, channel group g4) holds channels 32 t + 8 g4 .. +7 of k-step t.
    bf16x8 qf[D / 32];
    {
      const uint16_t* qrow = &kt[2 + (hq >> 5)][(hq & 31) * KP + 8 * g4];
#pragma unroll
      for (int t = 0; t < D / 32; ++t) qf[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + 32 * t));
    }
    float m_run = -INFINITY, l_run = 0.f;  // head hq; l_run over this lane's keys
    for (int t = 0; t <= nchunks; ++t) {
      phase_top(t);
      if (t == nchunks) break;
      const int bi = t & (NB - 1);
      const int32_t s0 = s_begin + t * KC;
      // S^T for the chunk's 32 keys (two 16-key tiles); the K fragments of step u + PD are read
      // while step u's MFMAs run. Chunk t + 2's rows are requested one every two steps (when there is
      // such a chunk), so the address unit takes them while the MFMAs run instead of holding up the
      // wave.
      f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      const uint16_t* krow = &kt[bi][c16 * KP + 8 * g4];
      constexpr int PD = 3;                // K-fragment steps requested ahead
      bf16x8 kf[PD + 1][2];
      auto qk = [&](auto with_rows) {
        constexpr bool ROWS = decltype(with_rows)::value;
        // The rows' sources first: a selected entry or a page-table entry is an LDS or scalar read,
        // whose wait (in order) would otherwise also wait for the K fragments in flight.
        uint64_t src[ROWS ? 8 : 1];
        if (ROWS) {
          const int32_t sel = sel_entries(t + 2);
#pragma unroll
          for (int i = 0; i < 8; ++i) src[i] = row_src(t + 2, i, sel);
        }
#pragma unroll
        for (int p = 0; p < PD; ++p)
#pragma unroll
          for (int n = 0; n < 2; ++n) kf[p][n] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow + 16 * n * KP + 32 * p));
#pragma unroll
        for (int u = 0; u < D / 32; ++u) {
          if (ROWS && u % 2 == 0) row_dma(t + 2, u / 2, src[u / 2]);
          if (u + PD < D / 32) {
#pragma unroll
            for (int n = 0; n < 2; ++n)
              kf[(u + PD) % (PD + 1)][n] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow + 16 * n * KP + 32 * (u + PD)));
          }
#pragma unroll
          for (int n = 0; n < 2; ++n) sacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[u % (PD + 1)][n], qf[u], sacc[n], 0, 0, 0);
        }
        // Keep the reads PD steps ahead of the MFMAs (the scheduler would otherwise pull each read
        // down to just before its use).
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * PD, 0);
#pragma unroll
        for (int u = 0; u < D / 32; ++u) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          if (u + PD < D / 32) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
      };
      if (!kConsumerRows && t + 2 < nchunks) qk(std::true_type{}); else qk(std::false_type{});
      // Register r of tile n of lane (c16, g4) holds key 16 n + 4 g4 + r of head hq.
      float x[8];
      float cm = -INFINITY;
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kr = 16 * n + 4 * g4 + r;
          const bool valid = (PAGED || TOPK) ? rowok[bi][kr] != 0 : s0 + kr < s_end;
          x[4 * n + r] = valid ? sacc[n][r] * a.scale_log2 : -INFINITY;
          cm = fmaxf(cm, x[4 * n + r]);
        }
      const auto mx = [](float p, float q) { return fmaxf(p, q); };
      cm = xor32(xor16(cm, mx), mx);
      // The reference maximum moves only when the chunk exceeds it by more than 2^8 (or on the first
      // keys): P stays at most 256, and most chunks leave alpha exactly 1, so the consumers skip the
      // rescale.
      const float mn = (cm > m_run + kD512Slack || m_run == -INFINITY) ? cm : m_run;
      const bool none = (mn == -INFINITY);
      const float alpha = none ? 1.f : fast_exp2(m_run - mn);
      float psum = 0.f;
      uint16_t* pw = &pb[t & 1][hq * PP + 4 * g4];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        uint32_t w2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          // Rounded to bf16 here so the running sum matches what the MFMA multiplies.
          const uint32_t lo = none ? 0u : f32_to_bf16(fast_exp2(x[4 * n + 2 * e] - mn));
          const uint32_t hi = none ? 0u : f32_to_bf16(fast_exp2(x[4 * n + 2 * e + 1] - mn));
          psum += bf16_to_f32((uint16_t)lo) + bf16_to_f32((uint16_t)hi);
          w2[e] = lo | (hi << 16);
        }
        *reinterpret_cast<uint2*>(pw + 16 * n) = make_uint2(w2[0], w2[1]);
      }
      l_run = l_run * alpha + psum;
      m_run = mn;
      if (g4 == 0) alph[t & 1][hq] = alpha;
    }
    // Running max (base 2) and sum per head.
    const auto add = [](float p, float q) { return p + q; };
    l_run = xor32(xor16(l_run, add), add);
    const int h = 64 * zg + hq;
    if (g4 == 0 && h < a.H) {
      a.part_ml[(pslot * a.H + h) * 2] = m_run;
      a.part_ml[(pslot * a.H + h) * 2 + 1] = l_run;
    }
  } else {
    // ---- consumer: O for all 64 heads and channels 64 cw .. +63, [head tile 32 hp][channel tile
    // 64 cw + 32 ct].
    const int cw = wave - 4;
    f32x16 o[2][2];
#pragma unroll
    for (int hp = 0; hp < 2; ++hp)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) o[hp][ct] = f32x16{};
    for (int t = 0; t <= nchunks; ++t) {
      phase_top(t);
      const bool req = kConsumerRows && t + 2 < nchunks;   // chunk t + 2 is requested this phase
      uint64_t src[kConsumerRows ? kRowsPerWave : 1];
      if (req) {
        const int32_t sel = sel_entries(t + 2);
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) src[i] = row_src(t + 2, i, sel);
      }
      if (t == 0) {
        if (req) {
#pragma unroll
          for (int i = 0; i < kRowsPerWave; ++i) row_dma(t + 2, i, src[i]);
        }
        continue;
      }
      const int c = t - 1;                 // the chunk the producers finished in phase t - 1
      const uint16_t* cur = kt[c & (NB - 1)];
      const uint16_t* pcur = pb[c & 1];
      // O rescaled by the chunk's factors; skipped when none of a 32-head tile's heads raised its
      // maximum (alpha exactly 1), the usual case once the running maxima settle.
#pragma unroll
      for (int hp = 0; hp < 2; ++hp) {
        float al[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(&alph[c & 1][32 * hp + 8 * q4 + 4 * lh]);
#pragma unroll
          for (int e = 0; e < 4; ++e) al[4 * q4 + e] = v[e];
        }
        bool moved = false;
#pragma unroll
        for (int r = 0; r < 16; ++r) moved |= al[r] != 1.f;
        if (__builtin_amdgcn_ballot_w64(moved) != 0) {
#pragma unroll
          for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[hp][ct][r] *= al[r];
        }
      }
      // Every P and V fragment of the chunk is requested first, then the 16 MFMAs run.
      bf16x8 pa[KC / 16][2], vb[KC / 16][2];
#pragma unroll
      for (int kk = 0; kk < KC / 16; ++kk) {
#pragma unroll
        for (int hp = 0; hp < 2; ++hp)
          pa[kk][hp] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&pcur[(32 * hp + l32) * PP + 16 * kk + 8 * lh]));
        // Lane (channel l32, key group lh): keys 16 kk + 8 lh .. +7 of its channel, as two
        // transposing reads of 4 keys each.
        const uint16_t* vrow = cur + (16 * kk + 8 * (g4 >> 1) + (c16 >> 2)) * KP + 64 * cw + 16 * (g4 & 1) + 4 * (c16 & 3);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_v4i16(vrow + 32 * ct));
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_v4i16(vrow + 4 * KP + 32 * ct));
          vb[kk][ct] = __builtin_bit_cast(bf16x8, v8i16{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        }
      }
#pragma unroll
      for (int kk = 0; kk < KC / 16; ++kk)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
          for (int hp = 0; hp < 2; ++hp) o[hp][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[kk][hp], vb[kk][ct], o[hp][ct], 0, 0, 0);
          if (req) row_dma(t + 2, 2 * kk + ct, src[2 * kk + ct]);
        }
    }
    // Unnormalised O in the 16-head-tile layout of the merge ([16-channel tile][lane 16 g + c][4]:
    // head 4 g + r of the tile, channel 16 j + c).
    f32x4* po = reinterpret_cast<f32x4*>(a.part_o) + (pslot * a.head_tiles * 4 + 4 * zg) * (D / 16) * 64;
#pragma unroll
    for (int hp = 0; hp < 2; ++hp)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int h0 = 32 * hp + 8 * q4 + 4 * lh;           // local head of register 4 q4
          const int ch = 64 * cw + 32 * ct + l32;
          const int64_t idx = (int64_t)(h0 >> 4) * (D / 16) * 64 + (ch >> 4) * 64 + 16 * ((h0 & 15) >> 2) + (ch & 15);
          const f32x4 v = {o[hp][ct][4 * q4], o[hp][ct][4 * q4 + 1], o[hp][ct][4 * q4 + 2], o[hp][ct][4 * q4 + 3]};
          __builtin_nontemporal_store(v, &po[idx]);
        }
  }
}

template <bool FP8, bool PAGED>
void launch_dense(int d, dim3 grid, hipStream_t s, const AttnArgs& a) {
  if (!FP8 && d == 512) {
    hipLaunchKernelGGL((attn_dense512_kernel<PAGED, false>), grid, dim3(kD512Threads), 0, s, a);
    return;
  }
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
// bf16 partials (MFMA layout): launch_combine (attn_core.h). Up to 8 splits, one thread per
// 16-byte accumulator (4 heads x 1 channel) merges them with every load in flight at once; more
// splits go to a workgroup per (group of 16 heads, 64 accumulator words, sequence) that computes
// the split weights once per head in LDS, four lanes of a quad summing a strided quarter of the
// splits each. Every load is a whole, coalesced 16-byte vector.
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
  SplitPlan p = plan_splits(dtype, batch, n_heads, d, window, k, max_comp);
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
  SplitPlan p = plan_splits(dtype, batch, n_heads, d, window, kk, max_comp);
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
  if (p.wide && kk > 0) {
    // Selected entries at many sequences: the 64-head kernel, its slots' entries from the top-k list.
    const dim3 grid(p.n_splits, batch, (n_heads + 63) / 64);
    if (paged)
      hipLaunchKernelGGL((attn_dense512_kernel<true, true>), grid, dim3(kD512Threads), 0, s, a);
    else
      hipLaunchKernelGGL((attn_dense512_kernel<false, true>), grid, dim3(kD512Threads), 0, s, a);
  } else if (dense_split(dtype, kk, n_heads)) {
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
    launch_combine(a, batch, n_heads, d, out, lse, s);
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
  SplitPlan p = plan_splits(CHS_BF16, batch, n_heads, d, window, kk, max_comp);
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
  launch_combine(a, batch, n_heads, d, out, lse, s);
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

