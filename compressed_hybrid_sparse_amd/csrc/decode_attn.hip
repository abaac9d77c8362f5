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
#include "common.h"

namespace chs {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

// An LDS address as the transposing load builtin takes it.
__device__ __forceinline__ __attribute__((address_space(3))) v4i16* lds_v4i16(const uint16_t* p) {
  return (__attribute__((address_space(3))) v4i16*)(p);
}

constexpr int kThreads = 256;
constexpr int kKeysPerChunk = 32;

struct AttnArgs {
  const void* q;            // [batch][H][D]
  const void* swa;          // [batch][W][D]
  const int32_t* swa_len;   // [batch]
  const void* comp;         // [*][D]
  const int64_t* cu_comp;   // [batch+1]
  const int32_t* topk;      // [batch][k] or NULL
  int32_t H, D, W, k;
  int64_t max_comp;
  float scale_log2;         // scale * log2(e)
  int32_t n_splits, kps;    // key slots per split
  int32_t head_tiles;       // ceil(H / 64) for bf16, H for fp32
  float* part_o;            // per (sequence, split): see the layout note below
  float* part_ml;           // [batch][n_splits][H][2]: running max (base 2), running sum
};

constexpr int kCombineSplits = 512;   // most splits one call may use

// Partial O of a split. bf16 (MFMA layout): per (sequence, split, 64-head tile, wave) the
// wave's accumulators as they sit in registers, [16-column tile j][lane][4]: lane 16g + c,
// element r hold head 16 * wave + 4g + r, channel 16j + c. fp32: [H][D].

// Key slots of sequence b: [0, swa_len) window rows, then k (C4) or G_b (C128) entries.
struct SlotMap {
  int64_t comp0, G;
  int32_t nswa, nextra;
  __device__ SlotMap(const AttnArgs& a, int b) {
    int32_t L = a.swa_len[b];
    nswa = L < 0 ? 0 : (L > a.W ? a.W : L);
    comp0 = a.cu_comp[b];
    G = a.cu_comp[b + 1] - comp0;
    if (G < 0) G = 0;
    if (a.topk) {
      nextra = a.k;
    } else {
      int64_t g = G < a.max_comp ? G : a.max_comp;
      nextra = (int32_t)g;
    }
  }
  __device__ int32_t nslots() const { return nswa + nextra; }
  // Element offset of slot s's row within its buffer; -1 if the slot holds no key.
  // *is_swa tells which buffer.
  __device__ int64_t row(const AttnArgs& a, int b, int32_t s, bool* is_swa) const {
    if (s < nswa) { *is_swa = true; return ((int64_t)b * a.W + s) * a.D; }
    *is_swa = false;
    int64_t j = s - nswa;
    if (a.topk) {
      j = a.topk[(int64_t)b * a.k + j];
      if (j < 0 || j >= G) return -1;
    }
    return (comp0 + j) * a.D;
  }
};

// Max / sum over the 16 lanes of a DPP row (lanes 16r .. 16r+15); every lane gets the result.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));
  return v;
}

// Source rows of a 32-slot chunk starting at slot s0 for a wave whose load i covers slot
// s0 + (4i + wave) * RPI + lr (null: no key there). Branch-free: the top-k entry is read at a
// clamped position whether or not the slot needs it, so the reads issue back to back. At
// d = 512 (RPI = 1) every operand is the same for the whole wave.
template <int D, int LOADS, int RPI>
__device__ __forceinline__ void chunk_rows(const AttnArgs& a, const SlotMap& sm, int b, int32_t s0, int32_t s_end,
                                           int wave, int lr, const uint16_t* (&rp)[LOADS]) {
  const uint16_t* swa = static_cast<const uint16_t*>(a.swa);
  const uint16_t* comp = static_cast<const uint16_t*>(a.comp);
  int32_t idx[LOADS];
  if (a.topk != nullptr && a.k > 0) {
    const int32_t* tk = a.topk + (int64_t)b * a.k;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) idx[i] = tk[min(max(s0 + (4 * i + wave) * RPI + lr - sm.nswa, 0), a.k - 1)];
  } else {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) idx[i] = s0 + (4 * i + wave) * RPI + lr - sm.nswa;
  }
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int32_t s = s0 + (4 * i + wave) * RPI + lr;
    const bool in_swa = s < sm.nswa;
    const bool ok = s < s_end && (in_swa || (idx[i] >= 0 && idx[i] < sm.G));
    const uint16_t* p = in_swa ? swa + ((int64_t)b * a.W + s) * D : comp + (sm.comp0 + idx[i]) * D;
    rp[i] = ok ? p : nullptr;
  }
}

// ---------------------------------------------------------------- bf16 MFMA split kernel
// One workgroup of 4 waves per (split, sequence, 16-head tile). The 16 heads are the MFMA
// rows. Each wave gathers a quarter of a chunk's 32 rows and contracts Q K^T over a quarter of
// the channels (d >= 128; all of them at d = 64). The four partial logit tiles are summed
// through LDS in a fixed order, so every wave holds bit-identical logits and runs the same
// softmax. Each wave then computes P.V for its quarter of the channels. A wave thus issues a
// handful of loads and 8 KiB of partial stores (d = 512).
template <int D>
__global__ __launch_bounds__(kThreads) void attn_bf16_kernel(AttnArgs a) {
  constexpr int KC = kKeysPerChunk;
  constexpr int KN_PITCH = D + 8;          // bf16 elements per row-major LDS row
  constexpr int P_PITCH = KC + 8;
  constexpr int VPR = D / 8;               // 16-byte vectors per row
  constexpr int RPI = 64 / VPR;            // rows one wave-wide load covers (1 at d = 512)
  constexpr int LOADS = KC / (4 * RPI);    // loads per wave per chunk
  constexpr int TPW = D / 64;              // 16-channel output tiles per wave
  constexpr bool SPLIT_S = D >= 128;       // logits contracted over a quarter of d per wave
  constexpr int QD = SPLIT_S ? D / 4 : D;  // channels of Q (and of the logit contraction) per wave
  static_assert(QD % 32 == 0, "k step");
  static_assert(VPR <= 64 && 64 % VPR == 0 && KC % (4 * RPI) == 0 && TPW >= 1, "tile");
  __shared__ __attribute__((aligned(16))) uint16_t kn[KC * KN_PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t pb[4][16 * P_PITCH];
  __shared__ int32_t rowok[KC];
  __shared__ __attribute__((aligned(16))) f32x4 spart[SPLIT_S ? 4 : 1][2][64];

  const int b = blockIdx.y, split = blockIdx.x;
  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = RPI > 1 ? lane / VPR : 0, cv = lane % VPR;
  const int h_base = blockIdx.z * 16;
  const SlotMap sm(a, b);
  const int32_t s_begin = split * a.kps;
  const int32_t s_end = min(s_begin + a.kps, sm.nslots());

  // Source row of load i of the first chunk (null: no key). These index reads go out before
  // the Q loads, so waiting for them does not wait for Q as well.
  const uint16_t* rp[LOADS];
  chunk_rows<D, LOADS, RPI>(a, sm, b, s_begin, s_end, wave, lr, rp);

  // Q fragment (A operand): row c of the 16 heads, d = d0 + 32t + 8g .. +8 (d0 = this wave's
  // quarter); head index clamped, then zeroed, so the loads are unconditional.
  const int d0 = SPLIT_S ? QD * wave : 0;
  bf16x8 qf[QD / 32];
  {
    const int h = h_base + c;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.H + min(h, a.H - 1)) * D + d0;
    u32x4 qv[QD / 32];
#pragma unroll
    for (int t = 0; t < QD / 32; ++t) qv[t] = *reinterpret_cast<const u32x4*>(qp + 32 * t + 8 * g);
#pragma unroll
    for (int t = 0; t < QD / 32; ++t) qf[t] = __builtin_bit_cast(bf16x8, h < a.H ? qv[t] : u32x4{0, 0, 0, 0});
  }
  f32x4 o[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) o[j] = f32x4{0, 0, 0, 0};
  float m_run[4], l_run[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) { m_run[r] = -INFINITY; l_run[r] = 0.f; }

  for (int32_t s0 = s_begin; s0 < s_end; s0 += KC) {
    // 1. gather the chunk's rows (coalesced 16-byte loads) into a row-major LDS tile.
    u32x4 v[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      v[i] = rp[i] ? *reinterpret_cast<const u32x4*>(rp[i] + 8 * cv) : u32x4{0, 0, 0, 0};
    __syncthreads();   // the previous chunk's LDS reads are done
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int r = (4 * i + wave) * RPI + lr;
      *reinterpret_cast<u32x4*>(&kn[r * KN_PITCH + 8 * cv]) = v[i];
      if (cv == 0) rowok[r] = rp[i] != nullptr;
    }
    if (s0 + KC < s_end) chunk_rows<D, LOADS, RPI>(a, sm, b, s0 + KC, s_end, wave, lr, rp);
    __syncthreads();
    // 2. S = Q K^T for keys 16n + c (n = 0, 1); lane holds heads 4g + r.
    f32x4 sacc[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      sacc[n] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int t = 0; t < QD / 32; ++t) {
        u32x4 kb = *reinterpret_cast<const u32x4*>(&kn[(16 * n + c) * KN_PITCH + d0 + 32 * t + 8 * g]);
        sacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[t], __builtin_bit_cast(bf16x8, kb), sacc[n], 0, 0, 0);
      }
    }
    if constexpr (SPLIT_S) {
      // Sum the four channel quarters in wave order, the same order in every wave.
      spart[wave][0][lane] = sacc[0];
      spart[wave][1][lane] = sacc[1];
      __syncthreads();
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        f32x4 t = spart[0][n][lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
          const f32x4 u = spart[w][n][lane];
#pragma unroll
          for (int r = 0; r < 4; ++r) t[r] += u[r];
        }
        sacc[n] = t;
      }
    }
    // 3. online softmax (base-2), per head row 4g + r.
    const bool valid0 = rowok[c] != 0, valid1 = rowok[16 + c] != 0;
    float p[2][4], alpha[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float x0 = valid0 ? sacc[0][r] * a.scale_log2 : -INFINITY;
      const float x1 = valid1 ? sacc[1][r] * a.scale_log2 : -INFINITY;
      const float cm = row16_max(fmaxf(x0, x1));
      const float mn = fmaxf(m_run[r], cm);
      const bool none = (mn == -INFINITY);
      alpha[r] = none ? 1.f : fast_exp2(m_run[r] - mn);
      // Round P to bf16 here so the running sum matches what the MFMA multiplies.
      p[0][r] = none ? 0.f : bf16_to_f32((uint16_t)f32_to_bf16(fast_exp2(x0 - mn)));
      p[1][r] = none ? 0.f : bf16_to_f32((uint16_t)f32_to_bf16(fast_exp2(x1 - mn)));
      l_run[r] = l_run[r] * alpha[r] + row16_sum(p[0][r] + p[1][r]);
      m_run[r] = mn;
    }
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
#pragma unroll
      for (int r = 0; r < 4; ++r) o[j][r] *= alpha[r];
    }
    // 4. P to this wave's LDS slice as [head][key], read back as the A operand (row c, keys
    // 8g .. 8g+7).
    uint16_t* pw = pb[wave];
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        pw[(4 * g + r) * P_PITCH + 16 * n + c] = (uint16_t)(__float_as_uint(p[n][r]) >> 16);
    __syncthreads();
    const bf16x8 pf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&pw[c * P_PITCH + 8 * g]));
    // B operand of P.V: column 16j + c of the tile, keys 8g .. 8g+7. ds_read_b64_tr_b16 gives
    // lane i of a 16-lane group element e of the group's 8-byte chunks read with stride 16,
    // so lane c addressing channels 16j + 4(c&3) .. +3 of key row 8g + (c>>2) (+4 for the
    // upper half) receives keys 8g .. 8g+3 (8g+4 .. 8g+7) of channel 16j + c.
    const uint16_t* vrow = &kn[(8 * g + (c >> 2)) * KN_PITCH + 4 * (c & 3) + 16 * TPW * wave];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_v4i16(vrow + 16 * j));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_v4i16(vrow + 4 * KN_PITCH + 16 * j));
      const v8i16 vb = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf, __builtin_bit_cast(bf16x8, vb), o[j], 0, 0, 0);
    }
  }
  // Partial result of this split: unnormalised O in the MFMA accumulator layout (one 16-byte
  // store per tile and lane, coalesced; wave w holds tiles TPW w ..), running max (base 2) and
  // sum per head. The slot of 16-head tile z is (64-head tile z / 4, quarter z % 4).
  const int64_t pslot = (int64_t)b * a.n_splits + split;
  f32x4* po = reinterpret_cast<f32x4*>(a.part_o) + (pslot * a.head_tiles * 4 + blockIdx.z) * (D / 16) * 64;
#pragma unroll
  for (int j = 0; j < TPW; ++j) po[(TPW * wave + j) * 64 + lane] = o[j];
  if (wave == 0 && c == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = h_base + 4 * g + r;
      if (h < a.H) {
        a.part_ml[(pslot * a.H + h) * 2] = m_run[r];
        a.part_ml[(pslot * a.H + h) * 2 + 1] = l_run[r];
      }
    }
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
// bf16 partials (MFMA layout): one workgroup per (group of 16 heads, 1024 accumulator words
// of their tile, sequence); each thread reads one 16-byte accumulator (4 heads x 1 channel)
// per split, so every load is a whole, coalesced vector. Split weights are computed once per
// head in LDS.
// Four lanes of a quad share one accumulator word, each summing a strided quarter of the
// splits, so a launch has four times as many workgroups as words / 256.
constexpr int kCombineLanes = 4;

__global__ __launch_bounds__(kThreads) void combine_mfma_kernel(AttnArgs a, float* out, float* lse) {
  __shared__ float wts[16][kCombineSplits];
  __shared__ float lpart[16][kCombineSplits];
  __shared__ float lsum[16];
  const int b = blockIdx.z, hg = blockIdx.y;          // heads 16 hg .. 16 hg + 15
  const int tid = threadIdx.x, D = a.D;
  const int ns = a.n_splits;
  const int sq = tid & (kCombineLanes - 1);           // this lane's quarter of the splits
  // Accumulator word index within the wave tile: (j, lane); this thread's 4 heads 4g + r.
  const int wraw = blockIdx.x * (kThreads / kCombineLanes) + tid / kCombineLanes;
  const int wpos = min(wraw, (D / 16) * 64 - 1);
  const int j = wpos >> 6, lane = wpos & 63, g = lane >> 4, c = lane & 15;
  const int tile = hg >> 2, wave = hg & 3;
  const f32x4* po = reinterpret_cast<const f32x4*>(a.part_o);
  const int64_t stride = (int64_t)a.head_tiles * 4 * (D / 16) * 64;   // one split, in f32x4
  const int64_t base = (((int64_t)b * ns * a.head_tiles + tile) * 4 + wave) * (D / 16) * 64 + wpos;
  // This lane's first splits (sq, sq + 4, ...) are requested before anything else, so they
  // arrive while the split weights are computed.
  constexpr int kBatch = 8;
  f32x4 v[kBatch];
#pragma unroll
  for (int q = 0; q < kBatch; ++q) v[q] = po[base + (int64_t)min(sq + kCombineLanes * q, ns - 1) * stride];
  // The 16 heads' (max, sum) pairs of every split come through LDS in one coalesced pass; then
  // head hl = tid / 16 is handled by the 16 lanes of one DPP row, each lane a strided subset of
  // the splits, and the head's maximum and weighted sum are row reductions.
  const int nh = min(16, a.H - 16 * hg);
  for (int e = tid; e < ns * nh; e += kThreads) {
    const int sp = e / nh, hl = e - sp * nh;
    const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + (((int64_t)b * ns + sp) * a.H + 16 * hg + hl) * 2);
    wts[hl][sp] = ml.x;
    lpart[hl][sp] = ml.y;
  }
  __syncthreads();
  {
    const int hl = tid >> 4, sl = tid & 15;
    const int h = 16 * hg + hl;
    float M = -INFINITY;
    if (hl < nh)
      for (int sp = sl; sp < ns; sp += 16) M = fmaxf(M, wts[hl][sp]);
    M = row16_max(M);
    float L = 0.f;
    for (int sp = sl; sp < ns; sp += 16) {
      const float ms = hl < nh ? wts[hl][sp] : -INFINITY;
      const float wgt = (ms == -INFINITY) ? 0.f : exp2f(ms - M);
      L += wgt * (hl < nh ? lpart[hl][sp] : 0.f);
      wts[hl][sp] = wgt;
    }
    L = row16_sum(L);
    if (sl == 0) {
      lsum[hl] = L;
      if (lse && hl < nh && blockIdx.x == 0) lse[(int64_t)b * a.H + h] = (L > 0.f) ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
    }
  }
  __syncthreads();
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int sp0 = 0; sp0 < ns; sp0 += kCombineLanes * kBatch) {
    if (sp0 > 0) {
#pragma unroll
      for (int q = 0; q < kBatch; ++q)
        v[q] = po[base + (int64_t)min(sp0 + sq + kCombineLanes * q, ns - 1) * stride];
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int sp = sp0 + sq + kCombineLanes * q;
      if (sp < ns) {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = fmaf(wts[4 * g + r][sp], v[q][r], acc[r]);
      }
    }
  }
  // Quad sum: the four lanes of a word hold disjoint split subsets.
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    acc[r] += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc[r]), 0xB1, 0xF, 0xF, false));
    acc[r] += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc[r]), 0x4E, 0xF, 0xF, false));
  }
  if (sq != 0 || wraw >= (D / 16) * 64) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int hl = 4 * g + r, h = 16 * hg + hl;
    if (h < a.H) {
      const float L = lsum[hl];
      out[((int64_t)b * a.H + h) * D + 16 * j + c] = (L > 0.f) ? acc[r] / L : 0.f;
    }
  }
}

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

struct SplitPlan {
  int32_t n_splits, kps;
};

SplitPlan plan_splits(chs_dtype dt, int32_t batch, int32_t H, int32_t window, int32_t k, int64_t max_comp) {
  const int64_t max_slots = (int64_t)window + (k > 0 ? k : max_comp);
  const int gran = dt == CHS_BF16 ? kKeysPerChunk : kThreads;
  // Aim at about 512 workgroups: bf16 runs one per 16-head tile, fp32 one per head.
  const int64_t blocks_per_split = (int64_t)batch * (dt == CHS_BF16 ? (H + 15) / 16 : H);
  int64_t want = (512 + blocks_per_split - 1) / blocks_per_split;
  const int64_t most = (max_slots + gran - 1) / gran;
  if (want > most) want = most;
  if (want > kCombineSplits) want = kCombineSplits;
  if (want < 1) want = 1;
  int64_t kps = (max_slots + want - 1) / want;
  kps = (kps + gran - 1) / gran * gran;
  if (kps < gran) kps = gran;
  SplitPlan p;
  p.kps = (int32_t)kps;
  p.n_splits = (int32_t)((max_slots + kps - 1) / kps);
  if (p.n_splits < 1) p.n_splits = 1;
  return p;
}

size_t ws_bytes(chs_dtype dt, int32_t batch, int32_t H, int32_t D, const SplitPlan& p, float** po, float** pml,
                char* base) {
  const size_t nparts = (size_t)batch * p.n_splits * H;
  const size_t hpad = dt == CHS_BF16 ? (size_t)(H + 63) / 64 * 64 : (size_t)H;
  size_t o_po = 0, o_ml = align_up((size_t)batch * p.n_splits * hpad * D * 4, 256);
  size_t total = align_up(o_ml + nparts * 2 * 4, 256);
  if (po) *po = reinterpret_cast<float*>(base + o_po);
  if (pml) *pml = reinterpret_cast<float*>(base + o_ml);
  return total;
}

}  // namespace
}  // namespace chs

extern "C" size_t chs_decode_attn_workspace_size(chs_dtype dtype, int32_t batch, int32_t n_heads, int32_t d,
                                                 int32_t window, int32_t k, int64_t max_comp) {
  using namespace chs;
  if (batch < 1 || n_heads < 1 || d < 1 || window < 0 || k < 0 || max_comp < 0) return 0;
  SplitPlan p = plan_splits(dtype, batch, n_heads, window, k, max_comp);
  return ws_bytes(dtype, batch, n_heads, d, p, nullptr, nullptr, nullptr);
}

extern "C" chs_status chs_decode_attn(chs_dtype dtype, int32_t batch, int32_t n_heads, int32_t d,
                                      int32_t window, int32_t k, float scale, const void* q,
                                      const void* swa_kv, const int32_t* swa_len, const void* comp_kv,
                                      const int64_t* cu_comp, const int32_t* topk, int64_t max_comp,
                                      float* out, float* lse, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  using namespace chs;
  if (!dtype_ok(dtype)) return CHS_ERR_DTYPE;
  if (batch < 1 || batch > 65535 || n_heads < 1 || n_heads > 128 || window < 0 || window > 4096 ||
      k < 0 || k > 2048 || max_comp < 0 || max_comp >= (1LL << 31) || !(scale > 0.f) || !(scale < INFINITY))
    return CHS_ERR_SHAPE;
  if (dtype == CHS_BF16) {
    if (d != 64 && d != 128 && d != 256 && d != 512) return CHS_ERR_SHAPE;
  } else if (d < 1 || d > 1024 || d % 4 != 0) {
    return CHS_ERR_SHAPE;
  }
  if (!q || !swa_len || !cu_comp || !out || !workspace) return CHS_ERR_NULL;
  if (window > 0 && !swa_kv) return CHS_ERR_NULL;
  if (!comp_kv && (topk ? k > 0 : max_comp > 0)) return CHS_ERR_NULL;
  const int kk = topk ? k : 0;
  SplitPlan p = plan_splits(dtype, batch, n_heads, window, kk, max_comp);
  AttnArgs a;
  a.q = q; a.swa = swa_kv; a.swa_len = swa_len; a.comp = comp_kv; a.cu_comp = cu_comp; a.topk = topk;
  a.H = n_heads; a.D = d; a.W = window; a.k = kk; a.max_comp = max_comp;
  a.scale_log2 = scale * kLog2e;
  a.n_splits = p.n_splits; a.kps = p.kps;
  a.head_tiles = dtype == CHS_BF16 ? (n_heads + 63) / 64 : n_heads;
  const size_t need = ws_bytes(dtype, batch, n_heads, d, p, &a.part_o, &a.part_ml, static_cast<char*>(workspace));
  if (workspace_bytes < need) return CHS_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == CHS_BF16) {
    dim3 grid(p.n_splits, batch, (n_heads + 15) / 16);
    switch (d) {
      case 64: hipLaunchKernelGGL(attn_bf16_kernel<64>, grid, dim3(kThreads), 0, s, a); break;
      case 128: hipLaunchKernelGGL(attn_bf16_kernel<128>, grid, dim3(kThreads), 0, s, a); break;
      case 256: hipLaunchKernelGGL(attn_bf16_kernel<256>, grid, dim3(kThreads), 0, s, a); break;
      default: hipLaunchKernelGGL(attn_bf16_kernel<512>, grid, dim3(kThreads), 0, s, a); break;
    }
  } else {
    dim3 grid(p.n_splits, batch, n_heads);
    hipLaunchKernelGGL(attn_f32_kernel, grid, dim3(kThreads), 0, s, a);
  }
  if (launch_status() != CHS_OK) return CHS_ERR_LAUNCH;
  if (dtype == CHS_BF16) {
    const int words_per_block = kThreads / kCombineLanes;
    const dim3 cgrid((unsigned)((d / 16 * 64 + words_per_block - 1) / words_per_block), (unsigned)((n_heads + 15) / 16),
                     (unsigned)batch);
    hipLaunchKernelGGL(combine_mfma_kernel, cgrid, dim3(kThreads), 0, s, a, out, lse);
  } else {
    hipLaunchKernelGGL(combine_rows_kernel, dim3(n_heads, batch), dim3(kThreads), 0, s, a, out, lse);
  }
  return launch_status();
}
