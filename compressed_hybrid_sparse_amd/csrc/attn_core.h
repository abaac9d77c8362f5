// Attention device code shared by the decode-attention kernels and the fused decode step:
// the key-slot map, the split body (gather, Q K^T, online softmax, P V) over one or several
// 16-head tiles, the log-sum-exp combine body, and the split plan. The design is described
// in decode_attn.hip.
#pragma once

#include <type_traits>

#include "common.h"

namespace chs {
namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

// Loads through pointers the compiler cannot place (a row pointer that may be null, a top-k row
// that may live in LDS) would otherwise be flat loads, which also hold the LDS counter: these
// name the address space.
__device__ __forceinline__ u32x4 load_global_u32x4(const void* p) {
  return *(const __attribute__((address_space(1))) u32x4*)(p);
}
__device__ __forceinline__ float load_global_f32(const float* p) {
  return *(const __attribute__((address_space(1))) float*)(p);
}
__device__ __forceinline__ int32_t load_global_i32(const int32_t* p) {
  return *(const __attribute__((address_space(1))) int32_t*)(p);
}
__device__ __forceinline__ int32_t load_lds_i32(const int32_t* p) {
  return *(const __attribute__((address_space(3))) int32_t*)(p);
}

// An LDS address as the transposing load builtin takes it.
__device__ __forceinline__ __attribute__((address_space(3))) v4i16* lds_v4i16(const uint16_t* p) {
  return (__attribute__((address_space(3))) v4i16*)(p);
}

constexpr int kAttnThreads = 256;       // threads of the standalone split and combine blocks
constexpr int kKeysPerChunk = 32;

// Paged pools (all NULL / 0: contiguous storage). The window of sequence b is page swa_page[b]
// of the window pool (rows page * W .. + W - 1) instead of slot b; compressed entry j of sequence
// b is pool row pt[b * pt_stride + j / 2^shift] * 2^shift + j mod 2^shift, and comp_len[b]
// entries exist. A window page outside [0, swa_pages) drops the window; an entry whose page is
// outside [0, pool_pages) is skipped.
struct Paging {
  const int32_t* swa_page;  // [batch] or NULL
  int64_t swa_pages;
  const int32_t* pt;        // [batch][pt_stride] or NULL
  const int64_t* comp_len;  // [batch] (with pt)
  int32_t pt_stride, shift;
  int64_t pool_pages;
};

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
  const float* swa_scale;   // FP8 storage: [batch][W] row scales of swa (else unused)
  const float* comp_scale;  // FP8 storage: [*] row scales of comp (else unused)
  Paging pg;                // paged pools (zeroed: contiguous)
};

constexpr int kCombineSplits = 512;   // most splits one call may use
constexpr int kCombineLanes = 4;      // lanes per output word in the combine

// Partial O of a split. bf16 (MFMA layout): per (sequence, split, 64-head tile, 16-head
// quarter z % 4) the 16-head tile's accumulators as they sit in registers, [16-column tile
// j][lane][4]: lane 16g + c, element r hold head 16z + 4g + r, channel 16j + c. fp32: [H][D].

// Key slots of sequence b: [0, swa_len) window rows, then k (C4) or G_b (C128) entries.
struct SlotMap {
  int64_t comp0, G;
  int64_t swa_row0;         // first row of the sequence's window in the window buffer
  int32_t nswa, nextra;
  __device__ SlotMap(const AttnArgs& a, int b) {
    int32_t L = a.swa_len[b];
    nswa = L < 0 ? 0 : (L > a.W ? a.W : L);
    swa_row0 = (int64_t)b * a.W;
    if (a.pg.swa_page) {
      const int64_t p = a.pg.swa_page[b];
      if (p < 0 || p >= a.pg.swa_pages) nswa = 0;
      swa_row0 = (p < 0 || p >= a.pg.swa_pages ? 0 : p) * a.W;
    }
    if (a.pg.pt) {
      comp0 = 0;
      G = a.pg.comp_len[b];
      const int64_t cap = (int64_t)a.pg.pt_stride << a.pg.shift;
      if (G > cap) G = cap;
    } else {
      comp0 = a.cu_comp[b];
      G = a.cu_comp[b + 1] - comp0;
    }
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
    if (s < nswa) { *is_swa = true; return (swa_row0 + s) * a.D; }
    *is_swa = false;
    int64_t j = s - nswa;
    if (a.topk) {
      j = a.topk[(int64_t)b * a.k + j];
      if (j < 0 || j >= G) return -1;
    }
    if (a.pg.pt) {
      const int64_t p = a.pg.pt[(int64_t)b * a.pg.pt_stride + (j >> a.pg.shift)];
      if (p < 0 || p >= a.pg.pool_pages) return -1;
      return ((p << a.pg.shift) | (j & ((1 << a.pg.shift) - 1))) * a.D;
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

// Source rows of a 32-slot chunk starting at slot s0 for a workgroup of NW waves: load i of
// wave w is wave-wide load li = i * NW + w of the chunk (none if li >= 32 / RPI), covering slot
// s0 + li * RPI + lr (null: no key there); with FP8 storage also the row's scale. Branch-free:
// the top-k entry is read at a clamped position whether or not the slot needs it, so the reads
// issue back to back. When a load is one whole row every operand is the same for the whole wave.
// PAGED: entries go through the page table (one more dependent read per row, clamped the same
// way), and the window through the sequence's window page.
// sel: the sequence's top-k row in LDS, read instead of a.topk when given.
template <int D, int LOADS, int RPI, int NW, typename ET, bool PAGED = false>
__device__ __forceinline__ void chunk_rows(const AttnArgs& a, const SlotMap& sm, int b, int32_t s0, int32_t s_end,
                                           int wave, int lr, const ET* (&rp)[LOADS], const float* (&rs)[LOADS],
                                           const int32_t* sel = nullptr) {
  constexpr int NLOADS = kKeysPerChunk / RPI;
  const ET* swa = static_cast<const ET*>(a.swa);
  const ET* comp = static_cast<const ET*>(a.comp);
  int32_t idx[LOADS];
  if (a.topk != nullptr && a.k > 0) {
    if (sel) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i)
        idx[i] = load_lds_i32(sel + min(max(s0 + (i * NW + wave) * RPI + lr - sm.nswa, 0), a.k - 1));
    } else {
      const int32_t* tk = a.topk + (int64_t)b * a.k;
#pragma unroll
      for (int i = 0; i < LOADS; ++i)
        idx[i] = load_global_i32(tk + min(max(s0 + (i * NW + wave) * RPI + lr - sm.nswa, 0), a.k - 1));
    }
  } else {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) idx[i] = s0 + (i * NW + wave) * RPI + lr - sm.nswa;
  }
  int64_t prow[LOADS];                                 // PAGED: pool row of the entry
  bool pok[LOADS];
  if (PAGED) {
    const int32_t* ptb = a.pg.pt + (int64_t)b * a.pg.pt_stride;
    const int32_t mask = (1 << a.pg.shift) - 1;
    const int64_t last = sm.G > 0 ? sm.G - 1 : 0;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int64_t j = idx[i] < 0 ? 0 : (idx[i] > last ? last : idx[i]);
      const int64_t p = ptb[j >> a.pg.shift];
      pok[i] = p >= 0 && p < a.pg.pool_pages;
      prow[i] = ((pok[i] ? p : 0) << a.pg.shift) | (j & mask);
    }
  }
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int32_t s = s0 + (i * NW + wave) * RPI + lr;
    const bool in_swa = s < sm.nswa;
    const bool ok = i * NW + wave < NLOADS && s < s_end &&
                    (in_swa || (idx[i] >= 0 && idx[i] < sm.G && (!PAGED || pok[i])));
    const int64_t row = in_swa ? sm.swa_row0 + s : (PAGED ? prow[i] : sm.comp0 + idx[i]);
    const ET* p = (in_swa ? swa : comp) + row * D;
    rp[i] = ok ? p : nullptr;
    if (sizeof(ET) == 1) rs[i] = ok ? (in_swa ? a.swa_scale : a.comp_scale) + row : nullptr;
  }
}

// LDS of one split body over TILES 16-head tiles: the chunk's row-major K (= V) tile, each
// wave's P, the partial logit tiles of the four channel quarters, and the rows' validity.
template <int D, int TILES>
struct alignas(16) AttnShared {
  uint16_t kn[kKeysPerChunk * (D + 8)];
  uint16_t pb[4 * TILES][16 * (kKeysPerChunk + 8)];
  f32x4 spart[D >= 128 ? TILES : 1][4][2][64];
  int32_t rowok[kKeysPerChunk];
  float rowsc[kKeysPerChunk];          // FP8 storage: the chunk's row scales
};

struct NoHook {
  __device__ __forceinline__ void operator()(int32_t) {}
};

// Split `split` of sequence b for the 16-head tiles z0 .. z0 + TILES - 1, run by 4 * TILES
// waves: wave w serves tile w / 4 and channel quarter w % 4. Every wave gathers a share of a
// chunk's 32 rows into one row-major LDS tile; contracts Q K^T over its quarter of the channels
// (d >= 128; all of them at d = 64), the four partial logit tiles of a head tile being summed
// through LDS in a fixed order, so all four waves hold bit-identical logits and run the same
// softmax; and computes P.V for its quarter. before_rows(s0) runs, uniformly over the
// workgroup, before the rows of the chunk at slot s0 are looked up.
// sm is sequence b's slot map (SlotMap(a, b)), passed in by callers that already hold it; sel,
// when given, is the sequence's top-k row in LDS (read instead of a.topk). PF = 1: a split of
// several chunks requests the next chunk's rows as soon as the current one is in LDS, so they
// arrive while it computes (PF = 0: each chunk's rows when its turn comes). A second register
// buffer (two chunks ahead) spills at 1024 threads.
template <int D, int TILES, typename Hook, bool FP8 = false, bool PAGED = false, int PF = 0>
__device__ __forceinline__ void attn_split_sm(const AttnArgs& a, const SlotMap& sm, int b, int split, int z0, int tid,
                                              AttnShared<D, TILES>& sh, Hook& before_rows,
                                              const int32_t* sel = nullptr) {
  constexpr int KC = kKeysPerChunk;
  constexpr int KN_PITCH = D + 8;          // bf16 elements per row-major LDS row
  constexpr int P_PITCH = KC + 8;
  constexpr int NW = 4 * TILES;            // waves
  typedef typename std::conditional<FP8, uint8_t, uint16_t>::type ET;   // storage element
  constexpr int EPV = 16 / (int)sizeof(ET);    // elements per 16-byte vector
  constexpr int VPR = D / EPV;             // 16-byte vectors per row
  constexpr int RPI = 64 / VPR;            // rows one wave-wide load covers (1 at d = 512)
  constexpr int NLOADS = KC / RPI;         // wave-wide loads per chunk
  constexpr int LOADS = (NLOADS + NW - 1) / NW;   // per wave
  constexpr int TPW = D / 64;              // 16-channel output tiles per wave
  constexpr bool SPLIT_S = D >= 128;       // logits contracted over a quarter of d per wave
  constexpr int QD = SPLIT_S ? D / 4 : D;  // channels of Q (and of the logit contraction) per wave
  static_assert(VPR <= 64 && 64 % VPR == 0 && KC % RPI == 0 && TPW >= 1 && QD % 32 == 0, "tile");

  const int lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = wave >> 2, quarter = wave & 3;
  const int z = z0 + tile;
  const int lr = RPI > 1 ? lane / VPR : 0, cv = lane % VPR;
  const int h_base = z * 16;
  const int32_t s_begin = split * a.kps;
  const int32_t s_end = min(s_begin + a.kps, sm.nslots());

  // Source row (and FP8 row scale) of load i of the first chunk (null: no key). These index
  // reads go out before the Q loads, so waiting for them does not wait for Q as well.
  const ET* rp[LOADS];
  const float* rs[LOADS];
  before_rows(s_begin);
  chunk_rows<D, LOADS, RPI, NW, ET, PAGED>(a, sm, b, s_begin, s_end, wave, lr, rp, rs, sel);

  // Q fragment (A operand): row c of the tile's 16 heads, d = d0 + 32t + 8g .. +8 (d0 = this
  // wave's quarter). A head past H reads head H - 1 (clamped, so the loads are unconditional);
  // its rows of S, P and O are never stored or combined, and every other head's rows are
  // computed independently of them. Nothing waits on Q before the first chunk's rows are
  // requested.
  const int d0 = SPLIT_S ? QD * quarter : 0;
  bf16x8 qf[QD / 32];
  {
    const int h = h_base + c;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.H + min(h, a.H - 1)) * D + d0;
#pragma unroll
    for (int t = 0; t < QD / 32; ++t) qf[t] = *reinterpret_cast<const bf16x8*>(qp + 32 * t + 8 * g);
  }
  f32x4 o[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) o[j] = f32x4{0, 0, 0, 0};
  float m_run[4], l_run[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) { m_run[r] = -INFINITY; l_run[r] = 0.f; }

  static_assert(PF == 0 || PF == 1, "prefetch depth");
  u32x4 v[LOADS];
  float vs[LOADS];
  auto load_rows = [&]() {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      v[i] = rp[i] ? load_global_u32x4(rp[i] + EPV * cv) : u32x4{0, 0, 0, 0};
      if (FP8) vs[i] = rp[i] ? load_global_f32(rs[i]) : 0.f;
    }
  };
  if (PF == 1) load_rows();
  // One chunk at slot s0: rows into LDS, then the next chunk's rows looked up (and requested).
  auto stage = [&](int32_t s0) {
    // 1. gather the chunk's rows (coalesced 16-byte loads) into a row-major LDS tile (with PF
    // they were requested during the previous chunk).
    if (PF == 0) load_rows();
    __syncthreads();   // the previous chunk's LDS reads are done
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int li = i * NW + wave;
      if (li < NLOADS) {
        const int r = li * RPI + lr;
        if (FP8) {
          // 16 E4M3 codes become 16 bf16 values, exactly (scale 1); the row scale is applied
          // to the logits and to P below.
          u32x4 lo, hi;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t x = v[i][e];
            const uint32_t p0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false));
            const uint32_t p1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true));
            if (e < 2) { lo[2 * e] = p0; lo[2 * e + 1] = p1; } else { hi[2 * e - 4] = p0; hi[2 * e - 3] = p1; }
          }
          *reinterpret_cast<u32x4*>(&sh.kn[r * KN_PITCH + 16 * cv]) = lo;
          *reinterpret_cast<u32x4*>(&sh.kn[r * KN_PITCH + 16 * cv + 8]) = hi;
          if (cv == 0) sh.rowsc[r] = vs[i];
        } else {
          *reinterpret_cast<u32x4*>(&sh.kn[r * KN_PITCH + 8 * cv]) = v[i];
        }
        if (cv == 0) sh.rowok[r] = rp[i] != nullptr;   // the row pointers are still this chunk's
      }
    }
    if (s0 + KC < s_end) {
      before_rows(s0 + KC);
      chunk_rows<D, LOADS, RPI, NW, ET, PAGED>(a, sm, b, s0 + KC, s_end, wave, lr, rp, rs, sel);
      if (PF == 1) load_rows();
    }
    __syncthreads();
    // 2. S = Q K^T for keys 16n + c (n = 0, 1); lane holds heads 4g + r.
    f32x4 sacc[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      sacc[n] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int t = 0; t < QD / 32; ++t) {
        u32x4 kb = *reinterpret_cast<const u32x4*>(&sh.kn[(16 * n + c) * KN_PITCH + d0 + 32 * t + 8 * g]);
        sacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[t], __builtin_bit_cast(bf16x8, kb), sacc[n], 0, 0, 0);
      }
    }
    if constexpr (SPLIT_S) {
      // Sum the four channel quarters in quarter order, the same order in every wave.
      sh.spart[tile][quarter][0][lane] = sacc[0];
      sh.spart[tile][quarter][1][lane] = sacc[1];
      __syncthreads();
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        f32x4 t = sh.spart[tile][0][n][lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
          const f32x4 u = sh.spart[tile][w][n][lane];
#pragma unroll
          for (int r = 0; r < 4; ++r) t[r] += u[r];
        }
        sacc[n] = t;
      }
    }
    // 3. online softmax (base-2), per head row 4g + r; FP8 rows scale their logits.
    const bool valid0 = sh.rowok[c] != 0, valid1 = sh.rowok[16 + c] != 0;
    const float rsc0 = FP8 ? sh.rowsc[c] : 1.f, rsc1 = FP8 ? sh.rowsc[16 + c] : 1.f;
    if (FP8) {
#pragma unroll
      for (int r = 0; r < 4; ++r) { sacc[0][r] *= rsc0; sacc[1][r] *= rsc1; }
    }
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
    // 8g .. 8g+7). An FP8 row's scale multiplies its weight here (the values are its codes).
    uint16_t* pw = sh.pb[wave];
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pv = FP8 ? p[n][r] * (n ? rsc1 : rsc0) : p[n][r];
        pw[(4 * g + r) * P_PITCH + 16 * n + c] = FP8 ? (uint16_t)f32_to_bf16(pv) : (uint16_t)(__float_as_uint(pv) >> 16);
      }
    __syncthreads();
    const bf16x8 pf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&pw[c * P_PITCH + 8 * g]));
    // B operand of P.V: column 16j + c of the tile, keys 8g .. 8g+7. ds_read_b64_tr_b16 gives
    // lane i of a 16-lane group element e of the group's 8-byte chunks read with stride 16,
    // so lane c addressing channels 16j + 4(c&3) .. +3 of key row 8g + (c>>2) (+4 for the
    // upper half) receives keys 8g .. 8g+3 (8g+4 .. 8g+7) of channel 16j + c.
    const uint16_t* vrow = &sh.kn[(8 * g + (c >> 2)) * KN_PITCH + 4 * (c & 3) + 16 * TPW * quarter];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_v4i16(vrow + 16 * j));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_v4i16(vrow + 4 * KN_PITCH + 16 * j));
      const v8i16 vb = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf, __builtin_bit_cast(bf16x8, vb), o[j], 0, 0, 0);
    }
  };
  for (int32_t s0 = s_begin; s0 < s_end; s0 += KC) stage(s0);
  // Partial result of this split: unnormalised O in the MFMA accumulator layout (one 16-byte
  // store per tile and lane, coalesced; quarter q holds tiles TPW q ..), running max (base 2)
  // and sum per head.
  const int64_t pslot = (int64_t)b * a.n_splits + split;
  f32x4* po = reinterpret_cast<f32x4*>(a.part_o) + (pslot * a.head_tiles * 4 + z) * (D / 16) * 64;
#pragma unroll
  for (int j = 0; j < TPW; ++j) __builtin_nontemporal_store(o[j], &po[(TPW * quarter + j) * 64 + lane]);
  if (quarter == 0 && c == 0) {
    // The lane's head group, taken again from the lane id: keeping g live to here made the
    // 1024-thread fused kernel spill it.
    const int gl = (int)(__lane_id() >> 4);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = h_base + 4 * gl + r;
      if (h < a.H) {
        a.part_ml[(pslot * a.H + h) * 2] = m_run[r];
        a.part_ml[(pslot * a.H + h) * 2 + 1] = l_run[r];
      }
    }
  }
}

template <int D, int TILES, typename Hook, bool FP8 = false, bool PAGED = false, int PF = 0>
__device__ __forceinline__ void attn_split(const AttnArgs& a, int b, int split, int z0, int tid,
                                           AttnShared<D, TILES>& sh, Hook& before_rows) {
  const SlotMap sm(a, b);
  attn_split_sm<D, TILES, Hook, FP8, PAGED, PF>(a, sm, b, split, z0, tid, sh, before_rows);
}

// LDS of one combine block that merges at most MAXS splits.
template <int MAXS>
struct CombineShared {
  float wts[16][MAXS];
  float lpart[16][MAXS];
  float lsum[16];
};

// Merges the splits of 16-head group hg of sequence b for output block bx (64 words of the
// MFMA-layout tile) with kAttnThreads threads (tid < kAttnThreads), by the log-sum-exp
// identity: out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, lse = (M + log2 L) ln 2.
// KB: partial loads a lane requests at once (its splits sq, sq + 4, ...; 4 * KB splits per
// round of loads).
template <int MAXS, int KB = 8>
__device__ __forceinline__ void combine_tile(const AttnArgs& a, float* out, float* lse, int bx, int hg, int b, int tid,
                                             CombineShared<MAXS>& sh) {
  float (&wts)[16][MAXS] = sh.wts;
  float (&lpart)[16][MAXS] = sh.lpart;
  float (&lsum)[16] = sh.lsum;
  const int D = a.D;
  const int ns = a.n_splits;
  const int sq = tid & (kCombineLanes - 1);           // this lane's quarter of the splits
  // Accumulator word index within the wave tile: (j, lane); this thread's 4 heads 4g + r.
  const int wraw = bx * (kAttnThreads / kCombineLanes) + tid / kCombineLanes;
  const int wpos = min(wraw, (D / 16) * 64 - 1);
  const int j = wpos >> 6, lane = wpos & 63, g = lane >> 4, c = lane & 15;
  const int tile = hg >> 2, wave = hg & 3;
  const f32x4* po = reinterpret_cast<const f32x4*>(a.part_o);
  const int64_t stride = (int64_t)a.head_tiles * 4 * (D / 16) * 64;   // one split, in f32x4
  const int64_t base = (((int64_t)b * ns * a.head_tiles + tile) * 4 + wave) * (D / 16) * 64 + wpos;
  // The 16 heads' (max, sum) pairs of every split come through LDS in one coalesced pass; then
  // head hl = tid / 16 is handled by the 16 lanes of one DPP row, each lane a strided subset of
  // the splits, and the head's maximum and weighted sum are row reductions. Up to 64 splits the
  // pairs (at most 4 per thread, at clamped positions so no load sits behind a branch) are
  // requested first: loads complete in order, so the weights then wait only for them while this
  // lane's partials (splits sq, sq + 4, ..., requested next) are still arriving. Before, with the
  // partials requested first, the weights waited for all of them (the 44-split merge at 4 x 1M
  // tokens 8.0 -> 7.6 us together with the exact load count in launch_combine).
  const int nh = min(16, a.H - 16 * hg);
  const int nml = ns * nh;
  constexpr int kMl = (16 * MAXS + kAttnThreads - 1) / kAttnThreads;
  constexpr bool kMlFirst = kMl <= 4;
  float2 mlv[kMlFirst ? kMl : 1];
  if constexpr (kMlFirst) {
#pragma unroll
    for (int i = 0; i < kMl; ++i) {
      const int e = min(tid + i * kAttnThreads, nml - 1);
      const int sp = e / nh, hl = e - sp * nh;
      mlv[i] = *reinterpret_cast<const float2*>(a.part_ml + (((int64_t)b * ns + sp) * a.H + 16 * hg + hl) * 2);
    }
  }
  constexpr int kBatch = KB;
  f32x4 v[kBatch];
#pragma unroll
  for (int q = 0; q < kBatch; ++q) v[q] = po[base + (int64_t)min(sq + kCombineLanes * q, ns - 1) * stride];
  if constexpr (kMlFirst) {
#pragma unroll
    for (int i = 0; i < kMl; ++i) {
      const int e = tid + i * kAttnThreads;
      if (e < nml) {
        const int sp = e / nh, hl = e - sp * nh;
        wts[hl][sp] = mlv[i].x;
        lpart[hl][sp] = mlv[i].y;
      }
    }
  } else {
    for (int e = tid; e < nml; e += kAttnThreads) {
      const int sp = e / nh, hl = e - sp * nh;
      const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + (((int64_t)b * ns + sp) * a.H + 16 * hg + hl) * 2);
      wts[hl][sp] = ml.x;
      lpart[hl][sp] = ml.y;
    }
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
      if (lse && hl < nh && bx == 0) lse[(int64_t)b * a.H + h] = (L > 0.f) ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
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

// ---- merge kernels, shared by chs_decode_attn and the fused decode step (one dispatch rule, so the
// two give the same bits)
constexpr int kFewSplits = 8;

// Exactly NS <= kFewSplits splits: one thread per accumulator word of a 16-head tile (4 heads x 1
// channel) requests its NS partials at once (a compile-time count, so no load sits behind a branch
// and waits for the one before); the tile's (max, sum) pairs come through LDS in one coalesced load
// (one per thread), so a thread is one round trip plus one barrier. Grid: (words / 256, 16-head
// tiles, sequences).
template <int NS>
__global__ __launch_bounds__(kAttnThreads) void combine_few_kernel(AttnArgs a, float* out, float* lse) {
  static_assert(NS >= 1 && NS <= kFewSplits, "splits");
  __shared__ float2 sml[NS][16];
  const int b = blockIdx.z, hg = blockIdx.y;
  const int D = a.D, H = a.H;
  constexpr int ns = NS;
  const int words = (D / 16) * 64;
  const int wpos = min((int)(blockIdx.x * kAttnThreads + threadIdx.x), words - 1);
  const int j = wpos >> 6, lane = wpos & 63, g = lane >> 4, c = lane & 15;
  const int tile = hg >> 2, quarter = hg & 3;
  const f32x4* po = reinterpret_cast<const f32x4*>(a.part_o);
  const int64_t stride = (int64_t)a.head_tiles * 4 * words;    // one split, in f32x4
  const int64_t base = (((int64_t)b * ns * a.head_tiles + tile) * 4 + quarter) * words + wpos;
  f32x4 v[NS];
#pragma unroll
  for (int sp = 0; sp < NS; ++sp) v[sp] = po[base + sp * stride];
  if ((int)threadIdx.x < ns * 16) {
    const int sp = threadIdx.x >> 4, h = min(16 * hg + (int)(threadIdx.x & 15), H - 1);
    sml[sp][threadIdx.x & 15] = *reinterpret_cast<const float2*>(a.part_ml + (((int64_t)b * ns + sp) * H + h) * 2);
  }
  __syncthreads();
  if ((int)(blockIdx.x * kAttnThreads + threadIdx.x) >= words) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float M = -INFINITY;
#pragma unroll
    for (int sp = 0; sp < NS; ++sp) M = fmaxf(M, sml[sp][4 * g + r].x);
    float L = 0.f, acc = 0.f;
#pragma unroll
    for (int sp = 0; sp < NS; ++sp) {
      const float2 ml = sml[sp][4 * g + r];
      const float wgt = (ml.x == -INFINITY) ? 0.f : exp2f(ml.x - M);
      L += wgt * ml.y;
      acc = fmaf(wgt, v[sp][r], acc);
    }
    const int h = 16 * hg + 4 * g + r;
    if (h < H) {
      out[((int64_t)b * H + h) * D + 16 * j + c] = (L > 0.f) ? acc / L : 0.f;
      if (lse && j == 0 && c == 0) lse[(int64_t)b * H + h] = (L > 0.f) ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
    }
  }
}

// More splits: a workgroup per (64 output words, 16-head tile, sequence), split weights once per
// head in LDS sized for at most MAXS splits (small LDS keeps many workgroups resident).
template <int KB, int MAXS>
__global__ __launch_bounds__(kAttnThreads) void combine_tile_kernel(AttnArgs a, float* out, float* lse) {
  __shared__ CombineShared<MAXS> sh;
  combine_tile<MAXS, KB>(a, out, lse, blockIdx.x, blockIdx.y, blockIdx.z, threadIdx.x, sh);
}

// The merge of a bf16 (MFMA-layout) split kernel's partials into out and lse.
inline void launch_combine(const AttnArgs& a, int32_t batch, int32_t n_heads, int32_t d, float* out, float* lse,
                           hipStream_t s) {
  const int words = d / 16 * 64;
  if (a.n_splits <= kFewSplits) {
    const dim3 grid((unsigned)((words + kAttnThreads - 1) / kAttnThreads), (unsigned)((n_heads + 15) / 16),
                    (unsigned)batch);
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(kAttnThreads), 0, s, a, out, lse); };
    switch (a.n_splits) {
      case 1: go(combine_few_kernel<1>); break;
      case 2: go(combine_few_kernel<2>); break;
      case 3: go(combine_few_kernel<3>); break;
      case 4: go(combine_few_kernel<4>); break;
      case 5: go(combine_few_kernel<5>); break;
      case 6: go(combine_few_kernel<6>); break;
      case 7: go(combine_few_kernel<7>); break;
      default: go(combine_few_kernel<8>); break;
    }
    return;
  }
  const int words_per_block = kAttnThreads / kCombineLanes;
  const dim3 grid((unsigned)((words + words_per_block - 1) / words_per_block), (unsigned)((n_heads + 15) / 16),
                  (unsigned)batch);
  // Each lane requests KB partials at once; up to 64 splits KB is the smallest listed count that
  // covers the splits (20 -> 5, 44 -> 11), since a load past the last split repeats it and costs
  // address-unit time (KB = 16 at 44 splits requested 45% more than needed).
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(kAttnThreads), 0, s, a, out, lse); };
  const int per_lane = (a.n_splits + kCombineLanes - 1) / kCombineLanes;
  if (per_lane <= 3) go(combine_tile_kernel<3, 64>);
  else if (per_lane <= 4) go(combine_tile_kernel<4, 64>);
  else if (per_lane <= 5) go(combine_tile_kernel<5, 64>);
  else if (per_lane <= 6) go(combine_tile_kernel<6, 64>);
  else if (per_lane <= 8) go(combine_tile_kernel<8, 64>);
  else if (per_lane <= 11) go(combine_tile_kernel<11, 64>);
  else if (per_lane <= 12) go(combine_tile_kernel<12, 64>);
  else if (per_lane <= 16) go(combine_tile_kernel<16, 64>);
  else go(combine_tile_kernel<16, kCombineSplits>);
}

// Host checks of chs_decode_attn's arguments (all but the workspace).
inline chs_status check_args(chs_dtype dtype, int32_t batch, int32_t n_heads, int32_t d, int32_t window, int32_t k,
                             float scale, const void* q, const void* swa_kv, const int32_t* swa_len,
                             const void* comp_kv, const int64_t* cu_comp, const int32_t* topk, int64_t max_comp,
                             const float* out) {
  if (!dtype_ok(dtype)) return CHS_ERR_DTYPE;
  if (batch < 1 || batch > 65535 || n_heads < 1 || n_heads > 128 || window < 0 || window > 4096 ||
      k < 0 || k > 2048 || max_comp < 0 || max_comp >= (1LL << 31) || !(scale > 0.f) || !(scale < INFINITY))
    return CHS_ERR_SHAPE;
  if (dtype == CHS_BF16) {
    if (d != 64 && d != 128 && d != 256 && d != 512) return CHS_ERR_SHAPE;
  } else if (d < 1 || d > 1024 || d % 4 != 0) {
    return CHS_ERR_SHAPE;
  }
  if (!q || !swa_len || !cu_comp || !out) return CHS_ERR_NULL;
  if (window > 0 && !swa_kv) return CHS_ERR_NULL;
  if (!comp_kv && (topk ? k > 0 : max_comp > 0)) return CHS_ERR_NULL;
  return CHS_OK;
}

struct SplitPlan {
  int32_t n_splits, kps;
  bool wide;
};

constexpr int kDenseThreads = 1024;   // dense split workgroup: 16 waves, four 16-head tiles
constexpr int kSparseBlocks = 1024;   // selected (C4) and fp32 split workgroups aimed at per call
// Dense split workgroups aimed at per call, fewer than the CUs: each split writes 128 KiB of fp32 partials
// per 64 heads, which the merge reads back. 192 against 256 (graph replays, the two builds interleaved):
// 64 sequences of ~1,570 keys 42.0-42.3 against 42.4-43.3 us (3 splits instead of 4), 8 sequences of 6,000
// keys 27.1-27.5 against 29.0-29.2 us, 16 of 4,096 keys 32.3-32.4 against 32.4-33.3 us; 32 sequences of
// 3,000 keys 39.0-39.4 against 38.6-39.1 us (6 splits instead of 8); 4 sequences the same plan.
constexpr int kDenseBlocks = 192;
constexpr int kWideSparseBlocks = 256;        // selected attention goes wide past this many 16-head workgroups
// Selected (C4) splits of the 64-head kernel aimed at per call: at 64 sequences of 200K tokens (640
// slots each) 192 gives 3 splits of 256 slots: step 186.9 us, against 188.6 (256), 188.2 (128) and 196 (384).
constexpr int kWideTopkBlocks = 192;
constexpr int kWideMaxSelected = 2048;        // most selected entries one wide split stages in LDS

// Dense bf16 (or FP8) attention over many heads (every compressed entry, no top-k) uses one
// workgroup per 64 heads, so each gathered row is read from HBM once, and streams the
// split's chunks with rows requested ahead (PF). Selected (C4) attention keeps one workgroup per 16 heads and
// one chunk per split: it is latency bound, and more workgroups start sooner.
inline bool dense_split(chs_dtype dt, int32_t k, int32_t H) { return dt == CHS_BF16 && k == 0 && H > 48; }

// kps (a multiple of gran) and the split count for about `target` workgroups of blocks_per_split
// each, at most kCombineSplits splits.
inline SplitPlan plan_for(int64_t max_slots, int64_t blocks_per_split, int64_t target, int gran) {
  int64_t want = (target + blocks_per_split - 1) / blocks_per_split;
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
  p.wide = false;
  return p;
}

// The split plan of one call, shared by the workspace queries and the launches (the same plan gives
// the same bits). wide: the 64-head d = 512 kernel (attn_dense512_kernel) runs the splits:
//   - dense bf16 with more than 48 heads at d = 512 always; its 64-key chunks set the granularity,
//     and it aims at kDenseBlocks workgroups;
//   - selected (C4) bf16 attention with more than 48 heads at d = 512 once its 16-head workgroups
//     would outnumber the CUs (many sequences): each split's rows are then read once for 64 heads
//     instead of once per 16-head tile; it aims at kWideTopkBlocks workgroups.
// Otherwise bf16 runs one workgroup per 16-head tile over 32-key chunks, aiming at kSparseBlocks (at
// 64 sequences of a C4 layer 1024 measured better than 512 and 2048; at batch 1 the chunk count caps
// the splits first), and fp32 one per head over 256-key chunks. FP8 calls take the bf16 plan.
inline SplitPlan plan_splits(chs_dtype dt, int32_t batch, int32_t H, int32_t d, int32_t window, int32_t k,
                             int64_t max_comp) {
  const int64_t max_slots = (int64_t)window + (k > 0 ? k : max_comp);
  const int64_t tiles16 = (H + 15) / 16, tiles64 = (H + 63) / 64;
  if (dense_split(dt, k, H)) {
    SplitPlan p = plan_for(max_slots, (int64_t)batch * tiles64, kDenseBlocks, 64);
    p.wide = d == 512;
    return p;
  }
  if (dt != CHS_BF16) return plan_for(max_slots, (int64_t)batch * H, kSparseBlocks, kAttnThreads);
  const SplitPlan narrow = plan_for(max_slots, (int64_t)batch * tiles16, kSparseBlocks, kKeysPerChunk);
  if (d == 512 && H > 48 && (int64_t)narrow.n_splits * batch * tiles16 > kWideSparseBlocks) {
    SplitPlan p = plan_for(max_slots, (int64_t)batch * tiles64, kWideTopkBlocks, 64);
    if (p.kps <= kWideMaxSelected) {
      p.wide = true;
      return p;
    }
  }
  return narrow;
}

inline size_t ws_bytes(chs_dtype dt, int32_t batch, int32_t H, int32_t D, const SplitPlan& p, float** po, float** pml,
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
}  // namespace attn
}  // namespace chs
