/* chs.h - C ABI of libchs.so: one decode step of one hybrid-sparse-attention layer on MI355X
 * (gfx950), as hand-written HIP kernels.
 *
 * The method (web pages, cited by title and section):
 *  - "DeepSeek-V4 本地部署，SGLang 把活做絕了", section V4 到底改了啥: every attention layer
 *    combines a 128-token sliding window (SWA) with one of two compressions: C4 pools groups
 *    of 4 tokens and attends to the top-512 of them; C128 pools groups of 128 tokens and
 *    attends to all of them.
 *  - same page, section Kernel 層一堆狠活: the window and the compressed ("extra") entries
 *    are attended in one kernel call (FlashMLA's new interface); the compressor is one fused
 *    pass (Flash Compressor); top-512 of 256K candidates is chosen by a radix select rather
 *    than a global sort (Lightning TopK).
 *  - "SGLang 如何为 DeepSeek V4 打造「Day-0」推理加速", section 创新 2: the compressor's stages
 *    (load tokens, score, softmax, weighted sum, store) fused into one on-chip pass; the top-k
 *    threshold is found from per-block radix histograms, and the compressor's output feeds the
 *    top-k with no copy. Section 创新 3: each C4 step touches about 0.2% of the entries, each
 *    C128 step reads all of them.
 * The pages print no formulas. This library computes the following readings of them:
 *  - compressor: for every complete group of m tokens and every channel c, a softmax over the
 *    group's gate logits plus a learned per-slot, per-channel bias B[i, c], then the weighted
 *    sum of the group's token vectors; a trailing partial group is left to the window;
 *  - indexer score: s_j = sum_h w_h * ReLU(q_h . k_j);
 *  - top-k: the k largest scores, ties to the lower index, returned as an ascending index set;
 *  - attention: one softmax over the window rows and the selected (C4) or all (C128) compressed
 *    entries; keys double as values (a shared latent), logits scaled by `scale` (1/sqrt(d)).
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers owned by the caller, except where marked (host).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Calls are asynchronous
 *    on it; they never synchronize, allocate, free or retain memory. Buffers must stay alive
 *    until the stream has drained the call.
 *  - Arguments passed by value are validated on the host before anything is launched; on
 *    failure the call returns the error and launches nothing. Device-side arrays (cu_*, swa_len,
 *    topk) are preconditions the host cannot see; out-of-range values there are clamped or
 *    skipped as each call documents, never used to address memory outside the stated buffers.
 *  - A failed launch returns CHS_ERR_LAUNCH. Faults inside a kernel surface, as usual for HIP,
 *    at the caller's next synchronization.
 *  - Workspaces are scratch memory the caller owns, sized by the matching *_workspace_size
 *    query. They need no initialisation and hold nothing between calls; calls that run
 *    concurrently must use distinct workspaces. No global mutable state exists.
 *  - dtype CHS_BF16 means bfloat16 storage with fp32 arithmetic; CHS_F32 means fp32 throughout.
 */
#ifndef CHS_H
#define CHS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CHS_OK = 0,
  CHS_ERR_NULL = 1,         /* a required pointer is NULL */
  CHS_ERR_SHAPE = 2,        /* a size argument is outside its documented range */
  CHS_ERR_DTYPE = 3,        /* unknown dtype code */
  CHS_ERR_WORKSPACE = 4,    /* workspace smaller than the size query returned */
  CHS_ERR_UNSUPPORTED = 5,  /* valid arguments this build has no kernel for */
  CHS_ERR_LAUNCH = 6,       /* a kernel launch failed */
  /* Range markers, never returned: with them every int32 value is a valid chs_status in C++ (whose
     enums otherwise only hold the values their enumerators span), so chs_status_string may be
     given any code. */
  CHS_STATUS_MIN_ = -0x7fffffff - 1,
  CHS_STATUS_MAX_ = 0x7fffffff
} chs_status;

/* The storage type of a call's tensors. Unknown codes are rejected with CHS_ERR_DTYPE; the range
   markers make every int32 value a valid chs_dtype in C++, so that check is defined behaviour. */
typedef enum {
  CHS_F32 = 0,
  CHS_BF16 = 1,
  CHS_DTYPE_MIN_ = -0x7fffffff - 1,
  CHS_DTYPE_MAX_ = 0x7fffffff
} chs_dtype;

/* Library version: major*10000 + minor*100 + patch. */
int32_t chs_version(void);

/* Human-readable name of a status code (static storage). */
const char* chs_status_string(chs_status s);

/* Zero-fill `bytes` bytes of device memory on `stream` with a kernel (no hipMemsetAsync, so it
 * can be captured in a HIP graph). bytes must be a multiple of 4. Not needed by the calls below;
 * a convenience for callers that want deterministic scratch contents. */
chs_status chs_workspace_clear(void* workspace, size_t bytes, void* stream);

/* ---- chs_compress: the fused group softmax-pool (Flash Compressor's role) ----------------
 * Source: "SGLang 如何为 DeepSeek V4 打造「Day-0」推理加速", 创新 2 (five stages fused into one
 * pass); "DeepSeek-V4 本地部署，SGLang 把活做絕了", V4 到底改了啥 (C4: m = 4, C128: m = 128).
 * For sequence b (tokens cu_tokens[b] .. cu_tokens[b+1]-1, N_b of them), every group
 * g < G_b = floor(N_b / m) and channel c < d:
 *   a_i = gate[t, c] + bias[i, c],  t = cu_tokens[b] + g*m + i  (i < m)
 *   out[cu_groups[b] + g, c] = sum_i softmax_i(a)[i] * x[t, c]
 * x, gate : [T, d] of `dtype`, row-major (T = cu_tokens[batch]).
 * bias    : [m, d] fp32.
 * cu_tokens, cu_groups : [batch + 1] int64, non-decreasing, element 0 = 0. cu_groups gives the
 *   first output row of each sequence; at most cu_groups[b+1] - cu_groups[b] rows are written
 *   for sequence b (so a packed layout is cu_groups = prefix sums of floor(N_b / m)).
 * max_groups (host): an upper bound on max_b G_b; it sizes the grid, and groups at or beyond
 *   it are not computed. 0 launches nothing.
 * out     : [cu_groups[batch], d] of `dtype` (fp32 arithmetic, rounded to nearest-even once).
 * Ranges: 1 <= batch <= 65535; 1 <= m <= 1024; 1 <= d <= 4096 with d*elem_size % 16 == 0. */
chs_status chs_compress(chs_dtype dtype, int32_t batch, int32_t d, int32_t m, const void* x,
                        const void* gate, const float* bias, const int64_t* cu_tokens,
                        const int64_t* cu_groups, int64_t max_groups, void* out, void* stream);

/* ---- FP8 (E4M3) writers: chs_quantize_e4m3, chs_compress_fp8, chs_append_fp8 ---------------------
 * Source: "DeepSeek-V4 本地部署，SGLang 把活做絕了", V4 到底改了啥 (the checkpoints keep attention in
 * FP8) and "SGLang 如何为 DeepSeek V4 打造「Day-0」推理加速", 4.3 部署配置建议 (an fp8 KV cache). The
 * pages fix neither the FP8 variant, the rounding nor a scale layout. Reading taken (the same one the
 * FP8 readers chs_index_topk_fp8 and chs_decode_attn_fp8 take): OCP 8-bit E4M3 codes with one fp32
 * scale per row, written as
 *   amax = max_c |v_c|,  scale = amax / 448,  inv = min(448 / amax, FLT_MAX),  code_c = E4M3(v_c * inv)
 * with every operation rounded once to fp32, E4M3() the nearest E4M3 value with ties to the even
 * code and magnitudes from 448 up saturating to 448 (no NaN is written); a row of zeros gets scale 0
 * and codes 0x00. The row then decodes as scale * decode(code), its largest element to +-448 * scale.
 *
 * chs_quantize_e4m3: rows the caller holds (the window after a prefill, index keys made elsewhere).
 * in: [n_rows, d] of `dtype` (16-byte aligned); codes: [n_rows, d] bytes (8-byte aligned); scales:
 * [n_rows] fp32. 0 <= n_rows <= 2^40; 8 <= d <= 4096, d % 8 == 0. n_rows = 0 launches nothing. */
chs_status chs_quantize_e4m3(chs_dtype dtype, int64_t n_rows, int32_t d, const void* in, uint8_t* codes,
                             float* scales, void* stream);

/* chs_compress_fp8: chs_compress with E4M3 output, in the same single pass: every pooled entry row
 * (the fp32 values chs_compress would round to its storage type) is quantised as above and written as
 * out_codes[cu_groups[b] + g, :] ([cu_groups[batch], d] bytes) and out_scales[cu_groups[b] + g]
 * ([cu_groups[batch]] fp32). Other arguments and ranges as chs_compress; in addition the row must be
 * at most 64 16-byte chunks, a power of two of them (bf16: d in {8, 16, ..., 512}; fp32: d in
 * {4, ..., 256}), else CHS_ERR_UNSUPPORTED. */
chs_status chs_compress_fp8(chs_dtype dtype, int32_t batch, int32_t d, int32_t m, const void* x,
                            const void* gate, const float* bias, const int64_t* cu_tokens,
                            const int64_t* cu_groups, int64_t max_groups, uint8_t* out_codes,
                            float* out_scales, void* stream);

/* chs_append_fp8: chs_append over an FP8 cache. For every sequence b, with t = n_tokens[b] before the
 * call (a negative count reads as 0) and page = ring_page[b]:
 *   swa_codes[b, t mod window, :], swa_scale[b, t mod window] = the quantised x_new[b, :];
 *   x_ring[page * ring_size + t mod ring_size, :] = x_new[b, :];  gate_ring[same row, :] = z_new[b, :];
 *   if (t + 1) mod m == 0, the group g = t / m (tokens t+1-m .. t) is pooled as chs_compress pools it,
 *   its token rows and gates read from x_ring and gate_ring (which must hold what earlier appends, or
 *   the caller after a prefill, wrote there), then quantised into comp_codes[comp_start[b] + g, :] and
 *   comp_scale[comp_start[b] + g];
 *   n_tokens, swa_len, comp_count as chs_append.
 * The window holds quantised rows, so the group's rows come from the state ring, which keeps them
 * in the storage type beside the gates. For m in {1, 2, 4, 8} the entries (codes and scales) are
 * bit-identical to chs_compress_fp8's over the same history; the window codes are bit-identical to
 * chs_quantize_e4m3 of the token rows.
 * x_new, z_new: [batch, d] of `dtype`; bias: [m, d] fp32; n_tokens: [batch] int64 (in/out);
 * swa_codes: [batch, window, d] bytes; swa_scale: [batch, window] fp32; swa_len: [batch] int32 or NULL;
 * x_ring, gate_ring: [ring_pages * ring_size, d] of `dtype`; ring_page: [batch] int32 (a page outside
 * [0, ring_pages) skips that sequence's ring writes and group); comp_codes: [comp_rows, d] bytes;
 * comp_scale: [comp_rows] fp32; comp_start: [batch] int64 (a group whose row falls outside
 * [0, comp_rows) is not written); comp_count: [batch] int64 or NULL.
 * Ranges as chs_append, plus the row limit of chs_compress_fp8 (else CHS_ERR_UNSUPPORTED). */
chs_status chs_append_fp8(chs_dtype dtype, int32_t batch, int32_t d, int32_t m, int32_t window,
                          int32_t ring_size, const void* x_new, const void* z_new, const float* bias,
                          int64_t* n_tokens, uint8_t* swa_codes, float* swa_scale, int32_t* swa_len,
                          void* x_ring, void* gate_ring, const int32_t* ring_page, int64_t ring_pages,
                          uint8_t* comp_codes, float* comp_scale, const int64_t* comp_start,
                          int64_t comp_rows, int64_t* comp_count, void* stream);

/* ---- chs_append: one decode-time token per sequence into the window and the state ring ----
 * Source: "DeepSeek-V4 本地部署，SGLang 把活做絕了", ShadowRadix (a compression state ring per
 * layer, nested in the sequence's SWA page at page * ring_size + position mod ring_size; 8 slots
 * for C4, 128 for C128, doubled for speculative decoding) and V4 到底改了啥 (128-token window;
 * C4 and C128 groups). The pooling is chs_compress's.
 * For every sequence b, with t = n_tokens[b] tokens before the call (a negative count reads as 0):
 *   swa_kv[b, t mod window, :]                  = x_new[b, :]
 *   gate_ring[ring_page[b]*ring_size + t mod ring_size, :] = z_new[b, :]
 *   if (t + 1) mod m == 0, the group g = t / m (tokens t+1-m .. t) is pooled as chs_compress pools
 *   it and written to comp_kv[comp_start[b] + g, :]; its earlier token rows are read from
 *   swa_kv (slot position mod window) and its gates from gate_ring, which therefore must hold
 *   what earlier appends (or the caller, after a prefill) wrote there;
 *   n_tokens[b] = t + 1;  swa_len[b] = min(t + 1, window);  comp_count[b] = floor((t + 1) / m).
 * The window is a ring: after the call its rows [0, swa_len[b]) are exactly the last
 * min(t + 1, window) tokens, in slot order rather than token order, which chs_decode_attn accepts
 * (one softmax over a set). For m <= 8 the new entry is bit-identical to chs_compress's.
 * x_new, z_new : [batch, d] of `dtype`: the new token's row (its KV latent) and gate logits.
 * bias         : [m, d] fp32, as for chs_compress.
 * n_tokens     : [batch] int64, read and advanced in place.
 * swa_kv       : [batch, window, d] of `dtype` (the layout chs_decode_attn reads).
 * swa_len      : [batch] int32 output, or NULL.
 * gate_ring    : [ring_pages * ring_size, d] of `dtype`; ring_page: [batch] int32. A page outside
 *                [0, ring_pages) makes the call skip that sequence's gate write and group.
 * comp_kv      : [comp_rows, d] of `dtype`; comp_start: [batch] int64, the row of each sequence's
 *                group 0. A group whose row falls outside [0, comp_rows) is not written.
 * comp_count   : [batch] int64 output, or NULL. For one sequence stored from row 0, pointing it
 *                at cu_comp + 1 keeps the cu arrays of chs_index_topk / chs_decode_attn current.
 * Row pointers must be 16-byte aligned. Sequences must be distinct entries (one token each);
 * n_tokens must not alias swa_len or comp_count.
 * Ranges: 1 <= batch <= 65535; 1 <= m <= 1024; m <= window <= 2^20; m <= ring_size <= 2^20;
 * ring_pages >= 1; comp_rows >= 0; 1 <= d <= 4096 with d*elem_size % 16 == 0. */
chs_status chs_append(chs_dtype dtype, int32_t batch, int32_t d, int32_t m, int32_t window,
                      int32_t ring_size, const void* x_new, const void* z_new, const float* bias,
                      int64_t* n_tokens, void* swa_kv, int32_t* swa_len, void* gate_ring,
                      const int32_t* ring_page, int64_t ring_pages, void* comp_kv,
                      const int64_t* comp_start, int64_t comp_rows, int64_t* comp_count,
                      void* stream);

/* ---- chs_append_multi: chs_append for several compressor streams in one launch --------------
 * The layer appends each new token to more than one compressed stream: the KV latent's and the
 * indexer's own ("SGLang 如何为 DeepSeek V4 打造「Day-0」推理加速", 创新 5: the compressor and the
 * indexer among the per-step preparation operators). Each stream is described by one
 * chs_append_stream and gets exactly what chs_append (page_table == NULL) or chs_append_paged
 * (page_table != NULL) would do for it; one launch covers them all. The streams share dtype, batch
 * and m; each has its own rows, rings, pools and counters, which must not overlap between streams.
 * 1 <= n_streams <= 4; `streams` is a host array, read during the call only. */
typedef struct {
  int32_t d, window, ring_size;
  const void* x_new;            /* [batch, d] */
  const void* z_new;            /* [batch, d] */
  const float* bias;            /* [m, d] */
  int64_t* n_tokens;            /* [batch], advanced in place */
  void* swa_kv;                 /* contiguous: [batch, window, d]; paged: the window pool */
  int32_t* swa_len;             /* [batch] or NULL */
  void* gate_ring;              /* the gate rings (pages of ring_size rows) */
  const int32_t* ring_page;     /* contiguous: [batch] */
  int64_t ring_pages;           /* contiguous: pages in gate_ring */
  void* comp_kv;                /* the compressed entries (pool) */
  const int64_t* comp_start;    /* contiguous: [batch] */
  int64_t comp_rows;            /* contiguous: rows of comp_kv */
  int64_t* comp_count;          /* [batch] or NULL */
  const int32_t* swa_page;      /* paged: [batch] window page (also the gate ring's page) */
  int64_t swa_pages;            /* paged: pages of the window pool */
  const int32_t* page_table;    /* paged: [batch, pt_stride]; NULL selects the contiguous form */
  int32_t pt_stride, page_size; /* paged */
  int64_t pool_pages;           /* paged: pages of comp_kv */
} chs_append_stream;

chs_status chs_append_multi(chs_dtype dtype, int32_t batch, int32_t m, int32_t n_streams,
                            const chs_append_stream* streams, void* stream);

/* ---- chs_index_topk: indexer scores, then exact top-k by radix select ------------------
 * Source: "SGLang 如何为 DeepSeek V4 打造「Day-0」推理加速", 创新 2 (Lightning TopK: per-block
 * radix histograms, a threshold, then each block scatters its entries above it; no global
 * sort) and 创新 5 (the indexer scores the candidates, then the top-k selects).
 * Sequence b's candidates are rows cu_cand[b] .. cu_cand[b+1]-1 (G_b of them). Scores:
 *   scores[cu_cand[b] + j] = sum_h w[b, h] * max(0, sum_t q_idx[b, h, t] * k_idx[cu_cand[b] + j, t])
 * computed in fp32, then topk[b, :] = the min(k, G_b) largest scores of the sequence (ties to
 * the lower index; -0.0 equals +0.0), as sequence-local indices in ascending order, padded
 * with -1 to length k. The selection is exact: given the same score array it is bit-identical
 * to a full sort.
 * q_idx   : [batch, n_heads, head_dim] of `dtype`, or NULL: then `scores` is an INPUT holding
 *           the scores (fp32) and w, k_idx are ignored (standalone top-k). NaN scores are
 *           outside the contract (the output is then some valid index set, unspecified).
 * w       : [batch, n_heads] fp32.
 * k_idx   : [cu_cand[batch], head_dim] of `dtype`.
 * cu_cand : [batch + 1] int64, non-decreasing, element 0 = 0.
 * max_cand (host): an upper bound on max_b G_b (sizes the grid; candidates beyond it are
 *           ignored).
 * scores  : [cu_cand[batch]] fp32. OUTPUT when q_idx != NULL (may then be NULL: the workspace
 *           holds them), INPUT when q_idx == NULL.
 * topk    : [batch, k] int32 output.
 * workspace: chs_index_topk_workspace_size(batch, max_cand, k) bytes.
 * Ranges: 1 <= batch <= 65535; 1 <= k <= 2048; 0 <= max_cand <= 4194304 (CHS_ERR_UNSUPPORTED
 *   above); with q_idx:
 *   1 <= n_heads <= 16, head_dim >= 8, head_dim*elem_size % 16 == 0 and <= 1024 bytes
 *   (bf16 up to 512, fp32 up to 256). */
size_t chs_index_topk_workspace_size(int32_t batch, int64_t max_cand, int32_t k);
chs_status chs_index_topk(chs_dtype dtype, int32_t batch, int32_t n_heads, int32_t head_dim,
                          int32_t k, const void* q_idx, const float* w, const void* k_idx,
                          const int64_t* cu_cand, int64_t max_cand, float* scores, int32_t* topk,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ---- chs_index_scores: the indexer scores alone ---------------------------------------------
 * Source: "SGLang 如何为 DeepSeek V4 打造「Day-0」推理加速", 创新 5 (the indexer scores every compressed
 * candidate ahead of the top-k). Computes exactly the scores chs_index_topk computes (the same kernel,
 * bit-identical values) and no selection:
 *   scores[cu_cand[b] + j] = sum_h w[b, h] * max(0, sum_t q_idx[b, h, t] * k_idx[cu_cand[b] + j, t]).
 * q_idx, w, k_idx, cu_cand, max_cand: as chs_index_topk (q_idx must not be NULL).
 * scores  : [cu_cand[batch]] fp32 output (not NULL).
 * workspace: chs_index_topk_workspace_size(batch, max_cand, 1) bytes (the kernel also leaves its
 *   per-group statistics there). Ranges and errors as chs_index_topk with q_idx given. */
chs_status chs_index_scores(chs_dtype dtype, int32_t batch, int32_t n_heads, int32_t head_dim,
                            const void* q_idx, const float* w, const void* k_idx, const int64_t* cu_cand,
                            int64_t max_cand, float* scores, void* workspace, size_t workspace_bytes,
                            void* stream);

/* ---- chs_index_topk_fp8: chs_index_topk with FP8 index keys --------------------------------
 * Source: "DeepSeek-V4 本地部署，SGLang 把活做絕了", V4 到底改了啥 (the checkpoints keep
 * attention in FP8) and "SGLang 如何为 DeepSeek V4 打造「Day-0」推理加速", 4.3 部署配置建议 (an
 * fp8 KV cache). The pages fix neither the FP8 variant nor a scale layout; this call takes the
 * OCP 8-bit E4M3 format (bias 7, exponent 0 subnormal, S.1111.111 NaN, no infinities) with one
 * fp32 scale per key row:
 *   key row j = k_scale[j] * decode(k_idx[j, :]),
 *   scores[cu_cand[b] + j] = sum_h w[b, h] * max(0, sum_t q_idx[b, h, t] * key[cu_cand[b] + j, t])
 * computed in fp32 (the FP8 values enter the products exactly), then the top-k exactly as
 * chs_index_topk selects it.
 * q_idx   : [batch, n_heads, head_dim] bf16.
 * k_idx   : [cu_cand[batch], head_dim] bytes, E4M3 codes.
 * k_scale : [cu_cand[batch]] fp32, each >= 0 and finite.
 * Other arguments as chs_index_topk (scores is an OUTPUT here, or NULL); the workspace is
 * chs_index_topk_workspace_size(batch, max_cand, k) bytes.
 * Ranges: 1 <= batch <= 65535; 1 <= k <= 2048; 0 <= max_cand <= 4194304; 1 <= n_heads <= 16;
 *   16 <= head_dim <= 512, head_dim % 16 == 0. NaN codes are outside the contract. */
chs_status chs_index_topk_fp8(int32_t batch, int32_t n_heads, int32_t head_dim, int32_t k,
                              const void* q_idx, const float* w, const void* k_idx,
                              const float* k_scale, const int64_t* cu_cand, int64_t max_cand,
                              float* scores, int32_t* topk, void* workspace, size_t workspace_bytes,
                              void* stream);

/* ---- chs_decode_attn: one softmax over the window and the compressed entries ------------
 * Source: "DeepSeek-V4 本地部署，SGLang 把活做絕了", Kernel 層一堆狠活 (window and extra
 * C4/C128 attention in one call) and V4 到底改了啥 (SWA = 128; C4 top-512; C128 dense);
 * "SGLang 如何为 DeepSeek V4 打造「Day-0」推理加速", 3.2 (MLA decode over a shared latent is
 * memory-bound; heads need no caller padding here: unused MFMA rows are masked in-kernel).
 * For sequence b and head h, over the key multiset
 *   K_b = { swa_kv[b, t] : t < swa_len[b] }  (+)  { comp_kv[cu_comp[b] + j] : j in S_b }
 * where S_b = { topk[b, i] : i < k, 0 <= topk[b, i] < G_b } (C4; out-of-range entries, -1
 * included, are skipped; repeats count twice) or S_b = { 0 .. G_b - 1 } when topk == NULL
 * (C128), G_b = cu_comp[b+1] - cu_comp[b]:
 *   l_i = scale * (q[b, h] . k_i),   lse[b, h] = log sum_i exp(l_i),
 *   out[b, h, :] = sum_i exp(l_i - lse[b, h]) * k_i          (keys are also the values)
 * An empty key set gives out = 0 and lse = -inf.
 * q       : [batch, n_heads, d] of `dtype`.
 * swa_kv  : [batch, window, d] of `dtype`: the window's rows (the last min(N_b, window) tokens,
 *           current token included), any order. swa_len: [batch] int32, clamped to [0, window].
 * comp_kv : [cu_comp[batch], d] of `dtype`; cu_comp: [batch + 1] int64 (element 0 = 0).
 * topk    : [batch, k] int32 (as chs_index_topk writes it) or NULL for the dense form.
 * max_comp (host): an upper bound on max_b G_b (sizes the grid for the dense form).
 * out     : [batch, n_heads, d] fp32;  lse: [batch, n_heads] fp32, or NULL.
 * workspace: chs_decode_attn_workspace_size(...) bytes with the same window, k (0 for dense),
 *           max_comp, batch, n_heads and d.
 * Ranges: 1 <= batch <= 65535; 1 <= n_heads <= 128; 0 <= window <= 4096; 0 <= k <= 2048;
 *   scale finite and > 0; bf16: d in {64, 128, 256, 512}; f32: 1 <= d <= 1024, d % 4 == 0. */
size_t chs_decode_attn_workspace_size(chs_dtype dtype, int32_t batch, int32_t n_heads, int32_t d,
                                      int32_t window, int32_t k, int64_t max_comp);
chs_status chs_decode_attn(chs_dtype dtype, int32_t batch, int32_t n_heads, int32_t d,
                           int32_t window, int32_t k, float scale, const void* q,
                           const void* swa_kv, const int32_t* swa_len, const void* comp_kv,
                           const int64_t* cu_comp, const int32_t* topk, int64_t max_comp,
                           float* out, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream);

/* ---- chs_decode_step: the C4 decode step (index scores, top-k, attention) in one call --------
 * Source: "DeepSeek-V4 本地部署，SGLang 把活做絕了", Kernel 層一堆狠活 (the indexer's top-512
 * feeds the attention over the window and the selected C4 entries) and "SGLang 如何为 DeepSeek
 * V4 打造「Day-0」推理加速", 创新 2 (the selected set goes to the attention with no copy).
 * Computes exactly chs_index_topk(CHS_BF16, batch, idx_heads, idx_dim, k, q_idx, w, k_idx,
 * cu_comp, max_comp, scores, topk, ...) followed by chs_decode_attn(CHS_BF16, batch, n_heads, d,
 * window, k, scale, q, swa_kv, swa_len, comp_kv, cu_comp, topk, max_comp, out, lse, ...): the
 * candidates are the compressed entries (cu_comp), and scores, topk, out and lse are
 * bit-identical to those two calls. The selection's second kernel runs inside the attention's
 * split kernel, so the step takes three launches instead of four.
 * Argument meanings, layouts and ranges are those of the two calls (bf16 storage only;
 * q_idx must not be NULL; scores may be NULL); topk [batch, k] is an output.
 * workspace: chs_decode_step_workspace_size(batch, n_heads, d, window, k, max_comp) bytes. */
size_t chs_decode_step_workspace_size(int32_t batch, int32_t n_heads, int32_t d, int32_t window, int32_t k,
                                      int64_t max_comp);
chs_status chs_decode_step(int32_t batch, int32_t n_heads, int32_t d, int32_t window, int32_t k, float scale,
                           int32_t idx_heads, int32_t idx_dim, const void* q_idx, const float* w,
                           const void* k_idx, const void* q, const void* swa_kv, const int32_t* swa_len,
                           const void* comp_kv, const int64_t* cu_comp, int64_t max_comp, float* scores,
                           int32_t* topk, float* out, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream);

/* ---- chs_decode_step_fp8: the C4 decode step over FP8 storage in one call ------------------------
 * Source: as chs_decode_step, with "SGLang 如何为 DeepSeek V4 打造「Day-0」推理加速", 4.3 部署配置建议
 * (an fp8 KV cache) and "DeepSeek-V4 本地部署，SGLang 把活做絕了", V4 到底改了啥 (attention kept in
 * FP8), in the reading of chs_index_topk_fp8 and chs_decode_attn_fp8 (OCP E4M3 codes, one fp32
 * scale per row).
 * Computes exactly chs_index_topk_fp8(batch, idx_heads, idx_dim, k, q_idx, w, k_codes, k_scale,
 * cu_comp, max_comp, scores, topk, ...) followed by chs_decode_attn_fp8(batch, n_heads, d, window, k,
 * scale, q, swa_codes, swa_scale, swa_len, comp_codes, comp_scale, cu_comp, topk, max_comp, out, lse,
 * ...): scores, topk, out and lse are bit-identical to those two calls, in three launches instead
 * of four (the selection's second kernel runs inside the attention's split kernel).
 * k_codes  : [cu_comp[batch], idx_dim] E4M3 codes; k_scale: [cu_comp[batch]] fp32 (>= 0, finite).
 * swa_codes: [batch, window, d] E4M3; swa_scale: [batch, window] fp32 (may be NULL when window = 0).
 * comp_codes: [cu_comp[batch], d] E4M3; comp_scale: [cu_comp[batch]] fp32.
 * q_idx, w, q, swa_len, cu_comp, scores, topk, out, lse and the ranges: as chs_decode_step (idx_dim
 * a multiple of 16 in [16, 512]). A NULL scale array returns CHS_ERR_NULL before any launch.
 * workspace: chs_decode_step_workspace_size(batch, n_heads, d, window, k, max_comp) bytes. */
chs_status chs_decode_step_fp8(int32_t batch, int32_t n_heads, int32_t d, int32_t window, int32_t k, float scale,
                               int32_t idx_heads, int32_t idx_dim, const void* q_idx, const float* w,
                               const void* k_codes, const float* k_scale, const void* q, const void* swa_codes,
                               const float* swa_scale, const int32_t* swa_len, const void* comp_codes,
                               const float* comp_scale, const int64_t* cu_comp, int64_t max_comp, float* scores,
                               int32_t* topk, float* out, float* lse, void* workspace, size_t workspace_bytes,
                               void* stream);

/* ---- chs_decode_step_noalloc: chs_decode_step for callers that cannot allocate ------------------
 * For callers that cannot call hipMalloc or pass a workspace: code under HIP graph capture that must
 * not allocate, tight serving loops, harnesses that forbid allocation. Computes exactly what
 * chs_decode_step computes (the same kernels; scores, topk, out and lse bit-identical), with the
 * workspace taken from a scratch array inside the library instead of the caller: one array of
 * CHS_NOALLOC_SCRATCH_BYTES per GPU, part of the library's device code, held by each GPU the call
 * runs on until the process ends. The call allocates and frees nothing; its first call on a device
 * looks the array's device address up once (hipGetSymbolAddress).
 * Arguments: as chs_decode_step, without the workspace. A call whose chs_decode_step workspace would
 * exceed CHS_NOALLOC_SCRATCH_BYTES returns CHS_ERR_WORKSPACE and launches nothing (at 1M tokens
 * and batch 1 the step needs about 3.8 MiB; 64 sequences of 200K tokens about 33 MiB).
 * Every call on a GPU shares that GPU's array, and the array keeps the last call's contents (the
 * step needs no initialised scratch): calls that overlap on one GPU, on different streams or from
 * different threads, race on it and must be serialised by the caller. */
#define CHS_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
chs_status chs_decode_step_noalloc(int32_t batch, int32_t n_heads, int32_t d, int32_t window, int32_t k,
                                   float scale, int32_t idx_heads, int32_t idx_dim, const void* q_idx,
                                   const float* w, const void* k_idx, const void* q, const void* swa_kv,
                                   const int32_t* swa_len, const void* comp_kv, const int64_t* cu_comp,
                                   int64_t max_comp, float* scores, int32_t* topk, float* out, float* lse,
                                   void* stream);

/* ---- Paged pools: chs_decode_attn_paged, chs_append_paged ----------------------------------
 * Source: "SGLang 如何为 DeepSeek V4 打造「Day-0」推理加速", 创新 1 (ShadowRadix: a per-request index
 * projected onto separate physical pools for the window, the C4 and the C128 entries, plus the
 * state rings, whose address is swa_page * ring_size + pos; the window pool frees a sequence's page
 * as it slides while its compressed entries stay shared) and "DeepSeek-V4 本地部署，SGLang 把活做絕
 * 了", ShadowRadix (the ring nested in the SWA page index).
 * The calls compute exactly what chs_decode_attn / chs_append compute; only the addressing differs:
 *   window of sequence b    : rows swa_page[b] * window .. + window - 1 of swa_pool
 *                             ([swa_pages * window, d]); its gate ring (chs_append_paged) is page
 *                             swa_page[b] of gate_ring ([swa_pages * ring_size, d]);
 *   compressed entry j of b : row page_table[b * pt_stride + j / page_size] * page_size
 *                             + j mod page_size of the pool ([pool_pages * page_size, d]);
 *   entries of b            : comp_len[b] (int64, capped at pt_stride * page_size), in place of the
 *                             cu_comp ranges. Top-k indices stay sequence-local.
 * page_size is a power of two, 1 .. 65536; page tables are [batch, pt_stride] int32. A window page
 * outside [0, swa_pages) drops that sequence's window (attention) or skips its writes (append);
 * an entry whose page is outside the pool is skipped (attention) or not written (append).
 * chs_decode_attn_paged takes the workspace of chs_decode_attn_workspace_size with the same
 * arguments; max_comp (host) must bound max_b comp_len[b] for a dense (C128) call. dtype CHS_BF16
 * or CHS_F32, d as for chs_decode_attn. One page table can serve the KV pool and the index-key pool
 * (chs_index_topk_paged): they hold the same entry numbering. */
chs_status chs_decode_attn_paged(chs_dtype dtype, int32_t batch, int32_t n_heads, int32_t d,
                                 int32_t window, int32_t k, float scale, const void* q,
                                 const void* swa_pool, const int32_t* swa_page, int64_t swa_pages,
                                 const int32_t* swa_len, const void* comp_pool, int64_t pool_pages,
                                 int32_t page_size, const int32_t* page_table, int32_t pt_stride,
                                 const int64_t* comp_len, const int32_t* topk, int64_t max_comp,
                                 float* out, float* lse, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* chs_decode_step_paged: chs_decode_step over the paged pools, addressed as above: computes exactly
 * chs_index_topk_paged(CHS_BF16, batch, idx_heads, idx_dim, k, q_idx, w, key_pool, pool_pages, page_size,
 * page_table, pt_stride, comp_len, max_comp, scores, topk, ...) followed by
 * chs_decode_attn_paged(CHS_BF16, batch, n_heads, d, window, k, scale, q, swa_pool, swa_page, swa_pages,
 * swa_len, comp_pool, pool_pages, page_size, page_table, pt_stride, comp_len, topk, max_comp, out, lse,
 * ...), one page table serving the index-key pool and the entry pool (the same entry numbering):
 * scores, topk, out and lse are bit-identical to those two calls, in three launches instead of four.
 * Ranges: those of the two calls (bf16; idx_dim 64, 128 or 256; page_size a power of two of at
 * least 64). workspace: chs_decode_step_workspace_size(batch, n_heads, d, window, k, max_comp) bytes. */
chs_status chs_decode_step_paged(int32_t batch, int32_t n_heads, int32_t d, int32_t window, int32_t k, float scale,
                                 int32_t idx_heads, int32_t idx_dim, const void* q_idx, const float* w,
                                 const void* key_pool, const void* q, const void* swa_pool, const int32_t* swa_page,
                                 int64_t swa_pages, const int32_t* swa_len, const void* comp_pool, int64_t pool_pages,
                                 int32_t page_size, const int32_t* page_table, int32_t pt_stride,
                                 const int64_t* comp_len, int64_t max_comp, float* scores, int32_t* topk, float* out,
                                 float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* chs_index_topk_paged: chs_index_topk with the index keys in a paged pool, addressed as above
 * (candidate j of sequence b at pool row page_table[b * pt_stride + j / page_size] * page_size +
 * j mod page_size; cand_len[b] candidates, capped at max_cand and pt_stride * page_size). scores, if
 * not NULL, is [batch, max_cand] fp32 with sequence b's scores from b * max_cand. The workspace is
 * chs_index_topk_workspace_size(batch, max_cand, k). Supported: CHS_BF16 keys, head_dim in
 * {64, 128, 256}, 1..16 heads, page_size a power of two >= 64 (a wave's keys then lie in one page);
 * other shapes return CHS_ERR_UNSUPPORTED. A page outside [0, pool_pages) reads page 0 (the scores of
 * its candidates are then unspecified; nothing outside the pool is read). */
chs_status chs_index_topk_paged(chs_dtype dtype, int32_t batch, int32_t n_heads, int32_t head_dim, int32_t k,
                                const void* q_idx, const float* w, const void* key_pool, int64_t pool_pages,
                                int32_t page_size, const int32_t* page_table, int32_t pt_stride,
                                const int64_t* cand_len, int64_t max_cand, float* scores, int32_t* topk,
                                void* workspace, size_t workspace_bytes, void* stream);

/* chs_index_topk_fp8_paged, chs_decode_attn_fp8_paged: the FP8 calls (chs_index_topk_fp8,
 * chs_decode_attn_fp8) over paged pools, addressed as above; each row's fp32 scale sits at the same
 * row index of a scale pool ([pool_pages * page_size] for keys and entries, [swa_pages * window] for
 * the windows). The index call supports head_dim 64, 128, 256 with page_size at least the keys a
 * wave scores (128, 64, 32 respectively; else CHS_ERR_SHAPE). Results are bit-identical to the
 * contiguous FP8 calls on the same rows. */
chs_status chs_index_topk_fp8_paged(int32_t batch, int32_t n_heads, int32_t head_dim, int32_t k,
                                    const void* q_idx, const float* w, const void* key_pool,
                                    const float* scale_pool, int64_t pool_pages, int32_t page_size,
                                    const int32_t* page_table, int32_t pt_stride, const int64_t* cand_len,
                                    int64_t max_cand, float* scores, int32_t* topk, void* workspace,
                                    size_t workspace_bytes, void* stream);

chs_status chs_decode_attn_fp8_paged(int32_t batch, int32_t n_heads, int32_t d, int32_t window, int32_t k,
                                     float scale, const void* q, const void* swa_pool,
                                     const float* swa_scale_pool, const int32_t* swa_page, int64_t swa_pages,
                                     const int32_t* swa_len, const void* comp_pool,
                                     const float* comp_scale_pool, int64_t pool_pages, int32_t page_size,
                                     const int32_t* page_table, int32_t pt_stride, const int64_t* comp_len,
                                     const int32_t* topk, int64_t max_comp, float* out, float* lse,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* chs_append_paged: chs_append with the window, the gate ring and the compressed pool paged as
 * above (n_tokens, swa_len, comp_count as in chs_append; comp_count counts entries, so it can feed
 * comp_len of chs_decode_attn_paged directly). */
chs_status chs_append_paged(chs_dtype dtype, int32_t batch, int32_t d, int32_t m, int32_t window,
                            int32_t ring_size, const void* x_new, const void* z_new, const float* bias,
                            int64_t* n_tokens, void* swa_pool, const int32_t* swa_page, int64_t swa_pages,
                            int32_t* swa_len, void* gate_ring, void* comp_pool, int64_t pool_pages,
                            int32_t page_size, const int32_t* page_table, int32_t pt_stride,
                            int64_t* comp_count, void* stream);

/* ---- chs_gather_selected: a HiSparse-style working-set gather --------------------------------
 * Source: "SGLang 如何为 DeepSeek V4 打造「Day-0」推理加速", 创新 3 (HiSparse: each C4 step touches about
 * 0.2% of the entries, so the full pool can be mirrored in pinned host memory while the GPU keeps a
 * working set of what each step hits; misses come in from the mirror) and "DeepSeek-V4 本地部署，SGLang
 * 把活做絕了", HiSparse 把不活躍 KV 甩到 CPU.
 * For every sequence b and slot i with j = topk[b, i] in [0, G_b), G_b = cu_comp[b+1] - cu_comp[b]:
 *   work[b*k + i, :] = cache[resident[cu_comp[b] + j], :]  if resident is not NULL and that value is in
 *                                                           [0, cache_rows),
 *                    = mirror[cu_comp[b] + j, :]            otherwise;
 *   work_topk[b, i]  = i; other slots get work_topk = -1 and their work row is left untouched.
 * chs_decode_attn over (work, cu = {0, k, 2k, ...}, work_topk) is then bit-identical to chs_decode_attn
 * over (mirror, cu_comp, topk). The residency map and the cache are the caller's (its eviction policy
 * decides them); the call only reads them.
 * mirror       : [cu_comp[batch], d] of `dtype`; device memory, or, with mirror_on_host = 1, pinned host
 *                memory allocated by the HIP runtime (hipHostMalloc; torch's pin_memory), read over PCIe.
 *                Host memory the runtime cannot map returns CHS_ERR_UNSUPPORTED before any launch.
 * cache        : [cache_rows, d] device rows, and resident: [cu_comp[batch]] int32, both or neither.
 * work         : [batch * k, d] device; work_topk: [batch, k] int32.
 * Ranges: 1 <= batch <= 65535; 1 <= k <= 2048; 1 <= d <= 4096 with d*elem_size % 16 == 0. */
chs_status chs_gather_selected(chs_dtype dtype, int32_t batch, int32_t d, int32_t k, const void* mirror,
                               int32_t mirror_on_host, const int64_t* cu_comp, const int32_t* topk,
                               const void* cache, const int32_t* resident, int64_t cache_rows, void* work,
                               int32_t* work_topk, void* stream);

/* ---- chs_decode_attn_fp8: chs_decode_attn over an FP8 KV cache ------------------------------
 * Source: as chs_decode_attn, with "SGLang 如何为 DeepSeek V4 打造「Day-0」推理加速", 4.3 部署配置
 * 建议 (an fp8 KV cache) and "DeepSeek-V4 本地部署，SGLang 把活做絕了", V4 到底改了啥 (attention
 * kept in FP8). Reading taken (the pages fix no format): window rows and compressed entries are
 * OCP E4M3 codes with one fp32 scale per row, row = scale * decode(codes); the query is bf16.
 * Computes chs_decode_attn's outputs for those rows (keys doubling as values).
 * q        : [batch, n_heads, d] bf16.
 * swa_kv   : [batch, window, d] E4M3 codes; swa_scale: [batch, window] fp32 (>= 0, finite).
 * comp_kv  : [cu_comp[batch], d] E4M3 codes; comp_scale: [cu_comp[batch]] fp32 (>= 0, finite).
 * Other arguments, ranges and the workspace as chs_decode_attn with dtype CHS_BF16
 * (chs_decode_attn_workspace_size(CHS_BF16, ...)). NaN codes are outside the contract. */
chs_status chs_decode_attn_fp8(int32_t batch, int32_t n_heads, int32_t d, int32_t window, int32_t k,
                               float scale, const void* q, const void* swa_kv, const float* swa_scale,
                               const int32_t* swa_len, const void* comp_kv, const float* comp_scale,
                               const int64_t* cu_comp, const int32_t* topk, int64_t max_comp,
                               float* out, float* lse, void* workspace, size_t workspace_bytes,
                               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CHS_H */
