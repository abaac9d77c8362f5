/* Plain CPU oracle for one decode step of one hybrid-sparse-attention layer.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg may load this library. It shares no code, header or table with the GPU library.
 *
 * Everything is computed in double precision with plain loops, one output at a time, in the
 * order the definitions state. OpenMP only spreads independent outputs over threads; each
 * output is computed by one thread in a fixed order, so results do not depend on the thread
 * count.
 *
 * Sources (web pages; cited by title and section):
 *  [P2] "DeepSeek-V4 本地部署，SGLang 把活做絕了", section "V4 到底改了啥" (hybrid sparse
 *       attention: every layer pairs a 128-token sliding window with either C4, 4:1 compression
 *       plus top-512 selection, or C128, 128:1 compression attended densely) and section
 *       "Kernel 層一堆狠活" (one attention call covers the window and the compressed entries;
 *       Lightning TopK picks 512 of 256K candidates at 1M context).
 *  [P3] "SGLang 如何为 DeepSeek V4 打造「Day-0」推理加速", section 创新 2 (the compressor's
 *       stages: load tokens, score, softmax, weighted sum, store; top-k by a radix threshold
 *       instead of a global sort) and section 创新 3 (C128 entries are all read each step).
 * The pages print no formulas. The readings used here are: per-channel softmax over each
 * group of gate logits plus a learned bias of shape [m, d]; score s_j = sum_h w_h ReLU(q_h.k_j);
 * top-k = the k largest, ties to the lower index, returned ascending; attention is one softmax
 * over window plus selected entries with K = V and logits scaled by 1/sqrt(d).
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---- Compressor ([P3] 创新 2, Flash Compressor; [P2] V4 到底改了啥) --------------------
 * For every complete group g of sequence b and every channel c:
 *   a_i = Z[t0 + g*m + i, c] + B[i, c]            (i < m, t0 = cu_tokens[b])
 *   w_i = exp(a_i - max_j a_j) / sum_j exp(a_j - max_j a_j)
 *   C[g, c] = sum_i w_i * X[t0 + g*m + i, c]
 * A trailing partial group (N_b mod m tokens) is not compressed. Output rows are packed:
 * sequence b's groups start at sum_{b'<b} floor(N_b'/m). X, Z: [T, d]; B: [m, d]. */
void oracle_compress(int32_t batch, int32_t d, int32_t m, const float* X, const float* Z,
                     const float* B, const int64_t* cu_tokens, double* out) {
  int64_t base = 0;
  for (int32_t b = 0; b < batch; ++b) {
    int64_t t0 = cu_tokens[b];
    int64_t n_groups = (cu_tokens[b + 1] - t0) / m;
    int64_t n_items = n_groups * d;
#pragma omp parallel for schedule(static)
    for (int64_t it = 0; it < n_items; ++it) {
      int64_t g = it / d;
      int32_t c = (int32_t)(it % d);
      double a[1024], w[1024];
      double mx = -INFINITY;
      for (int32_t i = 0; i < m; ++i) {
        a[i] = (double)Z[(t0 + g * m + i) * d + c] + (double)B[(int64_t)i * d + c];
        if (a[i] > mx) mx = a[i];
      }
      double den = 0.0;
      for (int32_t i = 0; i < m; ++i) den += exp(a[i] - mx);
      for (int32_t i = 0; i < m; ++i) w[i] = exp(a[i] - mx) / den;
      double acc = 0.0;
      for (int32_t i = 0; i < m; ++i) acc += w[i] * (double)X[(t0 + g * m + i) * d + c];
      out[(base + g) * d + c] = acc;
    }
    base += n_groups;
  }
}

/* ---- Indexer score ([P3] 创新 2 and 创新 5: the indexer scores every compressed candidate
 * and hands the scores to the top-k) ------------------------------------------------------
 *   s_j = sum_h w_h * max(0, sum_t q[h, t] * K[j, t])       q: [nh, dim], K: [n, dim] */
void oracle_index_scores(int32_t nh, int32_t dim, const float* q, const float* w, int64_t n,
                         const float* K, double* s) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) {
    double acc = 0.0;
    for (int32_t h = 0; h < nh; ++h) {
      double dot = 0.0;
      for (int32_t t = 0; t < dim; ++t) dot += (double)q[(int64_t)h * dim + t] * (double)K[j * dim + t];
      acc += (double)w[h] * (dot > 0.0 ? dot : 0.0);
    }
    s[j] = acc;
  }
}

/* ---- FP8 index keys ([P2] V4 到底改了啥: the checkpoints keep attention in FP8; [P3] 4.3 部署
 * 配置建议: an fp8 KV cache). The pages fix neither the FP8 variant nor a scale layout;
 * the reading taken here is the OCP 8-bit E4M3 format with one fp32 scale per key row.
 * E4M3 byte: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0. Exponent 0 encodes
 * subnormals m * 2^-9; exponent 15 with mantissa 7 is NaN; there are no infinities. */
double oracle_decode_e4m3(uint8_t b) {
  const int sign = b >> 7, e = (b >> 3) & 15, m = b & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m, -9);
  else v = ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -v : v;
}

void oracle_decode_e4m3_n(int64_t n, const uint8_t* in, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_decode_e4m3(in[i]);
}

/* The indexer score with FP8 keys: key row j is scale[j] * decode(K8[j, :]), and
 *   s_j = sum_h w_h * max(0, sum_t q[h, t] * (scale[j] * decode(K8[j, t]))). */
void oracle_index_scores_fp8(int32_t nh, int32_t dim, const float* q, const float* w, int64_t n,
                             const uint8_t* K8, const float* scale, double* s) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) {
    double acc = 0.0;
    for (int32_t h = 0; h < nh; ++h) {
      double dot = 0.0;
      for (int32_t t = 0; t < dim; ++t)
        dot += (double)q[(int64_t)h * dim + t] * ((double)scale[j] * oracle_decode_e4m3(K8[j * dim + t]));
      acc += (double)w[h] * (dot > 0.0 ? dot : 0.0);
    }
    s[j] = acc;
  }
}

/* ---- Top-k ([P3] 创新 2, Lightning TopK; [P2] Kernel 層一堆狠活) ------------------------
 * The definition a radix select must reproduce, computed by a full sort: order the pairs
 * (s_j, j) by s descending (compared as floats, so -0.0 equals +0.0), then j ascending; keep
 * the first min(k, n); return those indices in ascending order, padded with -1 to length k.
 * Returns the number selected, or -1 if a score is NaN (outside the contract). */
typedef struct { float s; int32_t j; } oracle_pair;

static int cmp_pair(const void* pa, const void* pb) {
  const oracle_pair* a = (const oracle_pair*)pa;
  const oracle_pair* b = (const oracle_pair*)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->j < b->j) ? -1 : (a->j > b->j);
}

static int cmp_i32(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a > b) - (a < b);
}

int32_t oracle_topk(const float* s, int64_t n, int32_t k, int32_t* out) {
  for (int64_t j = 0; j < n; ++j)
    if (isnan(s[j])) return -1;
  oracle_pair* p = (oracle_pair*)malloc(sizeof(oracle_pair) * (size_t)(n > 0 ? n : 1));
  for (int64_t j = 0; j < n; ++j) { p[j].s = s[j]; p[j].j = (int32_t)j; }
  qsort(p, (size_t)n, sizeof(oracle_pair), cmp_pair);
  int32_t cnt = (int32_t)(n < k ? n : k);
  for (int32_t i = 0; i < cnt; ++i) out[i] = p[i].j;
  qsort(out, (size_t)cnt, sizeof(int32_t), cmp_i32);
  for (int32_t i = cnt; i < k; ++i) out[i] = -1;
  free(p);
  return cnt;
}

/* ---- Attention over one key set ([P2] Kernel 層一堆狠活: the window and the compressed
 * entries go through one attention call; [P3] 3.2: MLA decode with a shared latent) --------
 * Keys double as values (K = V). For each head h:
 *   l_i = scale * sum_c q[h, c] * keys[i, c]
 *   lse_h = log sum_i exp(l_i)            (computed as max + log sum exp(l_i - max))
 *   out[h, c] = sum_i exp(l_i - lse_h) * keys[i, c]
 * With no keys, out = 0 and lse = -inf. */
static void attend_keys(int32_t H, int32_t d, const float* q, int64_t nkeys, const double* keys, double scale,
                        double* out, double* lse) {
#pragma omp parallel for schedule(static)
  for (int32_t h = 0; h < H; ++h) {
    double* l = (double*)malloc(sizeof(double) * (size_t)(nkeys > 0 ? nkeys : 1));
    double mx = -INFINITY;
    for (int64_t i = 0; i < nkeys; ++i) {
      double dot = 0.0;
      for (int32_t c = 0; c < d; ++c) dot += (double)q[(int64_t)h * d + c] * keys[i * d + c];
      l[i] = scale * dot;
      if (l[i] > mx) mx = l[i];
    }
    double sum = 0.0;
    for (int64_t i = 0; i < nkeys; ++i) sum += exp(l[i] - mx);
    double ls = (nkeys > 0) ? mx + log(sum) : -INFINITY;
    lse[h] = ls;
    for (int32_t c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int64_t i = 0; i < nkeys; ++i) acc += exp(l[i] - ls) * keys[i * d + c];
      out[(int64_t)h * d + c] = acc;
    }
    free(l);
  }
}

void oracle_attend(int32_t H, int32_t d, const float* q, int64_t nkeys, const float* keys,
                   double scale, double* out, double* lse) {
  double* kd = (double*)malloc(sizeof(double) * (size_t)(nkeys > 0 ? nkeys * d : 1));
  for (int64_t i = 0; i < nkeys * d; ++i) kd[i] = (double)keys[i];
  attend_keys(H, d, q, nkeys, kd, scale, out, lse);
  free(kd);
}

/* The same attention over FP8 key rows (see the FP8 index keys above): key row i is
 * scales[i] * decode(codes[i, :]), taken exactly in double. */
void oracle_attend_fp8(int32_t H, int32_t d, const float* q, int64_t nkeys, const uint8_t* codes,
                       const float* scales, double scale, double* out, double* lse) {
  double* kd = (double*)malloc(sizeof(double) * (size_t)(nkeys > 0 ? nkeys * d : 1));
  for (int64_t i = 0; i < nkeys; ++i)
    for (int32_t c = 0; c < d; ++c) kd[i * d + c] = (double)scales[i] * oracle_decode_e4m3(codes[i * d + c]);
  attend_keys(H, d, q, nkeys, kd, scale, out, lse);
  free(kd);
}

/* ---- Storage rounding ----------------------------------------------------------------
 * The compressed entries are stored in the input precision. bfloat16 keeps 8 significant
 * bits: round the double to 8 significant bits, ties to even (the default rounding mode). */
void oracle_round_bf16(const double* x, int64_t n, float* out) {
  for (int64_t j = 0; j < n; ++j) {
    double v = x[j];
    if (v == 0.0 || !isfinite(v)) { out[j] = (float)v; continue; }
    int e;
    double mant = frexp(v, &e);              /* |mant| in [0.5, 1) */
    double r = nearbyint(ldexp(mant, 8));    /* 8 significant bits */
    out[j] = (float)ldexp(r, e - 8);
  }
}

/* ---- FP8 E4M3 storage written by the library ([P2] V4 到底改了啥: attention kept in FP8; [P3]
 * 4.3 部署配置建议: an fp8 KV cache). The pages fix no rounding or scale rule; the reading taken here:
 * one fp32 scale per row, the row's largest magnitude mapped to the largest E4M3 value 448, every
 * element rounded to the nearest E4M3 value.
 *
 * Encoding of one value y (fp32): the nearest of the 254 finite E4M3 values (decode above), ties to
 * the even code (the code whose lowest mantissa bit is 0); magnitudes above 448 saturate to 448.
 * Written as the plain search over the non-negative codes 0x00 .. 0x7E (0x7F is NaN), in double,
 * where both y and every E4M3 value are exact. */
uint8_t oracle_encode_e4m3(float y) {
  const double a = fabs((double)y);
  const uint8_t sign = signbit(y) ? 0x80 : 0x00;      /* the sign is kept, zeros included */
  int best = 0;
  double best_err = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    const double err = fabs(oracle_decode_e4m3((uint8_t)c) - a);
    if (err < best_err || (err == best_err && (c & 1) == 0)) { best = c; best_err = err; }
  }
  if (a > 448.0) best = 0x7E;
  return (uint8_t)(sign | best);
}

void oracle_encode_e4m3_n(int64_t n, const float* y, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_encode_e4m3(y[i]);
}

/* Per-row quantisation of rows [n, d] of fp32 values:
 *   amax = max_c |x_c|,  scale = fp32(amax / 448),  inv = min(fp32(448 / amax), FLT_MAX),
 *   code_c = encode(fp32(x_c * inv)),
 * every operation rounded once to fp32 (a double quotient or product of two fp32 operands rounds to
 * the same fp32 value as the correctly rounded fp32 operation). A row with amax = 0 has scale 0 and
 * all codes 0. Row r decodes as scale_r * decode(code); inv and 1 / scale differ by at most a few
 * fp32 ulps, far below the E4M3 step. */
void oracle_quantize_e4m3_rows(int64_t n, int32_t d, const float* x, uint8_t* codes, float* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    float amax = 0.0f;
    for (int32_t c = 0; c < d; ++c) {
      const float v = fabsf(x[r * d + c]);
      if (v > amax) amax = v;
    }
    const float s = (float)((double)amax / 448.0);
    float inv = (float)(448.0 / (double)amax);
    if (!(inv <= FLT_MAX)) inv = FLT_MAX;
    scales[r] = s;
    for (int32_t c = 0; c < d; ++c)
      codes[r * d + c] = amax == 0.0f ? 0 : oracle_encode_e4m3((float)((double)x[r * d + c] * (double)inv));
  }
}
