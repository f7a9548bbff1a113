/*
 * dsa_oracle.c -- plain, slow CPU oracle for the DSA sparse-attention
 * verify step (lightning-indexer score -> per-row top-k -> sparse MLA ->
 * greedy acceptance, or rejection-sampling acceptance).
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code,
 * header, table or constant with the HIP library: every step below is
 * written from the pages' description of the method, in float64 unless the
 * step itself is defined in another precision.
 *
 * Sources (page title, then section):
 *  [P3] "MAX Pipeline 中的 DeepSeek-V3.2 架构实现解析", sections
 *       "Indexer 的结构与计算流程" (Hadamard rotation, block-128 dynamic FP8
 *       quantisation, top-k of shape (total_seq_len, index_topk)),
 *       "配置体系" (index_n_heads 64, index_head_dim 128, index_topk 2048,
 *       float8_e4m3fn indexer K cache with a per-token fp32 scale),
 *       "稀疏 MLA 的前向路径" (attention only over the selected positions).
 *  [P2] "GLM-5.3 推理全链路(十四):MTP 的三段前向", sections
 *       "验证段:6 行 batch 与一棵退化成链的树" (k+1 verify rows at
 *       consecutive positions, chain == plain causal mask, per-query top-k),
 *       "接受判定:greedy 与 rejection sampling" (greedy acceptance is the
 *       longest prefix where draft == target argmax),
 *       "GLM-5.3 的草稿层到底长什么样" (kv_lora_rank 512 + rope 64 latent).
 *  [P1] "MAX 中 GLM-5.2 (DeepSeek-V3.2 Sparse) 的统一 MTP 推测解码架构解析",
 *       "阶段 5" (step-0 top-k reused by gathering the accepted position).
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *  - score I[t,s] = sum_j w[t,j] * ReLU(q[t,j] . k[s]) over index heads, with
 *    q = s_q * q_hat and k = s_k * k_hat; the positive scales are factored
 *    out of the ReLU: I = s_k * sum_j (w*s_q) * ReLU(q_hat . k_hat);
 *  - Hadamard: Sylvester order, orthonormal 1/sqrt(D), applied to q and k
 *    head vectors before quantisation, computed in float32;
 *  - FP8: OCP e4m3fn, round-to-nearest-even, saturating at +-448;
 *    scale = amax/448 (float32), 1 when amax == 0; one block per vector
 *    (D <= 128);
 *  - row r of request b (R_b rows, L_b cached positions including the R_b
 *    verify rows) sits at position p = L_b - R_b + r and sees keys 0..p;
 *  - top-k ties go to the lower position; output ascending, -1 padded;
 *  - sparse MLA logits use all 576 dims, values are the first 512;
 *  - FP8 latent cache row (656 bytes, see its section): 512 e4m3fn latent
 *    codes in 4 blocks of 128 with one float32 scale each (amax/448, 1 when
 *    amax == 0), then the 64 rope values as bf16;
 *  - greedy: first maximum wins the argmax;
 *  - rejection sampling: softmax targets, given draft probabilities and
 *    uniforms, residual max(0, p - q), inverse-CDF draw (see that section).
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no fast-math:
 * every float operation below is meant exactly as written).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------ */
/* FP8 e4m3fn codec (format: 1 sign, 4 exponent bits with bias 7, 3     */
/* mantissa bits; no infinity; S.1111.111 is NaN; max finite 448).      */
/* ------------------------------------------------------------------ */

ORACLE_API double dsa_oracle_fp8_decode(uint8_t b) {
  int sign = (b >> 7) & 1;
  int e = (b >> 3) & 0xF;
  int m = b & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6); /* subnormal: (m/8) * 2^(1-7) */
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

/* Magnitudes of the 127 finite non-negative codes 0x00..0x7E, ascending. */
static double g_fp8_mag[127];
static int g_fp8_ready = 0;

static void fp8_table_init(void) {
  if (g_fp8_ready) return;
  for (int c = 0; c < 127; ++c) g_fp8_mag[c] = dsa_oracle_fp8_decode((uint8_t)c);
  g_fp8_ready = 1;
}

/* Round-to-nearest-even onto the e4m3fn grid, saturating at 448.        */
/* Nearest code found by bisection over the ascending magnitude table;  */
/* on an exact tie the code with an even (zero) low bit wins.           */
ORACLE_API uint8_t dsa_oracle_fp8_encode(float x) {
  fp8_table_init();
  if (isnan(x)) return 0x7F;
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs((double)x);
  if (a >= 448.0) return sign | 0x7E;
  int lo = 0, hi = 126; /* invariant: mag[lo] <= a < mag[hi] */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (g_fp8_mag[mid] <= a) lo = mid; else hi = mid;
  }
  double dlo = a - g_fp8_mag[lo], dhi = g_fp8_mag[hi] - a;
  int code;
  if (dlo < dhi) code = lo;
  else if (dhi < dlo) code = hi;
  else code = (lo & 1) ? hi : lo;
  return sign | (uint8_t)code;
}

/* ------------------------------------------------------------------ */
/* Quantiser: Sylvester Hadamard rotation, orthonormal scaling, dynamic  */
/* per-block amax scale, e4m3fn encode ([P3] "Indexer 的结构与计算流程"). */
/* ------------------------------------------------------------------ */

/* In-place fast Walsh-Hadamard transform in natural (Sylvester) order,  */
/* float32 butterflies (a, b) -> (a + b, a - b), strides 1, 2, 4, ...     */
ORACLE_API void dsa_oracle_fwht_f32(float* y, int n) {
  for (int h = 1; h < n; h *= 2)
    for (int i = 0; i < n; i += 2 * h)
      for (int j = i; j < i + h; ++j) {
        float a = y[j], b = y[j + h];
        y[j] = a + b;
        y[j + h] = a - b;
      }
}

/* x: [n_vec, dim] float32 -> x_fp8: [n_vec, dim] bytes, scale: [n_vec]. */
ORACLE_API int dsa_oracle_quantize(const float* x, int64_t n_vec, int dim,
                                   uint8_t* x_fp8, float* scale) {
  if (dim <= 0 || dim > 128 || (dim & (dim - 1))) return -1;
  const float c = (float)(1.0 / sqrt((double)dim)); /* RN(1/sqrt(D)) */
  fp8_table_init();
#pragma omp parallel for schedule(static)
  for (int64_t v = 0; v < n_vec; ++v) {
    float y[128];
    for (int i = 0; i < dim; ++i) y[i] = x[v * dim + i];
    dsa_oracle_fwht_f32(y, dim);
    float amax = 0.0f;
    for (int i = 0; i < dim; ++i) {
      y[i] = y[i] * c;
      float a = fabsf(y[i]);
      if (a > amax) amax = a;
    }
    float s = amax > 0.0f ? amax / 448.0f : 1.0f;
    scale[v] = s;
    for (int i = 0; i < dim; ++i) x_fp8[v * dim + i] = dsa_oracle_fp8_encode(y[i] / s);
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* Ragged layout helpers: q_row_offsets[B+1], kv_row_offsets[B+1] are    */
/* exclusive prefix sums ([P4] "Token 合并", ragged offsets).            */
/* ------------------------------------------------------------------ */

static int row_request(const int32_t* q_off, int B, int64_t t) {
  for (int b = 0; b < B; ++b)
    if (t >= q_off[b] && t < q_off[b + 1]) return b;
  return -1;
}

/* Number of keys row t may see: p_t + 1 with p_t = L_b - R_b + r. */
static int64_t row_visible(const int32_t* q_off, const int64_t* kv_off, int b, int64_t t) {
  int64_t L = kv_off[b + 1] - kv_off[b];
  int64_t R = q_off[b + 1] - q_off[b];
  int64_t r = t - q_off[b];
  int64_t v = L - R + r + 1;
  if (v < 0) v = 0;
  if (v > L) v = L;
  return v;
}

ORACLE_API int64_t dsa_oracle_row_visible(const int32_t* q_off, const int64_t* kv_off,
                                          int B, int64_t t) {
  int b = row_request(q_off, B, t);
  return b < 0 ? -1 : row_visible(q_off, kv_off, b, t);
}

/* ------------------------------------------------------------------ */
/* Lightning-indexer score ([P3] "Indexer 的结构与计算流程").            */
/*                                                                      */
/* For the listed rows, out[i, s] = I[t_i, s] for s < |V_t|, -inf after: */
/*   d_j = sum_c dec(q_hat[t,j,c]) * dec(k_hat[s,c])   (exact in fp64:   */
/*         every e4m3fn value is a multiple of 2^-9 of magnitude <= 448, */
/*         so each partial sum is a multiple of 2^-18 below 2^53 units)  */
/*   I   = s_k[s] * sum_{j ascending} (w[t,j] * s_q[t,j]) * max(d_j, 0)  */
/* ------------------------------------------------------------------ */
ORACLE_API int dsa_oracle_index_score_rows(
    const uint8_t* q_fp8, const float* q_scale, const float* w,
    const uint8_t* k_fp8, const float* k_scale,
    const int32_t* q_off, const int64_t* kv_off, int B, int H, int D,
    const int64_t* rows, int64_t n_rows, double* out, int64_t out_ld) {
  double dec[256];
  for (int c = 0; c < 256; ++c) dec[c] = dsa_oracle_fp8_decode((uint8_t)c);
  int bad = 0;
  for (int64_t i = 0; i < n_rows; ++i)
    if (row_request(q_off, B, rows[i]) < 0) bad = 1;
  if (bad) return -1;
  /* one task per (row, key); rows and keys are independent */
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t i = 0; i < n_rows; ++i) {
    for (int64_t s = 0; s < out_ld; ++s) {
      int64_t t = rows[i];
      int b = row_request(q_off, B, t);
      int64_t nv = row_visible(q_off, kv_off, b, t);
      double* o = out + i * out_ld;
      if (s >= nv) { o[s] = -INFINITY; continue; }
      const uint8_t* qt = q_fp8 + t * (int64_t)H * D;
      const uint8_t* ks = k_fp8 + (kv_off[b] + s) * (int64_t)D;
      double acc = 0.0;
      for (int j = 0; j < H; ++j) {
        double d = 0.0;
        for (int c = 0; c < D; ++c) d = d + dec[qt[j * D + c]] * dec[ks[c]];
        double r = d > 0.0 ? d : 0.0;
        double u = (double)w[t * H + j] * (double)q_scale[t * H + j];
        acc = acc + u * r;
      }
      o[s] = acc * (double)k_scale[kv_off[b] + s];
    }
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* Per-row top-k ([P3] "Indexer 的结构与计算流程": output shape          */
/* (total_seq_len, index_topk)). Order keys by (score desc, position     */
/* asc), keep the first min(k, n), emit positions ascending, pad -1.     */
/* ------------------------------------------------------------------ */
typedef struct { double v; int64_t pos; } scored_t;

static int cmp_score_desc_pos_asc(const void* a, const void* b) {
  const scored_t* x = (const scored_t*)a;
  const scored_t* y = (const scored_t*)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return (x->pos < y->pos) ? -1 : (x->pos > y->pos);
}

static int cmp_i32_asc(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* scores: [n_rows, ld] (f64); n_visible[i] keys of row i are candidates. */
ORACLE_API int dsa_oracle_topk(const double* scores, int64_t ld, const int64_t* n_visible,
                               int64_t n_rows, int k, int32_t* out) {
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < n_rows; ++i) {
    int64_t n = n_visible[i];
    int32_t* o = out + i * (int64_t)k;
    if (n < 0 || n > ld) { bad = 1; continue; }
    scored_t* tmp = (scored_t*)malloc(sizeof(scored_t) * (size_t)(n > 0 ? n : 1));
    if (!tmp) { bad = 1; continue; }
    for (int64_t s = 0; s < n; ++s) { tmp[s].v = scores[i * ld + s]; tmp[s].pos = s; }
    qsort(tmp, (size_t)n, sizeof(scored_t), cmp_score_desc_pos_asc);
    int64_t m = n < k ? n : k;
    for (int64_t j = 0; j < m; ++j) o[j] = (int32_t)tmp[j].pos;
    qsort(o, (size_t)m, sizeof(int32_t), cmp_i32_asc);
    for (int64_t j = m; j < k; ++j) o[j] = -1;
    free(tmp);
  }
  return bad ? -1 : 0;
}

/* ------------------------------------------------------------------ */
/* Sparse MLA decode over the selected latent rows ([P3] "稀疏 MLA 的前向 */
/* 路径"; latent 512 + rope 64 from [P2] "GLM-5.3 的草稿层到底长什么样").  */
/*                                                                      */
/* For each listed row t and head h, over valid indices (0 <= idx < L_b, */
/* -1 and out-of-range entries skipped):                                 */
/*   z_i = sm_scale * sum_{c<576} q[t,h,c] * C[kv_off_b + idx_i, c]       */
/*   out[t,h,:] = sum_i softmax(z)_i * C[., :512],  lse = m + ln(sum e^.) */
/* No valid index: out = 0, lse = -inf. Index-share ([P1] "阶段 5"): when */
/* share_base is given, every row of request b reads topk row            */
/* share_base[b] + num_accepted[b] instead of its own row.               */
/* ------------------------------------------------------------------ */
static double bf16_to_f64(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

ORACLE_API int dsa_oracle_sparse_mla_rows(
    const uint16_t* q, const uint16_t* kv, const int32_t* topk, int k,
    const int32_t* share_base, const int32_t* num_accepted,
    const int32_t* q_off, const int64_t* kv_off, int B, int H, float sm_scale,
    const int64_t* rows, int64_t n_rows, double* out, double* lse) {
  const int DQK = 576, DV = 512;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t ii = 0; ii < n_rows * H; ++ii) {
    int64_t i = ii / H;
    int h = (int)(ii % H);
    int64_t t = rows[i];
    int b = row_request(q_off, B, t);
    double* o = out + (i * H + h) * (int64_t)DV;
    if (b < 0) { bad = 1; continue; }
    int64_t L = kv_off[b + 1] - kv_off[b];
    int64_t trow = share_base ? (int64_t)share_base[b] + num_accepted[b] : t;
    const int32_t* idx = topk + trow * (int64_t)k;
    const uint16_t* qh = q + (t * (int64_t)H + h) * DQK;
    double* z = (double*)malloc(sizeof(double) * (size_t)k);
    if (!z) { bad = 1; continue; }
    double m = -INFINITY;
    int nvalid = 0;
    for (int j = 0; j < k; ++j) {
      int64_t p = idx[j];
      if (p < 0 || p >= L) { z[j] = NAN; continue; }
      const uint16_t* row = kv + (kv_off[b] + p) * (int64_t)DQK;
      double dot = 0.0;
      for (int c = 0; c < DQK; ++c) dot = dot + bf16_to_f64(qh[c]) * bf16_to_f64(row[c]);
      z[j] = (double)sm_scale * dot;
      if (z[j] > m) m = z[j];
      ++nvalid;
    }
    for (int c = 0; c < DV; ++c) o[c] = 0.0;
    if (nvalid == 0) {
      lse[i * H + h] = -INFINITY;
      free(z);
      continue;
    }
    double l = 0.0;
    for (int j = 0; j < k; ++j) {
      if (isnan(z[j])) continue;
      double pj = exp(z[j] - m);
      l = l + pj;
      const uint16_t* row = kv + (kv_off[b] + idx[j]) * (int64_t)DQK;
      for (int c = 0; c < DV; ++c) o[c] = o[c] + pj * bf16_to_f64(row[c]);
    }
    for (int c = 0; c < DV; ++c) o[c] = o[c] / l;
    lse[i * H + h] = m + log(l);
    free(z);
  }
  return bad ? -1 : 0;
}

/* ------------------------------------------------------------------ */
/* FP8 latent cache rows ([P2] the draft layer's KV pool: 656 bytes per   */
/* token per layer in the fp8_ds_mla layout; [P3] "配置体系": the caches  */
/* hold float8_e4m3fn with float32 scales).                              */
/*                                                                      */
/* Reading of the 656 bytes: 512 + 4*4 + 64*2, i.e.                      */
/*   bytes [0, 512)   e4m3fn codes of latent values 0..511               */
/*   bytes [512, 528) float32 scale of latent block b = 0..3 (128 values) */
/*   bytes [528, 656) the 64 rope values, bf16, copied bit for bit       */
/* Block b: amax = max |x| over its 128 values, scale = amax / 448 in    */
/* float32 (1 when amax == 0), code = e4m3fn(x / scale) with the division */
/* in float32 and the encoding of the indexer quantiser. The value a code */
/* stands for is decode(code) * scale, formed exactly in float64.        */
/* ------------------------------------------------------------------ */
static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* latent: [n, 576] bf16 rows -> out: [n, 656] bytes. */
ORACLE_API void dsa_oracle_mla_fp8_pack(const uint16_t* latent, int64_t n, uint8_t* out) {
  fp8_table_init();
  for (int64_t r = 0; r < n; ++r) {
    const uint16_t* x = latent + r * 576;
    uint8_t* o = out + r * 656;
    for (int b = 0; b < 4; ++b) {
      float amax = 0.0f;
      for (int i = 0; i < 128; ++i) {
        float a = fabsf(bf16_to_f32(x[128 * b + i]));
        if (a > amax) amax = a;
      }
      float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
      memcpy(o + 512 + 4 * b, &sc, sizeof sc);
      for (int i = 0; i < 128; ++i)
        o[128 * b + i] = dsa_oracle_fp8_encode(bf16_to_f32(x[128 * b + i]) / sc);
    }
    memcpy(o + 528, x + 512, 64 * sizeof(uint16_t));
  }
}

/* The 576 values a packed row stands for (float64, exact). */
static void fp8_row_values(const uint8_t* row, double* v) {
  float sc[4];
  memcpy(sc, row + 512, sizeof sc);
  for (int c = 0; c < 512; ++c) v[c] = dsa_oracle_fp8_decode(row[c]) * (double)sc[c / 128];
  for (int c = 0; c < 64; ++c) {
    uint16_t h;
    memcpy(&h, row + 528 + 2 * c, sizeof h);
    v[512 + c] = (double)bf16_to_f32(h);
  }
}

/* Sparse MLA as dsa_oracle_sparse_mla_rows, over packed FP8 rows kv8 [N, 656]. */
ORACLE_API int dsa_oracle_sparse_mla_fp8_rows(
    const uint16_t* q, const uint8_t* kv8, const int32_t* topk, int k,
    const int32_t* share_base, const int32_t* num_accepted,
    const int32_t* q_off, const int64_t* kv_off, int B, int H, float sm_scale,
    const int64_t* rows, int64_t n_rows, double* out, double* lse) {
  const int DQK = 576, DV = 512, RB = 656;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t ii = 0; ii < n_rows * H; ++ii) {
    int64_t i = ii / H;
    int h = (int)(ii % H);
    int64_t t = rows[i];
    int b = row_request(q_off, B, t);
    double* o = out + (i * H + h) * (int64_t)DV;
    if (b < 0) { bad = 1; continue; }
    int64_t L = kv_off[b + 1] - kv_off[b];
    int64_t trow = share_base ? (int64_t)share_base[b] + num_accepted[b] : t;
    const int32_t* idx = topk + trow * (int64_t)k;
    const uint16_t* qh = q + (t * (int64_t)H + h) * DQK;
    double* z = (double*)malloc(sizeof(double) * (size_t)k);
    double v[576];
    if (!z) { bad = 1; continue; }
    double m = -INFINITY;
    int nvalid = 0;
    for (int j = 0; j < k; ++j) {
      int64_t p = idx[j];
      if (p < 0 || p >= L) { z[j] = NAN; continue; }
      fp8_row_values(kv8 + (kv_off[b] + p) * (int64_t)RB, v);
      double dot = 0.0;
      for (int c = 0; c < DQK; ++c) dot = dot + (double)bf16_to_f32(qh[c]) * v[c];
      z[j] = (double)sm_scale * dot;
      if (z[j] > m) m = z[j];
      ++nvalid;
    }
    for (int c = 0; c < DV; ++c) o[c] = 0.0;
    if (nvalid == 0) {
      lse[i * H + h] = -INFINITY;
      free(z);
      continue;
    }
    double l = 0.0;
    for (int j = 0; j < k; ++j) {
      if (isnan(z[j])) continue;
      double pj = exp(z[j] - m);
      l = l + pj;
      fp8_row_values(kv8 + (kv_off[b] + idx[j]) * (int64_t)RB, v);
      for (int c = 0; c < DV; ++c) o[c] = o[c] + pj * v[c];
    }
    for (int c = 0; c < DV; ++c) o[c] = o[c] / l;
    lse[i * H + h] = m + log(l);
    free(z);
  }
  return bad ? -1 : 0;
}

/* ------------------------------------------------------------------ */
/* Greedy acceptance ([P2] "接受判定:greedy 与 rejection sampling").      */
/* Logits row b*(K+1)+i is the target distribution after verify row i    */
/* (row 0 = bonus token, rows 1..K = drafts).                            */
/*   a[b,i]   = smallest v with logits[row, v] == max (first max wins)   */
/*   n_b      = largest n <= K with draft[b, i] == a[b, i] for all i < n  */
/*   next[b]  = a[b, n_b]                                                */
/* dtype 0 = float32, 1 = bfloat16 (upcast exactly; -0 == +0).           */
/* ------------------------------------------------------------------ */
ORACLE_API int dsa_oracle_greedy_accept(const void* logits, int dtype, int64_t ld,
                                        const int32_t* draft, int B, int K, int V,
                                        int32_t* num_accepted, int32_t* next_token,
                                        int32_t* argmax_out) {
  if (dtype != 0 && dtype != 1) return -1;
  for (int b = 0; b < B; ++b) {
    int32_t a[1024];
    if (K + 1 > 1024) return -1;
    for (int i = 0; i <= K; ++i) {
      int64_t row = (int64_t)b * (K + 1) + i;
      double best = 0.0;
      int32_t arg = -1;
      for (int v = 0; v < V; ++v) {
        double x = dtype == 0 ? (double)((const float*)logits)[row * ld + v]
                              : bf16_to_f64(((const uint16_t*)logits)[row * ld + v]);
        if (arg < 0 || x > best) { best = x; arg = v; } /* strict: first max kept */
      }
      a[i] = arg;
      if (argmax_out) argmax_out[row] = arg;
    }
    int n = 0;
    while (n < K && draft[(int64_t)b * K + n] == a[n]) ++n;
    num_accepted[b] = n;
    next_token[b] = a[n];
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* Rejection-sampling acceptance ([P2] "接受判定:greedy 与 rejection       */
/* sampling": draft token i is kept with probability min(1, p/q), q the */
/* draft distribution and p the target's; at the first refused step a   */
/* token is drawn from the corrected distribution and becomes that      */
/* step's bonus). Readings (listed in the design notes):                */
/*  - p_i = softmax of logits row b*(K+1)+i over the V entries, float64; */
/*  - q_i = draft_probs[b, i, :] as given (float32 probabilities);        */
/*  - the uniforms are inputs: draft i is kept iff u[b,i] * q_i(x_i) <   */
/*    p_i(x_i), the event u < min(1, p/q) for u in [0, 1);               */
/*  - corrected distribution at the first refusal n: w(v) = max(0,      */
/*    p_n(v) - q_n(v)); when every draft is kept, w = p_K (bonus row);    */
/*    if w sums to 0, w = p_n;                                           */
/*  - the token is the smallest v with C(v) > us[b] * C(V-1), C the      */
/*    running sum of w in index order (inverse CDF).                     */
/* For the tests, acc_margin[b*K+i] = (p - u*q) / max(p, u*q) of every   */
/* decision taken (0 where none was), and samp_margin[b] = the distance  */
/* of us*W to the nearer of C(v-1), C(v) of the drawn v, divided by W.    */
/* ------------------------------------------------------------------ */
static double logit_at(const void* logits, int dtype, int64_t idx) {
  return dtype == 0 ? (double)((const float*)logits)[idx]
                    : bf16_to_f64(((const uint16_t*)logits)[idx]);
}

/* p[v] = softmax of one logits row, float64 */
static void softmax_row(const void* logits, int dtype, int64_t row_start, int V, double* p) {
  double m = -INFINITY;
  for (int v = 0; v < V; ++v) {
    double x = logit_at(logits, dtype, row_start + v);
    if (x > m) m = x;
  }
  double s = 0.0;
  for (int v = 0; v < V; ++v) {
    p[v] = exp(logit_at(logits, dtype, row_start + v) - m);
    s = s + p[v];
  }
  for (int v = 0; v < V; ++v) p[v] = p[v] / s;
}

ORACLE_API int dsa_oracle_rejection_accept(const void* logits, int dtype, int64_t ld,
                                           const float* draft_probs, const int32_t* draft,
                                           const float* u, const float* us, int B, int K, int V,
                                           int32_t* num_accepted, int32_t* next_token,
                                           double* acc_margin, double* samp_margin) {
  if ((dtype != 0 && dtype != 1) || V < 1 || K < 0) return -1;
  double* p = (double*)malloc(sizeof(double) * (size_t)V);
  double* w = (double*)malloc(sizeof(double) * (size_t)V);
  if (!p || !w) { free(p); free(w); return -1; }
  int bad = 0;
  for (int b = 0; b < B && !bad; ++b) {
    int n = 0;
    for (; n < K; ++n) {
      const int64_t row = (int64_t)b * (K + 1) + n;
      const int32_t x = draft[(int64_t)b * K + n];
      if (x < 0 || x >= V) { bad = 1; break; }
      softmax_row(logits, dtype, row * ld, V, p);
      const double pq = p[x];
      const double uq = (double)u[(int64_t)b * K + n] *
                        (double)draft_probs[((int64_t)b * K + n) * V + x];
      const double big = pq > uq ? pq : uq;
      if (acc_margin) acc_margin[(int64_t)b * K + n] = big > 0.0 ? (pq - uq) / big : 0.0;
      if (!(uq < pq)) break;  /* refused */
    }
    if (bad) break;
    for (int i = n + 1; i < K && acc_margin; ++i) acc_margin[(int64_t)b * K + i] = 0.0;
    const int64_t row = (int64_t)b * (K + 1) + n;
    softmax_row(logits, dtype, row * ld, V, p);
    double W = 0.0;
    for (int v = 0; v < V; ++v) {
      double d = n < K ? p[v] - (double)draft_probs[((int64_t)b * K + n) * V + v] : p[v];
      w[v] = d > 0.0 ? d : 0.0;
      W = W + w[v];
    }
    if (!(W > 0.0)) {
      W = 0.0;
      for (int v = 0; v < V; ++v) { w[v] = p[v]; W = W + w[v]; }
    }
    const double target = (double)us[b] * W;
    double c = 0.0, prev = 0.0;
    int tok = -1;
    for (int v = 0; v < V; ++v) {
      prev = c;
      c = c + w[v];
      if (c > target) { tok = v; break; }
    }
    if (tok < 0) { /* rounding left target at or above the total: the last positive entry */
      for (int v = V - 1; v >= 0; --v)
        if (w[v] > 0.0) { tok = v; break; }
      prev = c - w[tok];
    }
    num_accepted[b] = n;
    next_token[b] = tok;
    if (samp_margin) {
      double d0 = target - prev, d1 = c - target;
      samp_margin[b] = (d0 < d1 ? d0 : d1) / W;
    }
  }
  free(p);
  free(w);
  return bad ? -1 : 0;
}
