/*
 * dsa.h -- C ABI of libdsa.so: the DSA sparse-attention verify step on one
 * MI355X (gfx950).
 *
 * The step follows the pages' statement of the problem:
 *   "MAX Pipeline 中的 DeepSeek-V3.2 架构实现解析" (section
 *   "Indexer 的结构与计算流程"): q/k are Hadamard-rotated, dynamically
 *   quantised to FP8 (block 128), scored by the lightning indexer, and a
 *   top-k of shape (total_seq_len, index_topk) selects the positions sparse
 *   MLA attends to ("稀疏 MLA 的前向路径").
 *   "GLM-5.3 推理全链路(十四):MTP 的三段前向" (section "验证段"): each
 *   request contributes k+1 verify rows (bonus + drafts) at consecutive
 *   positions with a chain-causal mask; every row selects its own top-k;
 *   greedy acceptance keeps the longest draft prefix equal to the target
 *   argmax ("接受判定").
 *   "MAX 中 GLM-5.2 (DeepSeek-V3.2 Sparse) 的统一 MTP 推测解码架构解析"
 *   (section "阶段 5"): later draft steps reuse the step-0 top-k row at the
 *   accepted position (index_share_for_mtp_iteration).
 *   "MAX 推测解码配置指南解读 max.pipelines.speculative" (section
 *   "Token 合并"): ragged batches are described by exclusive-prefix row
 *   offsets [B+1].
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are DEVICE pointers unless documented otherwise; the caller
 *   owns every buffer (inputs, outputs and workspace). The library never
 *   allocates, frees, synchronises or reads device memory from the host.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream); every
 *   call only enqueues kernels on it, so calls are graph-capturable.
 * - Ragged batch: request b owns query rows [q_row_offsets[b],
 *   q_row_offsets[b+1]) (R_b rows) and cached positions [kv_row_offsets[b],
 *   kv_row_offsets[b+1]) (L_b positions, which include its R_b verify rows).
 *   Row r of request b sits at position p = L_b - R_b + r and sees positions
 *   0..p (chain-causal). Host scalars (B, T, max_q_rows, max_kv_len) size
 *   the launch; device offsets bound every access per row. The host scalars
 *   must be upper bounds of the device values: max_q_rows >= every R_b,
 *   max_kv_len >= every L_b, T == q_row_offsets[B]; rows longer than the score
 *   stride are clipped to it.
 * - Device array CONTENTS (offsets, indices) are trusted for ordering but
 *   every gather is bounds-checked against its request: out-of-range top-k
 *   entries are skipped like -1.
 * - Errors: invalid host arguments are rejected before any launch with a
 *   dsa_status and a thread-local message (dsa_last_error()). A failed
 *   launch returns DSA_ERR_HIP. No C++ exception crosses this boundary.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 7

/* Cache rows per entry of the key-scale table (dsa_key_scale_max). */
#define DSA_KEY_SCALE_CHUNK 2048

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARGUMENT = 1,
  DSA_ERR_UNSUPPORTED = 2,
  DSA_ERR_WORKSPACE_TOO_SMALL = 3,
  DSA_ERR_HIP = 4
} dsa_status;

typedef enum { DSA_F32 = 0, DSA_BF16 = 1 } dsa_dtype;

/* ABI version of the loaded library (DSA_ABI_VERSION). Host only. */
int dsa_abi_version(void);

/* Message of the last failed call on this thread ("" if none). Host only;
 * the string stays valid until the next call on this thread. */
const char* dsa_last_error(void);

/*
 * dsa_quantize_fp8 -- Hadamard rotation + dynamic FP8 quantisation.
 * ("MAX Pipeline 中的 DeepSeek-V3.2 架构实现解析", "Indexer 的结构与计算流程":
 * hadamard_transform in Sylvester order, then dynamic float8_e4m3fn
 * quantisation with block size 128 and an fp32 scale.)
 *
 * For each of the n_vec vectors x[v, 0:dim] (float32, dim in {64, 128},
 * one quantisation block per vector):
 *   y = FWHT(x) in float32 butterflies (a,b)->(a+b,a-b), strides 1,2,4,...
 *   y = y * RN_f32(1/sqrt(dim))
 *   scale[v] = amax(|y|) / 448 (float32 division), or 1 when amax == 0
 *   x_fp8[v, i] = e4m3fn(y[i] / scale[v]), round-to-nearest-even, saturating
 * Used for indexer queries [T*H_I vectors] and for index-cache keys [N].
 * Errors: DSA_ERR_INVALID_ARGUMENT (null pointer, n_vec < 0),
 * DSA_ERR_UNSUPPORTED (dim not 64/128).
 */
dsa_status dsa_quantize_fp8(const float* x, int64_t n_vec, int32_t dim, uint8_t* x_fp8,
                            float* scale, void* stream);

/*
 * dsa_verify_cache_write -- the verify step's cache writes, with its query
 * quantisation, in one launch.
 * ("GLM-5.3 推理全链路(十四)", the accept/rollback discussion: the verify segment
 * writes one indexer key per verify row into the indexer cache before the
 * acceptance decision, and the verify window's latent rows into the MLA cache;
 * "MAX Pipeline 中的 DeepSeek-V3.2 架构实现解析", "Indexer 的结构与计算流程" and
 * "配置体系": keys are rotated and quantised like queries, into the indexer K
 * cache and its fp32 per-token scale cache.)
 *
 * For each verify row t < T with cache row d = dst_rows[t]:
 *   k_cache[d, :], k_scale[d] = dsa_quantize_fp8 of k_new[t, :]
 *   kv_cache[d, :] = latent_new[t, :]  (576 bf16 copied bit for bit; skipped when
 *                                      latent_new is NULL)
 * and, when q is not NULL, q_fp8 / q_scale = dsa_quantize_fp8 of the T*H_I query
 * vectors q[t, j, :]. When k_scale_max is not NULL (the key-scale table of
 * dsa_key_scale_max), entry d / DSA_KEY_SCALE_CHUNK is raised to k_scale[d] if
 * below it (an atomic maximum), so the table stays an upper bound of its
 * chunks' scales.
 *   k_new [T, D_I] float32 (16-byte aligned); latent_new [T, 576] bf16 (16-byte
 *   aligned rows); dst_rows [T] int64 device array (distinct rows, trusted);
 *   k_cache [N, D_I] u8; k_scale [N] f32; kv_cache [N, 576] bf16;
 *   q [T, H_I, D_I] float32; q_fp8 [T, H_I, D_I] u8; q_scale [T, H_I] f32;
 *   k_scale_max [ceil(N / DSA_KEY_SCALE_CHUNK)] f32 (4-byte aligned) or NULL.
 * The caller decides the rows: under the ragged layout of dsa_index_score, row
 * t = q_off[b] + r is position L_b - R_b + r of request b, cache row
 * kv_row_offsets[b] + L_b - R_b + r.
 * Errors: DSA_ERR_INVALID_ARGUMENT (null or misaligned pointers, T < 0, q without
 * q_fp8/q_scale or H_I < 1), DSA_ERR_UNSUPPORTED (D_I not 64/128).
 */
dsa_status dsa_verify_cache_write(const float* k_new, const uint16_t* latent_new,
                                  const int64_t* dst_rows, int32_t T, int32_t D_I,
                                  uint8_t* k_cache, float* k_scale, uint16_t* kv_cache,
                                  const float* q, int32_t H_I, uint8_t* q_fp8, float* q_scale,
                                  float* k_scale_max, void* stream);

/*
 * dsa_index_score -- lightning-indexer scores of every verify row against
 * every visible cached index key.
 * ("MAX Pipeline 中的 DeepSeek-V3.2 架构实现解析", "Indexer 的结构与计算流程";
 * index_n_heads / index_head_dim from "配置体系".)
 *
 *   scores[t, s] = k_scale[s] * sum_j (w[t,j] * q_scale[t,j]) * ReLU(q_hat[t,j] . k_hat[s])
 * i.e. sum_j w[t,j] ReLU(q[t,j] . k[s]) with the positive FP8 scales
 * factored out. The FP8 products are exact, but the MFMA adds them at reduced
 * width: a head dot can differ from its exact value by up to 2^-9 *
 * max|q_hat_j| * max|k_hat| (128 products, each off by up to 2^-16 of the
 * largest; typical errors are far smaller). The ReLU, weights and head sum run
 * in float32. Written for s in [0, p_t] only; entries beyond are untouched.
 *
 *   q_fp8   [T, H_I, D_I] e4m3fn codes     q_scale, w [T, H_I] float32
 *   k_fp8   [N, D_I] e4m3fn codes          k_scale    [N] float32
 *   scores  [T, score_ld] float32, score_ld >= max_kv_len
 * Supported: D_I = 128 or 64, H_I in [1, 128].
 * Errors: DSA_ERR_INVALID_ARGUMENT, DSA_ERR_UNSUPPORTED.
 */
dsa_status dsa_index_score(const uint8_t* q_fp8, const float* q_scale, const float* w,
                           const uint8_t* k_fp8, const float* k_scale,
                           const int32_t* q_row_offsets, const int64_t* kv_row_offsets,
                           int32_t B, int32_t T, int32_t max_q_rows, int32_t H_I, int32_t D_I,
                           int64_t max_kv_len, float* scores, int64_t score_ld, void* stream);

/*
 * dsa_topk_refine -- inputs of the exact-boundary refine of dsa_topk: the
 * same FP8 queries, weights, keys and scales that dsa_index_score scored.
 * All pointers are device pointers (layouts as in dsa_index_score).
 *   err_scale  C of the error bound eps_t below; 0 selects 4
 *   status     [T] int32, nullable. Per row:
 *                >= 0  the row is refined; the value is the number of band keys
 *                      rescored exactly (0 when every visible key is selected)
 *                  -1  the band held more than 4096 keys: the float32 selection
 *                      is kept
 *                  -2  theta or eps is not finite, or the band cannot supply the
 *                      missing keys: the float32 selection is kept
 *                  -3  internal count mismatch: the float32 selection is kept
 *                  -4  the row is refined, but some band key's float32 score lies
 *                      farther than eps_t / 2 from its exact value, so the margin
 *                      the bound relies on is thinner than measured (treat the
 *                      set as possibly inexact)
 *   k_scale_max, k_scale_max_len  the caller's key-scale table (nullable). Set,
 *              smax_t below is taken from its entries covering cache rows
 *              kv_row_offsets[b] .. + p_t (an entry past the table gives an
 *              infinite eps_t, status -2); NULL, a pre-pass launch computes the
 *              per-request maxima in the workspace on every call.
 */
typedef struct dsa_topk_refine {
  const uint8_t* q_fp8;
  const float* q_scale;
  const float* w;
  const uint8_t* k_fp8;
  const float* k_scale;
  int32_t H_I;
  int32_t D_I;
  double err_scale;
  int32_t* status;
  const float* k_scale_max;  /* key-scale table (dsa_key_scale_max) or NULL */
  int64_t k_scale_max_len;   /* its entries (>= 1 when k_scale_max is set) */
} dsa_topk_refine;

/*
 * dsa_topk -- per-row top-k selection over the visible scores.
 * ("MAX Pipeline 中的 DeepSeek-V3.2 架构实现解析", "Indexer 的结构与计算流程": top-k
 * output of shape (total_seq_len, index_topk); "GLM-5.3 推理全链路(十四)",
 * "验证段的逐层算子": every verify query selects its own top-k.)
 *
 * For each row t, orders positions s in [0, p_t] by (scores[t,s] desc,
 * s asc) -- -0.0 equals +0.0, scores must not be NaN -- keeps the first
 * min(k, p_t+1), and writes them ASCENDING to topk[t, 0:k], padding with -1.
 * Positions are request-local.
 *
 * With refine != NULL the selection follows the exact scores instead of the
 * float32 ones: the set becomes the one obtained by ordering on
 *   I_exact[t,s] = s_k[s] * sum_{j ascending} u_j * max(d_j, 0),
 *   d_j = q_hat[t,j] . k_hat[s] (exact), u_j = w[t,j] * q_scale[t,j],
 * evaluated in float64 in exactly that order (one rounding per product and
 * per sum), provided every float32 score lies within
 *   eps_t = C * 2^-16 * 448 * smax_t * sum_j |u_j| * max_c |q_hat[t,j,c]|
 *           + (H_I + 3) * 2^-23 * |theta_t|
 * of its exact value (smax_t: the largest key scale of the 2048-position
 * chunks holding the row's visible keys, or an upper bound of it from the
 * key-scale table; theta_t: the k-th largest float32 score). The first term bounds the FP8 MFMA's accumulation error of each head
 * dot by C times 2^-16 of the largest possible product; the second, the float32
 * epilogue for nonnegative weights. EXACTNESS IS CONDITIONAL: with the default
 * C = 4 the bound is not derived but checked by measurement (the largest
 * observed |I_f32 - I_exact| / eps_t is 0.02-0.25 on the synthetic workloads),
 * and each refined row re-checks it on its own band keys (status -4).
 * C = 128 gives the worst case of the accumulation model (128 products each off
 * by up to 2^-16 of the largest), at the price of a band about 32 times wider.
 * Keys above theta_t + 2 eps_t are kept, keys below theta_t - 2 eps_t dropped,
 * and the band in between is rescored exactly and ranked by (I_exact desc,
 * s asc).
 *   scores [T, score_ld] float32 (as written by dsa_index_score)
 *   topk   [T, k] int32
 * Rows of up to 65536 visible scores take one block each. When max_kv_len
 * exceeds 65536, every row is first cut into 65536-position chunks whose own
 * top-k are selected in parallel (the row's top-k lies in their union), then
 * merged; with the refine, rows of up to 2^18 positions then classify and
 * rescore their band over many blocks (three more launches) before one block
 * per row ranks it.
 * Workspace: dsa_topk_workspace_size(B, T, max_kv_len, k, refine != NULL)
 * bytes, 16-byte aligned (0 bytes for rows of at most 65536 positions without a
 * refine; ws may then be NULL). Its contents need no initialisation.
 * Errors: DSA_ERR_INVALID_ARGUMENT (k < 1, k > 8192, refine with k > 4096,
 * D_I not 64/128, H_I not in [1, 128], ...), DSA_ERR_WORKSPACE_TOO_SMALL.
 */
dsa_status dsa_topk(const float* scores, int64_t score_ld, const int32_t* q_row_offsets,
                    const int64_t* kv_row_offsets, int32_t B, int32_t T, int32_t max_q_rows,
                    int64_t max_kv_len, int32_t k, const dsa_topk_refine* refine, int32_t* topk,
                    void* ws, size_t ws_bytes, void* stream);

size_t dsa_topk_workspace_size(int32_t B, int32_t T, int64_t max_kv_len, int32_t k,
                               int32_t refine);

/*
 * dsa_key_scale_max -- the key-scale table the refine of dsa_topk reads its
 * smax_t from, kept beside the index-key cache so that no call rescans the
 * scales. (The bound eps_t of dsa_topk needs the largest key scale among a
 * row's visible keys; "MAX Pipeline 中的 DeepSeek-V3.2 架构实现解析", "Indexer 的结构与计算流程":
 * the indexer K cache holds one fp32 scale per token.)
 *
 * For every chunk c = r / DSA_KEY_SCALE_CHUNK of a row r in [row_begin, row_end):
 *   k_scale_max[c] = max |k_scale[i]| over rows i of chunk c below N
 * (the whole chunk is recomputed, also rows outside [row_begin, row_end)).
 * Build it once over [0, N) after the cache is filled, again over a range after
 * writing that range in some other way; dsa_verify_cache_write with the table
 * keeps it up to date (raising entries only). Any entry at or above the true
 * maximum keeps the refine exact; a larger one only widens its band. Rows that
 * hold no key count with the scale stored there (0 keeps them out).
 *   k_scale [N] f32; k_scale_max [ceil(N / DSA_KEY_SCALE_CHUNK)] f32, both
 *   device pointers, 4-byte aligned; caller-owned.
 * Errors: DSA_ERR_INVALID_ARGUMENT (null pointers, not 0 <= row_begin <=
 * row_end <= N).
 */
dsa_status dsa_key_scale_max(const float* k_scale, int64_t N, int64_t row_begin, int64_t row_end,
                             float* k_scale_max, void* stream);

/*
 * dsa_index_topk -- the indexer scores and the refined top-k of every row in one call, with
 * no score row written to memory.
 * ("MAX Pipeline 中的 DeepSeek-V3.2 架构实现解析", "Indexer 的结构与计算流程": the indexer's
 * output is the top-k of shape (total_seq_len, index_topk), produced there by one fused
 * index-and-top-k operator.)
 *
 * Result: what dsa_index_score followed by dsa_topk with a refine gives (err_scale, status
 * as in dsa_topk_refine): each row's set by the exact scores, ascending, -1 padded; the
 * float32 scores are those of dsa_index_score's arithmetic. Steps:
 *   1. S evenly spaced keys of each request (S = 1024..8192, about one key in 32 of the
 *      longest request; positions floor(j n0 / S), n0 the first row's visible count) are
 *      scored;
 *   2. each row's threshold tau is the sample's m-th largest score, m = ceil(2.5 k S / n0)
 *      (-inf when m >= S: the row keeps every key);
 *   3. the scoring pass keeps only scores >= tau, with the largest key scale it saw;
 *   4. one block per row selects the k-th largest candidate theta and refines the band
 *      [theta - 2 eps, theta + 2 eps] exactly. A row with fewer than k or more than 8192
 *      candidates, or with theta - 2 eps < tau (band keys may lie below tau), is scored
 *      again in full by its own block and selected by the path of dsa_topk.
 *   path  [T] int32, nullable: 0 when the row was selected from its candidates, 1 when it
 *         was scored again (the result is the same either way).
 * Inputs as in dsa_index_score; k in [1, 4096].
 * Workspace: dsa_index_topk_workspace_size(B, T, max_q_rows, H_I, max_kv_len) bytes,
 * 256-byte aligned (at 32 x 65536 with 6 rows: about 105 MB).
 * Errors: DSA_ERR_INVALID_ARGUMENT, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE_TOO_SMALL.
 */
dsa_status dsa_index_topk(const uint8_t* q_fp8, const float* q_scale, const float* w,
                          const uint8_t* k_fp8, const float* k_scale,
                          const int32_t* q_row_offsets, const int64_t* kv_row_offsets, int32_t B,
                          int32_t T, int32_t max_q_rows, int32_t H_I, int32_t D_I,
                          int64_t max_kv_len, int32_t k, double err_scale, int32_t* status,
                          int32_t* path, int32_t* topk, void* ws, size_t ws_bytes, void* stream);

size_t dsa_index_topk_workspace_size(int32_t B, int32_t T, int32_t max_q_rows, int32_t H_I,
                                     int64_t max_kv_len);

/*
 * dsa_sparse_mla_decode -- attention of every query row over only its
 * selected latent rows.
 * ("MAX Pipeline 中的 DeepSeek-V3.2 架构实现解析", "稀疏 MLA 的前向路径"; latent row
 * = kv_lora_rank 512 + qk_rope_head_dim 64 from "GLM-5.3 推理全链路(十四)",
 * "GLM-5.3 的草稿层到底长什么样".)
 *
 * For row t (request b), head h, over the valid indices i of its top-k row
 * (entries < 0 or >= L_b are skipped):
 *   z_i = sm_scale * q[t,h,0:576] . kv[kv_row_offsets[b] + idx_i, 0:576]
 *   out[t,h,0:512] = sum_i softmax(z)_i * kv[., 0:512]   (bf16, fp32 accumulate)
 *   lse[t,h] = ln sum_i exp(z_i)  (natural log; optional)
 * No valid index: out = 0, lse = -inf.
 * Index sharing ("MAX 中 GLM-5.2 ... 统一 MTP 推测解码架构解析", "阶段 5"): when
 * share_base != NULL, every row of request b reads top-k row
 * share_base[b] + num_accepted[b] instead of row t (no copy is made).
 *   q [T, H, 576] bf16; kv [N, 576] bf16; topk [topk_rows, k] int32 (topk_rows >= T
 *   without a share map; a share map entry outside [0, topk_rows) selects nothing)
 *   out [T, H, 512] bf16; lse [T, H] float32 or NULL
 * H must be a multiple of 16, at most 128.
 * Workspace: dsa_sparse_mla_workspace_size() bytes, 0 unless a row's list is cut into
 * slices (small grids, or k > 2048): per (row, slice, head) the slice's normalised
 * output in bf16 and its (max, sum) in float32, merged by a second launch.
 * Errors: DSA_ERR_INVALID_ARGUMENT, DSA_ERR_UNSUPPORTED,
 * DSA_ERR_WORKSPACE_TOO_SMALL.
 */
dsa_status dsa_sparse_mla_decode(const uint16_t* q, const uint16_t* kv, const int32_t* topk,
                                 int32_t topk_rows, const int32_t* share_base, const int32_t* num_accepted,
                                 const int32_t* q_row_offsets, const int64_t* kv_row_offsets,
                                 int32_t B, int32_t T, int32_t max_q_rows, int32_t H, int32_t k,
                                 float sm_scale, uint16_t* out, float* lse, void* ws,
                                 size_t ws_bytes, void* stream);

size_t dsa_sparse_mla_workspace_size(int32_t T, int32_t H, int32_t k);

/*
 * dsa_mla_fp8_pack -- FP8 latent cache rows from bf16 latent rows.
 * ("GLM-5.3 推理全链路(十四)", the draft-layer section: the KV pool holds 656 bytes per
 * token per layer in the fp8_ds_mla layout; "MAX Pipeline 中的 DeepSeek-V3.2 架构实现解析",
 * "配置体系": float8_e4m3fn caches with float32 scales.)
 *
 * Row layout, 656 bytes (rows are 16-byte aligned when the array is):
 *   bytes [0, 512)   e4m3fn code of latent value c = 0..511
 *   bytes [512, 528) float32 scale of latent block b = 0..3 (values 128b .. 128b+127):
 *                    amax_b / 448 rounded to float32, 1 when amax_b == 0
 *   bytes [528, 656) the 64 rope values (latent dims 512..575), bf16 copied bit for bit
 * code = e4m3fn(x / scale_b): float32 division, round to nearest even, saturating at
 * +-448. A code stands for decode(code) * scale_b.
 * For i < n: row dst_rows[i] (row i when dst_rows is NULL) of kv_fp8 = pack(latent[i]).
 *   latent [n, 576] bf16; dst_rows [n] int64 device array or NULL (distinct rows,
 *   trusted); kv_fp8 [N, 656] u8. latent and kv_fp8 16-byte aligned.
 * Errors: DSA_ERR_INVALID_ARGUMENT (n < 0, null or misaligned pointers).
 */
dsa_status dsa_mla_fp8_pack(const uint16_t* latent, const int64_t* dst_rows, int64_t n,
                            uint8_t* kv_fp8, void* stream);

/*
 * dsa_sparse_mla_decode_fp8 -- dsa_sparse_mla_decode over an FP8 latent cache.
 * (The passages of dsa_sparse_mla_decode; the rows are those of dsa_mla_fp8_pack.)
 *
 * Same arguments, results, workspace and errors as dsa_sparse_mla_decode, with
 * kv_fp8 [N, 656] u8 (16-byte aligned) in place of kv: a row stands for
 * decode(code) * scale_b in its 512 latent dims and for its bf16 rope in the last 64.
 * The codes enter the bf16 MFMAs exactly; the scales are applied in float32, to each
 * block's partial logit and to the PV weights (which are rounded to bf16 after the
 * scale, as the bf16 path rounds its weights).
 */
dsa_status dsa_sparse_mla_decode_fp8(const uint16_t* q, const uint8_t* kv_fp8,
                                     const int32_t* topk, int32_t topk_rows,
                                     const int32_t* share_base, const int32_t* num_accepted,
                                     const int32_t* q_row_offsets, const int64_t* kv_row_offsets,
                                     int32_t B, int32_t T, int32_t max_q_rows, int32_t H, int32_t k,
                                     float sm_scale, uint16_t* out, float* lse, void* ws,
                                     size_t ws_bytes, void* stream);

/*
 * greedy_accept -- greedy acceptance of a chain of K drafts per request.
 * ("GLM-5.3 推理全链路(十四)", "接受判定:greedy 与 rejection sampling": the target
 * argmax of row i is compared with draft i, stopping at the first mismatch;
 * "验证输入是怎么拼出来的": verify rows are cat(bonus, drafts).)
 *
 * Logits row b*(K+1)+i is the target distribution after verify row i.
 *   a[b,i] = smallest v attaining max_v logits[b*(K+1)+i, v]  (values, -0 == +0)
 *   num_accepted[b] = largest n <= K with draft[b,i] == a[b,i] for all i < n
 *   next_token[b]   = a[b, num_accepted[b]]
 *   argmax[b*(K+1)+i] = a[b,i] (optional)
 * accept length (bonus included) is num_accepted + 1.
 *   logits [B*(K+1), logits_ld] float32 or bf16 (dtype); draft [B, K] int32
 * Workspace: greedy_accept_workspace_size() bytes. Logits must not be NaN.
 * Errors: DSA_ERR_INVALID_ARGUMENT, DSA_ERR_WORKSPACE_TOO_SMALL.
 */
dsa_status greedy_accept(const void* logits, int32_t dtype, int64_t logits_ld,
                         const int32_t* draft, int32_t B, int32_t K, int32_t V,
                         int32_t* num_accepted, int32_t* next_token, int32_t* argmax, void* ws,
                         size_t ws_bytes, void* stream);

size_t greedy_accept_workspace_size(int32_t B, int32_t K, int32_t V);

/*
 * greedy_accept_noalloc -- greedy_accept for callers that cannot allocate: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. Same inputs, outputs,
 * results and errors as greedy_accept, without the workspace arguments: the per-slice maxima
 * go to a fixed scratch array of DSA_NOALLOC_SCRATCH_BYTES in each device's memory, held
 * until the process ends (its address is looked up once per device, on the first call made
 * with that device current). The call allocates and frees nothing.
 * Limit: greedy_accept_workspace_size(B, K, V) <= DSA_NOALLOC_SCRATCH_BYTES (for V = 151552,
 * up to 3542 logits rows); larger batches return DSA_ERR_WORKSPACE_TOO_SMALL before any
 * launch. Every call on a device shares that device's array: calls that overlap on one
 * device (concurrent streams, or threads) race; calls on one stream are ordered.
 * Nothing in the array needs clearing between calls (each call writes every entry it reads).
 */
#define DSA_NOALLOC_SCRATCH_BYTES (1u << 20)

dsa_status greedy_accept_noalloc(const void* logits, int32_t dtype, int64_t logits_ld,
                                 const int32_t* draft, int32_t B, int32_t K, int32_t V,
                                 int32_t* num_accepted, int32_t* next_token, int32_t* argmax,
                                 void* stream);

/*
 * rejection_accept -- acceptance of a chain of K drafts per request by rejection
 * sampling.
 * ("GLM-5.3 推理全链路(十四)", "接受判定:greedy 与 rejection sampling": draft i is kept
 * with probability min(1, p/q), q the draft distribution and p the target's; at the
 * first refused step a token is drawn from the corrected distribution as that step's
 * bonus.)
 *
 * With p_i = softmax(logits row b*(K+1)+i) over V and the uniforms as inputs:
 *   draft i is kept iff u[b,i] * draft_probs[b,i,x_i] < p_i(x_i), x_i = draft[b,i]
 *   num_accepted[b] = n = the first refused i (K when none is refused)
 *   w(v) = max(0, p_n(v) - draft_probs[b,n,v]) if n < K, else p_K(v); w = p_n if it
 *          sums to 0
 *   next_token[b] = the smallest v with C(v) > us[b] * C(V-1), C the running sum of w
 *   logits [B*(K+1), logits_ld] float32 or bf16 (dtype); draft_probs [B, K, V] float32;
 *   draft [B, K] int32; u [B, K] and us [B] float32 in [0, 1).
 * Probabilities and sums are taken in float64 except the exponentials of the softmax
 * denominators (float32, summed in float64). A draft outside [0, V) counts as refused.
 * Workspace: rejection_accept_workspace_size() bytes, 8-byte aligned.
 * Errors: DSA_ERR_INVALID_ARGUMENT, DSA_ERR_WORKSPACE_TOO_SMALL.
 */
dsa_status rejection_accept(const void* logits, int32_t dtype, int64_t logits_ld,
                            const float* draft_probs, const int32_t* draft, const float* u,
                            const float* us, int32_t B, int32_t K, int32_t V,
                            int32_t* num_accepted, int32_t* next_token, void* ws, size_t ws_bytes,
                            void* stream);

size_t rejection_accept_workspace_size(int32_t B, int32_t K, int32_t V);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
