// topk.hip -- per-row top-k over the indexer scores (radix select in LDS).
//
// "MAX Pipeline 中的 DeepSeek-V3.2 架构实现解析", section "Indexer 的结构与计算流程": the
// indexer output is a top-k of shape (total_seq_len, index_topk); "GLM-5.3 推理全链路
// (十四)", section "验证段的逐层算子": each verify query selects its own 2048 keys.
//
// Selection order: (score desc, position asc). Scores map to order-preserving
// 32-bit keys (-0.0 canonicalised to +0.0, so equal values tie on position).
// One 1024-thread block per row:
//   1. three LDS histogram passes (11 + 11 + 10 key bits) find the exact k-th
//      largest key theta and how many keys lie strictly above it;
//   2. one ordered pass emits every position with key > theta plus the lowest
//      positions with key == theta, using block prefix sums in position order,
//      so the output comes out ascending with no sort.
// The row is read four times; after the first pass it is served from L2/MALL.
#include "common.hpp"

namespace dsa {
namespace {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x == 0.0f ? 0.0f : x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive block-wide prefix sum over TK_THREADS threads; *total gets the sum.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  if (wave == 0) {
    uint32_t s = lane < TK_WAVES ? tmp[lane] : 0u;
#pragma unroll
    for (int o = 1; o < TK_WAVES; o <<= 1) {
      uint32_t y = __shfl_up(s, o);
      if (lane >= o) s += y;
    }
    if (lane < TK_WAVES) tmp[TK_WAVES + lane] = s;  // inclusive wave totals
  }
  __syncthreads();
  const uint32_t before = wave ? tmp[TK_WAVES + wave - 1] : 0u;
  *total = tmp[2 * TK_WAVES - 1];
  __syncthreads();
  return before + x - v;
}

__global__ __launch_bounds__(TK_THREADS) void topk_kernel(const float* __restrict__ scores,
                                                          int64_t ld,
                                                          const int32_t* __restrict__ q_off,
                                                          const int64_t* __restrict__ kv_off,
                                                          int k, int32_t* __restrict__ topk) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t tmp[2 * TK_WAVES];
  __shared__ uint32_t sel_bin, sel_above;

  const int b = blockIdx.y, r = blockIdx.x;
  const RowInfo ri = load_row_info(q_off, kv_off, b);
  if (r >= ri.R) return;
  const int64_t t = ri.t0 + r;
  int64_t n = visible_count(ri, r);
  if (n > ld) n = ld;  // device lengths beyond the score stride are clipped
  int32_t* out = topk + t * k;
  const int tid = threadIdx.x;
  if (n <= k) {
    for (int i = tid; i < k; i += TK_THREADS) out[i] = i < n ? i : -1;
    return;
  }
  const float* srow = scores + t * ld;
  const int64_t n4 = n / 4;
  const float4* srow4 = reinterpret_cast<const float4*>(srow);

  // ---- 1. radix select of the k-th largest key ----
  uint32_t prefix = 0;       // high bits of theta fixed so far
  uint32_t need = k;         // keys still to take among those matching prefix
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
#pragma unroll 1
  for (int level = 0; level < 3; ++level) {
    const int sh = shifts[level], nb = 1 << widths[level];
    const int hi_sh = sh + widths[level];  // bits above this level must equal prefix
    for (int i = tid; i < nb; i += TK_THREADS) hist[i] = 0;
    __syncthreads();
    auto add = [&](float x) {
      const uint32_t key = order_key(x);
      if (level == 0 || (key >> hi_sh) == prefix) atomicAdd(&hist[(key >> sh) & (nb - 1)], 1u);
    };
    for (int64_t i = tid; i < n4; i += TK_THREADS) {
      const float4 v = srow4[i];
      add(v.x); add(v.y); add(v.z); add(v.w);
    }
    for (int64_t i = n4 * 4 + tid; i < n; i += TK_THREADS) add(srow[i]);
    __syncthreads();
    // bins in descending order: thread j covers desc slots 2j, 2j+1
    const int d0 = 2 * tid, d1 = 2 * tid + 1;
    const uint32_t c0 = d0 < nb ? hist[nb - 1 - d0] : 0u;
    const uint32_t c1 = d1 < nb ? hist[nb - 1 - d1] : 0u;
    uint32_t total;
    const uint32_t ex = block_excl_scan(c0 + c1, tmp, &total);
    if (ex < need && need <= ex + c0) {
      sel_bin = nb - 1 - d0;
      sel_above = ex;
    } else if (ex + c0 < need && need <= ex + c0 + c1) {
      sel_bin = nb - 1 - d1;
      sel_above = ex + c0;
    }
    __syncthreads();
    prefix = (prefix << widths[level]) | sel_bin;
    need -= sel_above;
    __syncthreads();
  }
  const uint32_t theta = prefix;  // exact key of the k-th largest score
  // keys > theta: k - need of them; ties at theta: take the `need` lowest positions

  // ---- 2. ordered emission ----
  uint32_t eq_seen = 0, emitted = 0;
  for (int64_t base = 0; base < n; base += 4 * TK_THREADS) {
    const int64_t p0 = base + 4 * tid;
    uint32_t key[4];
    bool live[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      live[j] = p0 + j < n;
      key[j] = live[j] ? order_key(srow[p0 + j]) : 0u;
    }
    uint32_t eqc = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) eqc += (live[j] && key[j] == theta) ? 1u : 0u;
    uint32_t eq_total;
    uint32_t eq_rank = eq_seen + block_excl_scan(eqc, tmp, &eq_total);
    bool sel[4];
    uint32_t selc = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool gt = live[j] && key[j] > theta;
      const bool eq = live[j] && key[j] == theta;
      sel[j] = gt || (eq && eq_rank < need);
      if (eq) ++eq_rank;
      selc += sel[j] ? 1u : 0u;
    }
    uint32_t sel_total;
    uint32_t pos = emitted + block_excl_scan(selc, tmp, &sel_total);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (sel[j] && pos < static_cast<uint32_t>(k)) out[pos++] = static_cast<int32_t>(p0 + j);
    eq_seen += eq_total;
    emitted += sel_total;
  }
}

}  // namespace
}  // namespace dsa

extern "C" size_t dsa_topk_workspace_size(int32_t, int64_t, int32_t) { return 0; }

extern "C" dsa_status dsa_topk(const float* scores, int64_t score_ld,
                               const int32_t* q_row_offsets, const int64_t* kv_row_offsets,
                               int32_t B, int32_t T, int32_t max_q_rows, int64_t max_kv_len,
                               int32_t k, int32_t* topk, void* ws, size_t ws_bytes,
                               void* stream) {
  using namespace dsa;
  (void)ws;
  (void)ws_bytes;
  DSA_REQUIRE(k >= 1 && k <= 8192, "dsa_topk: k must be in [1, 8192] (got %d)", k);
  DSA_REQUIRE(B >= 0 && T >= 0 && max_q_rows >= 0 && max_kv_len >= 0, "dsa_topk: negative size");
  DSA_REQUIRE(score_ld >= max_kv_len && score_ld % 4 == 0,
              "dsa_topk: score_ld must be >= max_kv_len and a multiple of 4");
  DSA_REQUIRE(max_kv_len < (int64_t(1) << 31), "dsa_topk: max_kv_len must be < 2^31");
  if (B == 0 || T == 0 || max_q_rows == 0) return ok();
  DSA_REQUIRE(scores && q_row_offsets && kv_row_offsets && topk, "dsa_topk: null pointer");
  DSA_REQUIRE((reinterpret_cast<uintptr_t>(scores) & 15) == 0,
              "dsa_topk: scores must be 16-byte aligned");
  DSA_REQUIRE(B <= 65535, "dsa_topk: B must be <= 65535");
  dim3 grid((unsigned)max_q_rows, (unsigned)B);
  hipLaunchKernelGGL(topk_kernel, grid, dim3(TK_THREADS), 0, as_stream(stream), scores, score_ld,
                     q_row_offsets, kv_row_offsets, k, topk);
  return check_launch("dsa_topk");
}
