// rejection_accept.hip -- acceptance of a draft chain by rejection sampling.
//
// "GLM-5.3 推理全链路(十四)", section "接受判定:greedy 与 rejection sampling": draft token i
// is kept with probability min(1, p/q), q being the draft distribution and p the target's;
// at the first refused step a token is drawn from the corrected distribution and is that
// step's bonus. Verify rows are cat(bonus, drafts) ("验证输入是怎么拼出来的"), so logits
// row b*(K+1)+i is the target distribution after verify row i.
//
// With p_i = softmax(logits row b*(K+1)+i) and the uniforms given as inputs:
//   draft i is kept iff u[b,i] * q_i(x_i) < p_i(x_i);
//   n_b = the first refused i (K if none);
//   w(v) = max(0, p_n(v) - q_n(v)) for n < K, p_K(v) for n = K; w = p_n if it sums to 0;
//   next_token[b] = the smallest v with C(v) > us[b] * C(V-1), C the running sum of w.
//
// Four launches, HBM-bound (the logits are read once in full, the draw's row twice):
//  1. stats: per (row, 4096-entry slice), the slice maximum m and sum_v exp(l_v - m)
//     (float32 exponentials summed in float64);
//  2. decide: one wave per request merges the slices of each row it needs (float64) and
//     takes the accept decisions in float64, stopping at the first refusal;
//  3. weights: per (request, slice) of the drawing row, the sums of w (and of p, for the
//     fallback) in float64, with p(v) = exp(l_v - M) / S in float64;
//  4. draw: one block per request finds the slice holding us * W, then the entry inside
//     it by a block scan in float64.
#include "common.hpp"

namespace dsa {
namespace {

constexpr int RA_THREADS = 256;
constexpr int RA_SLICE = 4096;                  // vocabulary entries per block
constexpr int RA_PER = RA_SLICE / RA_THREADS;   // entries per thread (16)

template <bool BF16>
__device__ __forceinline__ float logit(const void* lg, int64_t idx) {
  if constexpr (BF16)
    return bf16_bits_to_f32(static_cast<const uint16_t*>(lg)[idx]);
  else
    return static_cast<const float*>(lg)[idx];
}

__device__ __forceinline__ double block_sum_d(double x, double* red) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  const int wave = threadIdx.x / 64;
  if (threadIdx.x % 64 == 0) red[wave] = x;
  __syncthreads();
  double s = 0.0;
  for (int w = 0; w < RA_THREADS / 64; ++w) s += red[w];
  __syncthreads();
  return s;
}

__device__ __forceinline__ float block_max_f(float x, float* red) {
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  const int wave = threadIdx.x / 64;
  if (threadIdx.x % 64 == 0) red[wave] = x;
  __syncthreads();
  float m = red[0];
  for (int w = 1; w < RA_THREADS / 64; ++w) m = fmaxf(m, red[w]);
  __syncthreads();
  return m;
}

// 1. slice statistics of every logits row
template <bool BF16>
__global__ __launch_bounds__(RA_THREADS) void ra_stats_kernel(const void* __restrict__ logits,
                                                              int64_t ld, int V, int nslice,
                                                              float* __restrict__ ws_m,
                                                              double* __restrict__ ws_s) {
  __shared__ float redf[RA_THREADS / 64];
  __shared__ double redd[RA_THREADS / 64];
  const int slice = blockIdx.x;
  const int64_t row = blockIdx.y;
  const int v0 = slice * RA_SLICE;
  float x[RA_PER];
  float m = -INFINITY;
#pragma unroll
  for (int e = 0; e < RA_PER; ++e) {
    const int v = v0 + e * RA_THREADS + threadIdx.x;
    x[e] = v < V ? logit<BF16>(logits, row * ld + v) : -INFINITY;
    m = fmaxf(m, x[e]);
  }
  m = block_max_f(m, redf);
  double s = 0.0;
  if (m > -INFINITY) {
#pragma unroll
    for (int e = 0; e < RA_PER; ++e) s += static_cast<double>(expf(x[e] - m));
  }
  s = block_sum_d(s, redd);
  if (threadIdx.x == 0) {
    ws_m[row * nslice + slice] = m;
    ws_s[row * nslice + slice] = s;
  }
}

// (M, S) of one row from its slices, by one wave (every lane gets the result)
__device__ __forceinline__ void row_stats(const float* ws_m, const double* ws_s, int64_t row,
                                          int nslice, double* M, double* S) {
  const int lane = threadIdx.x % 64;
  float m = -INFINITY;
  for (int j = lane; j < nslice; j += 64) m = fmaxf(m, ws_m[row * nslice + j]);
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  double s = 0.0;
  for (int j = lane; j < nslice; j += 64) {
    const float mj = ws_m[row * nslice + j];
    if (mj > -INFINITY) s += ws_s[row * nslice + j] * exp(static_cast<double>(mj) - m);
  }
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  *M = m;
  *S = s;
}

// 2. accept decisions, one wave per request; writes n and the drawing row's (M, S)
template <bool BF16>
__global__ __launch_bounds__(64) void ra_decide_kernel(
    const void* __restrict__ logits, int64_t ld, const float* __restrict__ draft_probs,
    const int32_t* __restrict__ draft, const float* __restrict__ u, int K, int V, int nslice,
    const float* __restrict__ ws_m, const double* __restrict__ ws_s, int32_t* __restrict__ ws_n,
    double* __restrict__ ws_ms, int32_t* __restrict__ num_accepted) {
  const int b = blockIdx.x;
  int n = 0;
  double M = 0.0, S = 0.0;
  for (; n < K; ++n) {
    const int64_t row = static_cast<int64_t>(b) * (K + 1) + n;
    row_stats(ws_m, ws_s, row, nslice, &M, &S);
    const int32_t x = draft[static_cast<int64_t>(b) * K + n];
    if (x < 0 || x >= V) break;  // an out-of-range draft is refused
    const double p = exp(static_cast<double>(logit<BF16>(logits, row * ld + x)) - M) / S;
    const double uq = static_cast<double>(u[static_cast<int64_t>(b) * K + n]) *
                      static_cast<double>(draft_probs[(static_cast<int64_t>(b) * K + n) * V + x]);
    if (!(uq < p)) break;
  }
  if (n == K) row_stats(ws_m, ws_s, static_cast<int64_t>(b) * (K + 1) + K, nslice, &M, &S);
  if (threadIdx.x == 0) {
    ws_n[b] = n;
    ws_ms[2 * b] = M;
    ws_ms[2 * b + 1] = S;
    num_accepted[b] = n;
  }
}

// w(v) of the drawing row: corrected (rw) or target (pv) probability
template <bool BF16>
__device__ __forceinline__ void weights_at(const void* logits, int64_t ld, const float* draft_probs,
                                           int b, int n, int K, int V, double M, double S, int v,
                                           double* rw, double* pv) {
  const int64_t row = static_cast<int64_t>(b) * (K + 1) + n;
  const double p = v < V ? exp(static_cast<double>(logit<BF16>(logits, row * ld + v)) - M) / S : 0.0;
  double r = p;
  if (n < K && v < V) {
    const double d = p - static_cast<double>(draft_probs[(static_cast<int64_t>(b) * K + n) * V + v]);
    r = d > 0.0 ? d : 0.0;
  }
  *rw = r;
  *pv = p;
}

// 3. per (request, slice): sums of the corrected weights and of p over the drawing row
template <bool BF16>
__global__ __launch_bounds__(RA_THREADS) void ra_weights_kernel(
    const void* __restrict__ logits, int64_t ld, const float* __restrict__ draft_probs, int K,
    int V, int nslice, const int32_t* __restrict__ ws_n, const double* __restrict__ ws_ms,
    double* __restrict__ ws_w, double* __restrict__ ws_p) {
  __shared__ double redd[RA_THREADS / 64];
  const int slice = blockIdx.x, b = blockIdx.y;
  const int n = ws_n[b];
  const double M = ws_ms[2 * b], S = ws_ms[2 * b + 1];
  double sw = 0.0, sp = 0.0;
#pragma unroll 4
  for (int e = 0; e < RA_PER; ++e) {
    double rw, pv;
    weights_at<BF16>(logits, ld, draft_probs, b, n, K, V, M, S,
                     slice * RA_SLICE + e * RA_THREADS + static_cast<int>(threadIdx.x), &rw, &pv);
    sw += rw;
    sp += pv;
  }
  sw = block_sum_d(sw, redd);
  sp = block_sum_d(sp, redd);
  if (threadIdx.x == 0) {
    ws_w[static_cast<int64_t>(b) * nslice + slice] = sw;
    ws_p[static_cast<int64_t>(b) * nslice + slice] = sp;
  }
}

// 4. the draw, one block per request
template <bool BF16>
__global__ __launch_bounds__(RA_THREADS) void ra_draw_kernel(
    const void* __restrict__ logits, int64_t ld, const float* __restrict__ draft_probs, int K,
    int V, int nslice, const float* __restrict__ us, const int32_t* __restrict__ ws_n,
    const double* __restrict__ ws_ms, const double* __restrict__ ws_w,
    const double* __restrict__ ws_p, int32_t* __restrict__ next_token) {
  __shared__ double wsum[RA_THREADS / 64];
  __shared__ int pick[2];  // slice, then token
  const int b = blockIdx.x;
  const int n = ws_n[b];
  const double M = ws_ms[2 * b], S = ws_ms[2 * b + 1];
  const double* sl = ws_w + static_cast<int64_t>(b) * nslice;
  // corrected law unless it is empty; slice sums in index order by one thread
  if (threadIdx.x == 0) {
    double W = 0.0;
    for (int j = 0; j < nslice; ++j) W += sl[j];
    bool use_p = !(W > 0.0);
    if (use_p) {
      sl = ws_p + static_cast<int64_t>(b) * nslice;
      W = 0.0;
      for (int j = 0; j < nslice; ++j) W += sl[j];
    }
    const double target = static_cast<double>(us[b]) * W;
    double c = 0.0;
    int js = -1, last = 0;
    for (int j = 0; j < nslice; ++j) {
      if (sl[j] > 0.0) last = j;
      if (js < 0 && c + sl[j] > target) js = j;
      c += sl[j];
    }
    // rounding left the target at or above the total: the last slice with weight
    pick[0] = js >= 0 ? js : last;
    pick[1] = use_p ? 1 : 0;
    wsum[0] = target;
    double before = 0.0;
    for (int j = 0; j < pick[0]; ++j) before += sl[j];
    wsum[1] = before;
  }
  __syncthreads();
  const int js = pick[0];
  const bool use_p = pick[1] != 0;
  const double target = wsum[0], before = wsum[1];
  __syncthreads();
  // entries of slice js in index order: thread t holds 16 consecutive ones
  const int v0 = js * RA_SLICE + static_cast<int>(threadIdx.x) * RA_PER;
  double w[RA_PER];
  double tsum = 0.0;
#pragma unroll
  for (int e = 0; e < RA_PER; ++e) {
    double rw, pv;
    weights_at<BF16>(logits, ld, draft_probs, b, n, K, V, M, S, v0 + e, &rw, &pv);
    w[e] = use_p ? pv : rw;
    tsum += w[e];
  }
  // exclusive scan of the thread sums (block, float64)
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  double incl = tsum;
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  __shared__ double wtot[RA_THREADS / 64];
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  double c = before + incl - tsum;
  for (int x = 0; x < wave; ++x) c += wtot[x];
  int found = 0x7FFFFFFF, lastpos = -1;
#pragma unroll
  for (int e = 0; e < RA_PER; ++e) {
    const double cn = c + w[e];
    if (found == 0x7FFFFFFF && cn > target && w[e] > 0.0) found = v0 + e;
    if (w[e] > 0.0) lastpos = v0 + e;
    c = cn;
  }
  // the smallest qualifying entry, else the slice's last entry with weight
  for (int o = 32; o >= 1; o >>= 1) {
    found = min(found, __shfl_xor(found, o));
    lastpos = max(lastpos, __shfl_xor(lastpos, o));
  }
  __shared__ int fnd[RA_THREADS / 64], lst[RA_THREADS / 64];
  if (lane == 0) {
    fnd[wave] = found;
    lst[wave] = lastpos;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int f = 0x7FFFFFFF, l = -1;
    for (int x = 0; x < RA_THREADS / 64; ++x) {
      f = min(f, fnd[x]);
      l = max(l, lst[x]);
    }
    next_token[b] = f != 0x7FFFFFFF ? f : l;
  }
}

}  // namespace
}  // namespace dsa

extern "C" size_t rejection_accept_workspace_size(int32_t B, int32_t K, int32_t V) {
  if (B <= 0 || K < 0 || V <= 0) return 0;
  const int64_t ns = dsa::ceil_div(V, dsa::RA_SLICE);
  const int64_t rows = static_cast<int64_t>(B) * (K + 1);
  // doubles first (8-byte aligned), then floats and ints
  return static_cast<size_t>(rows * ns * 8 + 2 * B * 8 + 2 * B * ns * 8 + rows * ns * 4 + B * 4);
}

extern "C" dsa_status rejection_accept(const void* logits, int32_t dtype, int64_t logits_ld,
                                       const float* draft_probs, const int32_t* draft,
                                       const float* u, const float* us, int32_t B, int32_t K,
                                       int32_t V, int32_t* num_accepted, int32_t* next_token,
                                       void* ws, size_t ws_bytes, void* stream) {
  using namespace dsa;
  DSA_REQUIRE(dtype == DSA_F32 || dtype == DSA_BF16, "rejection_accept: dtype must be DSA_F32 or DSA_BF16");
  DSA_REQUIRE(B >= 0 && K >= 0 && K <= 63, "rejection_accept: need B >= 0 and 0 <= K <= 63");
  DSA_REQUIRE(V >= 1 && logits_ld >= V, "rejection_accept: need V >= 1 and logits_ld >= V");
  if (B == 0) return ok();
  DSA_REQUIRE(logits && us && num_accepted && next_token && (K == 0 || (draft_probs && draft && u)),
              "rejection_accept: null pointer");
  const int64_t rows = static_cast<int64_t>(B) * (K + 1);
  DSA_REQUIRE(rows <= 65535, "rejection_accept: B*(K+1) must be <= 65535");
  const size_t need = rejection_accept_workspace_size(B, K, V);
  if (!ws || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "rejection_accept: workspace needs %zu bytes (got %zu)",
                need, ws_bytes);
  DSA_REQUIRE((reinterpret_cast<uintptr_t>(ws) & 7) == 0, "rejection_accept: workspace must be 8-byte aligned");
  const int nslice = static_cast<int>(ceil_div(V, RA_SLICE));
  double* ws_s = static_cast<double*>(ws);
  double* ws_ms = ws_s + rows * nslice;
  double* ws_w = ws_ms + 2 * B;
  double* ws_p = ws_w + static_cast<int64_t>(B) * nslice;
  float* ws_m = reinterpret_cast<float*>(ws_p + static_cast<int64_t>(B) * nslice);
  int32_t* ws_n = reinterpret_cast<int32_t*>(ws_m + rows * nslice);
  hipStream_t st = as_stream(stream);
  const bool bf = dtype == DSA_BF16;
  if (bf)
    hipLaunchKernelGGL(ra_stats_kernel<true>, dim3((unsigned)nslice, (unsigned)rows), dim3(RA_THREADS), 0,
                       st, logits, logits_ld, V, nslice, ws_m, ws_s);
  else
    hipLaunchKernelGGL(ra_stats_kernel<false>, dim3((unsigned)nslice, (unsigned)rows), dim3(RA_THREADS), 0,
                       st, logits, logits_ld, V, nslice, ws_m, ws_s);
  dsa_status s = check_launch("rejection_accept(stats)");
  if (s != DSA_OK) return s;
  if (bf)
    hipLaunchKernelGGL(ra_decide_kernel<true>, dim3((unsigned)B), dim3(64), 0, st, logits, logits_ld,
                       draft_probs, draft, u, K, V, nslice, ws_m, ws_s, ws_n, ws_ms, num_accepted);
  else
    hipLaunchKernelGGL(ra_decide_kernel<false>, dim3((unsigned)B), dim3(64), 0, st, logits, logits_ld,
                       draft_probs, draft, u, K, V, nslice, ws_m, ws_s, ws_n, ws_ms, num_accepted);
  s = check_launch("rejection_accept(decide)");
  if (s != DSA_OK) return s;
  if (bf)
    hipLaunchKernelGGL(ra_weights_kernel<true>, dim3((unsigned)nslice, (unsigned)B), dim3(RA_THREADS), 0,
                       st, logits, logits_ld, draft_probs, K, V, nslice, ws_n, ws_ms, ws_w, ws_p);
  else
    hipLaunchKernelGGL(ra_weights_kernel<false>, dim3((unsigned)nslice, (unsigned)B), dim3(RA_THREADS), 0,
                       st, logits, logits_ld, draft_probs, K, V, nslice, ws_n, ws_ms, ws_w, ws_p);
  s = check_launch("rejection_accept(weights)");
  if (s != DSA_OK) return s;
  if (bf)
    hipLaunchKernelGGL(ra_draw_kernel<true>, dim3((unsigned)B), dim3(RA_THREADS), 0, st, logits, logits_ld,
                       draft_probs, K, V, nslice, us, ws_n, ws_ms, ws_w, ws_p, next_token);
  else
    hipLaunchKernelGGL(ra_draw_kernel<false>, dim3((unsigned)B), dim3(RA_THREADS), 0, st, logits, logits_ld,
                       draft_probs, K, V, nslice, us, ws_n, ws_ms, ws_w, ws_p, next_token);
  return check_launch("rejection_accept(draw)");
}
