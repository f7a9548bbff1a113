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
//  1. stats: per (row, 16384-entry slice, 16-byte loads), the slice maximum m and
//     sum_v exp(l_v - m): per-thread pairs merged in one block reduction (float32
//     exponentials, float64 sums);
//  2. decide: one block per request, wave i merging the slices of row i (float64) and
//     testing draft i; the first refusal ends the chain;
//  3. weights: per (request, slice) of the drawing row, the sums of w (and of p, for the
//     fallback) in float64, with p(v) = exp(l_v - M) / S (float32 exponential of the
//     exact float32 difference, float64 division);
//  4. draw: one block per request finds the slice holding us * W, then the entry inside
//     it by a block scan in float64.
#include "common.hpp"

namespace dsa {
namespace {

constexpr int RA_THREADS = 256;
constexpr int RA_SLICE = 16384;                 // vocabulary entries per block
constexpr int RA_PER = RA_SLICE / RA_THREADS;   // entries per thread (64)

// e^d for d <= 0 (a logit minus a maximum): 2^(d log2 e) with the product's rounding error
// and the constant's own error carried to first order, d*log2e = y + t, 2^(y+t) = 2^y (1 +
// t ln 2); about one ulp in a handful of instructions. Exactly 0 below -104 (where e^d is
// under the float32 range) and for -inf.
__device__ __forceinline__ float exp_nonpos(float d) {
  constexpr float L2E = 1.44269502163f;          // log2(e) rounded to float32
  constexpr float L2E_LO = 1.925963033e-8f;       // log2(e) - L2E
  constexpr float LN2 = 0.693147180560f;
  const bool live = d > -104.0f;
  const float dc = live ? d : -104.0f;
  const float y = dc * L2E;
  float t = fmaf(dc, L2E, -y);  // exact error of the rounded product
  t = fmaf(dc, L2E_LO, t);
  const float r = __builtin_amdgcn_exp2f(y);
  return live ? fmaf(r, t * LN2, r) : 0.0f;
}

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

// This thread's RA_PER consecutive-in-groups entries of a slice: 16-byte loads of 8 bf16
// (or 4 float32) at units threadIdx.x + j * RA_THREADS; entries past V read as -inf.
template <bool BF16>
__device__ __forceinline__ void load_slice(const void* lg, int64_t row_start, int v0, int V,
                                           float (&x)[RA_PER]) {
  constexpr int E = BF16 ? 8 : 4;  // entries per 16-byte unit
  constexpr int EB = BF16 ? 2 : 4;  // bytes per entry
  if (v0 + RA_SLICE <= V && (row_start * EB) % 16 == 0) {  // block-uniform: every load issued
    const i32x4* src = reinterpret_cast<const i32x4*>(static_cast<const uint8_t*>(lg) +
                                                      (row_start + v0) * EB);
    i32x4 d[RA_PER / E];
#pragma unroll
    for (int j = 0; j < RA_PER / E; ++j) d[j] = src[j * RA_THREADS + threadIdx.x];
#pragma unroll
    for (int j = 0; j < RA_PER / E; ++j)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint32_t wd = static_cast<uint32_t>(d[j][BF16 ? e / 2 : e]);
        x[j * E + e] = BF16 ? __uint_as_float((e & 1) ? (wd & 0xFFFF0000u) : (wd << 16))
                            : __uint_as_float(wd);
      }
    return;
  }
#pragma unroll
  for (int j = 0; j < RA_PER / E; ++j) {
    const int v = v0 + (j * RA_THREADS + static_cast<int>(threadIdx.x)) * E;
    if (v + E <= V && ((row_start + v) * (BF16 ? 2 : 4)) % 16 == 0) {
      const i32x4 d = reinterpret_cast<const i32x4*>(
          static_cast<const uint8_t*>(lg) + (row_start + v) * (BF16 ? 2 : 4))[0];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint32_t wd = static_cast<uint32_t>(d[BF16 ? e / 2 : e]);
        x[j * E + e] = BF16 ? __uint_as_float((e & 1) ? (wd & 0xFFFF0000u) : (wd << 16))
                            : __uint_as_float(wd);
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e)
        x[j * E + e] = v + e < V ? logit<BF16>(lg, row_start + v + e) : -INFINITY;
    }
  }
}

// (m, s) pairs merged to the larger reference: s = s1 e^(m1-M) + s2 e^(m2-M)
__device__ __forceinline__ void merge_ms(float& m, double& sum, float m2, double s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  sum = sum * static_cast<double>(exp_nonpos(m - M)) + s2 * static_cast<double>(exp_nonpos(m2 - M));
  m = M;
}

// 1. slice statistics of every logits row: per thread (max, sum of exponentials below it),
// merged over the block in one reduction
template <bool BF16>
__global__ __launch_bounds__(RA_THREADS) void ra_stats_kernel(const void* __restrict__ logits,
                                                              int64_t ld, int V, int nslice,
                                                              float* __restrict__ ws_m,
                                                              double* __restrict__ ws_s) {
  __shared__ float redm[RA_THREADS / 64];
  __shared__ double reds[RA_THREADS / 64];
  const int slice = blockIdx.x;
  const int64_t row = blockIdx.y;
  float x[RA_PER];
  load_slice<BF16>(logits, row * ld, slice * RA_SLICE, V, x);
  float m = -INFINITY;
#pragma unroll
  for (int e = 0; e < RA_PER; ++e) m = fmaxf(m, x[e]);
  double sum = 0.0;
  if (m > -INFINITY) {
#pragma unroll
    for (int e = 0; e < RA_PER; ++e) sum += static_cast<double>(exp_nonpos(x[e] - m));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) merge_ms(m, sum, __shfl_xor(m, o), __shfl_xor(sum, o));
  const int wave = threadIdx.x / 64;
  if (threadIdx.x % 64 == 0) {
    redm[wave] = m;
    reds[wave] = sum;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < RA_THREADS / 64; ++w) merge_ms(m, sum, redm[w], reds[w]);
    ws_m[row * nslice + slice] = m;
    ws_s[row * nslice + slice] = sum;
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

// 2. accept decisions: wave i of the request's block takes row i (its (M, S) and, for
// i < K, p_i(x_i)); wave 0 then walks the decisions up to the first refusal
template <bool BF16>
__global__ __launch_bounds__(1024) void ra_decide_kernel(
    const void* __restrict__ logits, int64_t ld, const float* __restrict__ draft_probs,
    const int32_t* __restrict__ draft, const float* __restrict__ u, int K, int V, int nslice,
    const float* __restrict__ ws_m, const double* __restrict__ ws_s, int32_t* __restrict__ ws_n,
    double* __restrict__ ws_ms, int32_t* __restrict__ num_accepted) {
  __shared__ double rm[64], rs[64];
  __shared__ int keep[64];
  const int b = blockIdx.x;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  for (int i = wave; i <= K; i += blockDim.x / 64) {
    const int64_t row = static_cast<int64_t>(b) * (K + 1) + i;
    double M, S;
    row_stats(ws_m, ws_s, row, nslice, &M, &S);
    int kept = 0;
    if (i < K) {
      const int32_t x = draft[static_cast<int64_t>(b) * K + i];
      if (x >= 0 && x < V) {  // an out-of-range draft is refused
        const double p = exp(static_cast<double>(logit<BF16>(logits, row * ld + x)) - M) / S;
        const double uq = static_cast<double>(u[static_cast<int64_t>(b) * K + i]) *
                          static_cast<double>(draft_probs[(static_cast<int64_t>(b) * K + i) * V + x]);
        kept = uq < p;
      }
    }
    if (lane == 0) {
      rm[i] = M;
      rs[i] = S;
      keep[i] = kept;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0;
    while (n < K && keep[n]) ++n;
    ws_n[b] = n;
    ws_ms[2 * b] = rm[n];
    ws_ms[2 * b + 1] = rs[n];
    num_accepted[b] = n;
  }
}

// N consecutive draft probabilities from v_begin (16-byte loads when aligned; 0 past V)
template <int N>
__device__ __forceinline__ void load_q_run(const float* qrow, int v_begin, int V, float (&q)[N]) {
  if (v_begin + N <= V && (reinterpret_cast<uintptr_t>(qrow + v_begin) & 15) == 0) {
    float4 d[N / 4];
#pragma unroll
    for (int j = 0; j < N / 4; ++j) d[j] = reinterpret_cast<const float4*>(qrow + v_begin)[j];
#pragma unroll
    for (int j = 0; j < N / 4; ++j) {
      q[4 * j] = d[j].x; q[4 * j + 1] = d[j].y; q[4 * j + 2] = d[j].z; q[4 * j + 3] = d[j].w;
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < N / 4; ++j) {
    const int v = v_begin + 4 * j;
    if (v + 4 <= V && (reinterpret_cast<uintptr_t>(qrow + v) & 15) == 0) {
      const float4 d = *reinterpret_cast<const float4*>(qrow + v);
      q[4 * j] = d.x; q[4 * j + 1] = d.y; q[4 * j + 2] = d.z; q[4 * j + 3] = d.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) q[4 * j + e] = v + e < V ? qrow[v + e] : 0.0f;
    }
  }
}

// N consecutive logits from v_begin (16-byte loads when aligned; -inf past V)
template <bool BF16, int N>
__device__ __forceinline__ void load_run(const void* lg, int64_t row_start, int v_begin, int V,
                                         float (&x)[N]) {
  constexpr int E = BF16 ? 8 : 4;
  constexpr int EB = BF16 ? 2 : 4;
  if (v_begin + N <= V && ((row_start + v_begin) * EB) % 16 == 0) {  // every load issued first
    const i32x4* src = reinterpret_cast<const i32x4*>(static_cast<const uint8_t*>(lg) +
                                                      (row_start + v_begin) * EB);
    i32x4 d[N / E];
#pragma unroll
    for (int j = 0; j < N / E; ++j) d[j] = src[j];
#pragma unroll
    for (int j = 0; j < N / E; ++j)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint32_t wd = static_cast<uint32_t>(d[j][BF16 ? e / 2 : e]);
        x[j * E + e] = BF16 ? __uint_as_float((e & 1) ? (wd & 0xFFFF0000u) : (wd << 16))
                            : __uint_as_float(wd);
      }
    return;
  }
#pragma unroll
  for (int j = 0; j < N / E; ++j) {
    const int v = v_begin + E * j;
    if (v + E <= V && ((row_start + v) * (BF16 ? 2 : 4)) % 16 == 0) {
      const i32x4 d = reinterpret_cast<const i32x4*>(
          static_cast<const uint8_t*>(lg) + (row_start + v) * (BF16 ? 2 : 4))[0];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint32_t wd = static_cast<uint32_t>(d[BF16 ? e / 2 : e]);
        x[j * E + e] = BF16 ? __uint_as_float((e & 1) ? (wd & 0xFFFF0000u) : (wd << 16))
                            : __uint_as_float(wd);
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) x[j * E + e] = v + e < V ? logit<BF16>(lg, row_start + v + e) : -INFINITY;
    }
  }
}

// p(v) and the corrected weight of one entry: l - M is one float32 subtraction (exact for
// bf16 logits within 2^16 of each other in magnitude, rounded once otherwise), then one
// float32 exponential, then float64 arithmetic
__device__ __forceinline__ void weight_of(float l, float q, float Mf, double invS, bool corrected,
                                          double* rw, double* pv) {
  const double p = static_cast<double>(exp_nonpos(l - Mf)) * invS;  // 0 for l = -inf (past V)
  const double d = p - static_cast<double>(q);
  *pv = p;
  *rw = corrected ? (d > 0.0 ? d : 0.0) : p;
}

// 3. per (request, slice): sums of the corrected weights and of p over the drawing row
template <bool BF16>
__global__ __launch_bounds__(RA_THREADS) void ra_weights_kernel(
    const void* __restrict__ logits, int64_t ld, const float* __restrict__ draft_probs, int K,
    int V, int nslice, const int32_t* __restrict__ ws_n, const double* __restrict__ ws_ms,
    double* __restrict__ ws_w, double* __restrict__ ws_p) {
  __shared__ double redd[RA_THREADS / 64];
  constexpr int E = BF16 ? 8 : 4;
  const int slice = blockIdx.x, b = blockIdx.y;
  const int n = ws_n[b];
  const float Mf = static_cast<float>(ws_ms[2 * b]);
  const double invS = 1.0 / ws_ms[2 * b + 1];
  const bool corrected = n < K;
  const int64_t row = static_cast<int64_t>(b) * (K + 1) + n;
  const float* qrow = draft_probs + (static_cast<int64_t>(b) * K + (corrected ? n : 0)) * V;
  // this thread's entries, in load_slice's layout: unit j * RA_THREADS + t of the slice
  float x[RA_PER], q[RA_PER];
  load_slice<BF16>(logits, row * ld, slice * RA_SLICE, V, x);
#pragma unroll
  for (int j = 0; j < RA_PER / E; ++j) {
    const int v = slice * RA_SLICE + (j * RA_THREADS + static_cast<int>(threadIdx.x)) * E;
    float qq[E];
    if (corrected) {
      load_q_run<E>(qrow, v, V, qq);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) qq[e] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) q[j * E + e] = qq[e];
  }
  double sw = 0.0, sp = 0.0;
#pragma unroll
  for (int e = 0; e < RA_PER; ++e) {
    double rw, pv;
    weight_of(x[e], q[e], Mf, invS, corrected, &rw, &pv);
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
  __shared__ double shd[2];  // target, weight before the chosen slice
  __shared__ int shi[2];     // chosen slice, law (0 corrected, 1 target)
  __shared__ double wtot[RA_THREADS / 64];
  __shared__ int fnd[RA_THREADS / 64], lst[RA_THREADS / 64];
  const int b = blockIdx.x;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int n = ws_n[b];
  const bool corrected = n < K;
  if (wave == 0) {
    // slice sums by lane (slices lane, lane + 64, ...); the corrected law unless it is empty
    const double* sw = ws_w + static_cast<int64_t>(b) * nslice;
    const double* sp = ws_p + static_cast<int64_t>(b) * nslice;
    double W = 0.0, P = 0.0;
    for (int j = lane; j < nslice; j += 64) {
      W += sw[j];
      P += sp[j];
    }
    for (int o = 32; o >= 1; o >>= 1) {
      W += __shfl_xor(W, o);
      P += __shfl_xor(P, o);
    }
    const bool use_p = !(W > 0.0);
    const double* sl = use_p ? sp : sw;
    const double target = static_cast<double>(us[b]) * (use_p ? P : W);
    // first slice whose running sum passes the target (chunks of 64 slices, in order)
    double base = 0.0;
    int js = -1, last = 0;
    for (int j0 = 0; j0 < nslice; j0 += 64) {
      const int j = j0 + lane;
      const double x = j < nslice ? sl[j] : 0.0;
      double incl = x;
      for (int o = 1; o < 64; o <<= 1) {
        const double y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      const uint64_t pass = __ballot(j < nslice && base + incl > target && js < 0);
      const uint64_t pos = __ballot(j < nslice && x > 0.0);
      if (pos) last = j0 + 63 - __builtin_clzll(pos);
      if (js < 0 && pass) {
        const int f = __builtin_ctzll(pass);
        js = j0 + f;
        const double incl_f = __shfl(incl, f), x_f = __shfl(x, f);
        if (lane == 0) shd[1] = base + incl_f - x_f;
      }
      base += __shfl(incl, 63);
    }
    if (js < 0) {  // rounding left the target at or above the total: the last slice with weight
      js = last;
      double before = 0.0;
      for (int j = lane; j < js; j += 64) before += sl[j];
      for (int o = 32; o >= 1; o >>= 1) before += __shfl_xor(before, o);
      if (lane == 0) shd[1] = before;
    }
    if (lane == 0) {
      shd[0] = target;
      shi[0] = js;
      shi[1] = use_p ? 1 : 0;
    }
  }
  __syncthreads();
  const int js = shi[0];
  const bool use_p = shi[1] != 0;
  const double target = shd[0], before = shd[1];
  const float Mf = static_cast<float>(ws_ms[2 * b]);
  const double invS = 1.0 / ws_ms[2 * b + 1];
  const int64_t row = static_cast<int64_t>(b) * (K + 1) + n;
  const float* qrow = draft_probs + (static_cast<int64_t>(b) * K + (corrected ? n : 0)) * V;
  // entries of slice js in index order: thread t holds RA_PER consecutive ones
  const int v0 = js * RA_SLICE + static_cast<int>(threadIdx.x) * RA_PER;
  float x[RA_PER], q[RA_PER];
  load_run<BF16, RA_PER>(logits, row * ld, v0, V, x);
  if (corrected && !use_p) {
    load_q_run<RA_PER>(qrow, v0, V, q);
  } else {
#pragma unroll
    for (int e = 0; e < RA_PER; ++e) q[e] = 0.0f;
  }
  double w[RA_PER];
  double tsum = 0.0;
#pragma unroll
  for (int e = 0; e < RA_PER; ++e) {
    double rw, pv;
    weight_of(x[e], q[e], Mf, invS, corrected, &rw, &pv);
    w[e] = use_p ? pv : rw;
    tsum += w[e];
  }
  // exclusive scan of the thread sums (block, float64)
  double incl = tsum;
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  double c = before + incl - tsum;
  for (int xw = 0; xw < wave; ++xw) c += wtot[xw];
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
  if (lane == 0) {
    fnd[wave] = found;
    lst[wave] = lastpos;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int f = 0x7FFFFFFF, l = -1;
    for (int xw = 0; xw < RA_THREADS / 64; ++xw) {
      f = min(f, fnd[xw]);
      l = max(l, lst[xw]);
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
  const dim3 dec_threads(64 * (K + 1 < 16 ? K + 1 : 16));  // one wave per row, at most 16
  if (bf)
    hipLaunchKernelGGL(ra_decide_kernel<true>, dim3((unsigned)B), dec_threads, 0, st, logits, logits_ld,
                       draft_probs, draft, u, K, V, nslice, ws_m, ws_s, ws_n, ws_ms, num_accepted);
  else
    hipLaunchKernelGGL(ra_decide_kernel<false>, dim3((unsigned)B), dec_threads, 0, st, logits, logits_ld,
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
