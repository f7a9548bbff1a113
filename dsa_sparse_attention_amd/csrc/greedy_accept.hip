// greedy_accept.hip -- greedy acceptance of a draft chain (split-vocab argmax + prefix scan).
//
// "GLM-5.3 推理全链路(十四)", section "接受判定:greedy 与 rejection sampling": the target
// argmax of verify row i is compared with draft token i; acceptance stops at the first
// mismatch, so the accepted length is the longest matching prefix. Verify rows are
// cat(bonus, drafts) ("验证输入是怎么拼出来的"), so logits row b*(K+1)+i follows row i.
//
// Pass 1 (HBM-bound): blocks of 256 threads scan a vocabulary slice of one logits row
// with 16-byte loads and keep (max, first index): a thread sees its indices in
// increasing order, so per 16-byte group it takes the group maximum only when strictly
// larger and then locates its first index; the merges across threads keep the lower
// index on ties. This reproduces "first maximum wins" exactly. Pass 2: one wave per request
// merges the slices of its K+1 rows in slice order, and a ballot over the K draft
// comparisons gives the first mismatch.
#include <atomic>

#include "common.hpp"

namespace dsa {
namespace {

constexpr int GA_THREADS = 256;
constexpr int GA_SLICE = 4096;  // vocabulary entries per block

struct ArgMax {
  float v;
  int32_t i;
};

__device__ __forceinline__ void take(ArgMax& a, float v, int32_t i) {
  if (v > a.v || (v == a.v && i < a.i)) { a.v = v; a.i = i; }
}

// A group of N values at indices i0..i0+N-1, later than every index `a` holds: its maximum
// replaces `a` only if it is larger (so the earlier index wins a tie), and then the first
// index holding it is located. The first group always replaces the empty state, so a
// row of -inf still yields its first index.
template <int N>
__device__ __forceinline__ void take_group(ArgMax& a, const float (&x)[N], int32_t i0) {
  float m = x[0];
#pragma unroll
  for (int e = 1; e < N; ++e) m = fmaxf(m, x[e]);
  if (m > a.v || a.i == 0x7FFFFFFF) {
    int k = N - 1;
#pragma unroll
    for (int e = N - 2; e >= 0; --e) k = x[e] == m ? e : k;
    a.v = m;
    a.i = i0 + k;
  }
}

template <bool BF16>
__global__ __launch_bounds__(GA_THREADS) void argmax_slices_kernel(const void* __restrict__ logits,
                                                                   int64_t ld, int V, int nslice,
                                                                   float* __restrict__ ws_v,
                                                                   int32_t* __restrict__ ws_i) {
  const int slice = blockIdx.x;
  const int64_t row = blockIdx.y;
  const int v0 = slice * GA_SLICE;
  const int v1 = v0 + GA_SLICE < V ? v0 + GA_SLICE : V;
  ArgMax best = {-INFINITY, 0x7FFFFFFF};
  if (BF16) {
    const uint16_t* lr = static_cast<const uint16_t*>(logits) + row * ld;
    // 8 bf16 per 16-byte load when the slice start is aligned; scalar tail
    const bool vec = ((reinterpret_cast<uintptr_t>(lr + v0) & 15) == 0);
    int v = v0;
    if (vec) {
      // every 16-byte load of the thread is issued before any is used (a whole slice is
      // in flight per block)
      constexpr int UNR = GA_SLICE / 8 / GA_THREADS;
      const int nvec = (v1 - v0) / 8;
      i32x4 d[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int j = threadIdx.x + u * GA_THREADS;
        if (j < nvec) d[u] = *reinterpret_cast<const i32x4*>(lr + v0 + 8 * j);
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int j = threadIdx.x + u * GA_THREADS;
        if (j < nvec) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t w = static_cast<uint32_t>(d[u][e]);
            x[2 * e] = __uint_as_float(w << 16);
            x[2 * e + 1] = __uint_as_float(w & 0xFFFF0000u);
          }
          take_group(best, x, v0 + 8 * j);
        }
      }
      v = v0 + 8 * nvec;
    }
    for (int j = v + threadIdx.x; j < v1; j += GA_THREADS) take(best, bf16_bits_to_f32(lr[j]), j);
  } else {
    const float* lr = static_cast<const float*>(logits) + row * ld;
    const bool vec = ((reinterpret_cast<uintptr_t>(lr + v0) & 15) == 0);
    int v = v0;
    if (vec) {
      constexpr int UNR = GA_SLICE / 4 / GA_THREADS;
      const int nvec = (v1 - v0) / 4;
      float4 d[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int j = threadIdx.x + u * GA_THREADS;
        if (j < nvec) d[u] = *reinterpret_cast<const float4*>(lr + v0 + 4 * j);
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int j = threadIdx.x + u * GA_THREADS;
        if (j < nvec) {
          const float x[4] = {d[u].x, d[u].y, d[u].z, d[u].w};
          take_group(best, x, v0 + 4 * j);
        }
      }
      v = v0 + 4 * nvec;
    }
    for (int j = v + threadIdx.x; j < v1; j += GA_THREADS) take(best, lr[j], j);
  }
  // -0.0 == +0.0 compare equal above; wave then block reduction, lower index on ties
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(best.v, o);
    const int32_t oi = __shfl_xor(best.i, o);
    take(best, ov, oi);
  }
  __shared__ float sv[GA_THREADS / 64];
  __shared__ int32_t si[GA_THREADS / 64];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  if (lane == 0) { sv[wave] = best.v; si[wave] = best.i; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < GA_THREADS / 64; ++w) take(best, sv[w], si[w]);
    ws_v[row * nslice + slice] = best.v;
    ws_i[row * nslice + slice] = best.i;
  }
}

// One block per request: wave w merges the slices of rows w, w + nwaves, .. (lane j takes
// slices j, j + 64, ..; the merge keeps the lower index on ties, so its order does not
// matter); wave 0 then finds the first mismatching draft with a ballot.
__global__ __launch_bounds__(1024) void accept_kernel(const float* __restrict__ ws_v,
                                                      const int32_t* __restrict__ ws_i,
                                                      int nslice, const int32_t* __restrict__ draft,
                                                      int K, int32_t* __restrict__ num_accepted,
                                                      int32_t* __restrict__ next_token,
                                                      int32_t* __restrict__ argmax) {
  __shared__ int32_t row_arg[64];
  const int b = blockIdx.x, lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int nwaves = blockDim.x / 64;
  for (int i = wave; i <= K; i += nwaves) {
    const int64_t row = static_cast<int64_t>(b) * (K + 1) + i;
    ArgMax best = {-INFINITY, 0x7FFFFFFF};
    for (int sl = lane; sl < nslice; sl += 64) take(best, ws_v[row * nslice + sl], ws_i[row * nslice + sl]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(best.v, o);
      const int32_t oi = __shfl_xor(best.i, o);
      take(best, ov, oi);
    }
    if (lane == 0) {
      row_arg[i] = best.i;
      if (argmax) argmax[row] = best.i;
    }
  }
  __syncthreads();
  if (wave == 0) {
    const int32_t a = lane <= K ? row_arg[lane] : -1;
    const bool miss = lane < K && draft[static_cast<int64_t>(b) * K + lane] != a;
    const uint64_t mask = __ballot(miss);
    const int n = mask ? __builtin_ctzll(mask) : K;  // first mismatching draft
    const int32_t an = __shfl(a, n);
    if (lane == 0) {
      num_accepted[b] = n;
      next_token[b] = an;
    }
  }
}

}  // namespace
}  // namespace dsa

extern "C" size_t greedy_accept_workspace_size(int32_t B, int32_t K, int32_t V) {
  if (B <= 0 || K < 0 || V <= 0) return 0;
  const int64_t nslice = dsa::ceil_div(V, dsa::GA_SLICE);
  return static_cast<size_t>(B) * (K + 1) * nslice * (sizeof(float) + sizeof(int32_t));
}

namespace dsa {
namespace {

// Argument checks and the two launches, on a workspace already sized and aligned.
dsa_status greedy_accept_launch(const void* logits, int32_t dtype, int64_t logits_ld,
                                const int32_t* draft, int32_t B, int32_t K, int32_t V,
                                int32_t* num_accepted, int32_t* next_token, int32_t* argmax,
                                void* ws, void* stream) {
  const int64_t rows = static_cast<int64_t>(B) * (K + 1);
  const int nslice = static_cast<int>(ceil_div(V, GA_SLICE));
  float* ws_v = static_cast<float*>(ws);
  int32_t* ws_i = reinterpret_cast<int32_t*>(ws_v + rows * nslice);
  hipStream_t st = as_stream(stream);
  dim3 grid((unsigned)nslice, (unsigned)rows);
  if (dtype == DSA_BF16)
    hipLaunchKernelGGL(argmax_slices_kernel<true>, grid, dim3(GA_THREADS), 0, st, logits, logits_ld,
                       V, nslice, ws_v, ws_i);
  else
    hipLaunchKernelGGL(argmax_slices_kernel<false>, grid, dim3(GA_THREADS), 0, st, logits, logits_ld,
                       V, nslice, ws_v, ws_i);
  dsa_status s = check_launch("greedy_accept(argmax)");
  if (s != DSA_OK) return s;
  const int acc_waves = K + 1 < 16 ? K + 1 : 16;  // one wave per verify row, at most 16
  hipLaunchKernelGGL(accept_kernel, dim3((unsigned)B), dim3(64 * acc_waves), 0, st, ws_v, ws_i, nslice, draft, K,
                     num_accepted, next_token, argmax);
  return check_launch("greedy_accept(accept)");
}

// Host-side checks shared by both entry points (before any launch).
dsa_status greedy_accept_check(const void* logits, int32_t dtype, int64_t logits_ld,
                               const int32_t* draft, int32_t B, int32_t K, int32_t V,
                               int32_t* num_accepted, int32_t* next_token) {
  DSA_REQUIRE(dtype == DSA_F32 || dtype == DSA_BF16, "greedy_accept: dtype must be DSA_F32 or DSA_BF16");
  DSA_REQUIRE(B >= 0 && K >= 0 && K <= 63, "greedy_accept: need B >= 0 and 0 <= K <= 63");
  DSA_REQUIRE(V >= 1 && logits_ld >= V, "greedy_accept: need V >= 1 and logits_ld >= V");
  if (B == 0) return ok();
  DSA_REQUIRE(logits && num_accepted && next_token && (K == 0 || draft),
              "greedy_accept: null pointer");
  DSA_REQUIRE(static_cast<int64_t>(B) * (K + 1) <= 65535, "greedy_accept: B*(K+1) must be <= 65535");
  return ok();
}

// Scratch of greedy_accept_noalloc: a fixed array in each device's memory for the whole life
// of the process. Its name is a host-side stand-in; the device address comes from
// hipGetSymbolAddress, resolved once per device with that device current.
__device__ __align__(256) uint8_t scratch[DSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

dsa_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(DSA_ERR_HIP, "greedy_accept_noalloc: no current device");
  if (dev >= kMaxDevices)
    return fail(DSA_ERR_UNSUPPORTED, "greedy_accept_noalloc: device index %d above %d", dev,
                kMaxDevices - 1);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {  // two threads racing here resolve the same address
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(DSA_ERR_HIP, "greedy_accept_noalloc: hipGetSymbolAddress failed: %s",
                  hipGetErrorString(e));
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return DSA_OK;
}

}  // namespace
}  // namespace dsa

extern "C" dsa_status greedy_accept(const void* logits, int32_t dtype, int64_t logits_ld,
                                    const int32_t* draft, int32_t B, int32_t K, int32_t V,
                                    int32_t* num_accepted, int32_t* next_token, int32_t* argmax,
                                    void* ws, size_t ws_bytes, void* stream) {
  using namespace dsa;
  dsa_status s = greedy_accept_check(logits, dtype, logits_ld, draft, B, K, V, num_accepted,
                                     next_token);
  if (s != DSA_OK || B == 0) return s;
  const size_t need = greedy_accept_workspace_size(B, K, V);
  if (!ws || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "greedy_accept: workspace needs %zu bytes (got %zu)", need,
                ws_bytes);
  DSA_REQUIRE((reinterpret_cast<uintptr_t>(ws) & 3) == 0, "greedy_accept: workspace must be 4-byte aligned");
  return greedy_accept_launch(logits, dtype, logits_ld, draft, B, K, V, num_accepted, next_token,
                              argmax, ws, stream);
}

extern "C" dsa_status greedy_accept_noalloc(const void* logits, int32_t dtype, int64_t logits_ld,
                                            const int32_t* draft, int32_t B, int32_t K, int32_t V,
                                            int32_t* num_accepted, int32_t* next_token,
                                            int32_t* argmax, void* stream) {
  using namespace dsa;
  dsa_status s = greedy_accept_check(logits, dtype, logits_ld, draft, B, K, V, num_accepted,
                                     next_token);
  if (s != DSA_OK || B == 0) return s;
  const size_t need = greedy_accept_workspace_size(B, K, V);
  if (need > DSA_NOALLOC_SCRATCH_BYTES)
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL,
                "greedy_accept_noalloc: B*(K+1) rows of %d logits need %zu bytes of scratch, above "
                "its fixed %zu bytes; call greedy_accept with a workspace instead",
                V, need, static_cast<size_t>(DSA_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  s = scratch_of_current_device(&ws);
  if (s != DSA_OK) return s;
  return greedy_accept_launch(logits, dtype, logits_ld, draft, B, K, V, num_accepted, next_token,
                              argmax, ws, stream);
}
