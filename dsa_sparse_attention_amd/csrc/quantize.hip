// quantize.hip -- Hadamard rotation + dynamic e4m3fn quantisation of indexer q/k vectors.
//
// "MAX Pipeline 中的 DeepSeek-V3.2 架构实现解析", section "Indexer 的结构与计算流程":
// q and k pass through a Sylvester-order Hadamard transform and are dynamically
// quantised to float8_e4m3fn with block size 128 and an fp32 scale before the
// indexer K cache is written / the scores are taken.
//
// Mapping: one vector of D floats is spread over D/4 lanes, four consecutive
// elements per lane (float4 loads, coalesced). FWHT strides 1 and 2 stay inside
// the lane; strides 4..D/2 pair lane i with lane i ^ (stride/4). Every
// butterfly is the same float32 (a+b, a-b) as the definition, so the result
// does not depend on the mapping. HBM-bound: 4*D bytes in, D+4 bytes out.
#include "common.hpp"

// Every float operation here must round exactly as written: no FMA contraction.
#pragma clang fp contract(off)

namespace dsa {
namespace {

// float32 -> e4m3fn code: round-to-nearest-even, saturate to +-448, NaN -> 0x7F.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float x) {
  uint32_t bits = __float_as_uint(x);
  uint32_t sign = (bits >> 24) & 0x80u;
  float a = fabsf(x);
  if (a != a) return 0x7Fu;
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f) {                   // below 2^-6: subnormal grid, step 2^-9
    float m = rintf(a * 512.0f);         // exact scaling; rintf rounds half to even
    return sign | static_cast<uint32_t>(m);  // m == 8 is the smallest normal, code 0x08
  }
  uint32_t ab = bits & 0x7FFFFFFFu;
  int e = static_cast<int>(ab >> 23) - 127;  // -6 .. 8
  uint32_t mant = ab & 0x7FFFFFu;
  uint32_t m3 = mant >> 20;
  uint32_t rem = mant & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) ++m3;
  if (m3 == 8u) { m3 = 0u; ++e; }
  return sign | (static_cast<uint32_t>(e + 7) << 3) | m3;
}

template <int D>
__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ x, int64_t n_vec,
                                                       float rsqrt_d, uint8_t* __restrict__ out,
                                                       float* __restrict__ scale) {
  constexpr int LPV = D / 4;  // lanes per vector
  const int lane_in_vec = threadIdx.x % LPV;
  const int64_t v = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / LPV;
  const bool live = v < n_vec;
  float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
  if (live) y = reinterpret_cast<const float4*>(x + v * D)[lane_in_vec];
  // stride 1: pairs (0,1), (2,3)
  float a0 = y.x + y.y, a1 = y.x - y.y, a2 = y.z + y.w, a3 = y.z - y.w;
  // stride 2: pairs (0,2), (1,3)
  float e0 = a0 + a2, e1 = a1 + a3, e2 = a0 - a2, e3 = a1 - a3;
  // strides 4 .. D/2 across lanes
#pragma unroll
  for (int m = 1; m < LPV; m <<= 1) {
    float o0 = __shfl_xor(e0, m), o1 = __shfl_xor(e1, m);
    float o2 = __shfl_xor(e2, m), o3 = __shfl_xor(e3, m);
    if (lane_in_vec & m) {  // upper half of the butterfly: a - b with a from the partner
      e0 = o0 - e0; e1 = o1 - e1; e2 = o2 - e2; e3 = o3 - e3;
    } else {
      e0 = e0 + o0; e1 = e1 + o1; e2 = e2 + o2; e3 = e3 + o3;
    }
  }
  e0 = e0 * rsqrt_d; e1 = e1 * rsqrt_d; e2 = e2 * rsqrt_d; e3 = e3 * rsqrt_d;
  float amax = fmaxf(fmaxf(fabsf(e0), fabsf(e1)), fmaxf(fabsf(e2), fabsf(e3)));
#pragma unroll
  for (int m = 1; m < LPV; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  if (!live) return;
  uint32_t packed = e4m3_rne_sat(e0 / s) | (e4m3_rne_sat(e1 / s) << 8) |
                    (e4m3_rne_sat(e2 / s) << 16) | (e4m3_rne_sat(e3 / s) << 24);
  reinterpret_cast<uint32_t*>(out + v * D)[lane_in_vec] = packed;
  if (lane_in_vec == 0) scale[v] = s;
}

}  // namespace
}  // namespace dsa

extern "C" dsa_status dsa_quantize_fp8(const float* x, int64_t n_vec, int32_t dim,
                                       uint8_t* x_fp8, float* scale, void* stream) {
  using namespace dsa;
  DSA_REQUIRE(n_vec >= 0, "dsa_quantize_fp8: n_vec must be >= 0 (got %lld)", (long long)n_vec);
  if (dim != 64 && dim != 128)
    return fail(DSA_ERR_UNSUPPORTED, "dsa_quantize_fp8: dim must be 64 or 128 (got %d)", dim);
  if (n_vec == 0) return ok();
  DSA_REQUIRE(x && x_fp8 && scale, "dsa_quantize_fp8: null pointer");
  DSA_REQUIRE((reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
                  (reinterpret_cast<uintptr_t>(x_fp8) & 3) == 0,
              "dsa_quantize_fp8: x must be 16-byte and x_fp8 4-byte aligned");
  // RN_f32(1/sqrt(D)): the exact constant rounded once to float32.
  const float rsqrt_d = static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(dim)));
  const int64_t vec_per_block = 256 / (dim / 4);
  const int64_t blocks = ceil_div(n_vec, vec_per_block);
  DSA_REQUIRE(blocks <= 0x7FFFFFFF, "dsa_quantize_fp8: too many vectors");
  if (dim == 128)
    hipLaunchKernelGGL(quantize_kernel<128>, dim3((unsigned)blocks), dim3(256), 0,
                       as_stream(stream), x, n_vec, rsqrt_d, x_fp8, scale);
  else
    hipLaunchKernelGGL(quantize_kernel<64>, dim3((unsigned)blocks), dim3(256), 0,
                       as_stream(stream), x, n_vec, rsqrt_d, x_fp8, scale);
  return check_launch("dsa_quantize_fp8");
}
