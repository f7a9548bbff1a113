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

// One vector of D floats over D/4 consecutive lanes (lane_in_vec = 0 .. D/4-1, four
// consecutive elements each); every lane of the group takes part in the shuffles, and only
// live groups load and store. codes/scale: this vector's destination.
template <int D>
__device__ __forceinline__ void quantize_vector(const float* __restrict__ src, bool live,
                                                int lane_in_vec, float rsqrt_d,
                                                uint8_t* __restrict__ codes,
                                                float* __restrict__ scale,
                                                unsigned int* smax = nullptr) {
  constexpr int LPV = D / 4;  // lanes per vector
  float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
  if (live) y = reinterpret_cast<const float4*>(src)[lane_in_vec];
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
  reinterpret_cast<uint32_t*>(codes)[lane_in_vec] = packed;
  if (lane_in_vec == 0) {
    *scale = s;
    // s > 0, so its bits order as the value does
    if (smax) atomicMax(smax, __float_as_uint(s));
  }
}

template <int D>
__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ x, int64_t n_vec,
                                                       float rsqrt_d, uint8_t* __restrict__ out,
                                                       float* __restrict__ scale) {
  constexpr int LPV = D / 4;
  const int64_t v = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / LPV;
  const bool live = v < n_vec;
  const int64_t vv = live ? v : 0;
  quantize_vector<D>(x + vv * D, live, threadIdx.x % LPV, rsqrt_d, out + vv * D, scale + vv);
}

constexpr int LATENT = 576;               // bf16 per latent row (512 + 64)
constexpr int LATENT_UNITS = LATENT / 8;  // 16-byte units per row

// The verify step's writes in one launch. Blocks [0, nbq): query vectors (as
// quantize_kernel); [nbq, nbq + nbk): the new index keys, quantised into cache row
// dst_rows[t]; the rest: the new latent rows, one 16-byte unit per thread, copied to the
// same cache rows. The block ranges are uniform per block.
template <int D>
__global__ __launch_bounds__(256) void verify_write_kernel(
    const float* __restrict__ q, int64_t nq, uint8_t* __restrict__ q_fp8,
    float* __restrict__ q_scale, const float* __restrict__ k_new,
    const int64_t* __restrict__ dst_rows, int T, uint8_t* __restrict__ k_cache,
    float* __restrict__ k_scale, unsigned int* __restrict__ k_scale_max,
    const uint16_t* __restrict__ latent_new, uint16_t* __restrict__ kv_cache, int nbq, int nbk,
    float rsqrt_d) {
  constexpr int LPV = D / 4;
  const int blk = blockIdx.x;
  if (blk < nbq + nbk) {
    const bool is_q = blk < nbq;
    const int64_t v = (static_cast<int64_t>(is_q ? blk : blk - nbq) * blockDim.x + threadIdx.x) / LPV;
    const bool live = v < (is_q ? nq : static_cast<int64_t>(T));
    const int64_t vv = live ? v : 0;
    if (is_q) {
      quantize_vector<D>(q + vv * D, live, threadIdx.x % LPV, rsqrt_d, q_fp8 + vv * D, q_scale + vv);
    } else {
      const int64_t d = live ? dst_rows[vv] : 0;
      quantize_vector<D>(k_new + vv * D, live, threadIdx.x % LPV, rsqrt_d, k_cache + d * D,
                         k_scale + d,
                         k_scale_max ? k_scale_max + d / DSA_KEY_SCALE_CHUNK : nullptr);
    }
    return;
  }
  const int64_t u = static_cast<int64_t>(blk - nbq - nbk) * blockDim.x + threadIdx.x;
  if (u >= static_cast<int64_t>(T) * LATENT_UNITS) return;
  const int64_t t = u / LATENT_UNITS;
  const int piece = static_cast<int>(u % LATENT_UNITS);
  const i32x4 val = reinterpret_cast<const i32x4*>(latent_new + t * LATENT)[piece];
  reinterpret_cast<i32x4*>(kv_cache + dst_rows[t] * LATENT)[piece] = val;
}

// FP8 latent cache rows ("GLM-5.3 推理全链路(十四)", the draft layer's KV pool: 656 bytes
// per token per layer): bytes [0, 512) e4m3fn codes of the 512 latent values, [512, 528)
// the float32 scale of each 128-value block (amax / 448, 1 when amax == 0), [528, 656) the
// 64 rope values copied as bf16. One wave per row: lane l quantises latent values
// 8l .. 8l+7 (its 16-lane group is one scale block); lanes 0..7 copy the rope.
constexpr int RB8 = 656;

__global__ __launch_bounds__(256) void mla_fp8_pack_kernel(const uint16_t* __restrict__ latent,
                                                           const int64_t* __restrict__ dst_rows,
                                                           int64_t n, uint8_t* __restrict__ out) {
  const int lane = threadIdx.x % 64;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / 64;
  const bool live = r < n;
  const int64_t rr = live ? r : 0;
  const uint16_t* src = latent + rr * LATENT;
  const i32x4 v = reinterpret_cast<const i32x4*>(src)[lane];
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_bits_to_f32(static_cast<uint16_t>(v[i] & 0xFFFF));
    x[2 * i + 1] = bf16_bits_to_f32(static_cast<uint16_t>(static_cast<uint32_t>(v[i]) >> 16));
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  if (!live) return;
  uint8_t* dst = out + (dst_rows ? dst_rows[r] : r) * RB8;
  uint32_t w0 = 0, w1 = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w0 |= e4m3_rne_sat(x[i] / s) << (8 * i);
    w1 |= e4m3_rne_sat(x[4 + i] / s) << (8 * i);
  }
  reinterpret_cast<uint2*>(dst)[lane] = make_uint2(w0, w1);
  if ((lane & 15) == 0) reinterpret_cast<float*>(dst + 512)[lane >> 4] = s;
  if (lane < 8)
    reinterpret_cast<i32x4*>(dst + 528)[lane] = reinterpret_cast<const i32x4*>(src + 512)[lane];
}

}  // namespace
}  // namespace dsa

extern "C" dsa_status dsa_mla_fp8_pack(const uint16_t* latent, const int64_t* dst_rows, int64_t n,
                                       uint8_t* kv_fp8, void* stream) {
  using namespace dsa;
  DSA_REQUIRE(n >= 0, "dsa_mla_fp8_pack: n must be >= 0 (got %lld)", (long long)n);
  if (n == 0) return ok();
  DSA_REQUIRE(latent && kv_fp8, "dsa_mla_fp8_pack: null pointer");
  DSA_REQUIRE((reinterpret_cast<uintptr_t>(latent) & 15) == 0 &&
                  (reinterpret_cast<uintptr_t>(kv_fp8) & 15) == 0,
              "dsa_mla_fp8_pack: latent and kv_fp8 must be 16-byte aligned");
  const int64_t blocks = ceil_div(n, 4);
  DSA_REQUIRE(blocks <= 0x7FFFFFFF, "dsa_mla_fp8_pack: too many rows");
  hipLaunchKernelGGL(mla_fp8_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream),
                     latent, dst_rows, n, kv_fp8);
  return check_launch("dsa_mla_fp8_pack");
}

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

extern "C" dsa_status dsa_verify_cache_write(const float* k_new, const uint16_t* latent_new,
                                             const int64_t* dst_rows, int32_t T, int32_t D_I,
                                             uint8_t* k_cache, float* k_scale, uint16_t* kv_cache,
                                             const float* q, int32_t H_I, uint8_t* q_fp8,
                                             float* q_scale, float* k_scale_max, void* stream) {
  using namespace dsa;
  DSA_REQUIRE(T >= 0, "dsa_verify_cache_write: T must be >= 0 (got %d)", T);
  if (D_I != 64 && D_I != 128)
    return fail(DSA_ERR_UNSUPPORTED, "dsa_verify_cache_write: D_I must be 64 or 128 (got %d)", D_I);
  if (T == 0) return ok();
  DSA_REQUIRE(k_new && dst_rows && k_cache && k_scale, "dsa_verify_cache_write: null pointer");
  DSA_REQUIRE(!latent_new == !kv_cache, "dsa_verify_cache_write: latent_new and kv_cache go together");
  DSA_REQUIRE(!q || (q_fp8 && q_scale && H_I >= 1),
              "dsa_verify_cache_write: q needs q_fp8, q_scale and H_I >= 1");
  DSA_REQUIRE((reinterpret_cast<uintptr_t>(k_scale_max) & 3) == 0,
              "dsa_verify_cache_write: k_scale_max must be 4-byte aligned");
  DSA_REQUIRE((reinterpret_cast<uintptr_t>(k_new) & 15) == 0 &&
                  (reinterpret_cast<uintptr_t>(k_cache) & 3) == 0 &&
                  (!q || ((reinterpret_cast<uintptr_t>(q) & 15) == 0 &&
                          (reinterpret_cast<uintptr_t>(q_fp8) & 3) == 0)) &&
                  (!latent_new || ((reinterpret_cast<uintptr_t>(latent_new) & 15) == 0 &&
                                   (reinterpret_cast<uintptr_t>(kv_cache) & 15) == 0)),
              "dsa_verify_cache_write: k_new, q, latent rows 16-byte and code arrays 4-byte aligned");
  const float rsqrt_d = static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(D_I)));
  const int64_t vec_per_block = 256 / (D_I / 4);
  const int64_t nq = q ? static_cast<int64_t>(T) * H_I : 0;
  const int64_t nbq = ceil_div(nq, vec_per_block);
  const int64_t nbk = ceil_div(T, vec_per_block);
  const int64_t nbl = latent_new ? ceil_div(static_cast<int64_t>(T) * LATENT_UNITS, 256) : 0;
  DSA_REQUIRE(nbq + nbk + nbl <= 0x7FFFFFFF, "dsa_verify_cache_write: too many rows");
  const dim3 grid(static_cast<unsigned>(nbq + nbk + nbl));
  if (D_I == 128)
    hipLaunchKernelGGL(verify_write_kernel<128>, grid, dim3(256), 0, as_stream(stream), q, nq, q_fp8,
                       q_scale, k_new, dst_rows, T, k_cache, k_scale,
                       reinterpret_cast<unsigned int*>(k_scale_max), latent_new, kv_cache,
                       static_cast<int>(nbq), static_cast<int>(nbk), rsqrt_d);
  else
    hipLaunchKernelGGL(verify_write_kernel<64>, grid, dim3(256), 0, as_stream(stream), q, nq, q_fp8,
                       q_scale, k_new, dst_rows, T, k_cache, k_scale,
                       reinterpret_cast<unsigned int*>(k_scale_max), latent_new, kv_cache,
                       static_cast<int>(nbq), static_cast<int>(nbk), rsqrt_d);
  return check_launch("dsa_verify_cache_write");
}
