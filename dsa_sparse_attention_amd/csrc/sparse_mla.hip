// sparse_mla.hip -- sparse MLA decode over the top-k selected latent rows (gfx950).
//
// "MAX Pipeline 中的 DeepSeek-V3.2 架构实现解析", section "稀疏 MLA 的前向路径": attention
// runs only over the positions the indexer selected; latent row = kv_lora_rank
// 512 + qk_rope_head_dim 64 ("GLM-5.3 推理全链路(十四)", "GLM-5.3 的草稿层到底长什么样").
// Index sharing: "MAX 中 GLM-5.2 ... 统一 MTP 推测解码架构解析", "阶段 5".
//
// Work split: a block owns one query row and one slice of its top-k list
// (split-K); wave w owns heads 16w..16w+15. Per 32-key chunk the block gathers
// 32 latent rows (1152 B each, 16-byte coalesced loads) into LDS, then
//   S^T[key, head] = K[32 x 576] . Q^T  (18 x 2 v_mfma_f32_16x16x32_bf16, Q^T
//                                        fragments held in registers)
//   online softmax per head in base 2 (one max / sum per lane, lane = head)
//   O^T[dim, head] += V^T[512 x 32] . P^T (32 MFMAs, P^T taken straight from the
//                                        S^T accumulator lanes, no shuffle)
// The transposed O^T layout keeps each head in one lane column, so the
// softmax rescale of O needs no cross-lane exchange. With more than one split
// the unnormalised partials (O, max, sum) go to the workspace and a combine
// kernel merges them.
#include "common.hpp"

namespace dsa {
namespace {

constexpr int DQK = 576, DV = 512;
constexpr int KC = 32;               // keys per chunk
constexpr int ROWB = DQK * 2 + 16;   // LDS row stride (bytes), padded against bank conflicts
constexpr int NCHUNK16 = DQK * 2 / 16;  // 72 16-byte pieces per latent row

__device__ __forceinline__ bf16x8 as_bf16x8(i32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int NW>
// Two waves per SIMD: caps the kernel at 256 registers per lane (Q^T 72, O^T 128, rest).
__global__ __launch_bounds__(NW * 64, NW == 1 ? 1 : 2) void mla_decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ topk, const int32_t* __restrict__ share_base,
    const int32_t* __restrict__ num_acc, const int32_t* __restrict__ q_off,
    const int64_t* __restrict__ kv_off, int H, int k, int topk_rows, float c2, int nsplit,
    int keys_per_split,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ ws_o,
    float* __restrict__ ws_ml) {
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(16))) uint8_t lds[KC * ROWB];
  __shared__ int32_t sidx[KC];

  const int split = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const RowInfo ri = load_row_info(q_off, kv_off, b);
  if (r >= ri.R) return;
  const int64_t t = ri.t0 + r;
  const int64_t trow = share_base ? static_cast<int64_t>(share_base[b]) + num_acc[b] : t;
  const bool trow_ok = trow >= 0 && trow < topk_rows;  // a bad share map selects nothing
  const int32_t* idx = topk + (trow_ok ? trow : 0) * k;
  const int i_begin = split * keys_per_split;
  const int i_end = !trow_ok ? i_begin : (i_begin + keys_per_split < k ? i_begin + keys_per_split : k);

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int g = lane / 16, c16 = lane % 16;
  const int head = wave * 16 + c16;

  // Q^T fragments: head `head`, dims 32*ks + 8*g .. +8
  bf16x8 qf[18];
  {
    const uint16_t* qrow = q + (t * H + head) * DQK + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qf[ks] = as_bf16x8(*reinterpret_cast<const i32x4*>(qrow + 32 * ks));
  }
  f32x4 o[DV / 16];
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) o[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;  // running max (base-2 logits) of this head
  float lsum = 0.0f;    // running sum of this lane's share of the keys

  for (int i0 = i_begin; i0 < i_end; i0 += KC) {
    if (tid < KC) {
      const int i = i0 + tid;
      const int p = i < i_end ? idx[i] : -1;
      sidx[tid] = (p >= 0 && p < ri.L) ? p : -1;
    }
    __syncthreads();
    for (int c = tid; c < KC * NCHUNK16; c += NT) {
      const int row = c / NCHUNK16, ch = c % NCHUNK16;
      const int p = sidx[row];
      i32x4 v = {0, 0, 0, 0};
      if (p >= 0) v = *reinterpret_cast<const i32x4*>(kv + (ri.kv_base + p) * DQK + ch * 8);
      *reinterpret_cast<i32x4*>(lds + row * ROWB + ch * 16) = v;
    }
    __syncthreads();

    // S^T for keys 0..15 (s0) and 16..31 (s1): lane holds keys 4g+i / 16+4g+i of head c16
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const bf16x8 a0 = as_bf16x8(*reinterpret_cast<const i32x4*>(lds + c16 * ROWB + ks * 64 + g * 16));
      const bf16x8 a1 = as_bf16x8(*reinterpret_cast<const i32x4*>(lds + (16 + c16) * ROWB + ks * 64 + g * 16));
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[ks], s1, 0, 0, 0);
    }
    float z[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = sidx[4 * g + i] >= 0 ? s0[i] * c2 : -INFINITY;
      z[4 + i] = sidx[16 + 4 * g + i] >= 0 ? s1[i] * c2 : -INFINITY;
    }
    float cm = z[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) cm = fmaxf(cm, z[i]);
    cm = fmaxf(cm, __shfl_xor(cm, 16));
    cm = fmaxf(cm, __shfl_xor(cm, 32));
    const float mn = fmaxf(m, cm);
    // all keys so far invalid for this head: nothing to add (p = 0, alpha = 1)
    const float alpha = (m == -INFINITY) ? (mn == -INFINITY ? 1.0f : 0.0f) : exp2f(m - mn);
    uint32_t pw[4];
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pa = z[2 * i] == -INFINITY ? 0.0f : exp2f(z[2 * i] - mn);
      const float pb = z[2 * i + 1] == -INFINITY ? 0.0f : exp2f(z[2 * i + 1] - mn);
      const uint16_t ha = f32_to_bf16_bits(pa), hb = f32_to_bf16_bits(pb);
      psum += bf16_bits_to_f32(ha) + bf16_bits_to_f32(hb);
      pw[i] = static_cast<uint32_t>(ha) | (static_cast<uint32_t>(hb) << 16);
    }
    lsum = lsum * alpha + psum;
    m = mn;
    if (__any(alpha != 1.0f)) {  // wave-uniform: skip the rescale once the max is stable
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt) o[dt] *= alpha;
    }
    const bf16x8 pf = as_bf16x8((i32x4){(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3]});
    // V^T fragments: dim 16*dt + c16, keys 4g..4g+3 then 16+4g..16+4g+3 (same slots as pf)
    const uint8_t* r0 = lds + (4 * g) * ROWB;
    const uint8_t* r1 = lds + (16 + 4 * g) * ROWB;
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) {
      const int off = (16 * dt + c16) * 2;
      uint32_t v[4];
      v[0] = *reinterpret_cast<const uint16_t*>(r0 + off) |
             (static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(r0 + ROWB + off)) << 16);
      v[1] = *reinterpret_cast<const uint16_t*>(r0 + 2 * ROWB + off) |
             (static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(r0 + 3 * ROWB + off)) << 16);
      v[2] = *reinterpret_cast<const uint16_t*>(r1 + off) |
             (static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(r1 + ROWB + off)) << 16);
      v[3] = *reinterpret_cast<const uint16_t*>(r1 + 2 * ROWB + off) |
             (static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(r1 + 3 * ROWB + off)) << 16);
      const bf16x8 vf = as_bf16x8((i32x4){(int)v[0], (int)v[1], (int)v[2], (int)v[3]});
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, o[dt], 0, 0, 0);
    }
    __syncthreads();
  }

  float l = lsum + __shfl_xor(lsum, 16);
  l += __shfl_xor(l, 32);
  if (nsplit == 1) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    uint16_t* orow = out + (t * H + head) * DV + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) {
      const uint32_t lo = f32_to_bf16_bits(o[dt][0] * inv) |
                          (static_cast<uint32_t>(f32_to_bf16_bits(o[dt][1] * inv)) << 16);
      const uint32_t hi = f32_to_bf16_bits(o[dt][2] * inv) |
                          (static_cast<uint32_t>(f32_to_bf16_bits(o[dt][3] * inv)) << 16);
      *reinterpret_cast<uint2*>(orow + 16 * dt) = make_uint2(lo, hi);
    }
    if (lse && g == 0) lse[t * H + head] = l > 0.0f ? (m + __log2f(l)) * 0.69314718055994531f : -INFINITY;
  } else {
    const int64_t slot = (t * nsplit + split) * H + head;
    float* orow = ws_o + slot * DV + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt)
      *reinterpret_cast<float4*>(orow + 16 * dt) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    if (g == 0) {
      ws_ml[2 * slot] = m;
      ws_ml[2 * slot + 1] = l;
    }
  }
}

// Merge split-K partials of one (row, head): 128 threads x 4 dims.
__global__ __launch_bounds__(128) void mla_combine_kernel(const float* __restrict__ ws_o,
                                                          const float* __restrict__ ws_ml,
                                                          int H, int nsplit,
                                                          uint16_t* __restrict__ out,
                                                          float* __restrict__ lse) {
  const int64_t t = blockIdx.x;
  const int head = blockIdx.y;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ws_ml[2 * ((t * nsplit + s) * H + head)]);
  float L = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (M != -INFINITY) {
    for (int s = 0; s < nsplit; ++s) {
      const int64_t slot = (t * nsplit + s) * H + head;
      const float ms = ws_ml[2 * slot];
      if (ms == -INFINITY) continue;
      const float f = exp2f(ms - M);
      L += ws_ml[2 * slot + 1] * f;
      const float4 v = reinterpret_cast<const float4*>(ws_o + slot * DV)[threadIdx.x];
      acc.x += v.x * f; acc.y += v.y * f; acc.z += v.z * f; acc.w += v.w * f;
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const uint32_t lo = f32_to_bf16_bits(acc.x * inv) | (static_cast<uint32_t>(f32_to_bf16_bits(acc.y * inv)) << 16);
  const uint32_t hi = f32_to_bf16_bits(acc.z * inv) | (static_cast<uint32_t>(f32_to_bf16_bits(acc.w * inv)) << 16);
  reinterpret_cast<uint2*>(out + (t * H + head) * DV)[threadIdx.x] = make_uint2(lo, hi);
  if (lse && threadIdx.x == 0) lse[t * H + head] = L > 0.0f ? (M + __log2f(L)) * 0.69314718055994531f : -INFINITY;
}

// Split count: enough blocks to cover the chip twice, at least 256 keys per split.
int choose_splits(int64_t rows, int k) {
  int s = 1;
  while (s < 8 && rows * s < 512 && (k + 2 * s - 1) / (2 * s) >= 256) s *= 2;
  return s;
}

int64_t keys_per_split(int k, int s) { return ceil_div(ceil_div(k, s), KC) * KC; }

}  // namespace
}  // namespace dsa

extern "C" size_t dsa_sparse_mla_workspace_size(int32_t T, int32_t H, int32_t k) {
  using namespace dsa;
  if (T <= 0 || H <= 0 || k <= 0) return 0;
  const int s = choose_splits(T, k);
  if (s == 1) return 0;
  return static_cast<size_t>(T) * s * H * (DV + 2) * sizeof(float);
}

extern "C" dsa_status dsa_sparse_mla_decode(const uint16_t* q, const uint16_t* kv,
                                            const int32_t* topk, int32_t topk_rows,
                                            const int32_t* share_base,
                                            const int32_t* num_accepted,
                                            const int32_t* q_row_offsets,
                                            const int64_t* kv_row_offsets, int32_t B, int32_t T,
                                            int32_t max_q_rows, int32_t H, int32_t k,
                                            float sm_scale, uint16_t* out, float* lse, void* ws,
                                            size_t ws_bytes, void* stream) {
  using namespace dsa;
  if (H < 16 || H > 128 || H % 16)
    return fail(DSA_ERR_UNSUPPORTED, "dsa_sparse_mla_decode: H must be a multiple of 16 in [16, 128] (got %d)", H);
  DSA_REQUIRE(k >= 1, "dsa_sparse_mla_decode: k must be >= 1 (got %d)", k);
  DSA_REQUIRE(topk_rows >= 0, "dsa_sparse_mla_decode: topk_rows must be >= 0");
  DSA_REQUIRE(share_base || topk_rows >= T, "dsa_sparse_mla_decode: topk needs T rows without a share map");
  DSA_REQUIRE(B >= 0 && T >= 0 && max_q_rows >= 0, "dsa_sparse_mla_decode: negative size");
  DSA_REQUIRE((share_base == nullptr) == (num_accepted == nullptr),
              "dsa_sparse_mla_decode: share_base and num_accepted go together");
  DSA_REQUIRE(sm_scale > 0.0f && sm_scale < 1e30f, "dsa_sparse_mla_decode: sm_scale must be positive");
  if (B == 0 || T == 0 || max_q_rows == 0) return ok();
  DSA_REQUIRE(q && kv && topk && q_row_offsets && kv_row_offsets && out,
              "dsa_sparse_mla_decode: null pointer");
  DSA_REQUIRE((reinterpret_cast<uintptr_t>(q) & 15) == 0 && (reinterpret_cast<uintptr_t>(kv) & 15) == 0 &&
                  (reinterpret_cast<uintptr_t>(out) & 15) == 0,
              "dsa_sparse_mla_decode: q, kv and out must be 16-byte aligned");
  DSA_REQUIRE(B <= 65535 && max_q_rows <= 65535, "dsa_sparse_mla_decode: B and max_q_rows must be <= 65535");
  const int s = choose_splits(T, k);
  const size_t need = dsa_sparse_mla_workspace_size(T, H, k);
  if (ws_bytes < need || (need && !ws))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "dsa_sparse_mla_decode: workspace needs %zu bytes (got %zu)",
                need, ws_bytes);
  DSA_REQUIRE(!need || (reinterpret_cast<uintptr_t>(ws) & 15) == 0,
              "dsa_sparse_mla_decode: workspace must be 16-byte aligned");
  const int kps = static_cast<int>(keys_per_split(k, s));
  const int nsplit = static_cast<int>(ceil_div(k, kps));
  float* ws_o = static_cast<float*>(ws);
  float* ws_ml = need ? ws_o + static_cast<size_t>(T) * nsplit * H * DV : nullptr;
  const float c2 = sm_scale * 1.4426950408889634f;  // natural -> base-2 logits
  hipStream_t st = as_stream(stream);
  dim3 grid((unsigned)nsplit, (unsigned)max_q_rows, (unsigned)B);
  const int nw = H / 16;
#define DSA_MLA_LAUNCH(NWV)                                                                     \
  hipLaunchKernelGGL(mla_decode_kernel<NWV>, grid, dim3(NWV * 64), 0, st, q, kv, topk,          \
                     share_base, num_accepted, q_row_offsets, kv_row_offsets, H, k, topk_rows, c2,  \
                     nsplit, kps, out, lse, ws_o, ws_ml)
  switch (nw) {
    case 1: DSA_MLA_LAUNCH(1); break;
    case 2: DSA_MLA_LAUNCH(2); break;
    case 3: DSA_MLA_LAUNCH(3); break;
    case 4: DSA_MLA_LAUNCH(4); break;
    case 5: DSA_MLA_LAUNCH(5); break;
    case 6: DSA_MLA_LAUNCH(6); break;
    case 7: DSA_MLA_LAUNCH(7); break;
    default: DSA_MLA_LAUNCH(8); break;
  }
#undef DSA_MLA_LAUNCH
  dsa_status stt = check_launch("dsa_sparse_mla_decode");
  if (stt != DSA_OK || nsplit == 1) return stt;
  hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)T, (unsigned)H), dim3(128), 0, st, ws_o,
                     ws_ml, H, nsplit, out, lse);
  return check_launch("dsa_sparse_mla_decode(combine)");
}
