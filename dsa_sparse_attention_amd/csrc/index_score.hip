// index_score.hip -- lightning-indexer scores on FP8 MFMA (gfx950).
//
// "MAX Pipeline 中的 DeepSeek-V3.2 架构实现解析", section "Indexer 的结构与计算流程":
// every verify row scores every cached index key with index_n_heads FP8 heads
// of index_head_dim; per-token fp32 scales come from the indexer scale cache
// ("配置体系", 双 KV 缓存). Score of row t against key s:
//     I[t,s] = k_scale[s] * sum_j (w[t,j] * q_scale[t,j]) * ReLU(q_hat[t,j] . k_hat[s])
//
// Work split: a block owns one request's key chunk and up to NW of its query
// rows (one wave per row). Keys stream HBM -> registers -> LDS in 64-key tiles
// (double-buffered, 16-byte chunks XOR-swizzled by key so the per-lane 32-byte
// reads are bank-conflict free); each key byte is fetched from HBM once per
// request and shared by all of its rows. Per 16-key sub-tile a wave issues one
// v_mfma_f32_16x16x128_f8f6f4 per 16-head tile (K = 128 = index_head_dim in one
// instruction): A = q codes [16 heads x 128], B = key codes [128 x 16 keys].
// The result lane layout (row = 4*(lane/16)+i, col = lane%16) puts 4 heads of
// one key in each lane, so the ReLU * weight head reduction is 4*HT in-lane
// FMAs plus two cross-lane adds. The four lane groups then store four
// different sub-tiles: one coalesced 256-byte store per 64 keys per row.
#include "common.hpp"

namespace dsa {
namespace {

constexpr int KT = 64;  // keys per LDS tile
constexpr int MAX_CHUNK = 4096;  // keys per block (key scales staged in LDS)

template <int D, int HT, int NW>
__global__ __launch_bounds__(NW * 64) void index_score_kernel(
    const uint8_t* __restrict__ q_fp8, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k_fp8,
    const float* __restrict__ k_scale, const int32_t* __restrict__ q_off,
    const int64_t* __restrict__ kv_off, int H, int64_t chunk, float* __restrict__ scores,
    int64_t ld) {
  constexpr int NCH = D / 16;                 // 16-byte chunks per key
  constexpr int CH = KT * NCH;                // chunks per tile
  constexpr int NT = NW * 64;
  constexpr int PER = (CH + NT - 1) / NT;     // chunk loads per thread per tile
  constexpr int NPRE = PER >= 4 ? 1 : 4 / PER;  // tiles in flight per block
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][KT * D];
  __shared__ float sscale[MAX_CHUNK];

  const int b = blockIdx.y;
  const RowInfo ri = load_row_info(q_off, kv_off, b);
  const int64_t key0 = static_cast<int64_t>(blockIdx.x) * chunk;
  const int row0 = blockIdx.z * NW;
  if (key0 >= ri.L || row0 >= ri.R) return;  // block-uniform
  int64_t key_end = key0 + chunk < ri.L ? key0 + chunk : ri.L;
  if (key_end > ld) key_end = ld;  // device lengths beyond the score stride are clipped

  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int g = lane / 16, c16 = lane % 16;
  const int r = row0 + wave;
  const bool row_live = r < ri.R;             // wave-uniform
  const int64_t nvis = row_live ? visible_count(ri, r) : 0;
  const int64_t t = ri.t0 + r;

  // A operands (q codes) and per-output-row weights u = w * q_scale.
  i32x8 qa[HT];
  float u[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int head = ht * 16 + c16;
    // branch-free loads from clamped addresses; invalid lanes are zeroed afterwards
    const bool qok = row_live && head < H && 32 * g < D;
    const int64_t tq = row_live ? t : ri.t0;
    const int hq = head < H ? head : H - 1;
    const int gq = 32 * g < D ? g : 0;
    const i32x4* p = reinterpret_cast<const i32x4*>(q_fp8 + (tq * H + hq) * D + 32 * gq);
    const i32x4 lo = p[0], hi = p[1];
    const i32x8 v = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    const i32x8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
    qa[ht] = qok ? v : zero8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h2 = ht * 16 + 4 * g + i;
      const int64_t o = tq * H + (h2 < H ? h2 : H - 1);
      const float uu = w[o] * q_scale[o];
      u[ht][i] = (row_live && h2 < H) ? uu : 0.0f;
    }
  }

  const uint8_t* kbase = k_fp8 + (ri.kv_base + key0) * D;
  const int64_t nkeys = key_end - key0;
  const int ntiles = static_cast<int>((nkeys + KT - 1) / KT);

  // Key scales of the whole chunk go to LDS once (chunk <= 4096 keys).
  for (int i0 = 0; i0 < nkeys; i0 += 4 * NT) {  // four independent loads per thread per step
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = i0 + j * NT + static_cast<int>(threadIdx.x);
      v[j] = k_scale[ri.kv_base + key0 + (i < nkeys ? i : nkeys - 1)];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = i0 + j * NT + static_cast<int>(threadIdx.x);
      if (i < nkeys) sscale[i] = v[j];
    }
  }

  // Register ring: each thread holds its 16-byte pieces of the next NPRE tiles, so
  // NPRE tiles per block are in flight while one is computed (the loop is unrolled
  // by NPRE so every ring slot is a fixed register).
  i32x4 pre[NPRE][PER];
  auto load_tile = [&](int it, i32x4* dst) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      // branch-free: keys past the chunk load the last key again (their scores are
      // never stored); pieces past the tile (idx >= CH) are never written to LDS
      const int idx = threadIdx.x + j * NT < CH ? threadIdx.x + j * NT : CH - 1;
      const int s = idx / NCH, c = idx % NCH;
      int64_t key = static_cast<int64_t>(it) * KT + s;
      key = key < nkeys ? key : nkeys - 1;
      dst[j] = *reinterpret_cast<const i32x4*>(kbase + key * D + c * 16);
    }
  };
  auto store_tile = [&](uint8_t* buf, const i32x4* src) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int idx = threadIdx.x + j * NT;
      if (idx < CH) {
        const int s = idx / NCH, c = idx % NCH;
        *reinterpret_cast<i32x4*>(buf + s * D + ((c ^ (s & (NCH - 1))) * 16)) = src[j];
      }
    }
  };

#pragma unroll
  for (int j = 0; j < NPRE; ++j)
    if (j < ntiles) load_tile(j, pre[j]);
  for (int base = 0; base < ntiles; base += NPRE) {
#pragma unroll
    for (int jr = 0; jr < NPRE; ++jr) {
      const int it = base + jr;
      if (it >= ntiles) break;  // block-uniform
      uint8_t* buf = lds[it & 1];
      store_tile(buf, pre[jr]);
      __syncthreads();  // tile `it` is in LDS; the other buffer (tile it-1) is no longer read
      if (it + NPRE < ntiles) load_tile(it + NPRE, pre[jr]);
      if (row_live) {
        float res[4];
#pragma unroll
        for (int sub = 0; sub < 4; ++sub) {
          const int s = sub * 16 + c16;
          i32x8 bfrag = {0, 0, 0, 0, 0, 0, 0, 0};
          if (32 * g < D) {
            const int c0 = 2 * g, c1 = 2 * g + 1;
            i32x4 lo = *reinterpret_cast<const i32x4*>(buf + s * D + ((c0 ^ (s & (NCH - 1))) * 16));
            i32x4 hi = *reinterpret_cast<const i32x4*>(buf + s * D + ((c1 ^ (s & (NCH - 1))) * 16));
            bfrag = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
          float part = 0.0f;
#pragma unroll
          for (int ht = 0; ht < HT; ++ht) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[ht], bfrag, acc, 0, 0, 0, 0,
                                                                   0, 0);
            // ReLU as med3(x, 0, FLT_MAX): one instruction (max(x, 0) for finite x)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              part = fmaf(u[ht][i], __builtin_amdgcn_fmed3f(acc[i], 0.0f, 3.402823466e38f), part);
          }
          part += __shfl_xor(part, 16);
          part += __shfl_xor(part, 32);
          res[sub] = part;
        }
        const float v = g == 0 ? res[0] : g == 1 ? res[1] : g == 2 ? res[2] : res[3];
        const int sl = it * KT + g * 16 + c16;         // key within the chunk
        const int64_t s = key0 + sl;                    // request-local position
        if (s < key_end && s < nvis) scores[t * ld + s] = v * sscale[sl];
      }
    }
  }
}

template <int D, int HT>
void launch_nw(int nw, dim3 grid, hipStream_t st, const uint8_t* q, const float* qs,
               const float* w, const uint8_t* k, const float* ks, const int32_t* qo,
               const int64_t* ko, int H, int64_t chunk, float* sc, int64_t ld) {
  switch (nw) {
    case 1: hipLaunchKernelGGL((index_score_kernel<D, HT, 1>), grid, dim3(64), 0, st, q, qs, w, k, ks, qo, ko, H, chunk, sc, ld); break;
    case 2: hipLaunchKernelGGL((index_score_kernel<D, HT, 2>), grid, dim3(128), 0, st, q, qs, w, k, ks, qo, ko, H, chunk, sc, ld); break;
    case 4: hipLaunchKernelGGL((index_score_kernel<D, HT, 4>), grid, dim3(256), 0, st, q, qs, w, k, ks, qo, ko, H, chunk, sc, ld); break;
    default: hipLaunchKernelGGL((index_score_kernel<D, HT, 8>), grid, dim3(512), 0, st, q, qs, w, k, ks, qo, ko, H, chunk, sc, ld); break;
  }
}

template <int D>
void launch_ht(int ht, int nw, dim3 grid, hipStream_t st, const uint8_t* q, const float* qs,
               const float* w, const uint8_t* k, const float* ks, const int32_t* qo,
               const int64_t* ko, int H, int64_t chunk, float* sc, int64_t ld) {
  switch (ht) {
    case 1: launch_nw<D, 1>(nw, grid, st, q, qs, w, k, ks, qo, ko, H, chunk, sc, ld); break;
    case 2: launch_nw<D, 2>(nw, grid, st, q, qs, w, k, ks, qo, ko, H, chunk, sc, ld); break;
    case 4: launch_nw<D, 4>(nw, grid, st, q, qs, w, k, ks, qo, ko, H, chunk, sc, ld); break;
    default: launch_nw<D, 8>(nw, grid, st, q, qs, w, k, ks, qo, ko, H, chunk, sc, ld); break;
  }
}

int pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

}  // namespace
}  // namespace dsa

extern "C" dsa_status dsa_index_score(const uint8_t* q_fp8, const float* q_scale, const float* w,
                                      const uint8_t* k_fp8, const float* k_scale,
                                      const int32_t* q_row_offsets,
                                      const int64_t* kv_row_offsets, int32_t B, int32_t T,
                                      int32_t max_q_rows, int32_t H_I, int32_t D_I,
                                      int64_t max_kv_len, float* scores, int64_t score_ld,
                                      void* stream) {
  using namespace dsa;
  if (D_I != 64 && D_I != 128)
    return fail(DSA_ERR_UNSUPPORTED, "dsa_index_score: D_I must be 64 or 128 (got %d)", D_I);
  if (H_I < 1 || H_I > 128)
    return fail(DSA_ERR_UNSUPPORTED, "dsa_index_score: H_I must be in [1, 128] (got %d)", H_I);
  DSA_REQUIRE(B >= 0 && T >= 0 && max_q_rows >= 0 && max_kv_len >= 0,
              "dsa_index_score: negative size");
  DSA_REQUIRE(score_ld >= max_kv_len, "dsa_index_score: score_ld (%lld) < max_kv_len (%lld)",
              (long long)score_ld, (long long)max_kv_len);
  if (B == 0 || T == 0 || max_q_rows == 0 || max_kv_len == 0) return ok();
  DSA_REQUIRE(q_fp8 && q_scale && w && k_fp8 && k_scale && q_row_offsets && kv_row_offsets &&
                  scores, "dsa_index_score: null pointer");
  DSA_REQUIRE((reinterpret_cast<uintptr_t>(q_fp8) & 15) == 0 &&
                  (reinterpret_cast<uintptr_t>(k_fp8) & 15) == 0,
              "dsa_index_score: q_fp8 and k_fp8 must be 16-byte aligned");
  DSA_REQUIRE(B <= 65535, "dsa_index_score: B must be <= 65535");
  const int ht = pow2_at_least((H_I + 15) / 16);
  const int nw = pow2_at_least(max_q_rows < 8 ? max_q_rows : 8);
  // Key chunk per block: enough blocks to fill the chip (~4 per CU), 256..4096 keys.
  int64_t chunk = 4096;
  const int64_t total_keys = static_cast<int64_t>(B) * max_kv_len;
  while (chunk > 256 && total_keys / chunk < 1024) chunk /= 2;
  const int64_t gx = ceil_div(max_kv_len, chunk);
  const int64_t gz = ceil_div(max_q_rows, nw);
  DSA_REQUIRE(gx <= 0x7FFFFFFF && gz <= 65535, "dsa_index_score: grid too large");
  dim3 grid((unsigned)gx, (unsigned)B, (unsigned)gz);
  hipStream_t st = as_stream(stream);
  if (D_I == 128)
    launch_ht<128>(ht, nw, grid, st, q_fp8, q_scale, w, k_fp8, k_scale, q_row_offsets,
                   kv_row_offsets, H_I, chunk, scores, score_ld);
  else
    launch_ht<64>(ht, nw, grid, st, q_fp8, q_scale, w, k_fp8, k_scale, q_row_offsets,
                  kv_row_offsets, H_I, chunk, scores, score_ld);
  return check_launch("dsa_index_score");
}
