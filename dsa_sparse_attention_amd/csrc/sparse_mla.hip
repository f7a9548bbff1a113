// sparse_mla.hip -- sparse MLA decode over the top-k selected latent rows (gfx950).
//
// "MAX Pipeline 中的 DeepSeek-V3.2 架构实现解析", section "稀疏 MLA 的前向路径": attention
// runs only over the positions the indexer selected; latent row = kv_lora_rank
// 512 + qk_rope_head_dim 64 ("GLM-5.3 推理全链路(十四)", "GLM-5.3 的草稿层到底长什么样").
// Index sharing: "MAX 中 GLM-5.2 ... 统一 MTP 推测解码架构解析", "阶段 5".
//
// Work split: a block owns one query row and one slice (<= 1024 entries) of its
// top-k list (split-K); wave w owns heads 16w..16w+15.
//  1. The slice's valid indices are compacted into LDS in list order (block
//     prefix sum), so -1 padding and out-of-range entries cost neither HBM
//     traffic nor MFMA work, and the accumulation order is deterministic.
//  2. Latent rows stream HBM -> LDS with 16-byte global_load_lds (LDS DMA, no
//     registers) in 32-row chunks, double-buffered: chunk c+1 is in flight
//     while chunk c is computed. Rows are stored unpadded (1152 B) with the
//     16-byte units of each 128-byte group XOR-swizzled by row, which keeps
//     both read patterns below free of bank conflicts.
//  3. S^T[key, head] = K[32 x 576] . Q^T with v_mfma_f32_16x16x32_bf16 (Q^T
//     fragments stay in registers); online softmax per head in base 2, one
//     head per lane column, with a lazy reference max: it moves (and the
//     accumulators are rescaled) only when a chunk's max exceeds it by more
//     than 2^8, so P <= 2^8 and the result is unchanged up to rounding.
//  4. O^T[dim, head] += V^T . P^T: P^T is the S^T accumulator itself (no data
//     movement); the V^T operand comes from ds_read_b64_tr_b16, which
//     transposes 4x4 blocks of bf16 across lanes while reading, so each 16x32
//     A operand is two 8-byte LDS reads per lane.
// With more than one split, unnormalised partials (O, max, sum) go to the
// workspace and a combine kernel merges them.
#include "common.hpp"

namespace dsa {
namespace {

constexpr int DQK = 576, DV = 512;
constexpr int KC = 32;                      // latent rows per chunk
constexpr int UNITS = DQK * 2 / 16;         // 72 16-byte units (8 dims each) per latent row
constexpr int UNIT_BYTES = KC * 16;         // 512: one unit of all 32 rows of a chunk
constexpr int CHUNK_BYTES = UNITS * UNIT_BYTES;  // 36864
constexpr int BLOCKS = CHUNK_BYTES / 1024;  // 36 wave-wide (64 x 16 B) DMA blocks per chunk
constexpr int MAX_KPS = 1024;               // top-k entries per split (LDS index staging)
constexpr float LAZY = 8.0f;                // reference-max slack, log2 units

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ bf16x8 as_bf16x8(i32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Chunk layout in LDS, unit-major: byte 512*u + 16*cell(r, u) holds dims 8u..8u+7 of the
// chunk's row r, with cell(r, u) = r ^ (4 * (u & 1)) (an involution in r).
//  - A K fragment read (16 lanes = rows 0..15 or 16..31 at one unit) is a contiguous
//    256-byte block: no bank conflicts.
//  - A transposing V read (16 lanes = 4 rows 4j..4j+3 x 2 adjacent units 2d, 2d+1)
//    lands on two disjoint 64-byte runs of the 256-byte bank window, thanks to the
//    4-row offset of odd units.
//  - A wave-wide DMA block m (1 KB) is units 2m and 2m+1: lane l writes cell l%32 of
//    unit 2m + l/32, so it loads chunk row (l%32) ^ (4*(l/32)) for every m -- one row
//    per lane per chunk, with a per-DMA offset of 32*m bytes in the source row.
__device__ __forceinline__ int cell(int row, int unit) { return row ^ (4 * (unit & 1)); }

template <int NW>
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    before += w < wave ? tmp[w] : 0;
    tot += tmp[w];
  }
  *total = tot;
  __syncthreads();
  return before + x - v;
}

// Two waves per SIMD: caps the kernel at 256 registers per lane (Q^T 72, O^T 128, rest).
// NW is a power of two (1, 2, 4, 8); heads past H are computed on zero queries and
// never stored.
template <int NW>
__global__ __launch_bounds__(NW * 64, NW == 1 ? 1 : 2) void mla_decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ topk, const int32_t* __restrict__ share_base,
    const int32_t* __restrict__ num_acc, const int32_t* __restrict__ q_off,
    const int64_t* __restrict__ kv_off, int H, int k, int topk_rows, float c2, int nsplit,
    int keys_per_split, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  constexpr int NT = NW * 64;
  constexpr int PER_T = (MAX_KPS + NT - 1) / NT;  // index entries per thread
  constexpr int DTW = (DV / 16) / NW;             // 16-dim output tiles per wave
  constexpr int DMA_PER = (BLOCKS + NW - 1) / NW; // DMA blocks per wave per chunk
  static_assert((NW & (NW - 1)) == 0 && NW <= 8, "NW must be 1, 2, 4 or 8");
  static_assert(DTW % 4 == 0, "a wave's first dim tile is a multiple of 4");
  __shared__ __attribute__((aligned(1024))) uint8_t kvbuf[2][CHUNK_BYTES];
  __shared__ int32_t sidx[MAX_KPS];
  __shared__ int scan_tmp[NW];
  __shared__ float sh_alpha[NW * 16]; // rescale factor of each head this chunk
  __shared__ int sh_resc[NW];         // wave h moved its reference this chunk
  // P^T operands of every wave (NW x 64 lanes x 16 B). Up to 4 KB they live in the rope
  // units (64..71, the last 4 KB) of the chunk being computed, dead once S^T is done;
  // 128 heads need a buffer of their own.
  constexpr bool P_IN_ROPE = NW <= 4;
  __shared__ i32x4 pbuf_own[P_IN_ROPE ? 1 : NW * 64];
  auto pslot = [&](const uint8_t* buf, int h, int ln) -> i32x4* {
    const int sl = h * 64 + ln;
    return P_IN_ROPE ? (i32x4*)(buf + 64 * UNIT_BYTES + 16 * sl) : &pbuf_own[sl];
  };

  const int split = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const RowInfo ri = load_row_info(q_off, kv_off, b);
  if (r >= ri.R) return;
  const int64_t t = ri.t0 + r;
  const int64_t trow = share_base ? static_cast<int64_t>(share_base[b]) + num_acc[b] : t;
  const bool trow_ok = trow >= 0 && trow < topk_rows && ri.L > 0;  // else nothing selected
  const int32_t* idx = topk + (trow_ok ? trow : 0) * k;
  const int i_begin = split * keys_per_split;
  const int i_end =
      !trow_ok ? i_begin : (i_begin + keys_per_split < k ? i_begin + keys_per_split : k);

  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // wave-uniform, kept in an SGPR
  const int g = lane / 16, c16 = lane % 16;
  const int head = wave * 16 + c16;  // head of this lane's column in the S/softmax phase
  const bool head_ok = head < H;

  // Q^T fragments: head `head`, dims 32*ks + 8*g .. +8 (loads overlap the index staging).
  // Heads past H read head H-1 and are zeroed.
  bf16x8 qf[18];
  {
    const uint16_t* qrow = q + (t * H + (head_ok ? head : H - 1)) * DQK + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const i32x4 v = *reinterpret_cast<const i32x4*>(qrow + 32 * ks);
      const i32x4 zero = {0, 0, 0, 0};
      qf[ks] = as_bf16x8(head_ok ? v : zero);
    }
  }

  // 1. compact the valid indices of the slice into sidx, in list order
  int mine[PER_T];
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < PER_T; ++j) {
    const int i = i_begin + tid * PER_T + j;
    int p = i < i_end ? idx[i] : -1;
    p = (p >= 0 && p < ri.L) ? p : -1;
    mine[j] = p;
    cnt += p >= 0;
  }
  int nvalid;
  int pos = block_excl_scan<NW>(cnt, scan_tmp, &nvalid);
#pragma unroll
  for (int j = 0; j < PER_T; ++j)
    if (mine[j] >= 0) sidx[pos++] = mine[j];
  const int nchunks = (nvalid + KC - 1) / KC;
  for (int i = nvalid + tid; i < nchunks * KC; i += NT) sidx[i] = -1;
  __syncthreads();

  // 2. chunk c -> LDS slot c&1 in wave-wide 1 KB DMA blocks m = wave + j*NW. Lane l
  // loads chunk row (l%32) ^ (4*(l/32)) for all of them: dims 8*(2m + l/32) .. +8.
  // `ln` is an opaque copy of the lane index (recomputed per chunk rather than hoisted
  // into registers held across the loop).
  const uint16_t* kvreq = kv + ri.kv_base * DQK;
  auto dma_src = [&](int c, int ln) {  // this lane's source for DMA block 0 of chunk c
    const int p = sidx[c * KC + ((ln & 31) ^ (4 * (ln >> 5)))];
    // padding rows load position 0 and are masked below
    return kvreq + static_cast<int64_t>(p < 0 ? 0 : p) * DQK + 8 * (ln >> 5);
  };
  auto dma_one = [&](int c, int j, const uint16_t* src) {
    const int m = wave + j * NW;
    if (m < BLOCKS)  // wave-uniform
      lds_dma16(src + 16 * m, (const lds_void*)((const lds_u8*)kvbuf[c & 1] + m * 1024));
  };

  f32x4 o[DTW][NW];  // O^T tiles: dims 16*(wave*DTW + d) .., heads 16h .. of the block
#pragma unroll
  for (int d = 0; d < DTW; ++d)
#pragma unroll
    for (int h = 0; h < NW; ++h) o[d][h] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;  // reference max (base-2 logits) of head `head`
  float lsum = 0.0f;        // running sum of this lane's share of the keys of `head`

  if (nchunks > 0) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const uint16_t* src = dma_src(0, ln);
#pragma unroll
    for (int j = 0; j < DMA_PER; ++j) dma_one(0, j, src);
  }
#pragma unroll 1
  for (int c = 0; c < nchunks; ++c) {
    DSA_WAIT_VMCNT(0);  // the only loads in flight: chunk c
    __syncthreads();    // chunk c is in LDS for every wave; chunk c-1's slot and pbuf are free
    const bool more = c + 1 < nchunks;
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const uint16_t* src = more ? dma_src(c + 1, ln) : kvreq;
    const uint8_t* buf = kvbuf[c & 1];

    // 3. S^T for keys 0..15 (s0) and 16..31 (s1): lane holds keys 4g+i / 16+4g+i of head
    // `head`. Chunk c+1's DMAs are spread over this loop, so the wave never stalls on a
    // burst of them.
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    // k-step ks: lane (g, c16) reads unit 4ks + g of rows c16 (s0) and 16 + c16 (s1)
    const uint8_t* kfrag = buf + g * UNIT_BYTES + 16 * cell(c16, g);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      if (more) {
#pragma unroll
        for (int j = ks * DMA_PER / 18; j < (ks + 1) * DMA_PER / 18; ++j) dma_one(c + 1, j, src);
      }
      const uint8_t* kp = kfrag + 4 * ks * UNIT_BYTES;
      const bf16x8 a0 = as_bf16x8(*reinterpret_cast<const i32x4*>(kp));
      const bf16x8 a1 = as_bf16x8(*reinterpret_cast<const i32x4*>(kp + 16 * 16));
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[ks], s1, 0, 0, 0);
    }

    // 4. softmax of this wave's 16 heads with a lazy reference max: it moves (and the
    // accumulators are rescaled) only when the chunk max exceeds it by more than
    // 2^LAZY; otherwise P <= 2^LAZY, and the reference cancels between numerator and
    // denominator.
    const int kb = c * KC;
    float z[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = kb + 4 * g + i < nvalid ? s0[i] * c2 : -INFINITY;
      z[4 + i] = kb + 16 + 4 * g + i < nvalid ? s1[i] * c2 : -INFINITY;
    }
    float cm = z[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) cm = fmaxf(cm, z[i]);
    cm = fmaxf(cm, __shfl_xor(cm, 16));
    cm = fmaxf(cm, __shfl_xor(cm, 32));  // finite: every chunk holds at least one valid key
    const bool resc = __any(cm > m_ref + LAZY);  // wave-uniform; always on the first chunk
    if (resc) {
      const float mn = cm > m_ref + LAZY ? cm : m_ref;
      const float alpha = exp2f(m_ref - mn);  // 0 on the first chunk, 1 if unchanged
      lsum *= alpha;
      m_ref = mn;
      if (g == 0) sh_alpha[head] = alpha;
    }
    if (lane == 0) sh_resc[wave] = resc;
    uint32_t pw[4];
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint16_t ha = f32_to_bf16_bits(exp2f(z[2 * i] - m_ref));  // masked keys: 0
      const uint16_t hb = f32_to_bf16_bits(exp2f(z[2 * i + 1] - m_ref));
      psum += bf16_bits_to_f32(ha) + bf16_bits_to_f32(hb);
      pw[i] = static_cast<uint32_t>(ha) | (static_cast<uint32_t>(hb) << 16);
    }
    lsum += psum;
    // The P^T operand of the 16x16x32 MFMA: lane (head c16, group g) holds keys
    // 4g..4g+3 and 16+4g..16+4g+3 (the K index order shared with the V^T operand).
    __syncthreads();  // every wave is done reading K (the rope columns take P^T)
    *pslot(buf, wave, lane) = (i32x4){(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3]};
    __syncthreads();  // every wave's P^T and rescale factors are in LDS

    // 5. O^T[dim, head] += V^T . P^T for this wave's dims and every head of the block. The
    // V^T operand comes from transposing reads: source lane s of group g points at row
    // key(g, s/4) and dims 16*dt + 4*(s%4) .. +4; the read hands lane i the value at dim
    // 16*dt + i of rows key(g, 0..3) -- keys 4g..4g+3, then 16+4g..16+4g+3.
    // Rescale the tiles of heads whose wave moved its reference this chunk.
#pragma unroll
    for (int h = 0; h < NW; ++h) {
      if (sh_resc[h]) {  // block-uniform
        const float a = sh_alpha[16 * h + c16];
#pragma unroll
        for (int d = 0; d < DTW; ++d) o[d][h] *= a;
      }
    }
    // Dim tile dt: source lane (group g, s = lane%16) points at row 4g + s/4 (+16 for
    // the second read), unit 2dt + (s%4)/2, byte 8*(s%2) of the unit cell. `ln` keeps the
    // lane-dependent base from being hoisted across the loop.
    const int g2 = ln >> 4, s2 = ln & 15;
    const int vu = (s2 & 3) >> 1;  // unit parity
    const lds_u8* vbase = (const lds_u8*)buf + vu * UNIT_BYTES +
                          16 * cell(4 * g2 + (s2 >> 2), vu) + 8 * (s2 & 1);
    auto v_operand = [&](int d) {
      const int dt = wave * DTW + d;
      const lds_u8* pa = vbase + 2 * dt * UNIT_BYTES;
      const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)pa);
      const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(pa + 16 * 16));
      const s16x4 v8[2] = {va, vb};
      return __builtin_bit_cast(bf16x8, v8);
    };
    if constexpr (NW <= 4) {  // all P^T operands in registers, one V^T operand at a time
      bf16x8 pf[NW];
#pragma unroll
      for (int h = 0; h < NW; ++h) pf[h] = as_bf16x8(*pslot(buf, h, lane));
#pragma unroll
      for (int d = 0; d < DTW; ++d) {
        const bf16x8 aop = v_operand(d);
#pragma unroll
        for (int h = 0; h < NW; ++h)
          o[d][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, pf[h], o[d][h], 0, 0, 0);
      }
    } else {  // 128 heads: all V^T operands in registers, one P^T operand at a time
      bf16x8 aop[DTW];
#pragma unroll
      for (int d = 0; d < DTW; ++d) aop[d] = v_operand(d);
#pragma unroll
      for (int h = 0; h < NW; ++h) {
        const bf16x8 pf = as_bf16x8(*pslot(buf, h, lane));
#pragma unroll
        for (int d = 0; d < DTW; ++d)
          o[d][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[d], pf, o[d][h], 0, 0, 0);
      }
    }
  }

  // Row sums of every head, for the waves that store its dims (slot 0 of the ring is
  // free once every wave is past the loop).
  float l = lsum + __shfl_xor(lsum, 16);
  l += __shfl_xor(l, 32);
  float* sh_l = reinterpret_cast<float*>(kvbuf[0]);
  __syncthreads();
  if (g == 0) sh_l[head] = l;
  __syncthreads();
  if (g == 0 && head_ok) {
    if (nsplit == 1) {
      if (lse) lse[t * H + head] = l > 0.0f ? (m_ref + __log2f(l)) * 0.69314718055994531f : -INFINITY;
    } else {
      const int64_t slot = (t * nsplit + split) * H + head;
      ws_ml[2 * slot] = m_ref;
      ws_ml[2 * slot + 1] = l;
    }
  }
  // this lane holds dims 16*dt + 4g .. +4 of head 16h + c16 in o[d][h]
#pragma unroll
  for (int h = 0; h < NW; ++h) {
    const int hd = 16 * h + c16;
    if (hd >= H) continue;
    if (nsplit == 1) {
      const float lh = sh_l[hd];
      const float inv = lh > 0.0f ? 1.0f / lh : 0.0f;
      uint16_t* orow = out + (t * H + hd) * DV + 4 * g;
#pragma unroll
      for (int d = 0; d < DTW; ++d) {
        const int dt = wave * DTW + d;
        const uint32_t lo = f32_to_bf16_bits(o[d][h][0] * inv) |
                            (static_cast<uint32_t>(f32_to_bf16_bits(o[d][h][1] * inv)) << 16);
        const uint32_t hi = f32_to_bf16_bits(o[d][h][2] * inv) |
                            (static_cast<uint32_t>(f32_to_bf16_bits(o[d][h][3] * inv)) << 16);
        *reinterpret_cast<uint2*>(orow + 16 * dt) = make_uint2(lo, hi);
      }
    } else {
      const int64_t slot = (t * nsplit + split) * H + hd;
      float* orow = ws_o + slot * DV + 4 * g;
#pragma unroll
      for (int d = 0; d < DTW; ++d) {
        const int dt = wave * DTW + d;
        *reinterpret_cast<float4*>(orow + 16 * dt) =
            make_float4(o[d][h][0], o[d][h][1], o[d][h][2], o[d][h][3]);
      }
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
  if (lse && threadIdx.x == 0)
    lse[t * H + head] = L > 0.0f ? (M + __log2f(L)) * 0.69314718055994531f : -INFINITY;
}

#ifndef DSA_MLA_TARGET_BLOCKS
#define DSA_MLA_TARGET_BLOCKS 256
#endif

// Split count: at least ceil(k / 1024) (LDS index staging), then doubled while the grid
// is below DSA_MLA_TARGET_BLOCKS blocks and each split keeps >= 256 entries.
int choose_splits(int64_t rows, int k) {
  int s = static_cast<int>(ceil_div(k, MAX_KPS));
  while (s < 16 && rows * s < DSA_MLA_TARGET_BLOCKS && ceil_div(k, 2 * s) >= 256) s *= 2;
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
    return fail(DSA_ERR_UNSUPPORTED,
                "dsa_sparse_mla_decode: H must be a multiple of 16 in [16, 128] (got %d)", H);
  DSA_REQUIRE(k >= 1 && k <= 16 * MAX_KPS, "dsa_sparse_mla_decode: k must be in [1, %d] (got %d)",
              16 * MAX_KPS, k);
  DSA_REQUIRE(topk_rows >= 0, "dsa_sparse_mla_decode: topk_rows must be >= 0");
  DSA_REQUIRE(B >= 0 && T >= 0 && max_q_rows >= 0, "dsa_sparse_mla_decode: negative size");
  DSA_REQUIRE((share_base == nullptr) == (num_accepted == nullptr),
              "dsa_sparse_mla_decode: share_base and num_accepted go together");
  DSA_REQUIRE(share_base || topk_rows >= T,
              "dsa_sparse_mla_decode: topk needs T rows without a share map");
  DSA_REQUIRE(sm_scale > 0.0f && sm_scale < 1e30f, "dsa_sparse_mla_decode: sm_scale must be positive");
  if (B == 0 || T == 0 || max_q_rows == 0) return ok();
  DSA_REQUIRE(q && kv && topk && q_row_offsets && kv_row_offsets && out,
              "dsa_sparse_mla_decode: null pointer");
  DSA_REQUIRE((reinterpret_cast<uintptr_t>(q) & 15) == 0 && (reinterpret_cast<uintptr_t>(kv) & 15) == 0 &&
                  (reinterpret_cast<uintptr_t>(out) & 15) == 0,
              "dsa_sparse_mla_decode: q, kv and out must be 16-byte aligned");
  DSA_REQUIRE(B <= 65535 && max_q_rows <= 65535,
              "dsa_sparse_mla_decode: B and max_q_rows must be <= 65535");
  const int s = choose_splits(T, k);
  const size_t need = dsa_sparse_mla_workspace_size(T, H, k);
  if (ws_bytes < need || (need && !ws))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL,
                "dsa_sparse_mla_decode: workspace needs %zu bytes (got %zu)", need, ws_bytes);
  DSA_REQUIRE(!need || (reinterpret_cast<uintptr_t>(ws) & 15) == 0,
              "dsa_sparse_mla_decode: workspace must be 16-byte aligned");
  const int kps = static_cast<int>(keys_per_split(k, s));
  const int nsplit = static_cast<int>(ceil_div(k, kps));
  float* ws_o = static_cast<float*>(ws);
  float* ws_ml = need ? ws_o + static_cast<size_t>(T) * nsplit * H * DV : nullptr;
  const float c2 = sm_scale * 1.4426950408889634f;  // natural -> base-2 logits
  hipStream_t st = as_stream(stream);
  dim3 grid((unsigned)nsplit, (unsigned)max_q_rows, (unsigned)B);
  const int nw = H <= 16 ? 1 : H <= 32 ? 2 : H <= 64 ? 4 : 8;  // waves of 16 heads, power of 2
#define DSA_MLA_LAUNCH(NWV)                                                                    \
  hipLaunchKernelGGL(mla_decode_kernel<NWV>, grid, dim3(NWV * 64), 0, st, q, kv, topk,         \
                     share_base, num_accepted, q_row_offsets, kv_row_offsets, H, k, topk_rows, \
                     c2, nsplit, kps, out, lse, ws_o, ws_ml)
  switch (nw) {
    case 1: DSA_MLA_LAUNCH(1); break;
    case 2: DSA_MLA_LAUNCH(2); break;
    case 4: DSA_MLA_LAUNCH(4); break;
    default: DSA_MLA_LAUNCH(8); break;
  }
#undef DSA_MLA_LAUNCH
  dsa_status stt = check_launch("dsa_sparse_mla_decode");
  if (stt != DSA_OK || nsplit == 1) return stt;
  hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)T, (unsigned)H), dim3(128), 0, st, ws_o,
                     ws_ml, H, nsplit, out, lse);
  return check_launch("dsa_sparse_mla_decode(combine)");
}
