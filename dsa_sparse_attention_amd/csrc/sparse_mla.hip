// sparse_mla.hip -- sparse MLA decode over the top-k selected latent rows (gfx950).
//
// "MAX Pipeline 中的 DeepSeek-V3.2 架构实现解析", section "稀疏 MLA 的前向路径": attention
// runs only over the positions the indexer selected; latent row = kv_lora_rank
// 512 + qk_rope_head_dim 64 ("GLM-5.3 推理全链路(十四)", "GLM-5.3 的草稿层到底长什么样").
// Index sharing: "MAX 中 GLM-5.2 ... 统一 MTP 推测解码架构解析", "阶段 5".
//
// Work split: a block owns one query row, one group of 64 heads and one slice (at most
// 2048 entries) of the row's top-k list; one block per CU, 16 waves in two roles:
//  - 8 S waves: wave (hq, kt) computes S^T[key, head] for keys 16kt..16kt+15 of a 32-key
//    chunk and heads 16hq..16hq+15 with v_mfma_f32_16x16x32_bf16 (its Q^T operand,
//    576 dims, stays in registers), then the online softmax of its heads: the chunk
//    max combines both key halves through LDS, and the reference max is lazy (it moves,
//    and the accumulators are rescaled, only when a chunk max exceeds it by more than
//    2^8, so P <= 2^8 and the result is unchanged up to rounding). P^T goes to LDS in
//    MFMA operand order, over the rope columns of the chunk (dead once S^T is done).
//  - 8 O waves: wave ow accumulates O^T[dim, head] for dims 64ow..64ow+63 of all 64
//    heads (four v_mfma_f32_32x32x16_bf16 tiles), one chunk behind the S waves; the V^T
//    operand comes from ds_read_b64_tr_b16, which transposes 4x4 blocks of bf16 across
//    lanes while reading. The O waves also stream the latent rows HBM -> LDS with
//    16-byte global_load_lds (LDS DMA, no registers), two chunks ahead, into a ring of
//    four 36 KB chunk buffers.
// The slice's valid indices are first compacted into LDS in list order (block prefix
// sum), so -1 padding and out-of-range entries cost neither HBM traffic nor MFMA work.
// With more than one slice per row, unnormalised partials (O, max, sum) go to the
// workspace and a combine kernel merges them.
#include <type_traits>

#include "common.hpp"

namespace dsa {
namespace {

constexpr int DQK = 576, DV = 512;
constexpr int KC = 32;                           // latent rows per chunk
constexpr int UNITS = DQK * 2 / 16;              // 72 16-byte units (8 dims each) per row
constexpr int CHUNK_BYTES = KC * UNITS * 16;     // 36864
constexpr int DMA_BLOCKS = CHUNK_BYTES / 1024;   // 36 wave-wide (64 x 16 B) DMAs per chunk
constexpr int NBUF = 4;                          // chunk ring: S, O, and two in flight
constexpr int MAX_KPS = 2048;                    // top-k entries per slice (LDS staging)
constexpr int HPB = 64;                          // heads per block
constexpr int NSW = 8, NOW = 8, NWAVE = NSW + NOW, NT = NWAVE * 64;
constexpr int KS = DQK / 32;                     // 18 k-steps of the S product
constexpr int KPF = 5;                           // K operand reads in flight ahead
constexpr int DMA_A = 2;  // O waves: DMA blocks issued before B1, the rest after
constexpr float LAZY = 8.0f;                     // reference-max slack, log2 units
constexpr float M_INIT = -1.0e30f;               // reference before any valid key (finite)

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ bf16x8 as_bf16x8(i32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// max / sum over lanes l, l^16, l^32, l^48 (the four lanes of one S^T column)
__device__ __forceinline__ float max_xor16_xor32(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float sum_xor16_xor32(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Chunk layout in LDS: 1 KB block 4 ug + rg holds rows 8rg..8rg+7 and dims 64ug..64ug+63
// (units 8ug..8ug+7 of 8 dims); row rr = r%8 of the block is 128 bytes at 128 rr, its unit
// uu = u%8 at 16 * (uu ^ rr ^ 2(rg & 1)).
//  - A DMA block (one wave-wide global_load_lds, 64 x 16 B) fills one block: lane l
//    copies unit (l%8) ^ (l/8) ^ 2(rg&1) of row 8rg + l/8, so the 8 lanes of a row read
//    one whole 128-byte line of it (8 lines per instruction, which keeps the address
//    path of the load unit from limiting the DMA rate).
//  - A K fragment read: 16 lanes = rows 0..15 or 16..31 at one unit; a transposing V
//    read: 16 lanes = 4 rows x 2 adjacent units. Measured on gfx950, this XOR keeps both
//    at the LDS peak for them (about 254 and 127 B/clk per CU).
// P^T of the chunk (32 keys x 64 heads bf16, 4 KB) overwrites the rope blocks 32..35
// after the S phase: byte 32768 + 1024 (2 ht + ko) + 16 l is lane l's B operand of head
// tile ht (32 heads), key step ko (16 keys).

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
  for (int w = 0; w < NWAVE; ++w) {
    before += w < wave ? tmp[w] : 0;
    tot += tmp[w];
  }
  *total = tot;
  __syncthreads();
  return before + x - v;
}

// Four waves per SIMD: at most 128 registers per lane.
__global__ __launch_bounds__(NT, 1) void mla_decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ topk, const int32_t* __restrict__ share_base,
    const int32_t* __restrict__ num_acc, const int32_t* __restrict__ q_off,
    const int64_t* __restrict__ kv_off, int H, int nhg, int k, int topk_rows, float c2,
    int nsplit, int keys_per_split, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  constexpr int PER_T = MAX_KPS / NT;  // index entries per thread
  __shared__ __attribute__((aligned(1024))) uint8_t kvbuf[NBUF][CHUNK_BYTES];
  __shared__ int32_t sidx[MAX_KPS];
  __shared__ int scan_tmp[NWAVE];
  __shared__ float sh_cm[2][HPB];     // chunk max of each head over one key half
  __shared__ float sh_alpha[2][HPB];  // rescale factor of each head, chunk parity
  __shared__ int sh_resc[2][4];       // head quarter moved its reference, chunk parity
  __shared__ float sh_m[HPB], sh_l[2][HPB];

  const int hg = blockIdx.x % nhg, split = blockIdx.x / nhg;
  const int r_row = blockIdx.y, b = blockIdx.z;
  const RowInfo ri = load_row_info(q_off, kv_off, b);
  if (r_row >= ri.R) return;
  const int64_t t = ri.t0 + r_row;
  const int64_t trow = share_base ? static_cast<int64_t>(share_base[b]) + num_acc[b] : t;
  const bool trow_ok = trow >= 0 && trow < topk_rows && ri.L > 0;  // else nothing selected
  const int32_t* idx = topk + (trow_ok ? trow : 0) * k;
  const int i_begin = split * keys_per_split;
  const int i_end =
      !trow_ok ? i_begin : (i_begin + keys_per_split < k ? i_begin + keys_per_split : k);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  const bool s_role = wave < NSW;

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
  int pos = block_excl_scan(cnt, scan_tmp, &nvalid);
#pragma unroll
  for (int j = 0; j < PER_T; ++j)
    if (mine[j] >= 0) sidx[pos++] = mine[j];
  const int nch = (nvalid + KC - 1) / KC;
  __syncthreads();
  // padding rows of the last chunk load the slice's first row (masked)
  for (int i = nvalid + tid; i < nch * KC; i += NT) sidx[i] = sidx[0];
  __syncthreads();

  const uint16_t* kvreq = kv + ri.kv_base * DQK;
  const int g = lane >> 4, c16 = lane & 15;  // 16x16 operand / accumulator coordinates
  const int h = lane >> 5, r = lane & 31;    // 32x32 operand / accumulator coordinates

  if (s_role) {
    // ================================ S waves ================================
    const int hq = wave >> 1, kt = wave & 1;
    const int head = min(HPB * hg + 16 * hq + c16, H - 1);  // heads past H repeat H-1
    i32x4 qf[KS];  // Q^T operand: head `head`, dims 32ks + 8g .. +8
    {
      const uint16_t* qrow = q + (t * H + head) * DQK + 8 * g;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const i32x4*>(qrow + 32 * ks);
    }
    float m_ref = M_INIT;  // reference max (base-2 logits) of head 16hq + c16
    float lsum = 0.0f;     // this lane's share of the row sum of that head
    // lane (g, c16) reads unit 4ks + g of chunk row 16kt + c16: block 4(ks/2) + 2kt + c16/8,
    // row c16%8, unit position (4(ks%2) + g) ^ sw with sw = (c16%8) ^ 2(c16/8)
    const int ksw = g ^ ((c16 & 7) ^ (2 * (c16 >> 3)));
    const int kb0 = 1024 * (2 * kt + (c16 >> 3)) + 128 * (c16 & 7) + 16 * ksw;
    const int kb1 = kb0 + 64 - 128 * (ksw >> 2);  // odd k-steps: position bit 2 flipped
#pragma unroll 1
    for (int i = 0; i <= nch; ++i) {
      __syncthreads();  // B0: chunk i is in LDS; P^T and factors of chunk i-1 are visible
      float cm = -INFINITY;
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
      const uint8_t* buf = kvbuf[i % NBUF];
      if (i < nch) {
        const uint8_t* ka0 = buf + kb0;
        const uint8_t* ka1 = buf + kb1;
        auto kread = [&](auto KSC) {
          constexpr int ks = decltype(KSC)::value;
          return *reinterpret_cast<const i32x4*>((ks & 1 ? ka1 : ka0) + 4096 * (ks >> 1));
        };
        i32x4 kr[KPF];
        static_for<0, KPF>([&](auto I) { kr[decltype(I)::value] = kread(I); });
        static_for<0, KS>([&](auto I) {
          constexpr int ks = decltype(I)::value;
          const i32x4 a = kr[ks % KPF];
          if constexpr (ks + KPF < KS)
            kr[ks % KPF] = kread(std::integral_constant<int, ks + KPF>{});
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(qf[ks]), s, 0, 0, 0);
        });
        // keys 32i + 16kt + 4g + j, j = 0..3
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool v = KC * i + 16 * kt + 4 * g + j < nvalid;
          s[j] = v ? s[j] * c2 : -INFINITY;
          cm = fmaxf(cm, s[j]);
        }
        cm = max_xor16_xor32(cm);
        if (g == 0) sh_cm[kt][16 * hq + c16] = cm;
      }
      __syncthreads();  // B1: every S wave is done with chunk i's K (rope takes P^T)
      if (i < nch) {
        cm = fmaxf(cm, sh_cm[kt ^ 1][16 * hq + c16]);
        const float mn = cm > m_ref + LAZY ? cm : m_ref;
        const bool resc = __any(mn != m_ref);  // wave-uniform; same in both key halves
        float alpha = 1.0f;
        if (resc) {
          alpha = exp2f(m_ref - mn);  // 0 at the first chunk, 1 if unchanged
          lsum *= alpha;
          m_ref = mn;
        }
        if (kt == 0) {
          if (g == 0) sh_alpha[i & 1][16 * hq + c16] = alpha;
          if (lane == 0) sh_resc[i & 1][hq] = resc;
        }
        // keys 4g .. 4g+3 of key step ko = kt are B operand slots 4g .. 4g+3 of lane
        // 32(g/2) + 16(hq%2) + c16, head tile hq/2, bytes 8(g%2) .. +8
        // The row sum takes the float32 weights; only the PV operand is rounded to bf16, so
        // lse carries float32 accuracy (a sum of bf16-rounded weights would move it by up to
        // 2^-9 when one key dominates).
        uint32_t pw[2];
        float psum = 0.0f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {  // masked keys: exp2(-inf) = 0; bf16 round to nearest even
          const float e0 = exp2f(s[2 * j] - m_ref), e1 = exp2f(s[2 * j + 1] - m_ref);
          const bf16x2 pp = __builtin_convertvector((f32x2){e0, e1}, bf16x2);
          psum += e0 + e1;
          pw[j] = __builtin_bit_cast(uint32_t, pp);
        }
        lsum += psum;
        uint8_t* pdst = const_cast<uint8_t*>(buf) + 32768 + 1024 * (2 * (hq >> 1) + kt) +
                        16 * (32 * (g >> 1) + 16 * (hq & 1) + c16) + 8 * (g & 1);
        *reinterpret_cast<uint2*>(pdst) = make_uint2(pw[0], pw[1]);
      }
    }
    // row sums and reference maxima for the O waves
    const float lt = sum_xor16_xor32(lsum);
    if (g == 0) {
      sh_l[kt][16 * hq + c16] = lt;
      if (kt == 0) sh_m[16 * hq + c16] = m_ref;
    }
    __syncthreads();
  } else {
    // ================================ O waves ================================
    const int ow = wave - NSW;
    const int ndma = ow < DMA_BLOCKS - 4 * NOW ? 5 : 4;  // blocks ow + 8j of a chunk
    // DMA block ow + 8j is (ug, rg) = (ow/4 + 2j, ow%4): this lane copies row
    // 8(ow%4) + l/8, unit 8ug + ((l%8) ^ (l/8) ^ 2(ow%2)).
    int ln = lane;
    const uint16_t* dsrc = kvreq;  // this lane's source for the chunk being issued
    auto dma_src = [&](int c) {
      asm volatile("" : "+v"(ln));
      const int p = sidx[c * KC + 8 * (ow & 3) + (ln >> 3)];
      const int uu = (ln & 7) ^ (ln >> 3) ^ (2 * (ow & 1));
      dsrc = kvreq + static_cast<int64_t>(p) * DQK + 64 * (ow >> 2) + 8 * uu;
    };
    // DMA blocks j0 <= j < j1 of chunk c (source row from dma_src(c))
    auto dma_part = [&](int c, auto J0, auto J1) {
      const lds_u8* dst = (const lds_u8*)kvbuf[c % NBUF] + 1024 * ow;
      static_for<decltype(J0)::value, decltype(J1)::value>([&](auto J) {
        constexpr int j = decltype(J)::value;
        if (j < 4 || ndma == 5)  // wave-uniform
          lds_dma16(dsrc + 128 * j, (const lds_void*)(dst + 8192 * j));
      });
    };
    auto dma_chunk = [&](int c) {
      dma_src(c);
      dma_part(c, std::integral_constant<int, 0>{}, std::integral_constant<int, 5>{});
    };
    f32x16 o[2][2];  // O^T tiles: dims 64ow + 32dt .., heads 32ht ..
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int ht = 0; ht < 2; ++ht)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][ht][e] = 0.0f;
    // V^T reads: 16-lane group g reads rows 16ko + 8(g/2) + 4rd + s/4 (read rd = 0/1) and
    // dims 64ow + 32dt + 16(g%2) + 4(s%4) .. +4 (s = lane%16): block 4ow + 2ko + g/2, row
    // 4rd + s/4, unit position (4dt + 2(g%2) + (s%4)/2) ^ (4rd + ((s/4) ^ 2(g/2))), which
    // is 4(dt ^ rd) + (low two bits, fixed per lane).
    const int vpos = (2 * (g & 1) + ((c16 & 3) >> 1)) ^ ((c16 >> 2) ^ (2 * (g >> 1)));
    const int vlane = 4096 * ow + 1024 * (g >> 1) + 128 * (c16 >> 2) + 16 * vpos + 8 * (c16 & 1);
    if (nch > 0) dma_chunk(0);
    if (nch > 1) dma_chunk(1);
#pragma unroll 1
    for (int i = 0; i <= nch; ++i) {
      // chunk i landed: only chunk i+1's DMAs may still be in flight
      if (i + 1 < nch) {
        if (ndma == 5) DSA_WAIT_VMCNT(5);
        else DSA_WAIT_VMCNT(4);
      } else {
        DSA_WAIT_VMCNT(0);
      }
      __syncthreads();  // B0
      if (i + 2 < nch) {
        dma_src(i + 2);
        dma_part(i + 2, std::integral_constant<int, 0>{}, std::integral_constant<int, DMA_A>{});
      }
      const int c = i - 1;  // chunk accumulated in this iteration
      const uint8_t* buf = kvbuf[(c + NBUF) % NBUF];
      auto o_step = [&](int ko) {
        const uint8_t* pb = buf + 32768 + 1024 * ko + 16 * lane;
        const i32x4 p0 = *reinterpret_cast<const i32x4*>(pb);         // heads 0..31
        const i32x4 p1 = *reinterpret_cast<const i32x4*>(pb + 2048);  // heads 32..63
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const lds_u8* pa = (const lds_u8*)buf + vlane + 2048 * ko;
          const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(pa + 64 * dt));
          const s16x4 x1 =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(pa + 512 + 64 * (dt ^ 1)));
          const s16x4 v8[2] = {x0, x1};
          const bf16x8 aop = __builtin_bit_cast(bf16x8, v8);
          o[dt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, as_bf16x8(p0), o[dt][0], 0, 0, 0);
          o[dt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, as_bf16x8(p1), o[dt][1], 0, 0, 0);
        }
      };
      if (c >= 0) {
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
          if (sh_resc[c & 1][2 * ht] | sh_resc[c & 1][2 * ht + 1]) {  // block-uniform
            const float a = sh_alpha[c & 1][32 * ht + r];
#pragma unroll
            for (int dt = 0; dt < 2; ++dt) o[dt][ht] *= a;
          }
        }
        o_step(0);
      }
      __syncthreads();  // B1
      if (i + 2 < nch)
        dma_part(i + 2, std::integral_constant<int, DMA_A>{}, std::integral_constant<int, 5>{});
      if (c >= 0) o_step(1);
    }
    __syncthreads();  // row sums and maxima from the S waves
    // this lane holds dims 64ow + 32dt + 8qd + 4h .. +4 of head 32ht + r in o[dt][ht]
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const int hd = HPB * hg + 32 * ht + r;
      if (hd >= H) continue;
      const float mh = sh_m[32 * ht + r];
      const float lh = sh_l[0][32 * ht + r] + sh_l[1][32 * ht + r];
      if (nsplit == 1) {
        const float inv = lh > 0.0f ? 1.0f / lh : 0.0f;
        uint16_t* orow = out + (t * H + hd) * DV + 64 * ow + 4 * h;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const f32x16& a = o[dt][ht];
            const uint32_t lo = f32_to_bf16_bits(a[4 * qd] * inv) |
                                (static_cast<uint32_t>(f32_to_bf16_bits(a[4 * qd + 1] * inv)) << 16);
            const uint32_t hi = f32_to_bf16_bits(a[4 * qd + 2] * inv) |
                                (static_cast<uint32_t>(f32_to_bf16_bits(a[4 * qd + 3] * inv)) << 16);
            *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * qd) = make_uint2(lo, hi);
          }
        if (lse && ow == 0 && h == 0)
          lse[t * H + hd] = lh > 0.0f ? (mh + __log2f(lh)) * 0.69314718055994531f : -INFINITY;
      } else {
        const int64_t slot = (t * nsplit + split) * H + hd;
        float* orow = ws_o + slot * DV + 64 * ow + 4 * h;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd)
            *reinterpret_cast<float4*>(orow + 32 * dt + 8 * qd) =
                make_float4(o[dt][ht][4 * qd], o[dt][ht][4 * qd + 1], o[dt][ht][4 * qd + 2],
                            o[dt][ht][4 * qd + 3]);
        if (ow == 0 && h == 0) {
          ws_ml[2 * slot] = mh;
          ws_ml[2 * slot + 1] = lh;
        }
      }
    }
  }
}

// Merge split partials of one (row, head): 128 threads x 4 dims.
__global__ __launch_bounds__(128) void mla_combine_kernel(const float* __restrict__ ws_o,
                                                          const float* __restrict__ ws_ml,
                                                          int H, int nsplit,
                                                          uint16_t* __restrict__ out,
                                                          float* __restrict__ lse) {
  const int64_t t = blockIdx.x;
  const int head = blockIdx.y;
  float M = M_INIT;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ws_ml[2 * ((t * nsplit + s) * H + head)]);
  float L = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < nsplit; ++s) {
    const int64_t slot = (t * nsplit + s) * H + head;
    const float f = exp2f(ws_ml[2 * slot] - M);  // 0 for a slice without valid keys
    L += ws_ml[2 * slot + 1] * f;
    const float4 v = reinterpret_cast<const float4*>(ws_o + slot * DV)[threadIdx.x];
    acc.x += v.x * f; acc.y += v.y * f; acc.z += v.z * f; acc.w += v.w * f;
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const uint32_t lo = f32_to_bf16_bits(acc.x * inv) | (static_cast<uint32_t>(f32_to_bf16_bits(acc.y * inv)) << 16);
  const uint32_t hi = f32_to_bf16_bits(acc.z * inv) | (static_cast<uint32_t>(f32_to_bf16_bits(acc.w * inv)) << 16);
  reinterpret_cast<uint2*>(out + (t * H + head) * DV)[threadIdx.x] = make_uint2(lo, hi);
  if (lse && threadIdx.x == 0)
    lse[t * H + head] = L > 0.0f ? (M + __log2f(L)) * 0.69314718055994531f : -INFINITY;
}

constexpr int64_t TARGET_BLOCKS = 160;  // grids below this many blocks take more slices

// Slices per row: at least ceil(k / 2048) (LDS index staging), then doubled while the
// grid is below TARGET_BLOCKS blocks (one per CU) and each slice keeps >= 256
// entries.
int choose_splits(int64_t blocks_per_split, int k) {
  int s = static_cast<int>(ceil_div(k, MAX_KPS));
  while (s < 16 && blocks_per_split * s < TARGET_BLOCKS && ceil_div(k, 2 * s) >= 256)
    s *= 2;
  return s;
}

int64_t keys_per_split(int k, int s) { return ceil_div(ceil_div(k, s), KC) * KC; }

}  // namespace
}  // namespace dsa

extern "C" size_t dsa_sparse_mla_workspace_size(int32_t T, int32_t H, int32_t k) {
  using namespace dsa;
  if (T <= 0 || H <= 0 || k <= 0) return 0;
  const int s = choose_splits(static_cast<int64_t>(T) * ceil_div(H, HPB), k);
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
  const int nhg = static_cast<int>(ceil_div(H, HPB));
  const int s = choose_splits(static_cast<int64_t>(T) * nhg, k);
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
  hipLaunchKernelGGL(mla_decode_kernel,
                     dim3((unsigned)(nsplit * nhg), (unsigned)max_q_rows, (unsigned)B), dim3(NT),
                     0, st, q, kv, topk, share_base, num_accepted, q_row_offsets, kv_row_offsets,
                     H, nhg, k, topk_rows, c2, nsplit, kps, out, lse, ws_o, ws_ml);
  dsa_status stt = check_launch("dsa_sparse_mla_decode");
  if (stt != DSA_OK || nsplit == 1) return stt;
  hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)T, (unsigned)H), dim3(128), 0, st, ws_o,
                     ws_ml, H, nsplit, out, lse);
  return check_launch("dsa_sparse_mla_decode(combine)");
}
