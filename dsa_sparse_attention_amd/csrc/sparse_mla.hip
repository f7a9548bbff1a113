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
//
// FP8 latent cache (mla_decode_kernel<true>; "GLM-5.3 推理全链路(十四)": 656 bytes per
// token per layer, the fp8_ds_mla layout): a row is 512 e4m3fn latent codes in four
// 128-value blocks with one float32 scale each, then the 64 rope values in bf16. The
// chunk lands in LDS as code blocks, rope blocks and the 32 rows' scales (21 DMAs instead
// of 36). Codes convert exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8 with scale 1), so the
// MFMAs stay bf16 and the scales are applied where they are exact in float32:
//  - S^T keeps one accumulator per scale block (and one for the rope); a key's logit is
//    sum_b scale_b * S_b + S_rope;
//  - the PV product takes P^T[key, head] * scale_b(key) as its B operand, one copy per
//    block b, and each O wave (64 dims, inside one block) reads its block's copy; its V^T
//    operand comes from ds_read_b64_tr_b8, which gathers 8 keys of one dim into a lane.
#include <type_traits>

#include "common.hpp"

namespace dsa {
namespace {

constexpr int DQK = 576, DV = 512;
constexpr int KC = 32;                           // latent rows per chunk
constexpr int UNITS = DQK * 2 / 16;              // 72 16-byte units (8 dims each) per row
constexpr int CHUNK_BYTES = KC * UNITS * 16;     // 36864
constexpr int DMA_BLOCKS = CHUNK_BYTES / 1024;   // 36 wave-wide (64 x 16 B) DMAs per chunk
constexpr int LEAD = 2;                          // chunks in flight ahead of the S waves
constexpr int NBUF = LEAD + 2;                   // chunk ring: S, O, and LEAD in flight
constexpr int MAX_KPS = 2048;                    // top-k entries per slice (LDS staging)
constexpr int MAX_SPLITS = 16;                   // slices per row (k <= 16 * MAX_KPS)
constexpr int HPB = 64;                          // heads per block
constexpr int NSW = 8, NOW = 8, NWAVE = NSW + NOW, NT = NWAVE * 64;
constexpr int KS = DQK / 32;                     // 18 k-steps of the S product
constexpr int KPF = 5;                           // K operand reads in flight ahead
constexpr int DMA_A = 2;  // O waves: DMA blocks issued before B1, the rest after
constexpr float LAZY = 8.0f;                     // reference-max slack, log2 units
// FP8 latent rows: byte layout of a cache row and of a chunk slot in LDS
constexpr int RB8 = 656;                 // bytes per row: 512 codes, 4 float32 scales, 64 bf16
constexpr int RB8_SCALE = 512, RB8_ROPE = 528;
constexpr int F8_ROPE = KC * 512;        // 16 code blocks (4 scale blocks x 4 row groups) first
constexpr int F8_SCALE = F8_ROPE + 4096; // then 4 rope blocks, then the rows' scales (1 KB)
constexpr int F8_SLOT = F8_SCALE + 1024;
constexpr int F8_DMA = F8_SLOT / 1024;   // 21 DMA blocks per chunk
constexpr int F8_PB = 4 * 4096;          // P^T of a chunk, one scaled copy per latent block
constexpr float M_INIT = -1.0e30f;               // reference before any valid key (finite)

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

__device__ __forceinline__ bf16x8 as_bf16x8(i32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// 2^x by v_exp_f32 alone: results below 2^-126 flush to +0 (exp2f would rescale them into
// denormals at five more instructions each). The softmax weights taken here never need
// them: the key that set the reference max weighs exactly 1, so the row sum is at least 1
// and a weight or a rescale factor below 2^-126 is below half an ulp of it, and of the
// output's float32 accumulation as well.
__device__ __forceinline__ float exp2_flush(float x) { return __builtin_amdgcn_exp2f(x); }

// The larger of two logits by one v_max_f32. fmaxf would first quiet each operand that the
// compiler cannot prove canonical (lane swaps, selects), one more instruction per operand;
// logits are never NaN here (-inf marks a padding row), so the plain instruction serves.
__device__ __forceinline__ float max_logit(float a, float b) {
  float r;
  asm("v_max_f32_e32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// max / sum over lanes l, l^16, l^32, l^48 (the four lanes of one S^T column)
__device__ __forceinline__ float max_xor16_xor32(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = max_logit(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return max_logit(__uint_as_float(b[0]), __uint_as_float(b[1]));
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

// Four waves per SIMD: at most 128 registers per lane. F8: kv holds FP8 rows of RB8 bytes,
// else bf16 rows of DQK values.
template <bool F8>
__global__ __launch_bounds__(NT, 1) void mla_decode_kernel(
    const uint16_t* __restrict__ q, const void* __restrict__ kv_rows,
    const int32_t* __restrict__ topk, const int32_t* __restrict__ share_base,
    const int32_t* __restrict__ num_acc, const int32_t* __restrict__ q_off,
    const int64_t* __restrict__ kv_off, int H, int nhg, int k, int topk_rows, float c2,
    int nsplit, int keys_per_split, int max_q_rows, int nwork, int per_xcd,
    uint16_t* __restrict__ out, float* __restrict__ lse, uint16_t* __restrict__ ws_o,
    float* __restrict__ ws_ml) {
  constexpr int PER_T = MAX_KPS / NT;  // index entries per thread
  constexpr int SLOT = F8 ? F8_SLOT : CHUNK_BYTES;
  constexpr int NB = NBUF, LD = LEAD;
  __shared__ __attribute__((aligned(1024))) uint8_t kvbuf[NB][SLOT];
  // F8: P^T of the last two chunks, one copy per latent scale block with each key's block
  // scale applied (bf16 keeps a single P^T over the chunk's rope columns)
  __shared__ __attribute__((aligned(1024))) uint8_t pbuf[F8 ? 2 : 1][F8 ? F8_PB : 16];
  __shared__ int32_t sidx[MAX_KPS];
  __shared__ int scan_tmp[NWAVE];
  __shared__ float sh_cm[2][HPB];     // chunk max of each head over one key half
  __shared__ float sh_alpha[2][HPB];  // rescale factor of each head, chunk parity
  __shared__ int sh_resc[2][4];       // head quarter moved its reference, chunk parity
  __shared__ float sh_m[HPB], sh_l[2][HPB];

  // Work item w = (split * nhg + hg) + nsplit * nhg * (row + max_q_rows * request): the
  // blocks of one query row (its head groups and slices) are consecutive. Block L goes to
  // XCD L % 8 (round-robin dispatch), and XCD x takes items x * per_xcd .. + per_xcd - 1, so
  // a row's blocks share one L2: the head groups' gathers of the same latent rows hit it.
  const int w = static_cast<int>(blockIdx.x % 8) * per_xcd + static_cast<int>(blockIdx.x / 8);
  if (w >= nwork) return;
  const int gx = nsplit * nhg;
  const int hg = (w % gx) % nhg, split = (w % gx) / nhg;
  const int r_row = (w / gx) % max_q_rows, b = (w / gx) / max_q_rows;
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

  const uint16_t* kvreq = static_cast<const uint16_t*>(kv_rows) + (F8 ? 0 : ri.kv_base * DQK);
  const uint8_t* kv8req = static_cast<const uint8_t*>(kv_rows) + (F8 ? ri.kv_base * RB8 : 0);
  const int g = lane >> 4, c16 = lane & 15;  // 16x16 operand / accumulator coordinates
  const int h = lane >> 5, r = lane & 31;    // 32x32 operand / accumulator coordinates

  if (s_role) {
    // ================================ S waves ================================
    const int hq = wave >> 1, kt = wave & 1;
    const int head = min(HPB * hg + 16 * hq + c16, H - 1);  // heads past H repeat H-1
    // Q^T operand: head `head`, dims 32ks + 8g .. +8. F8: the MFMA sum runs over the 512
    // latent dims in another order (any order shared by both operands gives the same
    // product): k-step ks < 16 takes dims 128(ks/4) + 16(4((ks/2)%2) + g) + 8(ks%2) .. +8,
    // the halves of the 16 codes its lane reads at once.
    i32x4 qf[KS];
    {
      const uint16_t* qrow = q + (t * H + head) * DQK;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int d = (F8 && ks < 16) ? 128 * (ks >> 2) + 16 * (4 * ((ks >> 1) & 1) + g) + 8 * (ks & 1)
                                      : 32 * ks + 8 * g;
        qf[ks] = *reinterpret_cast<const i32x4*>(qrow + d);
      }
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
      f32x4 s8[F8 ? 5 : 1];  // F8: S^T per latent scale block, and of the rope
      f32x4 ksc[F8 ? 4 : 1];  // F8: the four block scales of keys 16kt + 4g + j
      if constexpr (F8) {
#pragma unroll
        for (int bb = 0; bb < 5; ++bb) s8[bb] = (f32x4){0.f, 0.f, 0.f, 0.f};
      }
      const uint8_t* buf = kvbuf[i % NB];
      if (i < nch) {
        const uint8_t* ka0 = buf + kb0;
        const uint8_t* ka1 = buf + kb1;
        if constexpr (!F8) {
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
        } else {
          // reads r < 8: 16 codes of latent pair r (code block r/2, position bit 2 = r%2),
          // converted here to exact bf16; r = 8, 9: the rope k-steps 16, 17 (8 bf16 each)
          auto kread = [&](auto RC) {
            constexpr int r = decltype(RC)::value;
            if constexpr (r < 8)
              return *reinterpret_cast<const i32x4*>((r & 1 ? ka1 : ka0) + 4096 * (r >> 1));
            else
              return *reinterpret_cast<const i32x4*>((r & 1 ? ka1 : ka0) + F8_ROPE);
          };
          constexpr int KPF8 = 3;
          i32x4 kr[KPF8];
          static_for<0, KPF8>([&](auto I) { kr[decltype(I)::value] = kread(I); });
          static_for<0, 10>([&](auto I) {
            constexpr int r = decltype(I)::value;
            const i32x4 a = kr[r % KPF8];
            if constexpr (r + KPF8 < 10)
              kr[r % KPF8] = kread(std::integral_constant<int, r + KPF8>{});
            if constexpr (r < 8) {
              // e4m3 codes -> bf16, exact (scale 1): bytes 0..7 are k-step 2r, 8..15 2r+1
              static_for<0, 2>([&](auto HC) {
                constexpr int hf = decltype(HC)::value;
                const bf16x2 c0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(a[2 * hf], 1.0f, false);
                const bf16x2 c1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(a[2 * hf], 1.0f, true);
                const bf16x2 c2v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(a[2 * hf + 1], 1.0f, false);
                const bf16x2 c3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(a[2 * hf + 1], 1.0f, true);
                const bf16x8 op = {c0[0], c0[1], c1[0], c1[1], c2v[0], c2v[1], c3[0], c3[1]};
                s8[r >> 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op, as_bf16x8(qf[2 * r + hf]),
                                                                     s8[r >> 1], 0, 0, 0);
              });
            } else {
              s8[4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(qf[8 + r]),
                                                              s8[4], 0, 0, 0);
            }
          });
          // keys 16kt + 4g + j: logit = sum_b scale_b * S_b + S_rope
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            ksc[j] = *reinterpret_cast<const f32x4*>(buf + F8_SCALE + 16 * (16 * kt + 4 * g + j));
            float v = s8[4][j];
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) v = fmaf(ksc[j][bb], s8[bb][j], v);
            s[j] = v;
          }
        }
        // keys 32i + 16kt + 4g + j, j = 0..3; only the last chunk can hold padding rows
        if (KC * (i + 1) <= nvalid) {  // block-uniform
#pragma unroll
          for (int j = 0; j < 4; ++j) s[j] *= c2;
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            s[j] = KC * i + 16 * kt + 4 * g + j < nvalid ? s[j] * c2 : -INFINITY;
        }
        cm = max_logit(max_logit(s[0], s[1]), max_logit(s[2], s[3]));
        cm = max_xor16_xor32(cm);
        if (g == 0) sh_cm[kt][16 * hq + c16] = cm;
      }
      __syncthreads();  // B1: every S wave is done with chunk i's K (rope takes P^T)
      if (i < nch) {
        cm = max_logit(cm, sh_cm[kt ^ 1][16 * hq + c16]);
        const float mn = cm > m_ref + LAZY ? cm : m_ref;
        const bool resc = __any(mn != m_ref);  // wave-uniform; same in both key halves
        float alpha = 1.0f;
        if (resc) {
          alpha = exp2_flush(m_ref - mn);  // 0 at the first chunk, 1 if unchanged
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
        float ev[4];
#pragma unroll
        for (int j = 0; j < 2; ++j) {  // masked keys: exp2(-inf) = 0; bf16 round to nearest even
          const float e0 = exp2_flush(s[2 * j] - m_ref), e1 = exp2_flush(s[2 * j + 1] - m_ref);
          const bf16x2 pp = __builtin_convertvector((f32x2){e0, e1}, bf16x2);
          psum += e0 + e1;
          pw[j] = __builtin_bit_cast(uint32_t, pp);
          ev[2 * j] = e0;
          ev[2 * j + 1] = e1;
        }
        lsum += psum;
        const int poff = 1024 * (2 * (hq >> 1) + kt) + 16 * (32 * (g >> 1) + 16 * (hq & 1) + c16) +
                         8 * (g & 1);
        if constexpr (!F8) {
          *reinterpret_cast<uint2*>(const_cast<uint8_t*>(buf) + 32768 + poff) = make_uint2(pw[0], pw[1]);
        } else {
          // copy b of P^T carries each key's latent block-b scale (the row sum takes the
          // unscaled float32 weights above)
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            const bf16x2 p01 = __builtin_convertvector(
                (f32x2){ev[0] * ksc[0][bb], ev[1] * ksc[1][bb]}, bf16x2);
            const bf16x2 p23 = __builtin_convertvector(
                (f32x2){ev[2] * ksc[2][bb], ev[3] * ksc[3][bb]}, bf16x2);
            *reinterpret_cast<uint2*>(pbuf[i & 1] + F8_PB / 4 * bb + poff) =
                make_uint2(__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23));
          }
        }
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
    // DMA blocks ow + 8j of a chunk, j < ndma (bf16: 36 blocks, F8: 21)
    constexpr int NDMA_MAX = F8 ? 3 : 5;
    const int ndma = F8 ? (ow < F8_DMA - 2 * NOW ? 3 : 2) : (ow < DMA_BLOCKS - 4 * NOW ? 5 : 4);
    // bf16: DMA block ow + 8j is (ug, rg) = (ow/4 + 2j, ow%4): this lane copies row
    // 8(ow%4) + l/8, unit 8ug + ((l%8) ^ (l/8) ^ 2(ow%2)).
    // F8: blocks 0..15 are code blocks (ug, rg) = (blk/4, blk%4) of 8 rows x 128 codes,
    // 16..19 rope blocks rg = blk - 16, block 20 the chunk's 32 rows of scales. A wave's
    // code and rope blocks share the row group ow%4 and the unit rule above; its scale block
    // (wave 4) copies row l%32 (lanes 32..63 repeat rows 0..31 into the upper half).
    int ln = lane;
    const uint16_t* dsrc = kvreq;  // bf16: this lane's source for the chunk being issued
    const uint8_t* dsrc8 = kv8req; // F8: code / rope source of this lane's row
    const uint8_t* dscl8 = kv8req; // F8: scale source (wave 4)
    auto dma_src = [&](int c) {
      asm volatile("" : "+v"(ln));
      const int p = sidx[c * KC + 8 * (ow & 3) + (ln >> 3)];
      const int uu = (ln & 7) ^ (ln >> 3) ^ (2 * (ow & 1));
      if constexpr (!F8) {
        dsrc = kvreq + static_cast<int64_t>(p) * DQK + 64 * (ow >> 2) + 8 * uu;
      } else {
        dsrc8 = kv8req + static_cast<int64_t>(p) * RB8 + 16 * uu;
        if (ow == 4) dscl8 = kv8req + static_cast<int64_t>(sidx[c * KC + (ln & 31)]) * RB8 + RB8_SCALE;
      }
    };
    // DMA blocks j0 <= j < j1 of chunk c (source row from dma_src(c))
    auto dma_part = [&](int c, auto J0, auto J1) {
      const lds_u8* dst = (const lds_u8*)kvbuf[c % NB] + 1024 * ow;
      static_for<decltype(J0)::value, decltype(J1)::value>([&](auto J) {
        constexpr int j = decltype(J)::value;
        if constexpr (!F8) {
          if (j < 4 || ndma == 5)  // wave-uniform
            lds_dma16(dsrc + 128 * j, (const lds_void*)(dst + 8192 * j));
        } else if constexpr (j < 2) {  // code blocks ow, ow + 8: scale blocks ow/4 and ow/4 + 2
          lds_dma16(dsrc8 + 128 * (ow >> 2) + 256 * j, (const lds_void*)(dst + 8192 * j));
        } else {
          if (ow < 4)  // wave-uniform: rope block ow
            lds_dma16(dsrc8 + RB8_ROPE, (const lds_void*)(dst + 8192 * j));
          else if (ow == 4)
            lds_dma16(dscl8, (const lds_void*)(dst + 8192 * j));
        }
      });
    };
    auto dma_chunk = [&](int c) {
      dma_src(c);
      dma_part(c, std::integral_constant<int, 0>{}, std::integral_constant<int, NDMA_MAX>{});
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
    // F8 V^T reads (ds_read_b64_tr_b8): in each 16-lane group g, lane 2j + hf reads 8 codes of
    // key 8(g/2) + j (of key step ko), dims 64(ow%2) + 32dt + 16(g%2) + 8hf .. +8; the
    // transposed read hands lane s of the group the 8 keys at dim 16(g%2) + s of the tile,
    // which is the A layout of v_mfma_f32_32x32x16_bf16 (row l%32, keys 8(l/32) ..).
    // Code block (ow/2, 2ko + g/2), row j, unit 4(ow%2) + 2dt + g%2 at position
    // unit ^ j ^ 2((g/2)%2); dt flips position bit 1.
    const int v8pos = (4 * (ow & 1) + (g & 1)) ^ (c16 >> 1) ^ (2 * ((g >> 1) & 1));
    const int v8lane = 1024 * (4 * (ow >> 1) + (g >> 1)) + 128 * (c16 >> 1) + 16 * v8pos + 8 * (c16 & 1);
    const int v8dt = (v8pos & 2) ? -32 : 32;  // byte step from dt = 0 to dt = 1
    for (int c = 0; c < LD && c < nch; ++c) dma_chunk(c);
    // a chunk landed (this wave's DMAs of it): at most the DMAs of `after` (< LEAD) later
    // chunks may still be in flight, ndma each (wave-uniform: scalar branches to constant
    // counts)
    auto wait_chunk = [&](int after) {
      if constexpr (!F8) {
        if (after <= 0) DSA_WAIT_VMCNT(0);
        else if (ndma == 5) DSA_WAIT_VMCNT(5);
        else DSA_WAIT_VMCNT(4);
      } else {
        if (after <= 0) DSA_WAIT_VMCNT(0);
        else if (ndma == 3) DSA_WAIT_VMCNT(3);
        else DSA_WAIT_VMCNT(2);
      }
    };

#pragma unroll 1
    for (int i = 0; i <= nch; ++i) {
      // chunk i landed
      wait_chunk(nch - 1 - i < LD - 1 ? nch - 1 - i : LD - 1);
      __syncthreads();  // B0
      if (i + LD < nch) {
        dma_src(i + LD);
        dma_part(i + LD, std::integral_constant<int, 0>{}, std::integral_constant<int, DMA_A>{});
      }
      const int c = i - 1;  // chunk accumulated in this iteration
      const uint8_t* buf = kvbuf[(c + NB) % NB];
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
      // F8: every operand read of the chunk is issued at once, before the first MFMA (this
      // wave's scaled P^T copy and the V^T codes of both key steps; none waits for B1)
      i32x4 pop[F8 ? 2 : 1][2];
      i32x2 vop[F8 ? 2 : 1][2];
      if constexpr (F8) {
        if (c >= 0) {
#pragma unroll
          for (int ko = 0; ko < 2; ++ko)
#pragma unroll
            for (int ht = 0; ht < 2; ++ht)
              pop[ko][ht] = *reinterpret_cast<const i32x4*>(pbuf[c & 1] + F8_PB / 4 * (ow >> 1) +
                                                            1024 * ko + 2048 * ht + 16 * lane);
#pragma unroll
          for (int ko = 0; ko < 2; ++ko)
#pragma unroll
            for (int dt = 0; dt < 2; ++dt)
              vop[ko][dt] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                  (lds_i32x2*)((const lds_u8*)buf + v8lane + 2048 * ko + v8dt * dt));
        }
      }
      // V^T operand of key step ko: the codes as exact bf16 (the scales ride on P^T)
      auto f8_step = [&](int ko) {
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const i32x2 x = vop[ko][dt];
          const bf16x2 c0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.0f, false);
          const bf16x2 c1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.0f, true);
          const bf16x2 c2v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.0f, false);
          const bf16x2 c3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.0f, true);
          const bf16x8 aop = {c0[0], c0[1], c1[0], c1[1], c2v[0], c2v[1], c3[0], c3[1]};
          o[dt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, as_bf16x8(pop[ko][0]), o[dt][0], 0, 0, 0);
          o[dt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, as_bf16x8(pop[ko][1]), o[dt][1], 0, 0, 0);
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
        if constexpr (F8) f8_step(0);
        else o_step(0);
      }
      __syncthreads();  // B1
      if (i + LD < nch)
        dma_part(i + LD, std::integral_constant<int, DMA_A>{}, std::integral_constant<int, NDMA_MAX>{});
      if (c >= 0) {
        if constexpr (F8) f8_step(1);
        else o_step(1);
      }
    }
    __syncthreads();  // row sums and maxima from the S waves
    // this lane holds dims 64ow + 32dt + 8qd + 4h .. +4 of head 32ht + r in o[dt][ht]
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const int hd = HPB * hg + 32 * ht + r;
      if (hd >= H) continue;
      const float mh = sh_m[32 * ht + r];
      const float lh = sh_l[0][32 * ht + r] + sh_l[1][32 * ht + r];
      // the normalised output (bf16): the row's result, or with several slices this slice's
      // partial, which the combine kernel weighs by its (max, sum)
      const int64_t slot = (t * nsplit + split) * H + hd;
      const float inv = lh > 0.0f ? 1.0f / lh : 0.0f;
      uint16_t* orow = (nsplit == 1 ? out + (t * H + hd) * DV : ws_o + slot * DV) + 64 * ow + 4 * h;
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
      if (nsplit == 1) {
        if (lse && ow == 0 && h == 0)
          lse[t * H + hd] = lh > 0.0f ? (mh + __log2f(lh)) * 0.69314718055994531f : -INFINITY;
      } else if (ow == 0 && h == 0) {
        ws_ml[2 * slot] = mh;
        ws_ml[2 * slot + 1] = lh;
      }
    }
  }
}

// Merge the slices' normalised partials of one (row, head): 128 threads x 4 dims. Slice s
// (reference max m_s, row sum l_s) weighs l_s 2^(m_s - M), M the largest m_s.
__global__ __launch_bounds__(128) void mla_combine_kernel(const uint16_t* __restrict__ ws_o,
                                                          const float* __restrict__ ws_ml,
                                                          int H, int nsplit,
                                                          uint16_t* __restrict__ out,
                                                          float* __restrict__ lse) {
  const int64_t t = blockIdx.x;
  const int head = blockIdx.y;
  // every slice's (max, sum) and 4 outputs are loaded at once (at most MAX_SPLITS slices)
  float2 ml[MAX_SPLITS];
  uint2 v[MAX_SPLITS];
#pragma unroll
  for (int s = 0; s < MAX_SPLITS; ++s) {
    if (s < nsplit) {
      const int64_t slot = (t * nsplit + s) * H + head;
      ml[s] = reinterpret_cast<const float2*>(ws_ml)[slot];
      v[s] = reinterpret_cast<const uint2*>(ws_o + slot * DV)[threadIdx.x];
    }
  }
  float M = M_INIT;
#pragma unroll
  for (int s = 0; s < MAX_SPLITS; ++s)
    if (s < nsplit) M = fmaxf(M, ml[s].x);
  float L = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int s = 0; s < MAX_SPLITS; ++s) {
    if (s < nsplit) {
      const float f = ml[s].y * exp2f(ml[s].x - M);  // 0: no valid keys
      L += f;
      acc.x += bf16_bits_to_f32(static_cast<uint16_t>(v[s].x)) * f;
      acc.y += bf16_bits_to_f32(static_cast<uint16_t>(v[s].x >> 16)) * f;
      acc.z += bf16_bits_to_f32(static_cast<uint16_t>(v[s].y)) * f;
      acc.w += bf16_bits_to_f32(static_cast<uint16_t>(v[s].y >> 16)) * f;
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const uint32_t lo = f32_to_bf16_bits(acc.x * inv) | (static_cast<uint32_t>(f32_to_bf16_bits(acc.y * inv)) << 16);
  const uint32_t hi = f32_to_bf16_bits(acc.z * inv) | (static_cast<uint32_t>(f32_to_bf16_bits(acc.w * inv)) << 16);
  reinterpret_cast<uint2*>(out + (t * H + head) * DV)[threadIdx.x] = make_uint2(lo, hi);
  if (lse && threadIdx.x == 0)
    lse[t * H + head] = L > 0.0f ? (M + __log2f(L)) * 0.69314718055994531f : -INFINITY;
}

constexpr int64_t TARGET_BLOCKS = 160;  // grids below this many blocks take more slices
constexpr int64_t GRID_CUS = 256;       // compute units of the MI355X: one block each

// Slices per row: at least ceil(k / 2048) (LDS index staging). A grid below TARGET_BLOCKS
// blocks takes as many slices as still fit one block per CU (at most 16, each with >= 256
// entries).
int choose_splits(int64_t blocks_per_split, int k) {
  int s = static_cast<int>(ceil_div(k, MAX_KPS));
  if (blocks_per_split * s >= TARGET_BLOCKS) return s;
  int64_t fit = GRID_CUS / blocks_per_split;
  fit = fit < MAX_SPLITS ? fit : MAX_SPLITS;
  fit = fit < k / 256 ? fit : k / 256;
  return fit > s ? static_cast<int>(fit) : s;
}

int64_t keys_per_split(int k, int s) { return ceil_div(ceil_div(k, s), KC) * KC; }

}  // namespace
}  // namespace dsa

extern "C" size_t dsa_sparse_mla_workspace_size(int32_t T, int32_t H, int32_t k) {
  using namespace dsa;
  if (T <= 0 || H <= 0 || k <= 0) return 0;
  const int s = choose_splits(static_cast<int64_t>(T) * ceil_div(H, HPB), k);
  if (s == 1) return 0;
  return static_cast<size_t>(T) * s * H * (DV * sizeof(uint16_t) + 2 * sizeof(float));
}

namespace dsa {
namespace {

// Shared checks and launches of dsa_sparse_mla_decode (bf16 rows) and
// dsa_sparse_mla_decode_fp8 (FP8 rows); `name` prefixes the error messages.
template <bool F8>
dsa_status sparse_mla_launch(const char* name, const uint16_t* q, const void* kv,
                             const int32_t* topk, int32_t topk_rows, const int32_t* share_base,
                             const int32_t* num_accepted, const int32_t* q_row_offsets,
                             const int64_t* kv_row_offsets, int32_t B, int32_t T,
                             int32_t max_q_rows, int32_t H, int32_t k, float sm_scale,
                             uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                             void* stream) {
  if (H < 16 || H > 128 || H % 16)
    return fail(DSA_ERR_UNSUPPORTED, "%s: H must be a multiple of 16 in [16, 128] (got %d)", name, H);
  DSA_REQUIRE(k >= 1 && k <= MAX_SPLITS * MAX_KPS, "%s: k must be in [1, %d] (got %d)", name,
              MAX_SPLITS * MAX_KPS, k);
  DSA_REQUIRE(topk_rows >= 0, "%s: topk_rows must be >= 0", name);
  DSA_REQUIRE(B >= 0 && T >= 0 && max_q_rows >= 0, "%s: negative size", name);
  DSA_REQUIRE((share_base == nullptr) == (num_accepted == nullptr),
              "%s: share_base and num_accepted go together", name);
  DSA_REQUIRE(share_base || topk_rows >= T, "%s: topk needs T rows without a share map", name);
  DSA_REQUIRE(sm_scale > 0.0f && sm_scale < 1e30f, "%s: sm_scale must be positive", name);
  if (B == 0 || T == 0 || max_q_rows == 0) return ok();
  DSA_REQUIRE(q && kv && topk && q_row_offsets && kv_row_offsets && out, "%s: null pointer", name);
  DSA_REQUIRE((reinterpret_cast<uintptr_t>(q) & 15) == 0 && (reinterpret_cast<uintptr_t>(kv) & 15) == 0 &&
                  (reinterpret_cast<uintptr_t>(out) & 15) == 0,
              "%s: q, kv and out must be 16-byte aligned", name);
  DSA_REQUIRE(B <= 65535 && max_q_rows <= 65535, "%s: B and max_q_rows must be <= 65535", name);
  const int nhg = static_cast<int>(ceil_div(H, HPB));
  const int s = choose_splits(static_cast<int64_t>(T) * nhg, k);
  const size_t need = dsa_sparse_mla_workspace_size(T, H, k);
  if (ws_bytes < need || (need && !ws))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace needs %zu bytes (got %zu)", name, need,
                ws_bytes);
  DSA_REQUIRE(!need || (reinterpret_cast<uintptr_t>(ws) & 15) == 0,
              "%s: workspace must be 16-byte aligned", name);
  const int kps = static_cast<int>(keys_per_split(k, s));
  const int nsplit = static_cast<int>(ceil_div(k, kps));
  uint16_t* ws_o = static_cast<uint16_t*>(ws);
  float* ws_ml = need ? reinterpret_cast<float*>(ws_o + static_cast<size_t>(T) * nsplit * H * DV)
                      : nullptr;
  // one block per work item (slice, head group, row, request), XCD-ordered (see the kernel)
  const int64_t nwork = static_cast<int64_t>(nsplit) * nhg * max_q_rows * B;
  DSA_REQUIRE(nwork <= (int64_t{1} << 30), "%s: too many (row, head group, slice) blocks", name);
  const int per_xcd = static_cast<int>(ceil_div(nwork, 8));
  const float c2 = sm_scale * 1.4426950408889634f;  // natural -> base-2 logits
  hipStream_t st = as_stream(stream);
  hipLaunchKernelGGL(mla_decode_kernel<F8>, dim3(static_cast<unsigned>(8 * per_xcd)), dim3(NT), 0,
                     st, q, kv, topk, share_base, num_accepted, q_row_offsets, kv_row_offsets, H,
                     nhg, k, topk_rows, c2, nsplit, kps, max_q_rows, static_cast<int>(nwork),
                     per_xcd, out, lse, ws_o, ws_ml);
  dsa_status stt = check_launch(name);
  if (stt != DSA_OK || nsplit == 1) return stt;
  hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)T, (unsigned)H), dim3(128), 0, st, ws_o,
                     ws_ml, H, nsplit, out, lse);
  return check_launch(name);
}

}  // namespace
}  // namespace dsa

extern "C" dsa_status dsa_sparse_mla_decode(const uint16_t* q, const uint16_t* kv,
                                            const int32_t* topk, int32_t topk_rows,
                                            const int32_t* share_base,
                                            const int32_t* num_accepted,
                                            const int32_t* q_row_offsets,
                                            const int64_t* kv_row_offsets, int32_t B, int32_t T,
                                            int32_t max_q_rows, int32_t H, int32_t k,
                                            float sm_scale, uint16_t* out, float* lse, void* ws,
                                            size_t ws_bytes, void* stream) {
  return dsa::sparse_mla_launch<false>("dsa_sparse_mla_decode", q, kv, topk, topk_rows, share_base,
                                       num_accepted, q_row_offsets, kv_row_offsets, B, T,
                                       max_q_rows, H, k, sm_scale, out, lse, ws, ws_bytes, stream);
}

extern "C" dsa_status dsa_sparse_mla_decode_fp8(const uint16_t* q, const uint8_t* kv_fp8,
                                                const int32_t* topk, int32_t topk_rows,
                                                const int32_t* share_base,
                                                const int32_t* num_accepted,
                                                const int32_t* q_row_offsets,
                                                const int64_t* kv_row_offsets, int32_t B,
                                                int32_t T, int32_t max_q_rows, int32_t H,
                                                int32_t k, float sm_scale, uint16_t* out,
                                                float* lse, void* ws, size_t ws_bytes,
                                                void* stream) {
  return dsa::sparse_mla_launch<true>("dsa_sparse_mla_decode_fp8", q, kv_fp8, topk, topk_rows,
                                      share_base, num_accepted, q_row_offsets, kv_row_offsets, B,
                                      T, max_q_rows, H, k, sm_scale, out, lse, ws, ws_bytes,
                                      stream);
}
