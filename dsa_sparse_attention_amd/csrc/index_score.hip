// index_score.hip -- lightning-indexer scores on FP8 MFMA (gfx950).
//
// "MAX Pipeline 中的 DeepSeek-V3.2 架构实现解析", section "Indexer 的结构与计算流程":
// every verify row scores every cached index key with index_n_heads FP8 heads
// of index_head_dim; per-token fp32 scales come from the indexer scale cache
// ("配置体系", 双 KV 缓存). Score of row t against key s:
//     I[t,s] = k_scale[s] * sum_j (w[t,j] * q_scale[t,j]) * ReLU(q_hat[t,j] . k_hat[s])
//
// Work split: the keys of all requests, concatenated, are cut into equal ranges of whole
// 64-key tiles (up to 512 ranges, at least 256 keys each), so ragged context lengths and
// small batches still spread over all CUs. A block owns one range and up to 7 query rows
// of each request the range touches, and walks the range one request segment at a time:
// two compute waves per row (each takes 32 of every 64-key tile, so that 6 rows make
// 12 waves, 3 per SIMD: the MFMA load is spread evenly over the CU) plus one producer
// wave. Every key byte is fetched from HBM once per row group and shared by its rows.
//  1. The producer wave streams keys HBM -> LDS with LDS DMA (global_load_lds, no
//     registers) in 64-key tiles through a ring of NBUF slots (NBUF-2 tiles in flight),
//     together with the tile's 64 key scales. One 16-byte DMA instruction moves 1 KB of
//     consecutive keys (contiguous in HBM); in LDS a key keeps its row, with its
//     16-byte pieces XOR-permuted by (key >> 1) so that the MFMA operand reads (16
//     lanes = 16 keys at one piece) hit 16 distinct bank groups. The producer issues
//     nothing but these DMAs, so its s_waitcnt vmcnt counts are exact (the counter is
//     per wave: the compute waves' stores do not enter it).
//  2. Per 16-key sub-tile a compute wave issues one v_mfma_f32_16x16x128_f8f6f4 per
//     16-head tile (K = 128 = index_head_dim in one instruction), each into its own
//     accumulator: A = q codes [16 heads x 128], B = key codes [128 x 16 keys].
//     The result layout (row = 4*(lane/16)+i, col = lane%16) puts 4 heads of one key
//     in each lane: the ReLU * weight head sum is in-lane FMAs, then two lane-half
//     swaps (v_permlane32_swap / v_permlane16_swap, plain VALU) finish both sub-tiles
//     of a tile at once.
//  3. Each compute wave stores its row's 32 scores of the tile (key scale applied)
//     with one coalesced 128-byte store.
// One barrier per tile hands the tile after the current one to the compute waves (so a
// wave reads the next tile's first B operand before the barrier, and its MFMAs issue right
// after it) and the slot of the tile before the previous one back to the producer.
#include <atomic>

#include "common.hpp"
#include "fused.hpp"

namespace dsa {
namespace {

constexpr int KT = 64;                // keys per tile
constexpr int MIN_SHARE = 256;        // fewest keys per block (4 tiles)
constexpr int NBUF = 8;               // tile slots in LDS: NBUF - 2 tiles in flight
constexpr int MAX_ROWS = 7;           // rows per block: 2 compute waves each, plus a producer
constexpr int MAX_ROWS_H128 = 3;      // with 8 head tiles (registers: 256 per wave)

int max_rows_for(int ht) { return ht >= 8 ? MAX_ROWS_H128 : MAX_ROWS; }

// s_waitcnt vmcnt(n') for the largest constant n' <= n, n in [0, N] (wave-uniform n:
// scalar compares only).
template <int N>
__device__ __forceinline__ void wait_vm_at_most(int n) {
  if constexpr (N == 0) {
    DSA_WAIT_VMCNT(0);
  } else {
    if (n >= N) {
      DSA_WAIT_VMCNT(N);
    } else {
      wait_vm_at_most<N - 1>(n);
    }
  }
}

// Piece permutation of key k within its row in LDS (an involution on the piece index):
// 16 lanes reading keys 16j..16j+15 at one piece then cover all 256 bytes of the LDS
// bank window (keys alternate 128-byte halves for D = 128).
template <int NCH>
__device__ __forceinline__ int kswz(int k) { return (k >> 1) & (NCH - 1); }

template <int D>
struct Ring {
  static constexpr int NCH = D / 16;            // 16-byte pieces per key = K DMAs per tile
  static constexpr int KPB = 1024 / D;          // keys per 1 KB DMA block
  static constexpr int TILE_K = KT * D;         // key bytes per tile
  static constexpr int SLOT = TILE_K + KT * 4;  // + the tile's key scales
  static constexpr int DMAS = NCH + 1;          // producer DMAs per tile
  static_assert((NBUF - 2) * DMAS <= 63, "vmcnt holds at most 63");
};

// What a launch produces (kernel template argument):
//  SCORE   every visible score into scores[T, ld];
//  SAMPLE  scores of S evenly spaced keys per request, sample j at position
//          floor(j n0 / S) (n0 = the request's first row's visible count), into
//          samples[T, S] (the key segments are sample indices);
//  COMPACT only the scores >= tau[t] of each row, as (score bits, position) pairs in the
//          row's slice of cand for the block's key segment (no score row is written), with
//          the count and the largest key scale of every (row, range, wave half).
enum { SCORE = 0, SAMPLE = 1, COMPACT = 2 };

struct ModeArgs {
  int S;               // SAMPLE: samples per request (scores: the sample buffer, ld = S)
  const float* tau;    // COMPACT: [T] candidate threshold per row
  uint2* cand;         // COMPACT: [T, ldc] (float bits, request-local position)
  int64_t ldc;
  int32_t* cnt;        // COMPACT: [T, gx, 2] candidates of each (row, range, half)
  float* msc;          // COMPACT: [T, gx, 2] largest visible key scale of each
  int gx;              // COMPACT: number of key ranges (the grid's x)
};

// First row's visible count of a request (at least 1 when it has keys): sample positions
// are spread over the keys every row of the request sees.
__device__ __forceinline__ int64_t sample_span(const RowInfo& ri) {
  const int64_t n0 = ri.L - ri.R + 1;
  return n0 < 1 ? 1 : (n0 > ri.L ? ri.L : n0);
}

// Keys key0 .. key_end-1 (0 < key_end - key0 < 2^31) of request `ri` against its rows
// row0 .. row0+NR-1, by the whole block: the producer wave (producer_segment) streams the
// keys through the ring, the compute waves (compute_segment) score and store them. Each
// side passes one barrier per tile, so the block's barriers pair up one to one.
template <int D, int HT, int NR, int MODE>
__device__ __forceinline__ void producer_segment(
    uint8_t (&ring)[NBUF][Ring<D>::SLOT], const uint8_t* __restrict__ q_fp8,
    const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ k_fp8, const float* __restrict__ k_scale, const RowInfo& ri,
    int64_t key0, int64_t key_end, int row0, int H, float* __restrict__ scores, int64_t ld,
    int lane, int wave, const ModeArgs& ma) {
  constexpr int NCH = Ring<D>::NCH;
  constexpr int KPB = Ring<D>::KPB;
  constexpr int TILE_K = Ring<D>::TILE_K;
  constexpr int DMAS = Ring<D>::DMAS;
  const int nkeys = static_cast<int>(key_end - key0);
  const int ntiles = (nkeys + KT - 1) / KT;
  // ---- producer wave: tile `it` -> slot it % NBUF. DMA m < NCH moves keys KPB*m ..
  // KPB*m + KPB-1 of the tile: lane l writes physical piece l % NCH of key KPB*m + l/NCH,
  // i.e. loads logical piece (l % NCH) ^ kswz(key); keys past the chunk load its last
  // key again (their scores are never stored). DMA NCH moves the 64 key scales.
  // In a full tile, key KPB*m + l/NCH has kswz = (KPB*m/2 + l/(2*NCH)) % NCH, which only
  // depends on the parity of m (KPB*m/2 is a multiple of NCH for even m and NCH/2 more
  // for odd m): two per-lane byte offsets serve every DMA of every full tile.
  const uint8_t* kreq = k_fp8 + (ri.kv_base + key0) * D;
  const float* sreq = k_scale + ri.kv_base + key0;
  // SAMPLE: tile key i is sample key0 + i, at request position floor((key0 + i) n0 / S)
  const int64_t n0 = MODE == SAMPLE ? sample_span(ri) : 0;
  auto pos_of = [&](int i) -> int64_t {
    if constexpr (MODE == SAMPLE)
      return (key0 + i) * n0 / ma.S - key0;  // relative to kreq / sreq
    else
      return i;
  };
  const int ful = MODE == SAMPLE ? 0 : nkeys / KT;  // full (contiguous) tiles
  auto issue_tile = [&](int it) {
    int ln = lane;
    asm volatile("" : "+v"(ln));  // recomputed per tile, not held across the loop
    const lds_u8* slot = (const lds_u8*)ring[it % NBUF];
    if (it < ful) {
      const uint8_t* base = kreq + static_cast<int64_t>(it) * TILE_K + (ln / NCH) * D;
      const int off0 = 16 * ((ln % NCH) ^ kswz<NCH>(ln / NCH));
      const int off1 = 16 * ((ln % NCH) ^ kswz<NCH>(KPB + ln / NCH));
#pragma unroll
      for (int m = 0; m < NCH; ++m)
        lds_dma16(base + 1024 * m + ((m & 1) ? off1 : off0), (const lds_void*)(slot + 1024 * m));
      lds_dma4(sreq + it * KT + ln, (const lds_void*)(slot + TILE_K));
    } else {
#pragma unroll
      for (int m = 0; m < NCH; ++m) {
        const int kt = KPB * m + ln / NCH;  // key within the tile
        const int key = it * KT + kt < nkeys ? it * KT + kt : nkeys - 1;
        lds_dma16(kreq + pos_of(key) * D + 16 * ((ln % NCH) ^ kswz<NCH>(kt)),
                  (const lds_void*)(slot + 1024 * m));
      }
      const int key = it * KT + ln < nkeys ? it * KT + ln : nkeys - 1;
      lds_dma4(sreq + pos_of(key), (const lds_void*)(slot + TILE_K));
    }
  };
  // Barrier it hands over tile it+1 (tiles 0 and 1 at barrier 0): the compute waves read
  // a tile's sub-tile 0 between the barriers before it and its own, and the rest between its
  // own barrier and the next. Tile it+NBUF-2 goes into the slot of tile it-2, which every
  // compute wave finished reading before barrier it-1: the producer issues it before
  // barrier it, overlapped with the compute, and reaches the barrier as soon as tile it+1
  // is in.
  // Retire every load the compiler issued so far: its own wait bookkeeping does not see
  // the DMAs, and a wait it placed for one of its loads inside the loop would count them
  // wrongly and drain the whole DMA pipeline.
  DSA_WAIT_VMCNT(0);
#pragma unroll 1
  for (int j = 0; j < NBUF - 2 && j < ntiles; ++j) issue_tile(j);
#pragma unroll 1
  for (int it = 0; it < ntiles; ++it) {
    if (it + NBUF - 2 < ntiles) issue_tile(it + NBUF - 2);
    // tile it+1 has landed when at most the DMAs of the tiles after it are in flight
    const int last = it + NBUF - 2 < ntiles ? it + NBUF - 2 : ntiles - 1;  // last issued
    const int need = it + 1 < ntiles ? it + 1 : ntiles - 1;
    wait_vm_at_most<(NBUF - 3) * DMAS>((last - need) * DMAS);
    __syncthreads();  // hand tile it+1 over; every compute wave is done with tile it-1
  }
}

template <int D, int HT, int NR, int MODE>
__device__ __forceinline__ void compute_segment(
    uint8_t (&ring)[NBUF][Ring<D>::SLOT], const uint8_t* __restrict__ q_fp8,
    const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ k_fp8, const float* __restrict__ k_scale, const RowInfo& ri,
    int64_t key0, int64_t key_end, int row0, int H, float* __restrict__ scores, int64_t ld,
    int lane, int wave, const ModeArgs& ma) {
  constexpr int NCH = Ring<D>::NCH;
  constexpr int TILE_K = Ring<D>::TILE_K;
  const int nkeys = static_cast<int>(key_end - key0);
  const int ntiles = (nkeys + KT - 1) / KT;
  // lane-derived addresses are recomputed per segment rather than held (spilled) across them
  asm volatile("" : "+v"(lane));

  // ---- compute wave: row row0 + wave/2, keys 32*(wave%2) .. +32 of every tile
  const int g = lane / 16, c16 = lane % 16;
  const int kh = wave & 1;
  const int r = row0 + (wave >> 1);
  const bool row_live = r < ri.R;  // wave-uniform
  const int64_t nvis = row_live ? visible_count(ri, r) : 0;
  const int64_t t = ri.t0 + (row_live ? r : 0);  // a valid row for the (discarded) loads
  // scores stored for keys key0 .. key0 + nstore - 1 of this row (visible and in chunk;
  // every sample is visible to every row of its request)
  const int nstore =
      MODE == SAMPLE ? (row_live ? nkeys : 0)
                     : static_cast<int>(nvis - key0 < nkeys ? (nvis - key0 > 0 ? nvis - key0 : 0) : nkeys);

  // A operands (q codes) and per-output-row weights u = w * q_scale; all loads are issued
  // before any is used. Heads past H read head H-1 and are zeroed.
  i32x8 qa[HT];
  float u[HT][4];
  {
    i32x4 qlo[HT], qhi[HT];
    float wv[HT][4], qs[HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int head = ht * 16 + c16;
      const int gq = 32 * g < D ? g : 0;
      const i32x4* p = reinterpret_cast<const i32x4*>(q_fp8 + (t * H + (head < H ? head : H - 1)) * D + 32 * gq);
      qlo[ht] = p[0];
      qhi[ht] = p[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h2 = ht * 16 + 4 * g + i;
        const int64_t o = t * H + (h2 < H ? h2 : H - 1);
        wv[ht][i] = w[o];
        qs[ht][i] = q_scale[o];
      }
    }
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const bool qok = row_live && ht * 16 + c16 < H && 32 * g < D;
      const i32x8 v = {qlo[ht][0], qlo[ht][1], qlo[ht][2], qlo[ht][3],
                       qhi[ht][0], qhi[ht][1], qhi[ht][2], qhi[ht][3]};
      const i32x8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
      qa[ht] = qok ? v : zero8;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        u[ht][i] = (row_live && ht * 16 + 4 * g + i < H) ? wv[ht][i] * qs[ht][i] : 0.0f;
    }
  }
  float* srow = scores + t * ld + key0;
  // Lane groups 1 and 2 store the wave's 32 keys of a tile: key 32kh + 16(g-1) + c16 (the
  // other groups read a valid, unused scale).
  const int kt = 32 * kh + 16 * ((g - 1) & 1) + c16;
  // Byte offsets in a slot of this lane's two 16-byte B pieces of sub-tile 0: dims
  // 32g..32g+31 = logical pieces 2g and 2g+1 of key 32kh + c16. Sub-tile 1 is 16 keys =
  // 16 D bytes further on with the same permutation (kswz only sees key/2 mod NCH, and
  // 16/2 is a multiple of NCH).
  const int key_l = 32 * kh + c16;
  const int off_lo = key_l * D + 16 * ((2 * g) ^ kswz<NCH>(key_l));
  const int off_hi = key_l * D + 16 * ((2 * g + 1) ^ kswz<NCH>(key_l));

  // Software pipeline over 16-key sub-tiles (each wave owns sub-tiles 0 and 1 of its
  // 32-key half of every tile): the MFMAs of the next sub-tile are issued before the
  // current one is reduced. A tile's sub-tile 0 is read between the barrier that hands it
  // over and the tile's own barrier, the rest (sub-tile 1, key scales) before the barrier
  // after that, which is before the producer refills its slot.
  const bool live = row_live;
  auto live_tile = [&](int it) { return live && it * KT + 32 * kh < nstore; };  // wave-uniform
  // this lane's piece addresses in the current tile's slot (carried from sub-tile 0 of a
  // tile to its sub-tile 1)
  const uint8_t* a_lo = ring[0] + off_lo;
  const uint8_t* a_hi = ring[0] + off_hi;
  // B operand of sub-tile sb of the tile at a_lo / a_hi (for D = 128 every lane group holds
  // 32 of the key's dims: the load is unconditional, with no zero fill on the VALU)
  auto load_b = [&](int sb) {
    i32x8 bfrag = {0, 0, 0, 0, 0, 0, 0, 0};
    if (D >= 128 || 32 * g < D) {
      const i32x4 lo = *reinterpret_cast<const i32x4*>(a_lo + sb * 16 * D);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(a_hi + sb * 16 * D);
      bfrag = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    return bfrag;
  };
  auto mfma_sub = [&](const i32x8& bfrag, f32x4 (&acc)[HT]) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      acc[ht] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[ht], bfrag, zero, 0, 0, 0, 0,
                                                                 0, 0);
    }
  };
  // in-lane part of the ReLU * weight head sum of key c16 of a sub-tile (the lane's heads)
  auto partial = [&](const f32x4 (&acc)[HT]) {
    float part = 0.0f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int i = 0; i < 4; ++i)  // ReLU as med3(x, 0, FLT_MAX): max(x, 0) in one op
        part = fmaf(u[ht][i], __builtin_amdgcn_fmed3f(acc[ht][i], 0.0f, 3.402823466e38f), part);
    return part;
  };
  // Both sub-tiles' sums over the four lane groups with two lane-half swaps: the 32-lane
  // swap of (p0, p1) leaves p0's group pairs (0+2, 1+3) in lanes 0..31 and p1's in lanes
  // 32..63; the 16-lane swap then adds neighbouring groups, so groups 0 and 1 hold
  // sub-tile 0's sum and groups 2 and 3 sub-tile 1's.
  auto combine = [&](float p0, float p1) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false,
                                                    false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false,
                                                    false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
  };

  // COMPACT: the row's candidates of this segment go to cand[t, key0 .. key_end): the
  // first wave half fills it upwards from key0, the second downwards from key_end - 1 (each
  // keeps at most one entry per key it scores, so the two never meet); its running count,
  // and the largest key scale it saw
  uint2* creg = nullptr;
  int cdir = 1;
  float tau = 0.0f;
  int ccount = 0;
  float cmax = 0.0f;
  if constexpr (MODE == COMPACT) {
    creg = ma.cand + t * ma.ldc + (kh ? key_end - 1 : key0);
    cdir = kh ? -1 : 1;
    tau = ma.tau[t];
  }

  f32x4 acc0[HT], acc1[HT];  // sub-tile 0 / sub-tile 1 of the current tile
  if (ntiles > 0) {
    __syncthreads();  // tiles 0 and 1 are in LDS (the producer waited for them)
    if (live_tile(0)) mfma_sub(load_b(0), acc0);
  }
  // One tile: `slot` = it % NBUF. The loop below unrolls NBUF steps so that every slot
  // address is a constant offset from the ring's base.
  auto step = [&](const int it, const int slot) {
    const int nslot = (slot + 1) % NBUF;
    const bool lv = live_tile(it);
    float sc = 0.0f, p0 = 0.0f;
    const i32x8 b1 = load_b(1);
    if (lv) sc = reinterpret_cast<const float*>(ring[slot] + TILE_K)[kt];
    // sub-tile 0 of tile it+1, landed at the last barrier, read before the next one
    i32x8 bn = {0, 0, 0, 0, 0, 0, 0, 0};
    if (it + 1 < ntiles) {
      a_lo = ring[nslot] + off_lo;
      a_hi = ring[nslot] + off_hi;
      bn = load_b(0);
    }
    if (lv) {
      mfma_sub(b1, acc1);
      p0 = partial(acc0);
    }
    if (it + 1 < ntiles) {
      __syncthreads();  // tile it+2 is in LDS; every wave is done reading tile it
      if (live_tile(it + 1)) mfma_sub(bn, acc0);
    }
    if (live_tile(it)) {  // recomputed (scalar) rather than carried across the barrier
      const float sum = combine(p0, partial(acc1));
      const bool mine = (g == 1 || g == 2) && it * KT + kt < nstore;
      if constexpr (MODE == COMPACT) {
        const float v = sum * sc;
        const bool keep = mine && v >= tau;
        const uint64_t bk = __builtin_amdgcn_ballot_w64(keep);
        if (keep) {
          const int at = ccount + static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                                      static_cast<uint32_t>(bk >> 32),
                                      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bk), 0u)));
          creg[cdir * at] = make_uint2(__float_as_uint(v), static_cast<uint32_t>(key0 + it * KT + kt));
        }
        ccount += static_cast<int>(__popcll(bk));
        if (mine) cmax = fmaxf(cmax, sc);
      } else {
        // the tile's row base is wave-uniform (scalar arithmetic); the lane adds its key kt
        float* tile_row = srow + static_cast<int64_t>(__builtin_amdgcn_readfirstlane(it)) * KT;
        if (mine) tile_row[kt] = sum * sc;
      }
    }
  };
#pragma unroll 1
  for (int base = 0; base < ntiles; base += NBUF) {
#pragma unroll
    for (int k = 0; k < NBUF; ++k)
      if (base + k < ntiles) step(base + k, k);
  }
  if constexpr (MODE == COMPACT) {
    if (live) {
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) cmax = fmaxf(cmax, __shfl_xor(cmax, o));
      if (lane == 0) {
        const int64_t m = (t * ma.gx + blockIdx.x) * 2 + kh;
        ma.cnt[m] = ccount;
        ma.msc[m] = cmax;
      }
    }
  }
}

// The request holding global key position g (kv_off[0] <= g < kv_off[B]): the largest b
// with kv_off[b] <= g, which skips requests without keys. A 64-way search by the whole
// wave, one round of loads per factor of 64 in B; the result is wave-uniform.
__device__ __forceinline__ int request_of(const int64_t* __restrict__ kv_off, int B, int64_t g,
                                          int lane) {
  int lo = 0, hi = B;  // kv_off[lo] <= g; the answer lies in [lo, hi)
  while (hi - lo > 1) {
    const int step = (hi - lo + 63) / 64;
    const int idx = lo + lane * step;
    const bool ok = idx < hi && kv_off[idx < hi ? idx : lo] <= g;  // true for a lane prefix
    const uint64_t m = __builtin_amdgcn_ballot_w64(ok);             // lane 0 always set
    lo += (63 - __builtin_clzll(m)) * step;
    hi = lo + step < hi ? lo + step : hi;
  }
  return lo;
}

// Work split: the requests' keys, concatenated in request order (global positions
// kv_off[0] .. kv_off[B]), are cut into gridDim.x equal ranges, rounded up to whole
// 64-key tiles; block (x, 0, z) scores range x against rows z NR .. z NR + NR - 1 of every
// request the range touches, one segment per request. Ragged lengths thus spread evenly
// over the blocks, and a small batch still occupies many CUs.
template <int D, int HT, int NR, int MODE>
__global__ __launch_bounds__((2 * NR + 1) * 64) void index_score_kernel(
    const uint8_t* __restrict__ q_fp8, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k_fp8,
    const float* __restrict__ k_scale, const int32_t* __restrict__ q_off,
    const int64_t* __restrict__ kv_off, int B, int H, float* __restrict__ scores, int64_t ld,
    ModeArgs ma) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NBUF][Ring<D>::SLOT];
  const int lane = threadIdx.x % 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);  // wave-uniform (SGPR)
  const int row0 = blockIdx.z * NR;
  // key space cut into ranges: the requests' keys laid end to end, or (SAMPLE) S sample
  // slots per request
  const int64_t base = MODE == SAMPLE ? 0 : kv_off[0];
  const int64_t end = MODE == SAMPLE ? static_cast<int64_t>(B) * ma.S : kv_off[B];
  int64_t share = (end - base + gridDim.x - 1) / gridDim.x;
  share = (share + KT - 1) / KT * KT;
  const int64_t g0 = base + static_cast<int64_t>(blockIdx.x) * share;
  const int64_t g1 = g0 + share < end ? g0 + share : end;
  if (g0 >= g1) return;  // block-uniform
  // Both roles walk the same segments and pass the same barriers.
  auto for_segments = [&](auto&& body) {
    bool first = true;
    const int b_first = MODE == SAMPLE ? static_cast<int>(g0 / ma.S) : request_of(kv_off, B, g0, lane);
    for (int b = b_first; b < B; ++b) {
      const RowInfo ri = load_row_info(q_off, kv_off, b);
      const int64_t sbase = MODE == SAMPLE ? static_cast<int64_t>(b) * ma.S : ri.kv_base;
      const int64_t slen = MODE == SAMPLE ? (ri.L > 0 ? ma.S : 0) : ri.L;
      if (sbase >= g1) break;  // block-uniform, as every test below
      if (row0 >= ri.R) continue;
      const int64_t key0 = (g0 > sbase ? g0 : sbase) - sbase;
      int64_t key_end = (g1 < sbase + slen ? g1 : sbase + slen) - sbase;
      if (key_end > ld) key_end = ld;  // device lengths beyond the score stride are clipped
      if (key_end <= key0) continue;
      // every wave is done with the previous segment's tiles before the producer refills
      // their slots
      if (!first) __syncthreads();
      first = false;
      body(ri, key0, key_end);
    }
  };
  if (wave == 2 * NR) {
    for_segments([&](const RowInfo& ri, int64_t key0, int64_t key_end) {
      producer_segment<D, HT, NR, MODE>(ring, q_fp8, q_scale, w, k_fp8, k_scale, ri, key0,
                                        key_end, row0, H, scores, ld, lane, wave, ma);
    });
  } else {
    for_segments([&](const RowInfo& ri, int64_t key0, int64_t key_end) {
      compute_segment<D, HT, NR, MODE>(ring, q_fp8, q_scale, w, k_fp8, k_scale, ri, key0,
                                       key_end, row0, H, scores, ld, lane, wave, ma);
    });
  }
}

// Compute units of the current device (cached per device).
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  const int slot = dev < 64 ? dev : 63;
  int n = cache[slot].load(std::memory_order_relaxed);
  if (n <= 0 || dev >= 64) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 1;
    if (dev < 64) cache[slot].store(n, std::memory_order_relaxed);
  }
  return n;
}

// One launch of the scoring kernel: its arguments, and the grid before the cap below.
struct ScoreLaunch {
  dim3 grid;
  hipStream_t st;
  const uint8_t* q;
  const float* qs;
  const float* w;
  const uint8_t* k;
  const float* ks;
  const int32_t* qo;
  const int64_t* ko;
  int B, H;
  float* sc;
  int64_t ld;
  ModeArgs ma;
};

// grid.x on entry: the key ranges the sizes call for; it is capped at one wave of resident
// blocks (blocks per CU x CUs, shared by the grid.z row groups), so that every range starts
// at once and equal ranges finish together. Returns the capped grid.x; launches only when
// `launch` (COMPACT needs the count before its launch, to size and index its tables).
template <int D, int HT, int NRV, int MODE>
int64_t run_one(ScoreLaunch a, bool launch) {
  if constexpr (HT >= 8 && NRV > MAX_ROWS_H128) {
    return 0;  // never chosen: the host caps rows per block at MAX_ROWS_H128 for 8 head tiles
  } else {
    constexpr int threads = (2 * NRV + 1) * 64;
    static std::atomic<int> occ{0};  // resident blocks per CU of this instantiation
    int o = occ.load(std::memory_order_relaxed);
    if (o <= 0) {
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, index_score_kernel<D, HT, NRV, MODE>,
                                                       threads, 0) != hipSuccess || o < 1)
        o = 1;
      occ.store(o, std::memory_order_relaxed);
    }
    const int64_t cap = static_cast<int64_t>(o) * cu_count() / a.grid.z;
    if (static_cast<int64_t>(a.grid.x) > cap) a.grid.x = static_cast<unsigned>(cap > 1 ? cap : 1);
    if (launch) {
      if constexpr (MODE == COMPACT) a.ma.gx = static_cast<int>(a.grid.x);
      hipLaunchKernelGGL((index_score_kernel<D, HT, NRV, MODE>), a.grid, dim3(threads), 0, a.st, a.q,
                         a.qs, a.w, a.k, a.ks, a.qo, a.ko, a.B, a.H, a.sc, a.ld, a.ma);
    }
    return a.grid.x;
  }
}

template <int D, int HT, int MODE>
int64_t run_nr(int nr, const ScoreLaunch& a, bool launch) {
  switch (nr) {
    case 1: return run_one<D, HT, 1, MODE>(a, launch);
    case 2: return run_one<D, HT, 2, MODE>(a, launch);
    case 3: return run_one<D, HT, 3, MODE>(a, launch);
    case 4: return run_one<D, HT, 4, MODE>(a, launch);
    case 5: return run_one<D, HT, 5, MODE>(a, launch);
    case 6: return run_one<D, HT, 6, MODE>(a, launch);
    default: return run_one<D, HT, 7, MODE>(a, launch);
  }
}

template <int MODE>
int64_t run_scoring(int D, int ht, int nr, const ScoreLaunch& a, bool launch) {
  if (D == 128) {
    switch (ht) {
      case 1: return run_nr<128, 1, MODE>(nr, a, launch);
      case 2: return run_nr<128, 2, MODE>(nr, a, launch);
      case 4: return run_nr<128, 4, MODE>(nr, a, launch);
      default: return run_nr<128, 8, MODE>(nr, a, launch);
    }
  }
  switch (ht) {
    case 1: return run_nr<64, 1, MODE>(nr, a, launch);
    case 2: return run_nr<64, 2, MODE>(nr, a, launch);
    case 4: return run_nr<64, 4, MODE>(nr, a, launch);
    default: return run_nr<64, 8, MODE>(nr, a, launch);
  }
}

int pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Grid of a scoring launch over `keys_per_request` key slots per request (before the cap):
// row groups of at most max_rows_for(ht) rows, balanced (6 rows -> one group of 6, 8 -> 4 +
// 4), and one key range per MIN_SHARE keys of the largest batch the sizes allow.
void plan_scoring(int B, int max_q_rows, int H, int64_t keys_per_request, dim3* grid, int* nr) {
  const int ht = pow2_at_least((H + 15) / 16);
  const int64_t gz = ceil_div(max_q_rows, max_rows_for(ht));
  *nr = static_cast<int>(ceil_div(max_q_rows, gz));
  int64_t gx = ceil_div(static_cast<int64_t>(B) * keys_per_request, MIN_SHARE);
  gx = gx < 1 ? 1 : (gx > 0x7FFFFFFF ? 0x7FFFFFFF : gx);
  *grid = dim3((unsigned)gx, 1u, (unsigned)(gz > 65535 ? 65536 : gz));
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
  DSA_REQUIRE(score_ld < (int64_t(1) << 31), "dsa_index_score: score_ld must be < 2^31");
  ScoreLaunch a{};
  int nr = 0;
  plan_scoring(B, max_q_rows, H_I, max_kv_len, &a.grid, &nr);
  DSA_REQUIRE(a.grid.z <= 65535, "dsa_index_score: grid too large");
  a.st = as_stream(stream);
  a.q = q_fp8;
  a.qs = q_scale;
  a.w = w;
  a.k = k_fp8;
  a.ks = k_scale;
  a.qo = q_row_offsets;
  a.ko = kv_row_offsets;
  a.B = B;
  a.H = H_I;
  a.sc = scores;
  a.ld = score_ld;
  run_scoring<SCORE>(D_I, pow2_at_least((H_I + 15) / 16), nr, a, true);
  return check_launch("dsa_index_score");
}

namespace dsa {
namespace {

constexpr int64_t kFusedMaxRanges = 4096;  // key ranges the compaction tables are sized for

struct FusedLayout {
  int S;           // samples per request
  int64_t ldc;     // candidate row stride (entries)
  int64_t gxb;     // key ranges the count tables hold
  size_t samples, tau, cand, cnt, msc, total;  // byte offsets, then the size
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

FusedLayout fused_layout(int32_t B, int32_t T, int32_t max_q_rows, int32_t H, int64_t max_kv_len) {
  FusedLayout f{};
  f.S = fused_sample_count(max_kv_len);
  f.ldc = (max_kv_len + 3) / 4 * 4;
  if (f.ldc < 4) f.ldc = 4;
  dim3 grid;
  int nr = 0;
  plan_scoring(B, max_q_rows, H, max_kv_len, &grid, &nr);
  f.gxb = grid.x < kFusedMaxRanges ? grid.x : kFusedMaxRanges;
  size_t off = 0;
  f.samples = off;
  off = align256(off + static_cast<size_t>(T) * f.S * 4);
  f.tau = off;
  off = align256(off + static_cast<size_t>(T) * 4);
  f.cand = off;
  off = align256(off + static_cast<size_t>(T) * f.ldc * 8);
  f.cnt = off;
  off = align256(off + static_cast<size_t>(T) * f.gxb * 2 * 4);
  f.msc = off;
  off = align256(off + static_cast<size_t>(T) * f.gxb * 2 * 4);
  f.total = off;
  return f;
}

}  // namespace
}  // namespace dsa

extern "C" size_t dsa_index_topk_workspace_size(int32_t B, int32_t T, int32_t max_q_rows,
                                                int32_t H_I, int64_t max_kv_len) {
  using namespace dsa;
  if (B <= 0 || T <= 0 || max_q_rows <= 0 || H_I < 1 || max_kv_len < 0) return 0;
  return fused_layout(B, T, max_q_rows, H_I, max_kv_len).total;
}

extern "C" dsa_status dsa_index_topk(const uint8_t* q_fp8, const float* q_scale, const float* w,
                                     const uint8_t* k_fp8, const float* k_scale,
                                     const int32_t* q_row_offsets, const int64_t* kv_row_offsets,
                                     int32_t B, int32_t T, int32_t max_q_rows, int32_t H_I,
                                     int32_t D_I, int64_t max_kv_len, int32_t k, double err_scale,
                                     int32_t* status, int32_t* path, int32_t* topk, void* ws,
                                     size_t ws_bytes, void* stream) {
  using namespace dsa;
  if (D_I != 64 && D_I != 128)
    return fail(DSA_ERR_UNSUPPORTED, "dsa_index_topk: D_I must be 64 or 128 (got %d)", D_I);
  if (H_I < 1 || H_I > 128)
    return fail(DSA_ERR_UNSUPPORTED, "dsa_index_topk: H_I must be in [1, 128] (got %d)", H_I);
  DSA_REQUIRE(k >= 1 && k <= 4096, "dsa_index_topk: k must be in [1, 4096] (got %d)", k);
  DSA_REQUIRE(B >= 0 && T >= 0 && max_q_rows >= 0 && max_kv_len >= 0, "dsa_index_topk: negative size");
  DSA_REQUIRE(max_kv_len < (int64_t(1) << 31), "dsa_index_topk: max_kv_len must be < 2^31");
  DSA_REQUIRE(err_scale >= 0.0 && err_scale < 1e30, "dsa_index_topk: err_scale must be in [0, 1e30)");
  if (B == 0 || T == 0 || max_q_rows == 0) return ok();
  DSA_REQUIRE(q_fp8 && q_scale && w && k_fp8 && k_scale && q_row_offsets && kv_row_offsets && topk,
              "dsa_index_topk: null pointer");
  DSA_REQUIRE((reinterpret_cast<uintptr_t>(q_fp8) & 15) == 0 &&
                  (reinterpret_cast<uintptr_t>(k_fp8) & 15) == 0,
              "dsa_index_topk: q_fp8 and k_fp8 must be 16-byte aligned");
  DSA_REQUIRE(B <= 65535 && max_q_rows <= 65535, "dsa_index_topk: B and max_q_rows must be <= 65535");
  const FusedLayout f = fused_layout(B, T, max_q_rows, H_I, max_kv_len);
  if (!ws || ws_bytes < f.total)
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "dsa_index_topk: workspace needs %zu bytes (got %zu)",
                f.total, ws_bytes);
  DSA_REQUIRE((reinterpret_cast<uintptr_t>(ws) & 255) == 0, "dsa_index_topk: ws must be 256-byte aligned");
  uint8_t* wb = static_cast<uint8_t*>(ws);
  float* samples = reinterpret_cast<float*>(wb + f.samples);
  float* tau = reinterpret_cast<float*>(wb + f.tau);
  uint2* cand = reinterpret_cast<uint2*>(wb + f.cand);
  int32_t* cnt = reinterpret_cast<int32_t*>(wb + f.cnt);
  float* msc = reinterpret_cast<float*>(wb + f.msc);
  const int ht = pow2_at_least((H_I + 15) / 16);
  hipStream_t st = as_stream(stream);

  // 1. sample scores: S slots per request, scored like every other key
  ScoreLaunch a{};
  int nr = 0;
  plan_scoring(B, max_q_rows, H_I, f.S, &a.grid, &nr);
  DSA_REQUIRE(a.grid.z <= 65535, "dsa_index_topk: grid too large");
  a.st = st;
  a.q = q_fp8;
  a.qs = q_scale;
  a.w = w;
  a.k = k_fp8;
  a.ks = k_scale;
  a.qo = q_row_offsets;
  a.ko = kv_row_offsets;
  a.B = B;
  a.H = H_I;
  a.sc = samples;
  a.ld = f.S;
  a.ma.S = f.S;
  run_scoring<SAMPLE>(D_I, ht, nr, a, true);
  dsa_status s = check_launch("dsa_index_topk(sample)");
  if (s != DSA_OK) return s;
  // 2. each row's candidate threshold
  launch_sample_tau(samples, f.S, q_row_offsets, kv_row_offsets, B, max_q_rows, k, tau, st);
  s = check_launch("dsa_index_topk(threshold)");
  if (s != DSA_OK) return s;
  // 3. scores >= tau of every row, kept per key range
  plan_scoring(B, max_q_rows, H_I, max_kv_len, &a.grid, &nr);
  a.sc = nullptr;
  a.ld = f.ldc;
  a.ma = ModeArgs{};
  a.ma.tau = tau;
  a.ma.cand = cand;
  a.ma.ldc = f.ldc;
  a.ma.cnt = cnt;
  a.ma.msc = msc;
  const int64_t gx = run_scoring<COMPACT>(D_I, ht, nr, a, false);
  if (gx > f.gxb)
    return fail(DSA_ERR_UNSUPPORTED, "dsa_index_topk: %lld key ranges exceed the tables' %lld",
                (long long)gx, (long long)f.gxb);
  run_scoring<COMPACT>(D_I, ht, nr, a, true);
  s = check_launch("dsa_index_topk(score)");
  if (s != DSA_OK) return s;
  // 4. exact selection from the candidates (or from a rescored row)
  FusedSelectLaunch fsl{};
  fsl.cand = cand;
  fsl.ldc = f.ldc;
  fsl.cnt = cnt;
  fsl.msc = msc;
  fsl.tau = tau;
  fsl.path = path;
  fsl.gx = static_cast<int>(gx);
  fsl.q_fp8 = q_fp8;
  fsl.q_scale = q_scale;
  fsl.w = w;
  fsl.k_fp8 = k_fp8;
  fsl.k_scale = k_scale;
  fsl.status = status;
  fsl.err_scale = err_scale;
  fsl.H = H_I;
  fsl.D = D_I;
  launch_fused_select(fsl, q_row_offsets, kv_row_offsets, B, max_q_rows, k, topk, st);
  return check_launch("dsa_index_topk(select)");
}
