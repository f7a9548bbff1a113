// topk.hip -- per-row top-k over the indexer scores (radix select in LDS).
//
// "MAX Pipeline 中的 DeepSeek-V3.2 架构实现解析", section "Indexer 的结构与计算流程": the
// indexer output is a top-k of shape (total_seq_len, index_topk); "GLM-5.3 推理全链路
// (十四)", section "验证段的逐层算子": each verify query selects its own 2048 keys.
//
// Selection order: (score desc, position asc). Scores map to order-preserving 32-bit
// keys (-0.0 canonicalised to +0.0, so equal values tie on position). One 1024-thread
// block per row.
// Rows of up to 64K scores first try the register path: the row is loaded once into
// registers (lane l of wave w holds positions 4096w + 64r + l, r < 64), every eighth
// slot serves as a sample whose 16-bit key classes give a threshold admitting about
// 1.25 k keys, and one ballot pass compacts the keys at or above it into per-wave LDS
// regions, in position order. Three histogram selects over these few thousand
// candidates (16-bit class below the maximum, bits 15..5, bits 4..0) give theta and
// the number of theta-ties to take, and a ballot pass emits ascending positions. A
// sample that admits fewer than k keys, or more than a wave region holds, sends the
// row to the exact LDS path below, which needs no sampling:
// the top 16 bits of every key go
// to LDS (128 KB) together with the row maximum; a histogram of each key's distance
// below the maximum (keys spread over hundreds of bins, so LDS atomics rarely collide)
// gives the 16-bit class of the k-th largest key; the positions at or above that class
// (k plus the class population) are compacted in position order with per-wave ballots;
// their full keys are gathered and the last 16 bits, the ties and the ascending
// emission run in LDS. Longer rows, or rows whose candidates overflow, take the
// general path, three reads of the row:
//   1. histogram of key bits 31..21 into four privatised LDS histograms (one per
//      group of four waves: indexer scores pile into a few top-bit bins, and one
//      shared histogram would serialise its atomics), then the bin B1 holding the
//      k-th largest key;
//   2. histogram of bits 20..10 of the keys in B1 only, giving the second digit B2;
//   3. ordered compaction of every key whose top 22 bits are >= (B1, B2) into LDS, in
//      position order. There are k + (keys sharing theta's top 22 bits) of them, a
//      few thousand at most for real score distributions.
// The last 10 bits, the tie count at theta and the ascending emission then run on
// the LDS candidates only. If the candidates overflow LDS (massive exact ties), a
// slow path finishes the select and the emission with further reads of the row.
// Block-wide prefix sums use DPP row shifts and row broadcasts within each wave.
#include "common.hpp"

namespace dsa {
namespace {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int NSUB = 4;        // privatised level-1 histograms
constexpr int CAND = 8192;     // slow-path LDS candidate capacity (key + position)
constexpr int FAST_MAX = 65536;  // rows up to this length keep 16-bit keys in LDS
constexpr int FCAND = 5984;     // fast-path candidate capacity
constexpr int SSTEP = 8;        // register path: every eighth slot is a threshold sample
constexpr int CW = 1024;        // register path: candidates per wave region (8 B each)

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x == 0.0f ? 0.0f : x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum across the 64 lanes of a wave: Hillis-Steele steps of 1, 2, 4 and
// 8 lanes inside each 16-lane row (DPP row_shr; lanes with no source add 0), then row
// broadcasts of lane 15 into rows 1 and 3 and of lane 31 into rows 2 and 3.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x111, 0xF, 0xF, false));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x112, 0xF, 0xF, false));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x114, 0xF, 0xF, false));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x118, 0xF, 0xF, false));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x142, 0xA, 0xF, false));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x143, 0xC, 0xF, false));
  return x;
}

// Wave-wide sum and maximum (unsigned), returned in every lane.
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wave_incl_scan(x)), 63));
}

__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x111, 0xF, 0xF, false)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x112, 0xF, 0xF, false)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x114, 0xF, 0xF, false)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x118, 0xF, 0xF, false)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x142, 0xA, 0xF, false)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x143, 0xC, 0xF, false)));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 63));
}

// Number of set bits of a ballot in the lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint64_t b) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(b >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(b), 0u));
}

// Exclusive block-wide prefix sum over NW waves (the whole block); *total gets the sum.
template <int NW = TK_WAVES>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
  const int lane = threadIdx.x % 64;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / 64));
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  const uint32_t tw = wave_incl_scan(lane < NW ? tmp[lane] : 0u);  // inclusive wave totals
  const uint32_t before =
      wave ? static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(tw), wave - 1)) : 0u;
  *total = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(tw), NW - 1));
  __syncthreads();
  return before + x - v;
}

// Visit the row as float4s, UNR loads in flight per thread (the passes are
// latency-bound otherwise), then the scalar tail.
template <class F>
__device__ __forceinline__ void for_each_score(const float* srow, int64_t n, F f) {
  constexpr int UNR = 16;  // 16 x 16 B per thread: a 64K-score row is read in one sweep
  const int tid = threadIdx.x;
  const int64_t n4 = n / 4;
  const float4* srow4 = reinterpret_cast<const float4*>(srow);
  for (int64_t i = tid; i < n4; i += UNR * TK_THREADS) {
    float4 v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t j = i + u * TK_THREADS;
      v[u] = j < n4 ? srow4[j] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u)
      if (i + u * TK_THREADS < n4) {
        f(v[u].x); f(v[u].y); f(v[u].z); f(v[u].w);
      }
  }
  for (int64_t i = n4 * 4 + tid; i < n; i += TK_THREADS) f(srow[i]);
}

// Find the bin holding the need-th largest key of a histogram of nb (<= 2048) bins.
// Writes the bin and the number of keys in higher bins to *sel (all threads see it).
__device__ __forceinline__ void select_bin(const uint32_t* hist, int nb, uint32_t need,
                                           uint32_t* tmp, uint32_t* sel) {
  const int d0 = 2 * threadIdx.x, d1 = d0 + 1;  // descending slots
  const uint32_t c0 = d0 < nb ? hist[nb - 1 - d0] : 0u;
  const uint32_t c1 = d1 < nb ? hist[nb - 1 - d1] : 0u;
  uint32_t total;
  const uint32_t ex = block_excl_scan(c0 + c1, tmp, &total);
  if (ex < need && need <= ex + c0) {
    sel[0] = nb - 1 - d0;
    sel[1] = ex;
  } else if (ex + c0 < need && need <= ex + c0 + c1) {
    sel[0] = nb - 1 - d1;
    sel[1] = ex + c0;
  }
  __syncthreads();
}

// Ordered emission over n keys produced by key_at(i) (position pos_at(i)), i in
// [0, n) in ascending position order: every key > theta and the first `need` keys
// == theta. Writes ascending positions to out[0..k).
template <class KeyAt, class PosAt>
__device__ __forceinline__ void emit_ordered(int64_t n, uint32_t theta, uint32_t need, int k,
                                             int32_t* out, uint32_t* tmp, KeyAt key_at,
                                             PosAt pos_at) {
  const int tid = threadIdx.x;
  uint32_t eq_seen = 0, emitted = 0;
  for (int64_t base = 0; base < n; base += 4 * TK_THREADS) {
    const int64_t i0 = base + 4 * tid;
    uint32_t key[4];
    bool live[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      live[j] = i0 + j < n;
      key[j] = live[j] ? key_at(i0 + j) : 0u;
    }
    uint32_t eqc = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) eqc += (live[j] && key[j] == theta) ? 1u : 0u;
    uint32_t eq_total;
    uint32_t eq_rank = eq_seen + block_excl_scan(eqc, tmp, &eq_total);
    bool sel[4];
    uint32_t selc = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool gt = live[j] && key[j] > theta;
      const bool eq = live[j] && key[j] == theta;
      sel[j] = gt || (eq && eq_rank < need);
      if (eq) ++eq_rank;
      selc += sel[j] ? 1u : 0u;
    }
    uint32_t sel_total;
    uint32_t pos = emitted + block_excl_scan(selc, tmp, &sel_total);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (sel[j] && pos < static_cast<uint32_t>(k)) out[pos++] = pos_at(i0 + j);
    eq_seen += eq_total;
    emitted += sel_total;
  }
}

// Smallest float whose order key is at least c16 << 16 (the floor of a 16-bit key class).
__device__ __forceinline__ float class_floor(uint32_t c16) {
  const uint32_t key = c16 << 16;
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Bin holding the need-th largest key of an NB-bin histogram whose bin 0 holds the
// largest keys, computed by every wave on its own (no block barrier): *bin gets the bin
// and *above the count in bins before it. Returns false (uniformly) if the histogram holds
// fewer than `need` keys.
template <int NB>
__device__ __forceinline__ bool wave_select(const uint32_t* hist, uint32_t need, uint32_t* bin,
                                            uint32_t* above) {
  constexpr int PER = NB / 64;
  const int lane = threadIdx.x % 64;
  uint32_t c[PER];
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    c[j] = hist[PER * lane + j];
    sum += c[j];
  }
  const uint32_t incl = wave_incl_scan(sum);
  const uint32_t ex = incl - sum;
  const uint64_t hit = __builtin_amdgcn_ballot_w64(ex < need && need <= incl);
  if (!hit) return false;
  const int src = __builtin_ctzll(hit);
  uint32_t acc = ex, b = 0, ab = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (acc < need && need <= acc + c[j]) {
      b = PER * lane + j;
      ab = acc;
    }
    acc += c[j];
  }
  *bin = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b), src));
  *above = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(ab), src));
  return true;
}

// One histogram add per active lane of a wave. The lanes whose bin equals the first active
// lane's add once through that lane, so a run of identical keys does not serialise on one
// LDS address; every other active lane adds 1.
__device__ __forceinline__ void hist_add(uint32_t* h, bool act, uint32_t bin) {
  const uint64_t am = __builtin_amdgcn_ballot_w64(act);
  if (am == 0) return;
  const int first = __builtin_ctzll(am);
  const uint32_t b0 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(bin), first));
  const uint32_t same = static_cast<uint32_t>(__popcll(__builtin_amdgcn_ballot_w64(act && bin == b0)));
  const bool lead = static_cast<int>(threadIdx.x % 64) == first;
  if (act && (lead || bin != b0)) atomicAdd(&h[bin], lead ? same : 1u);
}

// Register path for a row of k < n <= 16 * 64 * RS visible scores (see the top of the
// file); wave w holds positions 64 RS w + 64 r + lane in slot r < RS (RS = 64 for rows
// up to 64K; shorter rows take fewer slots per lane, so their candidates still spread
// over all sixteen waves). Returns false, uniformly over
// the block, when the sampled threshold admits fewer than k keys or more than a wave
// region holds, or theta's class falls outside the class histogram; nothing has been
// written to `out` then. cand: 128 KB of LDS (16 wave regions of CW key bits followed by
// CW positions); hist: 1280 words; rs: 80 words.
template <int RS>
__device__ __forceinline__ bool select_in_registers(const float* __restrict__ srow, int n, int k,
                                                    int32_t* __restrict__ out, uint32_t* cand,
                                                    uint32_t* hist, uint32_t* rs) {
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int p0 = wave * (64 * RS) + lane;  // wave w holds positions [64 RS w, 64 RS (w + 1))
  const float* __restrict__ vrow = srow + p0;
  uint32_t* hs = hist;          // 256 bins: sample classes below the sample maximum
  uint32_t* h1 = hist + 256;    // 512 bins: candidate classes below R = sample max + 128
  uint32_t* h2 = hist + 768;    // 256 bins: bits 15..8 inside theta's class
  uint32_t* h3 = hist + 1024;   // 256 bins: bits 7..0

  // ---- load: sample slots first. A wave whose whole segment is visible loads with
  // immediate offsets; the wave holding the end of the row loads from positions clamped
  // to n - 1 and then sets the slots past the end to -inf (sample slots before the
  // threshold, the rest before the compaction); waves past the end load nothing. ----
  float v[RS];
  const int lim = n - p0;  // slot r is visible iff 64 r < lim
  const int seg0 = wave * (64 * RS);
  const bool partial = seg0 < n && seg0 + 64 * RS > n;  // wave-uniform
  if (seg0 + 64 * RS <= n) {
#pragma unroll
    for (int r = 0; r < RS; r += SSTEP) v[r] = vrow[64 * r];
    __builtin_amdgcn_sched_barrier(0);  // keep the sample loads ahead of the rest
#pragma unroll
    for (int r = 0; r < RS; ++r)
      if (r % SSTEP != 0) v[r] = vrow[64 * r];
  } else if (partial) {
#pragma unroll
    for (int r = 0; r < RS; r += SSTEP) v[r] = srow[min(p0 + 64 * r, n - 1)];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < RS; ++r)
      if (r % SSTEP != 0) v[r] = srow[min(p0 + 64 * r, n - 1)];
#pragma unroll
    for (int r = 0; r < RS; r += SSTEP) v[r] = 64 * r < lim ? v[r] : -__builtin_inff();
  } else {
#pragma unroll
    for (int r = 0; r < RS; ++r) v[r] = -__builtin_inff();
  }
  for (int i = tid; i < 1280; i += TK_THREADS) hist[i] = 0;

  // ---- threshold: 16-bit classes of the samples below their maximum ----
  uint32_t smax = 0, scount = 0;
#pragma unroll
  for (int r = 0; r < RS; r += SSTEP)
    if (64 * r < lim) {
      smax = max(smax, order_key(v[r]) >> 16);
      ++scount;
    }
  smax = wave_max(smax);
  scount = wave_sum(scount);
  if (lane == 0) {
    rs[wave] = smax;
    rs[16 + wave] = scount;
  }
  __syncthreads();
  const uint32_t m16 = wave_max(lane < TK_WAVES ? rs[lane] : 0u);
  const uint32_t ns = wave_sum(lane < TK_WAVES ? rs[16 + lane] : 0u);
#pragma unroll
  for (int r = 0; r < RS; r += SSTEP) {
    const uint32_t d = m16 - (order_key(v[r]) >> 16);
    hist_add(hs, 64 * r < lim, d < 255 ? d : 255);
  }
  __syncthreads();
  // aim at 1.25 times the samples' expected share of the top k, plus 16
  const uint64_t want = (5ull * k * ns + 4ull * n - 1) / (4ull * n) + 16;
  const uint32_t wsamp = want < ns ? static_cast<uint32_t>(want) : ns;
  uint32_t dcut, above_s;
  wave_select<256>(hs, wsamp, &dcut, &above_s);
  uint32_t c16 = m16 > dcut ? m16 - dcut : 0u;
  if (dcut == 255) {  // uniform: the wanted sample lies past a gap of 255+ classes below the
                      // maximum; classify the samples beyond the gap below their own maximum
    uint32_t smax2 = 0;
#pragma unroll
    for (int r = 0; r < RS; r += SSTEP)
      if (64 * r < lim) {
        const uint32_t c = order_key(v[r]) >> 16;
        if (m16 - c >= 255) smax2 = max(smax2, c);
      }
    smax2 = wave_max(smax2);
    if (lane == 0) rs[wave] = smax2;  // the first maxima were read before the last barrier
    __syncthreads();
    const uint32_t m2 = wave_max(lane < TK_WAVES ? rs[lane] : 0u);
#pragma unroll
    for (int r = 0; r < RS; r += SSTEP) {
      const uint32_t c = order_key(v[r]) >> 16;
      const uint32_t d = m2 - c;
      hist_add(h3, 64 * r < lim && m16 - c >= 255, d < 255 ? d : 255);
    }
    __syncthreads();
    uint32_t d2, a2;
    wave_select<256>(h3, wsamp - above_s, &d2, &a2);
    c16 = m2 > d2 ? m2 - d2 : 0u;
    __syncthreads();  // every wave has read h3 before it is cleared for select 3
    for (int i = tid; i < 256; i += TK_THREADS) h3[i] = 0;
  }
  if (c16 < 0x80u) c16 = 0x80u;  // keeps the threshold above -inf (the padding value)
  const float t_lo = class_floor(c16);
  if (partial) {
#pragma unroll
    for (int r = 0; r < RS; ++r)
      if (r % SSTEP != 0) v[r] = 64 * r < lim ? v[r] : -__builtin_inff();
  }

  // ---- compaction: keys >= t_lo into this wave's region, in position order ----
  uint32_t* region = cand + wave * (2 * CW);  // CW key bits, then CW positions
  uint32_t cnt = 0;
  if (seg0 < n) {
#pragma unroll
    for (int r = 0; r < RS; ++r) {
      const bool c = v[r] >= t_lo;  // padding holds -inf, below any finite t_lo
      const uint64_t b = __builtin_amdgcn_ballot_w64(c);
      if (b) {
        // an overflowing wave falls back below, so its extra keys may share the last slot
        const uint32_t idx = min(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(b >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(b), cnt)),
                                 static_cast<uint32_t>(CW - 1));
        if (c) {
          region[idx] = __float_as_uint(v[r]);
          region[CW + idx] = static_cast<uint32_t>(p0 + 64 * r);
        }
        cnt += static_cast<uint32_t>(__popcll(b));
      }
    }
  }
  if (lane == 0) rs[32 + wave] = cnt;
  __syncthreads();
  const uint32_t wc = lane < TK_WAVES ? rs[32 + lane] : 0u;
  const uint32_t total = wave_sum(wc);
  if (wave_max(wc) > static_cast<uint32_t>(CW) || total < static_cast<uint32_t>(k)) return false;
  const uint32_t cw = cnt;

  // this lane's candidate keys (region entries lane + 64 j); 0 marks no candidate, since
  // every candidate key is at least 0x80 << 16. The whole region is read (it is all in
  // LDS) so the reads issue back to back, and entries past cw are masked afterwards.
  constexpr int KJ = CW / 64;
  uint32_t kreg[KJ];
#pragma unroll
  for (int j = 0; j < KJ; ++j) kreg[j] = region[lane + 64 * j];
#pragma unroll
  for (int j = 0; j < KJ; ++j)
    if (64 * j < static_cast<int>(cw))
      kreg[j] = lane + 64 * j < cw ? order_key(__uint_as_float(kreg[j])) : 0u;
  // slots j with 64 j >= cw hold no candidate in any lane: the loops below skip them with
  // a scalar test, so a wave pays only for the slots it fills

  // ---- select 1: 16-bit class of theta. Bin b holds class R - b for R = sample max + 128
  // (bin 0 also every class above R) when R - c16 < 512; across a wider gap, bins 0..254
  // hold classes R..R-254, bins 256..511 classes c16+255..c16 (the threshold class, below
  // which no candidate lies) and bin 255 everything between. theta may not fall in bin 0
  // nor in the gap bin ----
  const int R = static_cast<int>(m16) + 128;
  const int lo = static_cast<int>(c16);
  const bool gap = R - lo > 511;  // uniform
#pragma unroll
  for (int j = 0; j < KJ; ++j)
    if (64 * j < static_cast<int>(cw)) {
      const int c = static_cast<int>(kreg[j] >> 16);
      const int d = R - c;
      int bin = d > 0 ? d : 0;
      if (gap && d >= 255) bin = c - lo < 256 ? 511 - (c - lo) : 255;
      hist_add(h1, kreg[j] != 0, static_cast<uint32_t>(bin < 511 ? bin : 511));
    }
  __syncthreads();
  uint32_t b1, above;
  wave_select<512>(h1, k, &b1, &above);
  if (b1 == 0 || (gap && b1 == 255)) return false;
  const uint32_t c16t = gap && b1 > 255 ? c16 + (511 - b1) : static_cast<uint32_t>(R) - b1;
  uint32_t need = k - above;
  // ---- select 2: bits 15..8 of the keys in theta's class ----
#pragma unroll
  for (int j = 0; j < KJ; ++j)
    if (64 * j < static_cast<int>(cw)) hist_add(h2, (kreg[j] >> 16) == c16t, 255 - ((kreg[j] >> 8) & 255));
  __syncthreads();
  uint32_t b2;
  wave_select<256>(h2, need, &b2, &above);
  const uint32_t p24 = (c16t << 8) | (255 - b2);
  need -= above;
  // ---- select 3: bits 7..0 ----
#pragma unroll
  for (int j = 0; j < KJ; ++j)
    if (64 * j < static_cast<int>(cw)) hist_add(h3, (kreg[j] >> 8) == p24, 255 - (kreg[j] & 255));
  __syncthreads();
  uint32_t b3;
  wave_select<256>(h3, need, &b3, &above);
  const uint32_t theta = (p24 << 8) | (255 - b3);
  need -= above;

  // ---- emission: keys > theta and the first `need` theta-ties, ascending positions ----
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < KJ; ++j)
    if (64 * j < static_cast<int>(cw)) {
      gt += kreg[j] > theta ? 1u : 0u;
      eq += kreg[j] == theta ? 1u : 0u;
    }
  gt = wave_sum(gt);
  eq = wave_sum(eq);
  if (lane == 0) {
    rs[48 + wave] = gt;
    rs[64 + wave] = eq;
  }
  uint32_t preg[KJ];  // positions, read while the counts settle
#pragma unroll
  for (int j = 0; j < KJ; ++j) preg[j] = region[CW + lane + 64 * j];
  __syncthreads();
  // lane w < 16 holds wave w's counts: ties before wave w, the ties it takes, and the
  // number of outputs before it
  const uint32_t eq_w = lane < TK_WAVES ? rs[64 + lane] : 0u;
  const uint32_t gt_w = lane < TK_WAVES ? rs[48 + lane] : 0u;
  const uint32_t ties_ex = wave_incl_scan(eq_w) - eq_w;
  const uint32_t left = ties_ex < need ? need - ties_ex : 0u;
  const uint32_t own = gt_w + (eq_w < left ? eq_w : left);
  const uint32_t out_ex = wave_incl_scan(own) - own;
  const uint32_t ties_before =
      static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(ties_ex), wave));
  const uint32_t out_before =
      static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(out_ex), wave));
  uint32_t run_eq = 0, run_sel = 0;
#pragma unroll
  for (int j = 0; j < KJ; ++j) {
    if (64 * j < static_cast<int>(cw)) {
      const uint32_t key = kreg[j];
      const bool is_eq = key == theta;
      const uint64_t be = __builtin_amdgcn_ballot_w64(is_eq);
      const uint32_t rank = ties_before + run_eq + lanes_below(be);
      const bool take = key > theta || (is_eq && rank < need);
      const uint64_t bt = __builtin_amdgcn_ballot_w64(take);
      const uint32_t o = out_before + run_sel + lanes_below(bt);
      if (take && o < static_cast<uint32_t>(k)) out[o] = static_cast<int32_t>(preg[j]);
      run_eq += static_cast<uint32_t>(__popcll(be));
      run_sel += static_cast<uint32_t>(__popcll(bt));
    }
  }
  return true;
}

// Top-k of one score row of n entries (entries 0..n-1 of srow) by (score desc, index asc),
// written ascending to out[0..k), -1 padded. Called by a whole TK_THREADS block.
__device__ __forceinline__ void select_row(const float* __restrict__ srow, int64_t n, int k,
                                           int32_t* __restrict__ out) {
  // Region A (128 KB): 16-bit keys of the fast path; reused by both paths afterwards.
  __shared__ __attribute__((aligned(16))) uint32_t regA[32768];
  __shared__ uint32_t fhist[2048];
  __shared__ int32_t fpos[FCAND];
  __shared__ uint32_t tmp[2 * TK_WAVES];
  __shared__ uint32_t sel[2];
  __shared__ uint32_t smax;
  __shared__ uint32_t rs[80];  // register path: per-wave maxima and counts
  uint32_t (*hist)[2048] = reinterpret_cast<uint32_t (*)[2048]>(regA);  // slow path: NSUB x 8 KB
  uint32_t* ckey = regA + NSUB * 2048;                                  // slow path: 32 KB
  int32_t* cpos = reinterpret_cast<int32_t*>(regA + NSUB * 2048 + CAND);  // slow path: 32 KB

  const int tid = threadIdx.x, wave = tid / 64;
  if (n <= k) {
    for (int i = tid; i < k; i += TK_THREADS) out[i] = i < n ? i : -1;
    return;
  }

  if (n <= FAST_MAX) {
    const int ni = static_cast<int>(n);
    const bool done = n <= 16 * 64 * 8    ? select_in_registers<8>(srow, ni, k, out, regA, fhist, rs)
                      : n <= 16 * 64 * 16 ? select_in_registers<16>(srow, ni, k, out, regA, fhist, rs)
                                          : select_in_registers<64>(srow, ni, k, out, regA, fhist, rs);
    if (done) return;
    __syncthreads();  // fall back to the exact LDS path (region A and fhist are reused)
    // ---- fast path A: one read of the row; top 16 key bits to LDS, row maximum ----
    uint16_t* k16 = reinterpret_cast<uint16_t*>(regA);
    if (tid == 0) smax = 0;
    __syncthreads();
    uint32_t lmax = 0;
    {
      constexpr int UNR = 8;
      const int64_t n4 = n / 4;
      const float4* s4 = reinterpret_cast<const float4*>(srow);
      for (int64_t i = tid; i < n4; i += UNR * TK_THREADS) {
        float4 v[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const int64_t j = i + u * TK_THREADS;
          v[u] = j < n4 ? s4[j] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const int64_t j = i + u * TK_THREADS;
          if (j < n4) {
            const uint32_t a = order_key(v[u].x) >> 16, bb = order_key(v[u].y) >> 16;
            const uint32_t c = order_key(v[u].z) >> 16, d = order_key(v[u].w) >> 16;
            reinterpret_cast<uint2*>(k16)[j] = make_uint2(a | (bb << 16), c | (d << 16));
            lmax = max(lmax, max(max(a, bb), max(c, d)));
          }
        }
      }
      for (int64_t i = n4 * 4 + tid; i < n; i += TK_THREADS) {
        const uint32_t a = order_key(srow[i]) >> 16;
        k16[i] = static_cast<uint16_t>(a);
        lmax = max(lmax, a);
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) lmax = max(lmax, static_cast<uint32_t>(__shfl_xor(lmax, o)));
    if ((tid & 63) == 0) atomicMax(&smax, lmax);
    for (int i = tid; i < 2048; i += TK_THREADS) fhist[i] = 0;
    __syncthreads();
    const uint32_t m16 = smax;

    // ---- fast path B: histogram of the distance below the maximum (bin 2047 - d) ----
    {
      auto bin = [&](uint32_t key16) {
        const uint32_t d = m16 - key16;
        atomicAdd(&fhist[2047 - (d < 2047 ? d : 2047)], 1u);
      };
      const int64_t n8 = n / 8;  // eight 16-bit keys per 16-byte LDS read
      for (int64_t i = tid; i < n8; i += TK_THREADS) {
        const uint4 v = reinterpret_cast<const uint4*>(k16)[i];
        bin(v.x & 0xFFFFu); bin(v.x >> 16); bin(v.y & 0xFFFFu); bin(v.y >> 16);
        bin(v.z & 0xFFFFu); bin(v.z >> 16); bin(v.w & 0xFFFFu); bin(v.w >> 16);
      }
      for (int64_t i = n8 * 8 + tid; i < n; i += TK_THREADS) bin(k16[i]);
    }
    __syncthreads();
    select_bin(fhist, 2048, k, tmp, sel);
    const uint32_t D = 2047 - sel[0];     // distance of theta's 16-bit class below the max
    const uint32_t above = sel[1];        // keys strictly closer to the max
    const uint32_t ncand = above + fhist[sel[0]];
    __syncthreads();
    if (D < 2047 && ncand <= FCAND) {
      const uint32_t c16 = m16 - D;
      // ---- fast path C: positions with key16 >= c16, compacted in order. Wave w owns a
      // contiguous segment; a lane takes 8 consecutive keys per 16-byte LDS read, so a
      // wave step covers 512 positions: count pass, block offsets, write pass.
      const int lane = tid & 63;
      const int64_t seg = ((n + TK_WAVES - 1) / TK_WAVES + 511) / 512 * 512;
      const int64_t lo = wave * seg, hi = lo + seg < n ? lo + seg : n;
      auto flags = [&](int64_t p0) -> uint32_t {  // bit j: position p0 + 8*lane + j is a candidate
        const int64_t q = p0 + 8 * lane;
        uint32_t f = 0;
        if (q + 7 < hi) {
          const uint4 v = *reinterpret_cast<const uint4*>(k16 + q);
          const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            f |= ((w4[j] & 0xFFFFu) >= c16 ? 1u : 0u) << (2 * j);
            f |= ((w4[j] >> 16) >= c16 ? 1u : 0u) << (2 * j + 1);
          }
        } else {
          for (int j = 0; j < 8; ++j)
            if (q + j < hi && k16[q + j] >= c16) f |= 1u << j;
        }
        return f;
      };
      uint32_t cnt = 0;
      for (int64_t p0 = lo; p0 < hi; p0 += 512) cnt += __popc(flags(p0));
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o);
      if (lane == 0) tmp[wave] = cnt;
      __syncthreads();
      uint32_t base = 0;
      for (int w = 0; w < wave; ++w) base += tmp[w];
      for (int64_t p0 = lo; p0 < hi; p0 += 512) {
        uint32_t f = flags(p0);
        const uint32_t c = __popc(f);
        uint32_t x = c;  // inclusive scan of the lane counts
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t y = __shfl_up(x, o);
          if (lane >= o) x += y;
        }
        uint32_t slot = base + x - c;
        const int64_t q = p0 + 8 * lane;
        while (f) {
          const int j = __ffs(f) - 1;
          f &= f - 1;
          fpos[slot++] = static_cast<int32_t>(q + j);
        }
        base += __shfl(x, 63);
      }
      __syncthreads();
      // ---- fast path D: full keys of the candidates (region A is free again) ----
      uint32_t* fkey = regA;
      for (uint32_t j = tid; j < ncand; j += TK_THREADS) fkey[j] = order_key(srow[fpos[j]]);
      uint32_t* h3 = regA + FCAND;
      for (int i = tid; i < 2048; i += TK_THREADS) h3[i] = 0;
      __syncthreads();
      // ---- fast path E: bits 15..5, then 4..0, of the keys in theta's class ----
      uint32_t need = k - above;
      for (uint32_t j = tid; j < ncand; j += TK_THREADS)
        if ((fkey[j] >> 16) == c16) atomicAdd(&h3[(fkey[j] >> 5) & 2047], 1u);
      __syncthreads();
      select_bin(h3, 2048, need, tmp, sel);
      const uint32_t p27 = (c16 << 11) | sel[0];
      need -= sel[1];
      __syncthreads();
      if (tid < 32) h3[tid] = 0;
      __syncthreads();
      for (uint32_t j = tid; j < ncand; j += TK_THREADS)
        if ((fkey[j] >> 5) == p27) atomicAdd(&h3[fkey[j] & 31], 1u);
      __syncthreads();
      select_bin(h3, 32, need, tmp, sel);
      const uint32_t theta = (p27 << 5) | sel[0];
      need -= sel[1];
      __syncthreads();
      emit_ordered(ncand, theta, need, k, out, tmp, [&](int64_t i) { return fkey[i]; },
                   [&](int64_t i) { return fpos[i]; });
      return;
    }
    __syncthreads();  // overflow: fall through to the general path (region A is reused)
  }

  // ---- 1. level-1 digit (bits 31..21) over privatised histograms ----
  for (int i = tid; i < NSUB * 2048; i += TK_THREADS) (&hist[0][0])[i] = 0;
  __syncthreads();
  {
    uint32_t* h = hist[wave % NSUB];
    for_each_score(srow, n, [&](float x) { atomicAdd(&h[order_key(x) >> 21], 1u); });
  }
  __syncthreads();
  for (int i = tid; i < 2048; i += TK_THREADS)
    hist[0][i] = hist[0][i] + hist[1][i] + hist[2][i] + hist[3][i];
  __syncthreads();
  select_bin(hist[0], 2048, k, tmp, sel);
  const uint32_t b1 = sel[0];
  uint32_t need = k - sel[1];  // keys still to take inside bin b1
  __syncthreads();

  // ---- 2. level-2 digit (bits 20..10) of the keys in b1 ----
  uint32_t* h2 = hist[1];
  for (int i = tid; i < 2048; i += TK_THREADS) h2[i] = 0;
  __syncthreads();
  auto add2 = [&](float x) {
    const uint32_t key = order_key(x);
    if ((key >> 21) == b1) atomicAdd(&h2[(key >> 10) & 2047], 1u);
  };
  for_each_score(srow, n, add2);
  __syncthreads();
  select_bin(h2, 2048, need, tmp, sel);
  const uint32_t p22 = (b1 << 11) | sel[0];  // top 22 bits of theta
  need -= sel[1];
  const uint32_t class_count = h2[sel[0]];    // keys sharing theta's top 22 bits
  const uint32_t ncand = (k - need) + class_count;
  __syncthreads();

  if (ncand <= CAND) {
    // ---- 3. compact candidates (top 22 bits >= p22) into LDS in position order ----
    uint32_t filled = 0;
    constexpr int PRE = 8;  // tiles loaded ahead of the ordered scans
    for (int64_t sbase = 0; sbase < n; sbase += PRE * 4 * TK_THREADS) {
      float4 v[PRE];
#pragma unroll
      for (int u = 0; u < PRE; ++u) {
        const int64_t p0 = sbase + u * 4 * TK_THREADS + 4 * tid;
        v[u] = p0 + 3 < n ? *reinterpret_cast<const float4*>(srow + p0) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < PRE; ++u) {
        const int64_t base = sbase + u * 4 * TK_THREADS;
        if (base >= n) break;  // block-uniform
        const int64_t p0 = base + 4 * tid;
        uint32_t key[4];
        bool c[4];
        uint32_t cc = 0;
        if (p0 + 3 < n) {
          key[0] = order_key(v[u].x); key[1] = order_key(v[u].y);
          key[2] = order_key(v[u].z); key[3] = order_key(v[u].w);
#pragma unroll
          for (int j = 0; j < 4; ++j) c[j] = (key[j] >> 10) >= p22;
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            key[j] = p0 + j < n ? order_key(srow[p0 + j]) : 0u;
            c[j] = p0 + j < n && (key[j] >> 10) >= p22;
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) cc += c[j] ? 1u : 0u;
        uint32_t tot;
        uint32_t slot = filled + block_excl_scan(cc, tmp, &tot);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (c[j]) {
            ckey[slot] = key[j];
            cpos[slot] = static_cast<int32_t>(p0 + j);
            ++slot;
          }
        filled += tot;
      }
    }
    __syncthreads();
    // level-3 digit (bits 9..0) among candidates of the theta class
    uint32_t* h3 = hist[2];
    for (int i = tid; i < 1024; i += TK_THREADS) h3[i] = 0;
    __syncthreads();
    for (uint32_t i = tid; i < ncand; i += TK_THREADS)
      if ((ckey[i] >> 10) == p22) atomicAdd(&h3[ckey[i] & 1023], 1u);
    __syncthreads();
    select_bin(h3, 1024, need, tmp, sel);
    const uint32_t theta = (p22 << 10) | sel[0];
    need -= sel[1];
    __syncthreads();
    emit_ordered(ncand, theta, need, k, out, tmp, [&](int64_t i) { return ckey[i]; },
                 [&](int64_t i) { return cpos[i]; });
    return;
  }

  // ---- slow path: level 3 and the emission read the row again ----
  uint32_t* h3 = hist[2];
  for (int i = tid; i < 1024; i += TK_THREADS) h3[i] = 0;
  __syncthreads();
  auto add3 = [&](float x) {
    const uint32_t key = order_key(x);
    if ((key >> 10) == p22) atomicAdd(&h3[key & 1023], 1u);
  };
  for_each_score(srow, n, add3);
  __syncthreads();
  select_bin(h3, 1024, need, tmp, sel);
  const uint32_t theta = (p22 << 10) | sel[0];
  need -= sel[1];
  __syncthreads();
  emit_ordered(n, theta, need, k, out, tmp, [&](int64_t i) { return order_key(srow[i]); },
               [&](int64_t i) { return static_cast<int32_t>(i); });
}

// One block per row: rows of up to FAST_MAX visible scores, and every row when the grid
// has no chunk stage.
__global__ __launch_bounds__(TK_THREADS) void topk_kernel(const float* __restrict__ scores,
                                                          int64_t ld,
                                                          const int32_t* __restrict__ q_off,
                                                          const int64_t* __restrict__ kv_off,
                                                          int k, int32_t* __restrict__ topk) {
  const int b = blockIdx.y, r = blockIdx.x;
  const RowInfo ri = load_row_info(q_off, kv_off, b);
  if (r >= ri.R) return;
  const int64_t t = ri.t0 + r;
  int64_t n = visible_count(ri, r);
  if (n > ld) n = ld;  // device lengths beyond the score stride are clipped
  select_row(scores + t * ld, n, k, topk + t * k);
}

// Grids with rows longer than FAST_MAX, stage 1: block (chunk c, row) selects the top-k of
// visible positions [c FAST_MAX, (c+1) FAST_MAX) as chunk-local indices into widx
// [T, nchunk, k] and their scores into the row's candidate scores cand_s (chunk c at
// offset c k; -inf where the index is -1). Every key of the row's top-k is in the top-k
// of its chunk. A row of at most FAST_MAX positions is finished here by its chunk-0 block.
__global__ __launch_bounds__(TK_THREADS) void topk_chunk_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ q_off,
    const int64_t* __restrict__ kv_off, int k, int nchunk, int64_t cstride,
    int32_t* __restrict__ widx, float* __restrict__ cand_s, int32_t* __restrict__ topk) {
  const int b = blockIdx.y, r = blockIdx.x / nchunk, c = blockIdx.x % nchunk;
  const RowInfo ri = load_row_info(q_off, kv_off, b);
  if (r >= ri.R) return;
  const int64_t t = ri.t0 + r;
  int64_t n = visible_count(ri, r);
  if (n > ld) n = ld;
  const float* srow = scores + t * ld;
  if (n <= FAST_MAX) {
    if (c == 0) select_row(srow, n, k, topk + t * k);
    return;
  }
  const int64_t c0 = static_cast<int64_t>(c) * FAST_MAX;
  if (c0 >= n) return;  // the merge reads only the chunks holding visible positions
  const int64_t nc = n - c0 < FAST_MAX ? n - c0 : FAST_MAX;
  int32_t* o = widx + (t * nchunk + c) * k;
  select_row(srow + c0, nc, k, o);
  __syncthreads();  // the block's index stores are visible to its own loads after this
  float* cs = cand_s + t * cstride + static_cast<int64_t>(c) * k;
  for (int i = threadIdx.x; i < k; i += TK_THREADS) {
    const int32_t j = o[i];
    cs[i] = j >= 0 ? srow[c0 + j] : -__builtin_inff();
  }
}

// Rows longer than FAST_MAX, stage 2: the candidate scores of the row's chunks, in chunk
// order, are in ascending position order (each chunk's list is ascending and only the
// last list ends in padding), so the top-k of that compact row, mapped back through the
// chunk indices, is the row's top-k: ties between equal scores still go to the lower
// position, and a -inf pad follows every visible -inf.
__global__ __launch_bounds__(TK_THREADS) void topk_merge_kernel(
    const int32_t* __restrict__ q_off, const int64_t* __restrict__ kv_off, int64_t ld, int k,
    int nchunk, int64_t cstride, const int32_t* __restrict__ widx,
    const float* __restrict__ cand_s, int32_t* __restrict__ topk) {
  const int b = blockIdx.y, r = blockIdx.x;
  const RowInfo ri = load_row_info(q_off, kv_off, b);
  if (r >= ri.R) return;
  const int64_t t = ri.t0 + r;
  int64_t n = visible_count(ri, r);
  if (n > ld) n = ld;
  if (n <= FAST_MAX) return;
  const int64_t m = (n + FAST_MAX - 1) / FAST_MAX * k;  // this row's chunks
  int32_t* out = topk + t * k;
  select_row(cand_s + t * cstride, m, k, out);
  __syncthreads();
  const int32_t* wrow = widx + t * nchunk * k;
  for (int i = threadIdx.x; i < k; i += TK_THREADS) {
    const int32_t j = out[i];
    if (j >= 0) out[i] = (j / k) * FAST_MAX + wrow[j];
  }
}

// ---------------------------------------------------------------------------------------
// Exact-boundary refine (see dsa_topk in dsa.h). One block per row, after topk_kernel:
//  1. theta = the smallest float32 score in the row's selection; eps from the row's FP8
//     queries, weights and the largest key scale among its visible keys;
//  2. one pass over the row: keys above theta + 2 eps are kept (they are all in the
//     selection already), keys in [theta - 2 eps, theta + 2 eps] form the band;
//  3. every band key is rescored in float64 (the head dots are exact; the weighted sum
//     over heads runs in ascending head order, one rounding per product and per sum);
//  4. the best k - |kept| band keys by (exact score desc, position asc) join the kept
//     keys, and the row is rewritten ascending.
constexpr int RF_THREADS = 1024;
constexpr int RF_WAVES = RF_THREADS / 64;
constexpr int BAND_CAP = 4096;
constexpr int RF_MAXK = 4096;

// e4m3fn code -> value (exact): normal (8 + m) 2^(e-10), subnormal m 2^-9; 0x7F/0xFF
// (NaN) are never produced by the quantiser and decode here as 0.
__device__ __forceinline__ double e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  double v = (e == 15u && m == 7u) ? 0.0
             : e ? __builtin_ldexp(static_cast<double>(8u + m), static_cast<int>(e) - 10)
                 : __builtin_ldexp(static_cast<double>(m), -9);
  return (c & 0x80u) ? -v : v;
}

__device__ __forceinline__ float block_min_f(float x, float* red) {
  for (int o = 32; o >= 1; o >>= 1) x = fminf(x, __shfl_xor(x, o));
  if (threadIdx.x % 64 == 0) red[threadIdx.x / 64] = x;
  __syncthreads();
  float y = red[0];
  for (int w = 1; w < RF_WAVES; ++w) y = fminf(y, red[w]);
  __syncthreads();
  return y;
}

__device__ __forceinline__ float block_max_f(float x, float* red) {
  return -block_min_f(-x, red);
}

// Bitonic sort of np2 (a power of two) LDS entries by `before`, one compare-exchange per
// pair and stage, the whole block taking part.
template <class Before, class Swap>
__device__ __forceinline__ void block_bitonic(int np2, Before before, Swap swap) {
  for (int size = 2; size <= np2; size <<= 1) {
    for (int stride = size / 2; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < np2 / 2; i += RF_THREADS) {
        const int a = 2 * i - (i & (stride - 1)), c = a + stride;
        const bool up = (a & size) == 0;
        if (up ? before(c, a) : before(a, c)) swap(a, c);
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

__global__ __launch_bounds__(RF_THREADS) void topk_refine_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ q_off,
    const int64_t* __restrict__ kv_off, int k, const uint8_t* __restrict__ q_fp8,
    const float* __restrict__ q_scale, const float* __restrict__ wt,
    const uint8_t* __restrict__ k_fp8, const float* __restrict__ k_scale, int H, int D,
    double err_scale, int32_t* __restrict__ topk, int32_t* __restrict__ status) {
  __shared__ double dtab[256];
  __shared__ int32_t band_pos[BAND_CAP];
  __shared__ double band_val[BAND_CAP];
  __shared__ int32_t in_pos[RF_MAXK];
  __shared__ int32_t sel_pos[RF_MAXK];
  __shared__ double kdec[RF_WAVES][128];  // one band key's decoded codes per wave
  __shared__ float redf[RF_WAVES];
  __shared__ double redd[RF_WAVES];
  __shared__ uint32_t tmp[2 * TK_WAVES];
  __shared__ int counters[4];  // band size

  const int b = blockIdx.y, r = blockIdx.x;
  const RowInfo ri = load_row_info(q_off, kv_off, b);
  if (r >= ri.R) return;
  const int64_t t = ri.t0 + r;
  int64_t n = visible_count(ri, r);
  if (n > ld) n = ld;
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  if (n <= k) {  // every visible key is selected whatever the scores
    if (tid == 0 && status) status[t] = 0;
    return;
  }
  const float* srow = scores + t * ld;
  int32_t* out = topk + t * k;
  const float* ksc = k_scale + ri.kv_base;
  for (int c = tid; c < 256; c += RF_THREADS) dtab[c] = e4m3_value(static_cast<uint32_t>(c));
  if (tid < 4) counters[tid] = 0;

  // ---- 1. theta, the largest visible key scale, and sum_j |u_j| max_c |q_hat[j,c]|;
  // loads are issued eight at a time per thread so the scans are not latency-bound ----
  constexpr int U = 8;
  float th = __builtin_inff();
  for (int i0 = tid; i0 < k; i0 += U * RF_THREADS) {
    int32_t pp[U];
#pragma unroll
    for (int u = 0; u < U; ++u) pp[u] = i0 + u * RF_THREADS < k ? out[i0 + u * RF_THREADS] : -1;
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      v[u] = __builtin_inff();
      if (pp[u] >= 0) v[u] = srow[pp[u]];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) th = fminf(th, v[u]);
  }
  th = block_min_f(th, redf);
  float smax = 0.0f;
  {
    // scalar head up to a 16-byte boundary, float4 body (four loads in flight), scalar tail
    const int64_t head = static_cast<int64_t>((16 - (reinterpret_cast<uintptr_t>(ksc) & 15)) & 15) / 4;
    const int64_t h0 = head < n ? head : n;
    if (tid < h0) smax = ksc[tid];
    const int64_t nb4 = (n - h0) / 4;
    const float4* k4 = reinterpret_cast<const float4*>(ksc + h0);
    for (int64_t i0 = tid; i0 < nb4; i0 += 4 * RF_THREADS) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i0 + u * RF_THREADS < nb4) v[u] = k4[i0 + u * RF_THREADS];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        smax = fmaxf(smax, fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w)));
    }
    for (int64_t s = h0 + 4 * nb4 + tid; s < n; s += RF_THREADS) smax = fmaxf(smax, ksc[s]);
  }
  smax = block_max_f(smax, redf);
  double asum = 0.0;  // sum_j |u_j| max_c |q_hat[j,c]|: 8 codes per thread and load, the
                      // D/8 threads of a head reduce with xor shuffles inside their group
  {
    const int per_head = D / 8;  // 16 or 8 threads
    const uint2* q8 = reinterpret_cast<const uint2*>(q_fp8 + t * H * D);
    for (int i0 = tid; i0 < H * per_head; i0 += RF_THREADS) {
      const uint2 v = q8[i0];
      uint32_t mc = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        mc = max(mc, (v.x >> (8 * e)) & 0x7Fu);
        mc = max(mc, (v.y >> (8 * e)) & 0x7Fu);
      }
      for (int o = per_head / 2; o >= 1; o >>= 1)
        mc = max(mc, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mc), o)));
      if (i0 % per_head == 0) {
        const int j = i0 / per_head;
        const double u = static_cast<double>(wt[t * H + j]) * static_cast<double>(q_scale[t * H + j]);
        asum += __builtin_fabs(u) * e4m3_value(mc);
      }
    }
    for (int o = 32; o >= 1; o >>= 1) asum += __shfl_xor(asum, o);
  }
  if (lane == 0) redd[wave] = asum;
  __syncthreads();
  double A = 0.0;
  for (int w = 0; w < RF_WAVES; ++w) A += redd[w];
  const double C = err_scale > 0.0 ? err_scale : 4.0;
  const double eps = C * 0x1p-16 * 448.0 * static_cast<double>(smax) * A;
  const double hi = static_cast<double>(th) + 2.0 * eps, lo = static_cast<double>(th) - 2.0 * eps;

  // ---- 2. kept keys (counted) and the band (collected); float4 loads, four in flight ----
  uint32_t nin = 0;
  auto classify = [&](float xf, int64_t s) {
    const double x = static_cast<double>(xf);
    if (x > hi) {
      ++nin;
    } else if (x >= lo) {
      const int slot = atomicAdd(&counters[0], 1);
      if (slot < BAND_CAP) band_pos[slot] = static_cast<int32_t>(s);
    }
  };
  const int64_t n4 = n / 4;
  const float4* s4 = reinterpret_cast<const float4*>(srow);  // rows are 16-byte aligned
  for (int64_t i0 = tid; i0 < n4; i0 += 4 * RF_THREADS) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i0 + u * RF_THREADS < n4) v[u] = s4[i0 + u * RF_THREADS];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + u * RF_THREADS;
      if (i < n4) {
        classify(v[u].x, 4 * i);
        classify(v[u].y, 4 * i + 1);
        classify(v[u].z, 4 * i + 2);
        classify(v[u].w, 4 * i + 3);
      }
    }
  }
  for (int64_t s = 4 * n4 + tid; s < n; s += RF_THREADS) classify(srow[s], s);
  uint32_t nin_total;
  block_excl_scan<RF_WAVES>(nin, tmp, &nin_total);  // ends with a barrier: counters[0] is final
  const int nb = counters[0];
  const int need = k - static_cast<int>(nin_total);
  if (nb > BAND_CAP || need < 1 || need > nb) {  // uniform: keep the float32 selection
    if (tid == 0 && status) status[t] = nb > BAND_CAP ? -1 : -2;
    return;
  }

  // ---- 3. exact rescore, one band key per wave at a time; lane j owns heads j and j+64.
  // A key's codes are prefetched one iteration ahead; the weighted head sum runs in
  // ascending head order over readlane. ----
  double uh[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int j = lane + 64 * hh;
    uh[hh] = j < H ? static_cast<double>(wt[t * H + j]) * static_cast<double>(q_scale[t * H + j]) : 0.0;
  }
  auto key_codes = [&](int i) -> uint32_t {  // two codes of band key i per lane (D <= 128)
    uint32_t c2 = 0;
    if (i < nb && 2 * lane < D)
      c2 = *reinterpret_cast<const uint16_t*>(k_fp8 + (ri.kv_base + band_pos[i]) * D + 2 * lane);
    return c2;
  };
  uint32_t kc = key_codes(wave);
  for (int i = wave; i < nb; i += RF_WAVES) {
    const int32_t p = band_pos[i];
    if (2 * lane < D) {
      kdec[wave][2 * lane] = dtab[kc & 0xFFu];
      kdec[wave][2 * lane + 1] = dtab[(kc >> 8) & 0xFFu];
    }
    kc = key_codes(i + RF_WAVES);  // next key of this wave, in flight during this one
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    double tj[2] = {0.0, 0.0};
    for (int hh = 0; hh < (H > 64 ? 2 : 1); ++hh) {  // wave-uniform
      uint4 qv[8];  // this lane's head codes (reloaded per key: cache hits)
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        qv[v] = make_uint4(0u, 0u, 0u, 0u);
        if (lane + 64 * hh < H && v < D / 16)
          qv[v] = reinterpret_cast<const uint4*>(q_fp8 + (t * H + lane + 64 * hh) * D)[v];
      }
      // exact: every partial sum is a multiple of 2^-18 below 2^53 units, so the four
      // interleaved partial sums and their total are exact in any order
      double d4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        if (v < D / 16) {
          const uint32_t wd[4] = {qv[v].x, qv[v].y, qv[v].z, qv[v].w};
#pragma unroll
          for (int e = 0; e < 16; ++e)
            d4[e % 4] = __builtin_fma(dtab[(wd[e / 4] >> (8 * (e % 4))) & 0xFFu],
                                      kdec[wave][16 * v + e], d4[e % 4]);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep each group's table reads local
      }
      const double d = (d4[0] + d4[1]) + (d4[2] + d4[3]);
      tj[hh] = __dmul_rn(uh[hh], d > 0.0 ? d : 0.0);
    }
    double acc = 0.0;  // heads 0..H-1 in order: lane j's tj[0], then lane j's tj[1] (j + 64)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int lo_w = __double2loint(tj[hh]), hi_w = __double2hiint(tj[hh]);
#pragma unroll
      for (int j = 0; j < 64; ++j)
        if (64 * hh + j < H)
          acc = __dadd_rn(acc, __hiloint2double(__builtin_amdgcn_readlane(hi_w, j),
                                                __builtin_amdgcn_readlane(lo_w, j)));
    }
    if (lane == 0) band_val[i] = __dmul_rn(acc, static_cast<double>(ksc[p]));
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  __syncthreads();

  // ---- 4. the best `need` band keys by (exact score desc, position asc), as ascending
  // positions in sel_pos; then a merge with the kept keys ----
  if (nb <= 64) {  // one wave ranks the band with register broadcasts: no block barriers
    if (wave == 0) {
      const bool live = lane < nb;
      const double v = live ? band_val[lane] : -__builtin_inf();
      const int32_t p = live ? band_pos[lane] : 0x7FFFFFFF;
      const int vlo = __double2loint(v), vhi = __double2hiint(v);
      int rank = 0;
      for (int m = 0; m < nb; ++m) {
        const double vm = __hiloint2double(__builtin_amdgcn_readlane(vhi, m),
                                           __builtin_amdgcn_readlane(vlo, m));
        const int32_t pm = __builtin_amdgcn_readlane(p, m);
        rank += (vm > v || (vm == v && pm < p)) ? 1 : 0;
      }
      const bool take = live && rank < need;
      int at = 0;  // rank by position among the taken keys
      for (int m = 0; m < nb; ++m) {
        const int32_t pm = __builtin_amdgcn_readlane(p, m);
        const bool tm = __builtin_amdgcn_readlane(take ? 1 : 0, m) != 0;
        at += (tm && pm < p) ? 1 : 0;
      }
      if (take) sel_pos[at] = p;
    }
    __syncthreads();
  } else {
    // pad the band to a power of two with entries that sort last, then bitonic sorts
    const int np2 = next_pow2(nb);
    for (int i = nb + tid; i < np2; i += RF_THREADS) {
      band_val[i] = -__builtin_inf();
      band_pos[i] = 0x7FFFFFFF;
    }
    __syncthreads();
    block_bitonic(
        np2,
        [&](int x, int y) {
          return band_val[x] > band_val[y] ||
                 (band_val[x] == band_val[y] && band_pos[x] < band_pos[y]);
        },
        [&](int x, int y) {
          const double v = band_val[x];
          band_val[x] = band_val[y];
          band_val[y] = v;
          const int32_t q = band_pos[x];
          band_pos[x] = band_pos[y];
          band_pos[y] = q;
        });
    const int ns2 = next_pow2(need > 1 ? need : 2);
    for (int i = tid; i < ns2; i += RF_THREADS) sel_pos[i] = i < need ? band_pos[i] : 0x7FFFFFFF;
    __syncthreads();
    block_bitonic(
        ns2, [&](int x, int y) { return sel_pos[x] < sel_pos[y]; },
        [&](int x, int y) {
          const int32_t q = sel_pos[x];
          sel_pos[x] = sel_pos[y];
          sel_pos[y] = q;
        });
  }
  // kept keys in the current (ascending) selection, order preserved; k <= RF_MAXK, so at
  // most four entries per thread, taken as one contiguous run
  constexpr int PER = RF_MAXK / RF_THREADS;
  int32_t mine[PER];
  uint32_t cnt = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid * PER + j;
    mine[j] = -1;
    if (i < k) {
      const int32_t p = out[i];
      if (static_cast<double>(srow[p]) > hi) {
        mine[j] = p;
        ++cnt;
      }
    }
  }
  uint32_t kept;
  uint32_t at = block_excl_scan<RF_WAVES>(cnt, tmp, &kept);  // ends with a barrier
  if (kept != nin_total) {  // uniform; cannot happen for a correct float32 selection
    if (tid == 0 && status) status[t] = -3;
    return;
  }
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (mine[j] >= 0) in_pos[at++] = mine[j];
  __syncthreads();
  auto count_below = [](const int32_t* a, int len, int32_t p) {  // a ascending
    int lo_i = 0, hi_i = len;
    while (lo_i < hi_i) {
      const int mid = (lo_i + hi_i) / 2;
      if (a[mid] < p) lo_i = mid + 1;
      else hi_i = mid;
    }
    return lo_i;
  };
  for (int i = tid; i < static_cast<int>(kept); i += RF_THREADS)
    out[i + count_below(sel_pos, need, in_pos[i])] = in_pos[i];
  for (int i = tid; i < need; i += RF_THREADS)
    out[i + count_below(in_pos, static_cast<int>(kept), sel_pos[i])] = sel_pos[i];
  if (tid == 0 && status) status[t] = nb;
}

}  // namespace
}  // namespace dsa

namespace dsa {
namespace {
// Chunks of rows longer than FAST_MAX, and the stride of the compact candidate rows.
int64_t topk_nchunk(int64_t max_kv_len) { return max_kv_len > FAST_MAX ? ceil_div(max_kv_len, FAST_MAX) : 1; }
int64_t topk_cstride(int64_t nchunk, int k) { return (nchunk * k + 3) / 4 * 4; }
}  // namespace
}  // namespace dsa

extern "C" size_t dsa_topk_workspace_size(int32_t T, int64_t max_kv_len, int32_t k) {
  using namespace dsa;
  if (T <= 0 || k <= 0) return 0;
  const int64_t nc = topk_nchunk(max_kv_len);
  if (nc <= 1) return 0;
  // chunk indices [T, nc, k] (padded to 16 bytes), then candidate scores [T, cstride]
  return static_cast<size_t>((static_cast<int64_t>(T) * nc * k + 3) / 4 * 4 +
                             static_cast<int64_t>(T) * topk_cstride(nc, k)) * 4;
}

extern "C" dsa_status dsa_topk(const float* scores, int64_t score_ld,
                               const int32_t* q_row_offsets, const int64_t* kv_row_offsets,
                               int32_t B, int32_t T, int32_t max_q_rows, int64_t max_kv_len,
                               int32_t k, const dsa_topk_refine* refine, int32_t* topk, void* ws,
                               size_t ws_bytes, void* stream) {
  using namespace dsa;
  DSA_REQUIRE(k >= 1 && k <= 8192, "dsa_topk: k must be in [1, 8192] (got %d)", k);
  DSA_REQUIRE(B >= 0 && T >= 0 && max_q_rows >= 0 && max_kv_len >= 0, "dsa_topk: negative size");
  DSA_REQUIRE(score_ld >= max_kv_len && score_ld % 4 == 0,
              "dsa_topk: score_ld must be >= max_kv_len and a multiple of 4");
  DSA_REQUIRE(max_kv_len < (int64_t(1) << 31), "dsa_topk: max_kv_len must be < 2^31");
  if (refine) {
    DSA_REQUIRE((reinterpret_cast<uintptr_t>(refine->q_fp8) & 15) == 0,
                "dsa_topk: refine q_fp8 must be 16-byte aligned");
    DSA_REQUIRE(k <= RF_MAXK, "dsa_topk: the refine supports k <= %d (got %d)", RF_MAXK, k);
    DSA_REQUIRE(refine->D_I == 64 || refine->D_I == 128, "dsa_topk: refine D_I must be 64 or 128");
    DSA_REQUIRE(refine->H_I >= 1 && refine->H_I <= 128, "dsa_topk: refine H_I must be in [1, 128]");
    DSA_REQUIRE(refine->err_scale >= 0.0, "dsa_topk: refine err_scale must be >= 0");
  }
  if (B == 0 || T == 0 || max_q_rows == 0) return ok();
  DSA_REQUIRE(scores && q_row_offsets && kv_row_offsets && topk, "dsa_topk: null pointer");
  DSA_REQUIRE(!refine || (refine->q_fp8 && refine->q_scale && refine->w && refine->k_fp8 &&
                          refine->k_scale),
              "dsa_topk: null refine pointer");
  DSA_REQUIRE((reinterpret_cast<uintptr_t>(scores) & 15) == 0,
              "dsa_topk: scores must be 16-byte aligned");
  DSA_REQUIRE(B <= 65535, "dsa_topk: B must be <= 65535");
  dim3 grid((unsigned)max_q_rows, (unsigned)B);
  const int64_t nchunk = topk_nchunk(max_kv_len);
  if (nchunk > 1) {
    const size_t need = dsa_topk_workspace_size(T, max_kv_len, k);
    if (ws_bytes < need || !ws)
      return fail(DSA_ERR_WORKSPACE_TOO_SMALL,
                  "dsa_topk: rows longer than %d need a %zu-byte workspace (got %zu)", FAST_MAX,
                  need, ws_bytes);
    DSA_REQUIRE((reinterpret_cast<uintptr_t>(ws) & 15) == 0, "dsa_topk: ws must be 16-byte aligned");
    DSA_REQUIRE(max_q_rows * nchunk <= 0x7FFFFFFF, "dsa_topk: too many chunks");
    int32_t* widx = static_cast<int32_t*>(ws);
    const int64_t cstride = topk_cstride(nchunk, k);
    float* cand_s = reinterpret_cast<float*>(widx + (static_cast<int64_t>(T) * nchunk * k + 3) / 4 * 4);
    hipLaunchKernelGGL(topk_chunk_kernel, dim3((unsigned)(max_q_rows * nchunk), (unsigned)B),
                       dim3(TK_THREADS), 0, as_stream(stream), scores, score_ld, q_row_offsets,
                       kv_row_offsets, k, (int)nchunk, cstride, widx, cand_s, topk);
    hipLaunchKernelGGL(topk_merge_kernel, grid, dim3(TK_THREADS), 0, as_stream(stream),
                       q_row_offsets, kv_row_offsets, score_ld, k, (int)nchunk, cstride, widx,
                       cand_s, topk);
  } else {
    hipLaunchKernelGGL(topk_kernel, grid, dim3(TK_THREADS), 0, as_stream(stream), scores,
                       score_ld, q_row_offsets, kv_row_offsets, k, topk);
  }
  if (refine)
    hipLaunchKernelGGL(topk_refine_kernel, grid, dim3(RF_THREADS), 0, as_stream(stream), scores,
                       score_ld, q_row_offsets, kv_row_offsets, k, refine->q_fp8, refine->q_scale,
                       refine->w, refine->k_fp8, refine->k_scale, refine->H_I, refine->D_I,
                       refine->err_scale, topk, refine->status);
  return check_launch("dsa_topk");
}
