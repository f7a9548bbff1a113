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
#include "fused.hpp"

namespace dsa {
namespace {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int NSUB = 4;        // privatised level-1 histograms
constexpr int CAND = 8192;     // slow-path LDS candidate capacity (key + position)
constexpr int FAST_MAX = 65536;  // rows up to this length keep 16-bit keys in LDS
constexpr int FCAND = 5952;     // fast-path candidate capacity
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

// ---------------------------------------------------------------------------------------
// Exact-boundary refine (see dsa_topk in dsa.h). With theta the k-th largest float32
// score of a row and eps a bound on |I_f32 - I_exact| for every visible key, keys above
// theta + 2 eps are in the exact top-k, keys below theta - 2 eps are not, and the band in
// between is rescored exactly and ranked by (exact score desc, position asc).
//  - The register path refines in place: the row is still in registers, so one pass
//    over them marks the kept keys in a position bitmap and lists the band.
//  - Every other path (rows whose sample missed, rows longer than 64K) runs the generic
//    refine after its float32 selection is written: one more read of the row.
// eps needs the largest key scale among the row's visible keys (an upper bound of it serves
// too: the band only widens). No row rescans them: either the caller keeps a table of the
// maxima of every SC_CHUNK consecutive cache rows (dsa_key_scale_max, updated by the cache
// write), or a pre-pass stores the maximum of every SC_CHUNK scales of each request.
constexpr int BAND_CAP = 4096;   // band keys rescored per row
constexpr int RF_MAXK = 4096;    // k supported by the refine
constexpr int SC_CHUNK = 2048;   // key scales per stored maximum
static_assert(SC_CHUNK == DSA_KEY_SCALE_CHUNK, "the caller's table uses the header's chunk");

struct Refine {  // kernel argument; q_fp8 == nullptr: no refine
  const uint8_t* q_fp8;
  const float* q_scale;
  const float* w;
  const uint8_t* k_fp8;
  const float* k_scale;
  const float* kmax;  // [B, nsc] maxima of SC_CHUNK key scales each, or nullptr
  const float* kglob; // maxima of SC_CHUNK consecutive cache rows' scales (kept by the
                      // caller), or nullptr
  int64_t kglob_len;  // entries of kglob
  int32_t* status;    // [T] or nullptr
  double C;
  int H, D, nsc;
  float smax_given;   // the row's largest visible key scale when kmax and kglob are nullptr
};

struct RowRef {  // one row of a refine
  Refine rf;
  int64_t t;        // query row
  int b;            // request
  int64_t kv_base;  // first cache row of the request
};

// LDS of the refine, overlaid on the 128 KB candidate region once a selection no longer
// needs it.
constexpr int RS_TERMS = 4096;   // u_j max(d_j, 0) of one rescoring round: [head][key]
struct RefineLds {
  double band_val[BAND_CAP];      // exact band scores
  double terms[RS_TERMS];
  uint32_t digits[256];           // e4m3fn code -> its three signed base-128 digits (bytes 0..2)
  int32_t band_pos[BAND_CAP];
  int32_t sel_pos[RF_MAXK];
  int32_t in_pos[RF_MAXK];
  uint32_t bitmap[FAST_MAX / 32];  // register path: selected positions
  double redd[TK_WAVES];
  float redf[TK_WAVES];
  uint32_t cnt[TK_WAVES];
  int counters[4];
  double eps;  // register path -> finish_register_refine
  int nb, need;
};
static_assert(RF_MAXK >= BAND_CAP, "band scales and scores are staged in sel_pos / in_pos");
static_assert(sizeof(RefineLds) <= 32768 * 4, "refine LDS overlays the 128 KB region");

// e4m3fn code -> value (exact): normal (8 + m) 2^(e-10), subnormal m 2^-9; 0x7F/0xFF
// (NaN) are never produced by the quantiser and decode here as 0.
__device__ __forceinline__ double e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  double v = (e == 15u && m == 7u) ? 0.0
             : e ? __builtin_ldexp(static_cast<double>(8u + m), static_cast<int>(e) - 10)
                 : __builtin_ldexp(static_cast<double>(m), -9);
  return (c & 0x80u) ? -v : v;
}

__device__ __forceinline__ double block_max_d(double x, double* red) {
  for (int o = 32; o >= 1; o >>= 1) x = fmax(x, __shfl_xor(x, o));
  if (threadIdx.x % 64 == 0) red[threadIdx.x / 64] = x;
  __syncthreads();
  double y = red[0];
  for (int w = 1; w < TK_WAVES; ++w) y = fmax(y, red[w]);
  __syncthreads();
  return y;
}

// eps of a row (every thread gets it):
//   C 2^-16 448 smax A  +  (H + 3) 2^-23 |theta|
// A = sum_j |u_j| max_c |q_hat[t,j,c]| (u = w q_scale), smax = the largest key scale of the
// SC_CHUNK chunks that hold the row's n visible keys. The first term is the FP8 MFMA's
// accumulation error per head dot (up to C 2^-16 of the largest possible product, 448
// max|q_hat_j|) weighted by |u_j| and the key scale; the second the float32 epilogue (H
// products, H sums, the scale multiply) for nonnegative weights.
// refine_prefetch leaves per-wave partial sums of A and maxima of smax in pa / ps (no block
// barrier; issued before the selection so that its loads overlap the row's), and
// refine_eps combines them once a block barrier has passed.
__device__ __forceinline__ void refine_prefetch(const RowRef& rr, int64_t n, double* pa, float* ps) {
  const Refine& rf = rr.rf;
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int H = rf.H, D = rf.D;
  const int per_head = D / 8;  // threads per head, 8 codes each (16 or 8, a divisor of 64)
  const uint2* q8 = reinterpret_cast<const uint2*>(rf.q_fp8 + rr.t * H * D);
  double asum = 0.0;
  for (int i0 = tid; i0 < H * per_head; i0 += TK_THREADS) {  // whole head groups stay together
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
      const double u = static_cast<double>(rf.w[rr.t * H + j]) *
                       static_cast<double>(rf.q_scale[rr.t * H + j]);
      asum += __builtin_fabs(u) * e4m3_value(mc);  // codes with the sign bit cleared
    }
  }
  float sm = 0.0f;
  if (rf.kglob) {
    // the table entries of cache rows kv_base .. kv_base + n - 1; a row outside the table
    // makes eps infinite (the float32 selection is kept)
    if (n > 0) {
      const int64_t c0 = rr.kv_base >= 0 ? rr.kv_base / SC_CHUNK : -1;
      const int64_t c1 = rr.kv_base >= 0 ? (rr.kv_base + n - 1) / SC_CHUNK : -1;
      for (int64_t c = c0 + tid; c <= c1; c += TK_THREADS)
        sm = fmaxf(sm, c >= 0 && c < rf.kglob_len ? rf.kglob[c] : __builtin_inff());
    }
  } else if (rf.kmax) {
    int nc = static_cast<int>((n + SC_CHUNK - 1) / SC_CHUNK);
    if (nc > rf.nsc) nc = rf.nsc;  // rows are clipped to the score stride; stay in the table
    for (int c = tid; c < nc; c += TK_THREADS)
      sm = fmaxf(sm, rf.kmax[static_cast<int64_t>(rr.b) * rf.nsc + c]);
  } else {
    sm = rf.smax_given;
  }
  for (int o = 32; o >= 1; o >>= 1) {
    asum += __shfl_xor(asum, o);
    sm = fmaxf(sm, __shfl_xor(sm, o));
  }
  if (lane == 0) {
    pa[wave] = asum;
    ps[wave] = sm;
  }
}

__device__ __forceinline__ double refine_eps(const Refine& rf, float theta, const double* pa,
                                             const float* ps) {
  double A = 0.0, smax = 0.0;
  for (int w = 0; w < TK_WAVES; ++w) {  // fixed order: the same value in every thread
    A += pa[w];
    smax = fmax(smax, static_cast<double>(ps[w]));
  }
  const double C = rf.C > 0.0 ? rf.C : 4.0;
  return C * 0x1p-16 * 448.0 * smax * A +
         (rf.H + 3) * 0x1p-23 * __builtin_fabs(static_cast<double>(theta));
}

// The next float above / below a finite x (one ulp; -0 and +0 step to the smallest
// subnormals).
__device__ __forceinline__ float float_up(float x) {
  const uint32_t u = __float_as_uint(x);
  if (x == 0.0f) return __uint_as_float(1u);
  return __uint_as_float((u & 0x80000000u) ? u - 1u : u + 1u);
}

__device__ __forceinline__ float float_down(float x) { return -float_up(-x); }

// Float thresholds around theta: x > hi_f implies x > theta + 2 eps, and x >= lo_f holds for
// every x >= theta - 2 eps (rounded outwards, so the band can only grow). Finite inputs.
__device__ __forceinline__ void band_edges(float theta, double eps, float* lo_f, float* hi_f) {
  const double hi = static_cast<double>(theta) + 2.0 * eps;
  const double lo = static_cast<double>(theta) - 2.0 * eps;
  float h = static_cast<float>(hi), l = static_cast<float>(lo);
  if (static_cast<double>(h) < hi) h = float_up(h);
  if (static_cast<double>(l) > lo) l = float_down(l);
  *hi_f = h;
  *lo_f = l;
}

// The exact value of e4m3fn code c times 2^9 is an integer of magnitude below 2^18: (8 + m)
// 2^(e-1) for a normal code, m for a subnormal one. Written x = x0 + 2^7 x1 + 2^14 x2 in base
// 128, each digit carrying the code's sign, it packs into one word as three signed bytes
// (|x0|, |x1| <= 127, |x2| <= 15).
__device__ __forceinline__ uint32_t e4m3_digit_word(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const uint32_t x = e ? (8u + m) << (e - 1u) : m;
  const bool neg = (c & 0x80u) != 0u;
  uint32_t word = 0;
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    const uint32_t dgt = (x >> (7 * p)) & 127u;
    word |= ((neg ? 0u - dgt : dgt) & 0xFFu) << (8 * p);
  }
  return word;
}

// The digit words (e4m3_digit_word, from the LDS table) of sixteen codes (one 16-byte load).
__device__ __forceinline__ void digit_words(i32x4 codes, const uint32_t* table, uint32_t (&wd)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i)
    wd[i] = table[(static_cast<uint32_t>(codes[i / 4]) >> (8 * (i % 4))) & 0xFFu];
}

// Digit plane p of sixteen codes as an int8 MFMA operand: byte i of the operand is digit p of
// code i. Three byte permutes per word: v_perm_b32(x, y, sel) picks byte sel_i of the eight
// bytes {x, y} (y bytes 0..3, x bytes 4..7; selector 0x0c gives 0).
template <int P>
__device__ __forceinline__ i32x4 digit_plane(const uint32_t (&wd)[16]) {
  constexpr uint32_t pair = P | ((4 + P) << 8) | 0x0c0c0000u;  // [y byte P, x byte P, 0, 0]
  i32x4 out;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t lo = __builtin_amdgcn_perm(wd[4 * w + 1], wd[4 * w], pair);
    const uint32_t hi = __builtin_amdgcn_perm(wd[4 * w + 3], wd[4 * w + 2], pair);
    out[w] = static_cast<int>(__builtin_amdgcn_perm(hi, lo, 0x05040100u));
  }
  return out;
}

// Exact scores of the nb band keys (positions in L.band_pos, request-local) into
// L.band_val; returns (to thread 0) the largest |I_f32 - I_exact| over the band, I_f32
// read from srow (or given in band_f32 when srow is null). band_sk and band_f32 are LDS
// staging arrays of at least nb entries, free until the band is chosen.
//   I_exact = s_k * sum_{j ascending} u_j * max(d_j, 0), d_j = q_hat[t,j] . k_hat (exact),
// evaluated in float64 with one rounding per product and per sum.
// The head dots are exact integer arithmetic on the int8 MFMA: every e4m3fn value times 2^9
// is an integer below 2^18, split into three base-128 digits; the nine digit-plane products
// (v_mfma_i32_16x16x64_i8) chain into five int32 accumulators, one per digit-weight 2^(7s)
// (s = a + b, |sum| < 3 * 2^21). They recombine exactly: lo = acc_0 + 2^7 acc_1 and
// hi = acc_2 + 2^7 acc_3 + 2^14 acc_4 stay below 2^30 in int32 (the top digits are below 16),
// and d 2^18 = lo + 2^14 hi (|d| 2^18 < 2^44) is one exact float64 fma. A
// wave takes one tile of 16 heads x 16 band keys per round, with the next round's key codes
// already loading; the u_j max(d_j, 0) terms of a round go to LDS, and one thread per key
// then adds them in ascending head order.
template <class Lds>
__device__ __forceinline__ double rescore_band(const RowRef& rr, const float* __restrict__ srow,
                                               int nb, Lds& L, bool table_ready,
                                               float* band_sk, float* band_f32) {
  const Refine& rf = rr.rf;
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int H = rf.H, D = rf.D;
  const int HT = H <= 16 ? 1 : H <= 32 ? 2 : H <= 64 ? 4 : 8;  // 16-head tiles (padded)
  const int KPR = 256 / HT;            // keys per round: (16 / HT) tiles of 16
  const int ht = wave % HT, kt = wave / HT;
  const int c16 = lane % 16, g = lane / 16;
  const int64_t t = rr.t;
  const uint8_t* __restrict__ kreq = rf.k_fp8 + rr.kv_base * D;
  const float* __restrict__ ksc = rf.k_scale + rr.kv_base;
  const int halves = D / 64;           // K = 64 per MFMA
  const int slot = 16 * kt + c16;      // this lane's key within a round
  // B operand codes of band key base + slot: dims 64 h + 16 g .. + 16 (zeros past the band)
  auto load_keys = [&](int base, i32x4 (&kc)[2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      kc[h] = (i32x4){0, 0, 0, 0};
      if (h < halves && base + slot < nb)
        kc[h] = *reinterpret_cast<const i32x4*>(
            kreq + static_cast<int64_t>(L.band_pos[base + slot]) * D + 64 * h + 16 * g);
    }
  };
  // every global load of the first round is issued before any is used: the first round's
  // key codes, this lane's query codes (head 16 ht + c16, dims 64 h + 16 g .. + 16; heads
  // past H are 0) and the weights of its output heads 16 ht + 4 g + i
  i32x4 kc[2];
  load_keys(0, kc);
  i32x4 qc[2];
  {
    const int head = 16 * ht + c16;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      qc[h] = (i32x4){0, 0, 0, 0};
      if (h < halves && head < H)
        qc[h] = *reinterpret_cast<const i32x4*>(rf.q_fp8 + (t * H + head) * D + 64 * h + 16 * g);
    }
  }
  double u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int head = 16 * ht + 4 * g + i;
    u[i] = head < H ? static_cast<double>(rf.w[t * H + head]) * static_cast<double>(rf.q_scale[t * H + head])
                    : 0.0;
  }
  // every band key's scale (and float32 score, unless band_f32 already holds them: srow
  // null) staged in LDS while the loads above are in flight
  for (int i = tid; i < nb; i += TK_THREADS) {
    const int32_t p = L.band_pos[i];
    band_sk[i] = ksc[p];
    if (srow) band_f32[i] = srow[p];
  }
  if (!table_ready) {  // block-uniform
    for (int c = tid; c < 256; c += TK_THREADS) L.digits[c] = e4m3_digit_word(static_cast<uint32_t>(c));
    __syncthreads();
  }
  i32x4 qa[2][3];  // A operands: the query digit planes
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t wd[16];
    digit_words(qc[h], L.digits, wd);
    qa[h][0] = digit_plane<0>(wd);
    qa[h][1] = digit_plane<1>(wd);
    qa[h][2] = digit_plane<2>(wd);
  }
  double worst = 0.0;
  // A band of one round with at most 64 keys is summed, ranked and read back by wave 0 alone
  // (thread i sums key i and writes band_val[i]): no barrier after its sums, and its error
  // maximum is a wave reduction.
  const bool one_wave = nb <= KPR && KPR <= 64;  // block-uniform
  for (int base = 0; base < nb; base += KPR) {  // block-uniform rounds
    if (base + 16 * kt < nb) {  // wave-uniform: the tile holds at least one band key
      i32x4 kb[2][3];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t wd[16];
        digit_words(kc[h], L.digits, wd);
        kb[h][0] = digit_plane<0>(wd);
        kb[h][1] = digit_plane<1>(wd);
        kb[h][2] = digit_plane<2>(wd);
      }
      if (base + KPR < nb) load_keys(base + KPR, kc);  // the next round's codes, in flight
      i32x4 acc[5];  // digit weight 2^(7s): sum of the (a, b) plane products with a + b = s
#pragma unroll
      for (int sw = 0; sw < 5; ++sw) acc[sw] = (i32x4){0, 0, 0, 0};
      // both halves unconditionally: with D = 64 the second half's codes are all 0
#pragma unroll
      for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int b = 0; b < 3; ++b) {
          acc[a + b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[0][a], kb[0][b], acc[a + b], 0, 0, 0);
          acc[a + b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[1][a], kb[1][b], acc[a + b], 0, 0, 0);
        }
      // heads past H (padding of the last tile) have u = 0 and so a +0 term
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int head = 16 * ht + 4 * g + i;
        // the exact dot of head 4 g + i and key c16 (2^18 d = lo + 2^14 hi, exact)
        const int32_t lo = acc[0][i] + acc[1][i] * 128;
        const int32_t hi = acc[2][i] + acc[3][i] * 128 + acc[4][i] * 16384;
        const double d = __builtin_fma(static_cast<double>(hi), 16384.0, static_cast<double>(lo));
        const double dj = __builtin_ldexp(d, -18);
        L.terms[head * KPR + slot] = __dmul_rn(u[i], dj > 0.0 ? dj : 0.0);
      }
    }
    __syncthreads();
    if (tid < KPR && base + tid < nb) {  // one thread per key: heads in ascending order
      const float sk = band_sk[base + tid], f32 = band_f32[base + tid];
      // all 16 HT heads: the sum starts at +0 and so never is -0, and the +0 terms of the
      // padding heads at its end leave it unchanged. Eight terms are read ahead of the
      // eight being added.
      const int nh = 16 * HT;
      double acc = 0.0;
      double tv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) tv[j] = L.terms[j * KPR + tid];
      for (int j0 = 0; j0 < nh; j0 += 8) {
        double nx[8];
        if (j0 + 8 < nh) {  // block-uniform
#pragma unroll
          for (int j = 0; j < 8; ++j) nx[j] = L.terms[(j0 + 8 + j) * KPR + tid];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = __dadd_rn(acc, tv[j]);
#pragma unroll
        for (int j = 0; j < 8; ++j) tv[j] = nx[j];
      }
      const double ex = __dmul_rn(acc, static_cast<double>(sk));
      L.band_val[base + tid] = ex;
      worst = fmax(worst, __builtin_fabs(static_cast<double>(f32) - ex));
    }
    if (!one_wave) __syncthreads();
  }
  if (one_wave) {
    if (wave == 0)
      for (int o = 32; o >= 1; o >>= 1) worst = fmax(worst, __shfl_xor(worst, o));
    return worst;
  }
  return block_max_d(worst, L.redd);
}

// Bitonic sort of np2 (a power of two) LDS entries by `before`, one compare-exchange per
// pair and stage, the whole block taking part.
template <class Before, class Swap>
__device__ __forceinline__ void block_bitonic(int np2, Before before, Swap swap) {
  for (int size = 2; size <= np2; size <<= 1) {
    for (int stride = size / 2; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < np2 / 2; i += TK_THREADS) {
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

// The best `need` of the nb band keys by (exact score desc, position asc). With SORTED,
// their positions go to L.sel_pos in ascending order; otherwise each is set in L.bitmap.
template <bool SORTED>
__device__ __forceinline__ void choose_band(int nb, int need, RefineLds& L) {
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  if (nb <= 64) {  // one wave ranks the band with register broadcasts: no block barriers
    if (wave == 0) {
      const bool live = lane < nb;
      const double v = live ? L.band_val[lane] : -__builtin_inf();
      const int32_t p = live ? L.band_pos[lane] : 0x7FFFFFFF;
      const int vlo = __double2loint(v), vhi = __double2hiint(v);
      int rank = 0;
      for (int m = 0; m < nb; ++m) {
        const double vm = __hiloint2double(__builtin_amdgcn_readlane(vhi, m),
                                           __builtin_amdgcn_readlane(vlo, m));
        const int32_t pm = __builtin_amdgcn_readlane(p, m);
        rank += (vm > v || (vm == v && pm < p)) ? 1 : 0;
      }
      const bool take = live && rank < need;
      if constexpr (SORTED) {
        int at = 0;  // rank by position among the taken keys
        for (int m = 0; m < nb; ++m) {
          const int32_t pm = __builtin_amdgcn_readlane(p, m);
          const bool tm = __builtin_amdgcn_readlane(take ? 1 : 0, m) != 0;
          at += (tm && pm < p) ? 1 : 0;
        }
        if (take) L.sel_pos[at] = p;
      } else {
        if (take) atomicOr(&L.bitmap[p >> 5], 1u << (p & 31));
      }
    }
    __syncthreads();
    return;
  }
  // pad the band to a power of two with entries that sort last, then bitonic sorts
  const int np2 = next_pow2(nb);
  for (int i = nb + tid; i < np2; i += TK_THREADS) {
    L.band_val[i] = -__builtin_inf();
    L.band_pos[i] = 0x7FFFFFFF;
  }
  __syncthreads();
  block_bitonic(
      np2,
      [&](int x, int y) {
        return L.band_val[x] > L.band_val[y] ||
               (L.band_val[x] == L.band_val[y] && L.band_pos[x] < L.band_pos[y]);
      },
      [&](int x, int y) {
        const double v = L.band_val[x];
        L.band_val[x] = L.band_val[y];
        L.band_val[y] = v;
        const int32_t q = L.band_pos[x];
        L.band_pos[x] = L.band_pos[y];
        L.band_pos[y] = q;
      });
  if constexpr (SORTED) {
    const int ns2 = next_pow2(need > 1 ? need : 2);
    for (int i = tid; i < ns2; i += TK_THREADS) L.sel_pos[i] = i < need ? L.band_pos[i] : 0x7FFFFFFF;
    __syncthreads();
    block_bitonic(
        ns2, [&](int x, int y) { return L.sel_pos[x] < L.sel_pos[y]; },
        [&](int x, int y) {
          const int32_t q = L.sel_pos[x];
          L.sel_pos[x] = L.sel_pos[y];
          L.sel_pos[y] = q;
        });
  } else {
    for (int i = tid; i < need; i += TK_THREADS)
      atomicOr(&L.bitmap[L.band_pos[i] >> 5], 1u << (L.band_pos[i] & 31));
    __syncthreads();
  }
}

// Status of a refined row: the band size, or -4 when a band key's float32 score is off
// its exact value by more than eps / 2 (the set is the refined one, but the margin the
// bound assumes is not there).
__device__ __forceinline__ int32_t refine_status(int nb, double worst, double eps) {
  return worst > 0.5 * eps ? -4 : nb;
}

// Register path for a row of k < n <= 16 * 64 * RS visible scores (see the top of the
// file); wave w holds positions 64 RS w + 64 r + lane in slot r < RS (RS = 64 for rows
// up to 64K; shorter rows take fewer slots per lane, so their candidates still spread
// over all sixteen waves). Returns false, uniformly over
// the block, when the sampled threshold admits fewer than k keys or more than a wave
// region holds, or theta's class falls outside the class histogram; nothing has been
// written to `out` then. cand: 128 KB of LDS (16 wave regions of CW key bits followed by
// CW positions); hist: 1280 words; rs: 80 words; tmp: 32 words.
// Returns REG_DONE with the selection written, REG_FALLBACK as described, or, with
// `refine`, REG_BAND: the kept keys are in the refine's position bitmap and the band in its
// list (one pass over the registers), and finish_register_refine completes the row. A band
// that cannot be resolved here (it overflows, or eps is not finite) gives REG_FALLBACK, and
// the generic refine decides after the LDS path.
constexpr int REG_FALLBACK = 0, REG_DONE = 1, REG_BAND = 2;

template <int RS>
__device__ __forceinline__ int select_in_registers(const float* __restrict__ srow, int n, int k,
                                                    int32_t* __restrict__ out, uint32_t* cand,
                                                    uint32_t* hist, uint32_t* rs, uint32_t* tmp,
                                                    const RowRef& rr, bool refine, double* pa,
                                                    float* ps) {
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
  // the refine's query-side bound: its loads queue behind the row's, whose wait comes next
  if (refine) refine_prefetch(rr, n, pa, ps);

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
  if (wave_max(wc) > static_cast<uint32_t>(CW) || total < static_cast<uint32_t>(k)) return REG_FALLBACK;
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
  if (b1 == 0 || (gap && b1 == 255)) return REG_FALLBACK;
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

  if (refine) {
    // ---- refine in registers: theta's band lies among the compacted candidates unless it
    // reaches below their threshold class (then the generic refine decides). Kept keys go
    // to a position bitmap, band keys to a list; finish_register_refine rescores the band,
    // adds its best keys to the bitmap and emits it in ascending order ----
    RefineLds& L = *reinterpret_cast<RefineLds*>(cand);
    uint32_t preg[KJ];  // this lane's candidate positions, read before L overlays the regions
#pragma unroll
    for (int j = 0; j < KJ; ++j) preg[j] = region[CW + lane + 64 * j];
    __syncthreads();  // every wave is done with its region
    const float th = __uint_as_float((theta & 0x80000000u) ? (theta & 0x7FFFFFFFu) : ~theta);
    if (tid < 4) L.counters[tid] = 0;
    for (int i = tid; i < FAST_MAX / 32; i += TK_THREADS) L.bitmap[i] = 0u;
    if (tid < 256) L.digits[tid] = e4m3_digit_word(static_cast<uint32_t>(tid));  // for the rescore
    const double eps = refine_eps(rr.rf, th, pa, ps);
    if (!__builtin_isfinite(th) || !__builtin_isfinite(eps)) return REG_FALLBACK;  // uniform
    __syncthreads();  // the cleared counters and bitmap are visible
    float lo_f, hi_f;
    band_edges(th, eps, &lo_f, &hi_f);
    const uint32_t lo_k = order_key(lo_f), hi_k = order_key(hi_f);
    if (lo_k < (c16 << 16)) return REG_FALLBACK;  // uniform: the band reaches below the candidates
    uint32_t kept_w = 0;
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      if (64 * j < static_cast<int>(cw)) {  // wave-uniform
        const uint32_t key = kreg[j];       // 0: no candidate
        const bool kp = key != 0u && key > hi_k;
        const bool bd = key != 0u && !kp && key >= lo_k;
        const int p = static_cast<int>(preg[j]);
        if (kp) atomicOr(&L.bitmap[p >> 5], 1u << (p & 31));
        kept_w += static_cast<uint32_t>(__popcll(__builtin_amdgcn_ballot_w64(kp)));
        const uint64_t bb = __builtin_amdgcn_ballot_w64(bd);
        if (bb) {
          int base = 0;
          if (lane == 0) base = atomicAdd(&L.counters[0], static_cast<int>(__popcll(bb)));
          base = __builtin_amdgcn_readfirstlane(base);
          if (bd) {
            const int slot = base + static_cast<int>(lanes_below(bb));
            if (slot < BAND_CAP) L.band_pos[slot] = p;
          }
        }
      }
    }
    if (lane == 0) L.cnt[wave] = kept_w;
    __syncthreads();
    const int nb = L.counters[0];
    int kept = 0;
    for (int w2 = 0; w2 < TK_WAVES; ++w2) kept += static_cast<int>(L.cnt[w2]);
    const int need_b = k - kept;
    if (nb > BAND_CAP || need_b < 1 || need_b > nb) return REG_FALLBACK;  // uniform
    if (tid == 0) {
      L.eps = eps;
      L.nb = nb;
      L.need = need_b;
    }
    __syncthreads();
    return REG_BAND;
  }

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
  return REG_DONE;
}

// LDS of one top-k block (one row at a time).
struct TopkLds {
  uint32_t regA[32768];  // 128 KB: register-path regions, 16-bit keys, slow-path histograms
                         // and candidates, or the refine (RefineLds)
  uint32_t fhist[2048];
  int32_t fpos[FCAND];
  uint32_t tmp[2 * TK_WAVES];
  uint32_t sel[2];
  uint32_t smax;
  uint32_t rs[80];  // register path: per-wave maxima and counts
  double rf_a[TK_WAVES];  // refine: per-wave partials of eps (refine_prefetch)
  float rf_s[TK_WAVES];
};

// Float32 top-k of one score row by the LDS paths (every row length): writes the
// selection ascending to out[0..k), -1 padded. Requires n > k.
__device__ __forceinline__ void select_row_lds(const float* __restrict__ srow, int64_t n, int k,
                                               int32_t* __restrict__ out, TopkLds& S) {
  uint32_t* regA = S.regA;
  uint32_t* fhist = S.fhist;
  int32_t* fpos = S.fpos;
  uint32_t* tmp = S.tmp;
  uint32_t* sel = S.sel;
  uint32_t& smax = S.smax;
  uint32_t (*hist)[2048] = reinterpret_cast<uint32_t (*)[2048]>(regA);  // slow path: NSUB x 8 KB
  uint32_t* ckey = regA + NSUB * 2048;                                  // slow path: 32 KB
  int32_t* cpos = reinterpret_cast<int32_t*>(regA + NSUB * 2048 + CAND);  // slow path: 32 KB

  const int tid = threadIdx.x, wave = tid / 64;
  if (n <= FAST_MAX) {
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

__device__ __forceinline__ void refine_generic(const float* __restrict__ srow, int64_t n, int k,
                                               int32_t* __restrict__ out, const RowRef& rr,
                                               RefineLds& L, uint32_t* tmp, const double* pa,
                                               const float* ps);

// The rest of a register-path refine (REG_BAND): rescore the band, add its best keys to the
// bitmap, and emit the bitmap's positions in ascending order (thread i takes words 2i and
// 2i + 1, positions 64 i .. 64 i + 63).
__device__ __forceinline__ void finish_register_refine(const float* __restrict__ srow, int n,
                                                       int k, int32_t* __restrict__ out,
                                                       const RowRef& rr, RefineLds& L,
                                                       uint32_t* tmp) {
  const int tid = threadIdx.x;
  const int nb = L.nb, need = L.need;
  const double eps = L.eps;
  const double worst = rescore_band(rr, srow, nb, L, true, reinterpret_cast<float*>(L.sel_pos),
                                    reinterpret_cast<float*>(L.in_pos));
  choose_band<false>(nb, need, L);
  const int nw = (n + 31) / 32;
  const uint32_t wd0 = 2 * tid < nw ? L.bitmap[2 * tid] : 0u;
  const uint32_t wd1 = 2 * tid + 1 < nw ? L.bitmap[2 * tid + 1] : 0u;
  uint32_t total;
  uint32_t o = block_excl_scan(static_cast<uint32_t>(__popc(wd0) + __popc(wd1)), tmp, &total);
  auto emit = [&](uint32_t wd, int pos0) {
    while (wd) {
      const int j = __builtin_ctz(wd);
      wd &= wd - 1;
      if (o < static_cast<uint32_t>(k)) out[o] = pos0 + j;
      ++o;
    }
  };
  emit(wd0, 64 * tid);
  emit(wd1, 64 * tid + 32);
  if (tid == 0 && rr.rf.status)
    rr.rf.status[rr.t] = total == static_cast<uint32_t>(k) ? refine_status(nb, worst, eps) : -3;
}

// Top-k of one score row of n entries (entries 0..n-1 of srow) by (score desc, index asc),
// written ascending to out[0..k), -1 padded; with `refine`, by the exact scores (see the
// refine section). Called by a whole TK_THREADS block.
__device__ __forceinline__ void select_row(const float* __restrict__ srow, int64_t n, int k,
                                           int32_t* __restrict__ out, TopkLds& S,
                                           const RowRef& rr, bool refine) {
  const int tid = threadIdx.x;
  if (n <= k) {
    for (int i = tid; i < k; i += TK_THREADS) out[i] = i < n ? i : -1;
    if (refine && tid == 0 && rr.rf.status) rr.rf.status[rr.t] = 0;
    return;
  }
  if (n <= FAST_MAX) {
    const int ni = static_cast<int>(n);
    const int rc =
        n <= 16 * 64 * 8    ? select_in_registers<8>(srow, ni, k, out, S.regA, S.fhist, S.rs, S.tmp, rr, refine, S.rf_a, S.rf_s)
        : n <= 16 * 64 * 16 ? select_in_registers<16>(srow, ni, k, out, S.regA, S.fhist, S.rs, S.tmp, rr, refine, S.rf_a, S.rf_s)
                            : select_in_registers<64>(srow, ni, k, out, S.regA, S.fhist, S.rs, S.tmp, rr, refine, S.rf_a, S.rf_s);
    if (rc == REG_DONE) return;
    if (rc == REG_BAND) {
      finish_register_refine(srow, ni, k, out, rr, *reinterpret_cast<RefineLds*>(S.regA), S.tmp);
      return;
    }
    __syncthreads();  // fall back to the exact LDS path (region A and fhist are reused)
  }
  select_row_lds(srow, n, k, out, S);
  if (refine) {
    refine_prefetch(rr, n, S.rf_a, S.rf_s);
    __syncthreads();  // the block's selection stores are visible to its own loads after this
    refine_generic(srow, n, k, out, rr, *reinterpret_cast<RefineLds*>(S.regA), S.tmp, S.rf_a,
                   S.rf_s);
  }
}

// Generic refine of a row whose float32 selection is already in out[0..k) (written by this
// block): theta is the smallest selected score; one pass over the row counts the kept keys
// and collects the band; the band is rescored exactly and its best keys are merged with the
// kept ones, ascending. On a band it cannot resolve (more than BAND_CAP keys, or counts
// that disagree) the float32 selection stays and the status says why.
__device__ __forceinline__ void refine_generic(const float* __restrict__ srow, int64_t n, int k,
                                               int32_t* __restrict__ out, const RowRef& rr,
                                               RefineLds& L, uint32_t* tmp, const double* pa,
                                               const float* ps) {
  const int tid = threadIdx.x;
  int32_t* status = rr.rf.status;
  // ---- 1. theta; loads are issued eight at a time per thread ----
  constexpr int U = 8;
  float th = __builtin_inff();
  for (int i0 = tid; i0 < k; i0 += U * TK_THREADS) {
    int32_t pp[U];
#pragma unroll
    for (int u = 0; u < U; ++u) pp[u] = i0 + u * TK_THREADS < k ? out[i0 + u * TK_THREADS] : -1;
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      v[u] = __builtin_inff();
      if (pp[u] >= 0) v[u] = srow[pp[u]];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) th = fminf(th, v[u]);
  }
  if (tid < 4) L.counters[tid] = 0;
  th = static_cast<float>(-block_max_d(-static_cast<double>(th), L.redd));  // publishes counters
  const double eps = refine_eps(rr.rf, th, pa, ps);
  if (!__builtin_isfinite(th) || !__builtin_isfinite(eps)) {
    if (tid == 0 && status) status[rr.t] = -2;
    return;
  }
  float lo_f, hi_f;
  band_edges(th, eps, &lo_f, &hi_f);

  // ---- 2. kept keys (counted) and the band (collected); float4 loads, four in flight ----
  uint32_t nin = 0;
  auto classify = [&](float x, int64_t s) {
    if (x > hi_f) {
      ++nin;
    } else if (x >= lo_f) {
      const int slot = atomicAdd(&L.counters[0], 1);
      if (slot < BAND_CAP) L.band_pos[slot] = static_cast<int32_t>(s);
    }
  };
  const int64_t n4 = n / 4;
  const float4* s4 = reinterpret_cast<const float4*>(srow);  // rows are 16-byte aligned
  for (int64_t i0 = tid; i0 < n4; i0 += 4 * TK_THREADS) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i0 + u * TK_THREADS < n4) v[u] = s4[i0 + u * TK_THREADS];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + u * TK_THREADS;
      if (i < n4) {
        classify(v[u].x, 4 * i);
        classify(v[u].y, 4 * i + 1);
        classify(v[u].z, 4 * i + 2);
        classify(v[u].w, 4 * i + 3);
      }
    }
  }
  for (int64_t s = 4 * n4 + tid; s < n; s += TK_THREADS) classify(srow[s], s);
  uint32_t nin_total;
  block_excl_scan(nin, tmp, &nin_total);  // ends with a barrier: the counter is final
  const int nb = L.counters[0];
  const int need = k - static_cast<int>(nin_total);
  if (nb > BAND_CAP || need < 1 || need > nb) {  // uniform: keep the float32 selection
    if (tid == 0 && status) status[rr.t] = nb > BAND_CAP ? -1 : -2;
    return;
  }

  // ---- 3. exact rescore; 4. the best `need` band keys, ascending, in sel_pos ----
  const double worst = rescore_band(rr, srow, nb, L, false, reinterpret_cast<float*>(L.sel_pos),
                                    reinterpret_cast<float*>(L.in_pos));
  choose_band<true>(nb, need, L);

  // ---- 5. merge with the kept keys of the current (ascending) selection; k <= RF_MAXK, so
  // at most four entries per thread, taken as one contiguous run ----
  constexpr int PER = RF_MAXK / TK_THREADS;
  int32_t mine[PER];
  uint32_t cnt = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid * PER + j;
    mine[j] = -1;
    if (i < k) {
      const int32_t p = out[i];
      if (srow[p] > hi_f) {
        mine[j] = p;
        ++cnt;
      }
    }
  }
  uint32_t kept;
  uint32_t at = block_excl_scan(cnt, tmp, &kept);  // ends with a barrier
  if (kept != nin_total) {  // uniform; cannot happen for a correct float32 selection
    if (tid == 0 && status) status[rr.t] = -3;
    return;
  }
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (mine[j] >= 0) L.in_pos[at++] = mine[j];
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
  for (int i = tid; i < static_cast<int>(kept); i += TK_THREADS)
    out[i + count_below(L.sel_pos, need, L.in_pos[i])] = L.in_pos[i];
  for (int i = tid; i < need; i += TK_THREADS)
    out[i + count_below(L.in_pos, static_cast<int>(kept), L.sel_pos[i])] = L.sel_pos[i];
  if (tid == 0 && status) status[rr.t] = refine_status(nb, worst, eps);
}

// ---------------------------------------------------------------------------------------
// Long-row refine. Rows longer than FAST_MAX (up to LR_MAX_N positions) refine over three
// more launches after the merge, so that the band, which massive exact ties can make
// thousands of keys long, is classified and rescored by the whole GPU rather than by the
// row's one block:
//  - the merge kernel (one block per row) writes theta, eps and the band edges (LongRow);
//  - topk_band_classify_kernel (LR_CLS positions per block) counts the kept keys, writes
//    their bitmap, and appends the band's positions (unordered) to the row's band list;
//  - topk_band_rescore_kernel (one rescoring round of a row's band per block) writes the
//    exact scores and the largest |I_f32 - I_exact|;
//  - topk_band_finish_kernel (one block per row) picks the best `need` band keys by a radix
//    select on (exact score desc, then position asc) and writes the kept and the chosen keys
//    in ascending position order through LDS position bitmaps (the kept bitmap from the
//    classify stage, so the float32 selection is not read again).
// Longer rows keep the single-block refine (refine_generic) in the merge kernel.
constexpr int64_t LR_MAX_N = int64_t{1} << 18;  // positions the finishing bitmaps cover
constexpr int LR_CLS = 16384;                   // positions classified per block
constexpr int LR_KPR_MIN = 32;                  // band keys per rescoring block at 128 heads
// Rescoring rounds per block: a block's first round waits on a chain of dependent loads
// (band positions, then scattered key rows, scales and scores) that costs several times a
// later round, whose key codes load during the previous one, so a block takes five.
constexpr int LR_ROUNDS = 5;
constexpr int LR_RESCORE_X = (BAND_CAP + LR_KPR_MIN * LR_ROUNDS - 1) / (LR_KPR_MIN * LR_ROUNDS);

struct LongRow {  // per query row, in the workspace
  double eps;
  float theta, lo_f, hi_f;
  int32_t state;             // 0: the row refines on this path; otherwise it does not
  uint32_t nb;               // band keys found (atomic)
  uint32_t kept;             // keys above the band (atomic)
  unsigned long long worst;  // largest |I_f32 - I_exact| over the band, as double bits (atomic max)
  uint32_t pad[2];
};
static_assert(sizeof(LongRow) == 48, "LongRow layout");

struct LongRefine {   // kernel argument; rows == nullptr: no long-row path
  LongRow* rows;      // [T]
  int32_t* band_pos;  // [T, BAND_CAP] request-local positions
  double* band_ex;    // [T, BAND_CAP] exact scores
  uint32_t* kept;     // [T, LR_MAX_N / 32] bitmap of the keys above the band
};

// Long-row path, stage 1 (in the merge kernel, after the float32 selection): theta = the
// smallest selected score (th: this thread's share of the minimum), eps and the band edges
// go to the row's LongRow, with its counters cleared. pa / ps: refine_prefetch's partials;
// red: TK_WAVES doubles of LDS.
__device__ __forceinline__ void long_row_open(float th, const RowRef& rr, LongRow& row,
                                              const double* pa, const float* ps, double* red) {
  const int tid = threadIdx.x;
  th = static_cast<float>(-block_max_d(-static_cast<double>(th), red));
  const double eps = refine_eps(rr.rf, th, pa, ps);
  if (tid != 0) return;
  row.nb = 0;
  row.kept = 0;
  row.worst = 0;
  if (!__builtin_isfinite(th) || !__builtin_isfinite(eps)) {
    row.state = 2;
    if (rr.rf.status) rr.rf.status[rr.t] = -2;
    return;
  }
  float lo_f, hi_f;
  band_edges(th, eps, &lo_f, &hi_f);
  row.eps = eps;
  row.theta = th;
  row.lo_f = lo_f;
  row.hi_f = hi_f;
  row.state = 0;
}

__device__ __forceinline__ RowRef row_ref(const Refine& rf, int64_t t, int b, int64_t kv_base) {
  RowRef rr;
  rr.rf = rf;
  rr.t = t;
  rr.b = b;
  rr.kv_base = kv_base;
  return rr;
}

// One block per row: rows of up to FAST_MAX visible scores, and every row when the grid
// has no chunk stage.
__global__ __launch_bounds__(TK_THREADS) void topk_kernel(const float* __restrict__ scores,
                                                          int64_t ld,
                                                          const int32_t* __restrict__ q_off,
                                                          const int64_t* __restrict__ kv_off,
                                                          int k, int32_t* __restrict__ topk,
                                                          Refine rf) {
  __shared__ __attribute__((aligned(16))) TopkLds S;
  const int b = blockIdx.y, r = blockIdx.x;
  const RowInfo ri = load_row_info(q_off, kv_off, b);
  if (r >= ri.R) return;
  const int64_t t = ri.t0 + r;
  int64_t n = visible_count(ri, r);
  if (n > ld) n = ld;  // device lengths beyond the score stride are clipped
  select_row(scores + t * ld, n, k, topk + t * k, S, row_ref(rf, t, b, ri.kv_base),
             rf.q_fp8 != nullptr);
}

// Grids with rows longer than FAST_MAX, stage 1: block (chunk c, row) selects the top-k of
// visible positions [c FAST_MAX, (c+1) FAST_MAX) as chunk-local indices into widx
// [T, nchunk, k] and their scores into the row's candidate scores cand_s (chunk c at
// offset c k; -inf where the index is -1). Every key of the row's float32 top-k is in the
// top-k of its chunk. A row of at most FAST_MAX positions is finished here by its chunk-0
// block (refine included).
__global__ __launch_bounds__(TK_THREADS) void topk_chunk_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ q_off,
    const int64_t* __restrict__ kv_off, int k, int nchunk, int64_t cstride,
    int32_t* __restrict__ widx, float* __restrict__ cand_s, int32_t* __restrict__ topk,
    Refine rf) {
  __shared__ __attribute__((aligned(16))) TopkLds S;
  const int b = blockIdx.y, r = blockIdx.x / nchunk, c = blockIdx.x % nchunk;
  const RowInfo ri = load_row_info(q_off, kv_off, b);
  if (r >= ri.R) return;
  const int64_t t = ri.t0 + r;
  int64_t n = visible_count(ri, r);
  if (n > ld) n = ld;
  const float* srow = scores + t * ld;
  const RowRef rr = row_ref(rf, t, b, ri.kv_base);
  if (n <= FAST_MAX) {
    if (c == 0) select_row(srow, n, k, topk + t * k, S, rr, rf.q_fp8 != nullptr);
    return;
  }
  const int64_t c0 = static_cast<int64_t>(c) * FAST_MAX;
  if (c0 >= n) return;  // the merge reads only the chunks holding visible positions
  const int64_t nc = n - c0 < FAST_MAX ? n - c0 : FAST_MAX;
  int32_t* o = widx + (t * nchunk + c) * k;
  select_row(srow + c0, nc, k, o, S, rr, false);
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
// position, and a -inf pad follows every visible -inf. The refine then reads the row itself.
__global__ __launch_bounds__(TK_THREADS) void topk_merge_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ q_off,
    const int64_t* __restrict__ kv_off, int64_t ld, int k, int nchunk, int64_t cstride,
    const int32_t* __restrict__ widx, const float* __restrict__ cand_s,
    int32_t* __restrict__ topk, Refine rf, LongRefine lr) {
  __shared__ __attribute__((aligned(16))) TopkLds S;
  const int b = blockIdx.y, r = blockIdx.x;
  const RowInfo ri = load_row_info(q_off, kv_off, b);
  if (r >= ri.R) return;
  const int64_t t = ri.t0 + r;
  int64_t n = visible_count(ri, r);
  if (n > ld) n = ld;
  if (n <= FAST_MAX) return;
  const int64_t m = (n + FAST_MAX - 1) / FAST_MAX * k;  // this row's chunks
  int32_t* out = topk + t * k;
  const RowRef rr = row_ref(rf, t, b, ri.kv_base);
  // the refine's query-side loads overlap the selection (its partials stay in rf_a / rf_s)
  if (rf.q_fp8 != nullptr) refine_prefetch(rr, n, S.rf_a, S.rf_s);
  const float* crow = cand_s + t * cstride;
  select_row(crow, m, k, out, S, rr, false);
  __syncthreads();
  // candidate indices -> positions; theta's share of this thread from the candidates'
  // scores (loaded in the same round as their positions)
  const int32_t* wrow = widx + t * nchunk * k;
  float th = __builtin_inff();
  for (int i = threadIdx.x; i < k; i += TK_THREADS) {
    const int32_t j = out[i];
    if (j >= 0) {
      out[i] = (j / k) * FAST_MAX + wrow[j];
      th = fminf(th, crow[j]);
    }
  }
  if (rf.q_fp8 != nullptr) {
    __syncthreads();
    if (lr.rows != nullptr && n <= LR_MAX_N) {
      long_row_open(th, rr, lr.rows[t], S.rf_a, S.rf_s, reinterpret_cast<double*>(S.regA));
    } else {
      if (lr.rows != nullptr && threadIdx.x == 0) lr.rows[t].state = 1;
      refine_generic(scores + t * ld, n, k, out, rr, *reinterpret_cast<RefineLds*>(S.regA), S.tmp,
                     S.rf_a, S.rf_s);
    }
  }
}

// Long-row path, stage 2 (every position chunk of every long row): the kept keys are
// counted and marked in the row's kept bitmap, the band's positions appended to its list.
__global__ __launch_bounds__(TK_THREADS) void topk_band_classify_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ q_off,
    const int64_t* __restrict__ kv_off, int64_t ld, int ncls, LongRefine lr) {
  __shared__ int32_t bpos[LR_CLS];
  __shared__ uint32_t kbits[LR_CLS / 32];  // this block's words of the kept bitmap
  __shared__ uint32_t cnt[2], base_s;
  const int c = static_cast<int>(blockIdx.x) % ncls, r = static_cast<int>(blockIdx.x) / ncls;
  const int b = blockIdx.y;
  const RowInfo ri = load_row_info(q_off, kv_off, b);
  if (r >= ri.R) return;
  const int64_t t = ri.t0 + r;
  int64_t n = visible_count(ri, r);
  if (n > ld) n = ld;
  if (n <= FAST_MAX || n > LR_MAX_N) return;
  const LongRow& row = lr.rows[t];
  if (row.state != 0) return;
  const int64_t c0 = static_cast<int64_t>(c) * LR_CLS;
  if (c0 >= n) return;
  const int nc = static_cast<int>(n - c0 < LR_CLS ? n - c0 : LR_CLS);
  const float lo_f = row.lo_f, hi_f = row.hi_f;
  const int tid = threadIdx.x;
  if (tid < 2) cnt[tid] = 0;
  for (int w = tid; w < LR_CLS / 32; w += TK_THREADS) kbits[w] = 0u;
  __syncthreads();
  const float* srow = scores + t * ld + c0;
  uint32_t kept = 0;
  auto classify = [&](float x, int i) {
    if (x > hi_f) {
      ++kept;
      atomicOr(&kbits[i >> 5], 1u << (i & 31));
    } else if (x >= lo_f) {
      bpos[atomicAdd(&cnt[0], 1u)] = static_cast<int32_t>(c0 + i);
    }
  };
  constexpr int PER = LR_CLS / 4 / TK_THREADS;  // float4 loads per thread, all in flight
  const int n4 = nc / 4;
  float4 v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = tid + u * TK_THREADS;
    v[u] = i < n4 ? reinterpret_cast<const float4*>(srow)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = tid + u * TK_THREADS;
    if (i < n4) {
      classify(v[u].x, 4 * i);
      classify(v[u].y, 4 * i + 1);
      classify(v[u].z, 4 * i + 2);
      classify(v[u].w, 4 * i + 3);
    }
  }
  if (tid < nc - 4 * n4) classify(srow[4 * n4 + tid], 4 * n4 + tid);
  kept = wave_sum(kept);
  if (tid % 64 == 0 && kept) atomicAdd(&cnt[1], kept);
  __syncthreads();
  LongRow& rw = lr.rows[t];
  if (tid == 0) {
    base_s = cnt[0] ? atomicAdd(&rw.nb, cnt[0]) : 0u;
    if (cnt[1]) atomicAdd(&rw.kept, cnt[1]);
  }
  __syncthreads();
  int32_t* dst = lr.band_pos + t * BAND_CAP;
  for (uint32_t i = tid; i < cnt[0]; i += TK_THREADS)
    if (base_s + i < static_cast<uint32_t>(BAND_CAP)) dst[base_s + i] = bpos[i];
  // the block's words of the row's kept bitmap (c0 is a multiple of 32; bits past n are 0)
  uint32_t* kdst = lr.kept + t * (LR_MAX_N / 32) + c0 / 32;
  for (int w = tid; w < (nc + 31) / 32; w += TK_THREADS) kdst[w] = kbits[w];
}

// LDS of one rescoring round (the members rescore_band uses)
struct RescoreLds {
  double band_val[256 * LR_ROUNDS];
  double terms[RS_TERMS];
  uint32_t digits[256];
  int32_t band_pos[256 * LR_ROUNDS];
  double redd[TK_WAVES];
  float sk[256 * LR_ROUNDS], f32[256 * LR_ROUNDS];
};

// Long-row path, stage 3: block x rescores band keys x KR .. x KR + KR - 1 of its row, KR =
// LR_ROUNDS rounds of rescore_band (KPR = 256 / head tiles keys each; the next round's key
// codes load during the current one). Blocks are numbered piece-major: launch order
// L = x + gridDim.x y holds piece L / (rows B) of row (L % rows, request (L / rows) % B),
// so a band's first pieces, which every row has, are the first blocks dispatched and the
// blocks past a short band (which return at once) come last instead of between them.
__global__ __launch_bounds__(TK_THREADS) void topk_band_rescore_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ q_off,
    const int64_t* __restrict__ kv_off, int64_t ld, int max_q_rows, int B, Refine rf,
    LongRefine lr) {
  __shared__ __attribute__((aligned(16))) RescoreLds L;
  const int64_t lin = blockIdx.x + static_cast<int64_t>(gridDim.x) * blockIdx.y;
  const int64_t per_piece = static_cast<int64_t>(max_q_rows) * B;
  const int piece = static_cast<int>(lin / per_piece);
  const int r = static_cast<int>(lin % per_piece % max_q_rows);
  const int b = static_cast<int>(lin % per_piece / max_q_rows);
  const RowInfo ri = load_row_info(q_off, kv_off, b);
  if (r >= ri.R) return;
  const int64_t t = ri.t0 + r;
  int64_t n = visible_count(ri, r);
  if (n > ld) n = ld;
  if (n <= FAST_MAX || n > LR_MAX_N) return;
  LongRow& row = lr.rows[t];
  if (row.state != 0) return;
  const int nb = static_cast<int>(row.nb);
  if (nb > BAND_CAP) return;  // the finishing stage reports the overflow
  const int HT = rf.H <= 16 ? 1 : rf.H <= 32 ? 2 : rf.H <= 64 ? 4 : 8;
  const int KR = LR_ROUNDS * (256 / HT);
  const int base = piece * KR;
  if (base >= nb) return;
  const int cnt = nb - base < KR ? nb - base : KR;
  const int32_t* src = lr.band_pos + t * BAND_CAP + base;
  for (int i = threadIdx.x; i < cnt; i += TK_THREADS) L.band_pos[i] = src[i];
  __syncthreads();
  const double worst = rescore_band(row_ref(rf, t, b, ri.kv_base), scores + t * ld, cnt, L, false,
                                    L.sk, L.f32);
  double* ex = lr.band_ex + t * BAND_CAP + base;
  for (int i = threadIdx.x; i < cnt; i += TK_THREADS) ex[i] = L.band_val[i];
  if (threadIdx.x == 0)
    atomicMax(&row.worst, static_cast<unsigned long long>(__double_as_longlong(worst)));
}

// Order-preserving 64-bit key of a double (larger value, larger key).
__device__ __forceinline__ uint64_t order_key64(double x) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x == 0.0 ? 0.0 : x));
  return (u >> 63) ? ~u : (u | (uint64_t{1} << 63));
}

struct FinishLds {
  uint64_t key[BAND_CAP];
  int32_t pos[BAND_CAP];
  uint32_t sel[LR_MAX_N / 32];   // positions taken
  uint32_t tie[LR_MAX_N / 32];   // band positions tied with the selection's last exact score
  uint32_t hist[256];
  uint64_t kmin[TK_WAVES], kmax[TK_WAVES];
  uint32_t tmp[2 * TK_WAVES];
  uint64_t prefix;
  uint32_t want;
  uint32_t kept2;
};

// Ordered walk over the first nw words of a position bitmap: each thread takes a contiguous
// run of words; f(position, rank) is called for every set bit, rank = its order among them.
// Returns the number of set bits (to every thread).
template <class F>
__device__ __forceinline__ uint32_t bitmap_walk(const uint32_t* bits, int nw, uint32_t* tmp, F f) {
  const int tid = threadIdx.x;
  const int per = (nw + TK_THREADS - 1) / TK_THREADS;
  const int w0 = tid * per, w1 = w0 + per < nw ? w0 + per : nw;
  uint32_t c = 0;
  for (int w = w0; w < w1; ++w) c += static_cast<uint32_t>(__popc(bits[w]));
  uint32_t total;
  uint32_t rank = block_excl_scan(c, tmp, &total);
  for (int w = w0; w < w1; ++w) {
    uint32_t x = bits[w];
    while (x) {
      const int bit = __builtin_ctz(x);
      x &= x - 1u;
      f(32 * w + bit, rank++);
    }
  }
  return total;
}

// Long-row path, stage 4 (one block per long row).
__global__ __launch_bounds__(TK_THREADS) void topk_band_finish_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ q_off,
    const int64_t* __restrict__ kv_off, int64_t ld, int k, int32_t* __restrict__ topk,
    int32_t* __restrict__ status, LongRefine lr) {
  __shared__ __attribute__((aligned(16))) FinishLds F;
  const int r = blockIdx.x, b = blockIdx.y;
  const RowInfo ri = load_row_info(q_off, kv_off, b);
  if (r >= ri.R) return;
  const int64_t t = ri.t0 + r;
  int64_t n = visible_count(ri, r);
  if (n > ld) n = ld;
  if (n <= FAST_MAX || n > LR_MAX_N) return;
  const LongRow& row = lr.rows[t];
  if (row.state != 0) return;
  const int tid = threadIdx.x;
  const int nb = static_cast<int>(row.nb);
  const int kept = static_cast<int>(row.kept);
  const int need = k - kept;
  if (nb > BAND_CAP || need < 1 || need > nb) {  // uniform: keep the float32 selection
    if (tid == 0 && status) status[t] = nb > BAND_CAP ? -1 : -2;
    return;
  }
  int32_t* out = topk + t * k;
  const int nw = static_cast<int>((n + 31) / 32);
  // the band's keys, and the kept keys' bitmap from the classify stage (both contiguous)
  uint64_t kmin = ~uint64_t{0}, kmax = 0;
  for (int i = tid; i < nb; i += TK_THREADS) {
    const uint64_t x = order_key64(lr.band_ex[t * BAND_CAP + i]);
    F.key[i] = x;
    F.pos[i] = lr.band_pos[t * BAND_CAP + i];
    kmin = x < kmin ? x : kmin;
    kmax = x > kmax ? x : kmax;
  }
  uint32_t kc = 0;
  const uint32_t* kbits = lr.kept + t * (LR_MAX_N / 32);
  for (int w = tid; w < nw; w += TK_THREADS) {
    const uint32_t x = kbits[w];
    F.sel[w] = x;
    F.tie[w] = 0u;
    kc += static_cast<uint32_t>(__popc(x));
  }
  for (int o = 32; o >= 1; o >>= 1) {
    const uint64_t a = __shfl_xor(kmin, o), c = __shfl_xor(kmax, o);
    kmin = a < kmin ? a : kmin;
    kmax = c > kmax ? c : kmax;
  }
  kc = wave_sum(kc);
  if (tid % 64 == 0) {
    F.kmin[tid / 64] = kmin;
    F.kmax[tid / 64] = kmax;
  }
  if (tid == 0) F.kept2 = 0;
  __syncthreads();
  if (tid % 64 == 0 && kc) atomicAdd(&F.kept2, kc);
  kmin = F.kmin[0];
  kmax = F.kmax[0];
  for (int w = 1; w < TK_WAVES; ++w) {
    kmin = F.kmin[w] < kmin ? F.kmin[w] : kmin;
    kmax = F.kmax[w] > kmax ? F.kmax[w] : kmax;
  }
  // Every key shares the bytes above the highest one where the smallest and largest keys
  // differ, so the radix select starts at that byte with those bytes as its prefix; an
  // all-tied band (kmin == kmax) needs no pass.
  const uint64_t diff = kmin ^ kmax;
  const int s0 = diff ? 8 * ((63 - __builtin_clzll(diff)) / 8) : -8;
  if (tid == 0) {
    F.prefix = s0 < 0 ? kmax : s0 == 56 ? 0 : (kmax >> (s0 + 8)) << (s0 + 8);
    F.want = static_cast<uint32_t>(need);
  }
  __syncthreads();
  // the need-th largest exact key, eight bits at a time from byte s0 down: bin 255 - d
  // holds digit d, so that bin 0 holds the largest keys
  for (int shift = s0; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += TK_THREADS) F.hist[i] = 0u;
    __syncthreads();
    const uint64_t prefix = F.prefix;
    for (int i0 = 0; i0 < nb; i0 += TK_THREADS) {  // wave-aggregated: exact ties share a bin
      const int i = i0 + tid;
      const uint64_t x = i < nb ? F.key[i] : 0;
      const bool act = i < nb && (shift == 56 || (x >> (shift + 8)) == (prefix >> (shift + 8)));
      hist_add(F.hist, act, 255u - static_cast<uint32_t>((x >> shift) & 255u));
    }
    __syncthreads();
    if (tid < 64) {
      uint32_t bin = 0, above = 0;
      wave_select<256>(F.hist, F.want, &bin, &above);
      if (tid == 0) {
        F.prefix = prefix | (static_cast<uint64_t>(255u - bin) << shift);
        F.want -= above;
      }
    }
    __syncthreads();
  }
  const uint64_t thk = F.prefix;  // the need-th largest exact key; F.want of its ties are taken
  const uint32_t want = F.want;
  // band keys above it are taken, its ties wait for the position order
  for (int i = tid; i < nb; i += TK_THREADS) {
    const int32_t p = F.pos[i];
    if (F.key[i] > thk) atomicOr(&F.sel[p >> 5], 1u << (p & 31));
    else if (F.key[i] == thk) atomicOr(&F.tie[p >> 5], 1u << (p & 31));
  }
  __syncthreads();
  if (F.kept2 != static_cast<uint32_t>(kept)) {  // uniform; cannot happen for a correct selection
    if (tid == 0 && status) status[t] = -3;
    return;
  }
  // the first `want` ties in position order
  bitmap_walk(F.tie, nw, F.tmp, [&](int p, uint32_t rank) {
    if (rank < want) atomicOr(&F.sel[p >> 5], 1u << (p & 31));
  });
  __syncthreads();
  const uint32_t total = bitmap_walk(F.sel, nw, F.tmp, [&](int p, uint32_t rank) {
    if (rank < static_cast<uint32_t>(k)) out[rank] = p;
  });
  if (tid == 0 && status) {
    const double worst = __longlong_as_double(static_cast<long long>(row.worst));
    status[t] = total == static_cast<uint32_t>(k) ? refine_status(nb, worst, row.eps) : -3;
  }
}

// Refine pre-pass: kmax[b, c] = the largest |k_scale| of positions [c SC_CHUNK, (c+1)
// SC_CHUNK) of request b (0 past its keys).
__global__ __launch_bounds__(256) void topk_scale_max_kernel(const float* __restrict__ k_scale,
                                                             const int64_t* __restrict__ kv_off,
                                                             int nsc, float* __restrict__ kmax) {
  constexpr int PER = SC_CHUNK / 256;  // scales per thread, all loads issued before use
  __shared__ float red[4];
  const int c = blockIdx.x, b = blockIdx.y;
  const int64_t base = kv_off[b], L = kv_off[b + 1] - base;
  const int64_t s0 = static_cast<int64_t>(c) * SC_CHUNK + threadIdx.x;
  if (static_cast<int64_t>(c) * SC_CHUNK >= L) {  // block-uniform: no key of the request here
    if (threadIdx.x == 0) kmax[static_cast<int64_t>(b) * nsc + c] = 0.0f;
    return;
  }
  // positions past the request's end load its last scale (in bounds, unconditionally, so
  // the loads issue back to back) and are masked afterwards
  float v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int64_t s = s0 + 256 * u;
    v[u] = k_scale[base + (s < L ? s : L - 1)];
  }
  float m = 0.0f;
#pragma unroll
  for (int u = 0; u < PER; ++u) m = fmaxf(m, s0 + 256 * u < L ? fabsf(v[u]) : 0.0f);
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (threadIdx.x % 64 == 0) red[threadIdx.x / 64] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    kmax[static_cast<int64_t>(b) * nsc + c] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}



// Key-scale table kept beside the cache: kglob[c] = the largest |k_scale| of cache rows
// [c SC_CHUNK, (c+1) SC_CHUNK) below N, for chunks c0 + blockIdx.x.
__global__ __launch_bounds__(256) void key_scale_table_kernel(const float* __restrict__ k_scale,
                                                              int64_t N, int64_t c0,
                                                              float* __restrict__ kglob) {
  constexpr int PER = SC_CHUNK / 256;
  __shared__ float red[4];
  const int64_t c = c0 + blockIdx.x;
  const int64_t r0 = c * SC_CHUNK + threadIdx.x;
  float v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {  // rows past N load row N - 1 (in bounds) and are masked
    const int64_t r = r0 + 256 * u;
    v[u] = k_scale[r < N ? r : N - 1];
  }
  float m = 0.0f;
#pragma unroll
  for (int u = 0; u < PER; ++u) m = fmaxf(m, r0 + 256 * u < N ? fabsf(v[u]) : 0.0f);
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (threadIdx.x % 64 == 0) red[threadIdx.x / 64] = m;
  __syncthreads();
  if (threadIdx.x == 0) kglob[c] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// The need-th largest of the order keys key[0..PER) of every thread (entries with live false
// excluded), by the whole block: the 16-bit class (key >> 16) counted below the largest class
// (2048 bins, the last one gathering every class 2047 or more below; keys drawn from the top of
// a distribution span few classes, and bins relative to the maximum keep them apart), then
// bits 15..8 and 7..0 inside the chosen class. Adds of lanes sharing a bin are merged
// (hist_add). hist: 2048 words; tmp: 2 * TK_WAVES words; sel: 2 words; mx: 1 word. The count
// of live keys must be at least need.
template <int PER>
__device__ __forceinline__ uint32_t block_kth_largest(const uint32_t (&key)[PER], const bool (&live)[PER],
                                                      uint32_t need, uint32_t* hist, uint32_t* tmp,
                                                      uint32_t* sel, uint32_t* mx) {
  const int tid = threadIdx.x;
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (live[j]) m = max(m, key[j] >> 16);
  m = wave_max(m);
  if (tid == 0) *mx = 0;
  for (int i = tid; i < 2048; i += TK_THREADS) hist[i] = 0;
  __syncthreads();
  if (tid % 64 == 0) atomicMax(mx, m);
  __syncthreads();
  const uint32_t top = *mx;
  // round 1: classes below the top, bin 2047 - d (the histogram ascends in key order)
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const uint32_t d = top - (key[j] >> 16);
    hist_add(hist, live[j], 2047u - (d < 2047u ? d : 2047u));
  }
  __syncthreads();
  select_bin(hist, 2048, need, tmp, sel);
  const uint32_t d1 = 2047u - sel[0];
  need -= sel[1];
  __syncthreads();
  // a class 2047 or more below the top gathers several classes in its bin: fall back to
  // the plain 16-bit class digit there (rare: a row spanning that many classes)
  const bool gathered = d1 == 2047u;
  uint32_t c16 = top - d1;
  if (gathered) {
    for (int i = tid; i < 2048; i += TK_THREADS) hist[i] = 0;
    __syncthreads();
    // the classes at or below top - 2047, by their top 11 bits relative to class 0
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const uint32_t c = key[j] >> 16;
      hist_add(hist, live[j] && top - c >= 2047u, c >> 5);
    }
    __syncthreads();
    select_bin(hist, 2048, need, tmp, sel);
    const uint32_t hi11 = sel[0];
    need -= sel[1];
    __syncthreads();
    for (int i = tid; i < 32; i += TK_THREADS) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const uint32_t c = key[j] >> 16;
      hist_add(hist, live[j] && top - c >= 2047u && (c >> 5) == hi11, c & 31u);
    }
    __syncthreads();
    select_bin(hist, 32, need, tmp, sel);
    c16 = (hi11 << 5) | sel[0];
    need -= sel[1];
    __syncthreads();
  }
  // rounds 2 and 3: bits 15..8, then 7..0, of the keys in class c16
  uint32_t prefix = c16;
#pragma unroll
  for (int round = 0; round < 2; ++round) {
    const int sh = round == 0 ? 8 : 0;
    for (int i = tid; i < 256; i += TK_THREADS) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PER; ++j)
      hist_add(hist, live[j] && (key[j] >> (sh + 8)) == prefix, (key[j] >> sh) & 255u);
    __syncthreads();
    select_bin(hist, 256, need, tmp, sel);
    prefix = (prefix << 8) | sel[0];
    need -= sel[1];
    __syncthreads();
  }
  return prefix;
}

// ---------------------------------------------------------------------------------------
// Fused scoring and selection (dsa_index_topk). dsa_index_score's kernel first scores S
// evenly spaced keys per request; sample_tau_kernel turns each row's sample into a threshold
// tau expected to leave about 2.5 k keys above it; the scoring kernel then keeps only
// the scores >= tau, and fused_select_kernel selects from those candidates with the
// exact-boundary refine. A row whose candidates cannot be trusted to hold its top-k and
// band (fewer than k, more than CCAP, or theta - 2 eps below tau) is scored again by its own
// block and selected by the standard path, so every row's set is exact.
constexpr int CCAP = 8192;      // candidates a row's block selects from in LDS
constexpr int MAX_SEGS = 1024;  // key ranges one row's candidates may come from

// 1 block per row: tau[t] = the sample's m-th largest score, m = ceil(2.5 k S / n0) (n0 the
// sampled span), or -inf when that leaves no sample out (the row keeps every key).
__global__ __launch_bounds__(TK_THREADS) void sample_tau_kernel(
    const float* __restrict__ samples, int S, const int32_t* __restrict__ q_off,
    const int64_t* __restrict__ kv_off, int k, float* __restrict__ tau) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t tmp[2 * TK_WAVES];
  __shared__ uint32_t sel[2];
  const int b = blockIdx.y, r = blockIdx.x;
  const RowInfo ri = load_row_info(q_off, kv_off, b);
  if (r >= ri.R) return;
  const int64_t t = ri.t0 + r;
  const int tid = threadIdx.x;
  int64_t n0 = ri.L - ri.R + 1;
  n0 = n0 < 1 ? 1 : (n0 > ri.L ? ri.L : n0);
  const int64_t m = (5 * static_cast<int64_t>(k) * S + 2 * n0 - 1) / (2 * n0);
  if (ri.L <= 0 || m >= S) {
    if (tid == 0) tau[t] = -__builtin_inff();
    return;
  }
  constexpr int PER = 8;  // S <= 8192
  uint32_t key[PER];
  bool live[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid + TK_THREADS * j;
    live[j] = i < S;
    key[j] = live[j] ? order_key(samples[t * S + i]) : 0u;
  }
  __shared__ uint32_t mx;
  const uint32_t prefix = block_kth_largest<PER>(key, live, static_cast<uint32_t>(m), hist, tmp, sel, &mx);
  if (tid == 0) tau[t] = __uint_as_float((prefix & 0x80000000u) ? (prefix & 0x7FFFFFFFu) : ~prefix);
}

// Scores of the row of rr (its n visible keys) into frow by the whole block, with the FP8
// MFMA and float32 epilogue of dsa_index_score (one 16-key sub-tile per wave at a time, the
// query operand reloaded per head tile); the largest visible key scale goes to *smax.
__device__ __forceinline__ void score_row_block(const RowRef& rr, int64_t n, float* __restrict__ frow,
                                                float* smax, double* red) {
  const Refine& rf = rr.rf;
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int g = lane / 16, c16 = lane % 16;
  const int H = rf.H, D = rf.D;
  const int nht = (H + 15) / 16;
  const int64_t t = rr.t;
  const uint8_t* __restrict__ kreq = rf.k_fp8 + rr.kv_base * D;
  const float* __restrict__ ksc = rf.k_scale + rr.kv_base;
  float sm = 0.0f;
  for (int64_t s0 = 16 * wave; s0 < n; s0 += 16 * TK_WAVES) {
    const int64_t key = s0 + c16;
    const bool valid = key < n;
    i32x8 bfrag = {0, 0, 0, 0, 0, 0, 0, 0};
    if (valid && 32 * g < D) {
      const i32x4* p = reinterpret_cast<const i32x4*>(kreq + key * D + 32 * g);
      const i32x4 lo = p[0], hi = p[1];
      bfrag = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    float part = 0.0f;
    for (int ht = 0; ht < nht; ++ht) {  // wave-uniform
      const int head = 16 * ht + c16;
      i32x8 qa = {0, 0, 0, 0, 0, 0, 0, 0};
      if (head < H && 32 * g < D) {
        const i32x4* p = reinterpret_cast<const i32x4*>(rf.q_fp8 + (t * H + head) * D + 32 * g);
        const i32x4 lo = p[0], hi = p[1];
        qa = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      const f32x4 acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa, bfrag, zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h2 = 16 * ht + 4 * g + i;
        const float u = h2 < H ? rf.w[t * H + h2] * rf.q_scale[t * H + h2] : 0.0f;
        part = fmaf(u, __builtin_amdgcn_fmed3f(acc[i], 0.0f, 3.402823466e38f), part);
      }
    }
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    if (g == 0 && valid) {
      const float sc = ksc[key];
      frow[key] = part * sc;
      sm = fmaxf(sm, sc);
    }
  }
  const double mx = block_max_d(static_cast<double>(sm), red);
  *smax = static_cast<float>(mx);
}

struct FusedSel {  // kernel argument of fused_select_kernel
  uint2* cand;          // [T, ldc] candidates from the scoring kernel (then a fallback row)
  int64_t ldc;
  const int32_t* cnt;   // [T, gx, 2]
  const float* msc;     // [T, gx, 2]
  const float* tau;     // [T]
  int32_t* path;        // [T] or nullptr: 0 selected from the candidates, 1 row rescored
  int gx;
};

// Ascending emission of the kept positions (kept_pos, any order) and the chosen band
// positions (sel_pos, ascending) of a row of n positions, in windows of FAST_MAX positions
// through the position bitmap.
__device__ __forceinline__ void emit_selected(int64_t n, int k, int32_t* __restrict__ out,
                                              const int32_t* kept_pos, int nkept,
                                              const int32_t* sel_pos, int nsel, RefineLds& L,
                                              uint32_t* tmp) {
  const int tid = threadIdx.x;
  uint32_t done = 0;
  for (int64_t w0 = 0; w0 < n; w0 += FAST_MAX) {  // block-uniform
    for (int i = tid; i < FAST_MAX / 32; i += TK_THREADS) L.bitmap[i] = 0u;
    __syncthreads();
    auto mark = [&](int32_t p) {
      if (p >= w0 && p < w0 + FAST_MAX) {
        const int q = static_cast<int>(p - w0);
        atomicOr(&L.bitmap[q >> 5], 1u << (q & 31));
      }
    };
    for (int i = tid; i < nkept; i += TK_THREADS) mark(kept_pos[i]);
    for (int i = tid; i < nsel; i += TK_THREADS) mark(sel_pos[i]);
    __syncthreads();
    const uint32_t wd0 = L.bitmap[2 * tid], wd1 = L.bitmap[2 * tid + 1];
    uint32_t total;
    uint32_t o = done + block_excl_scan(static_cast<uint32_t>(__popc(wd0) + __popc(wd1)), tmp, &total);
    auto emit = [&](uint32_t wd, int64_t pos0) {
      while (wd) {
        const int j = __builtin_ctz(wd);
        wd &= wd - 1;
        if (o < static_cast<uint32_t>(k)) out[o] = static_cast<int32_t>(pos0 + j);
        ++o;
      }
    };
    emit(wd0, w0 + 64 * tid);
    emit(wd1, w0 + 64 * tid + 32);
    done += total;
  }
  for (uint32_t i = done + tid; i < static_cast<uint32_t>(k); i += TK_THREADS) out[i] = -1;
}

__global__ __launch_bounds__(TK_THREADS) void fused_select_kernel(
    FusedSel fs, Refine rf, const int32_t* __restrict__ q_off, const int64_t* __restrict__ kv_off,
    int B, int k, int32_t* __restrict__ topk) {
  __shared__ __attribute__((aligned(16))) TopkLds S;
  const int b = blockIdx.y, r = blockIdx.x;
  const RowInfo ri = load_row_info(q_off, kv_off, b);
  if (r >= ri.R) return;
  const int64_t t = ri.t0 + r;
  int64_t n = visible_count(ri, r);
  if (n > fs.ldc) n = fs.ldc;  // device lengths beyond the host bound are clipped
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  int32_t* out = topk + t * k;
  RowRef rr = row_ref(rf, t, b, ri.kv_base);
  if (n <= k) {  // every visible key is selected
    for (int i = tid; i < k; i += TK_THREADS) out[i] = i < n ? i : -1;
    if (tid == 0) {
      if (rf.status) rf.status[t] = 0;
      if (fs.path) fs.path[t] = 0;
    }
    return;
  }
  RefineLds& L = *reinterpret_cast<RefineLds*>(S.regA);
  // candidate keys and positions overlay band_val / terms, which the rescoring uses only
  // after the candidates have been classified
  uint32_t* ckey = reinterpret_cast<uint32_t*>(L.band_val);
  int32_t* cpos = reinterpret_cast<int32_t*>(L.terms);
  static_assert(sizeof(L.band_val) >= CCAP * 4 && sizeof(L.terms) >= CCAP * 4, "candidate arrays");
  int* seg_k0 = S.fpos;  // per key range of the row: first key, end, the two counts, offset
  int* seg_ke = S.fpos + MAX_SEGS;
  int* seg_c0 = S.fpos + 2 * MAX_SEGS;
  int* seg_c1 = S.fpos + 3 * MAX_SEGS;
  int* seg_of = S.fpos + 4 * MAX_SEGS;
  static_assert(5 * MAX_SEGS <= FCAND, "segment table");
  bool fallback = false;
  float eps_f = 0.0f;
  // ---- 1. the row's key ranges in the scoring grid, their counts and key-scale maxima ----
  const int64_t base = kv_off[0], end = kv_off[B];
  int64_t share = (end - base + fs.gx - 1) / fs.gx;
  share = (share + 63) / 64 * 64;
  const int64_t x0 = (ri.kv_base - base) / share;
  const int64_t x1 = (ri.kv_base + ri.L - 1 - base) / share;
  const int nseg = static_cast<int>(x1 - x0 + 1);
  if (nseg > MAX_SEGS || nseg < 1) fallback = true;  // uniform
  uint32_t C = 0;
  float sm = 0.0f;
  if (!fallback) {
    uint32_t c = 0;
    int sk0 = 0, ske = 0, sc0 = 0, sc1 = 0;
    if (tid < nseg) {
      const int64_t x = x0 + tid;
      const int64_t g0 = base + x * share, g1 = g0 + share < end ? g0 + share : end;
      const int64_t k0 = (g0 > ri.kv_base ? g0 : ri.kv_base) - ri.kv_base;
      int64_t ke = (g1 < ri.kv_base + ri.L ? g1 : ri.kv_base + ri.L) - ri.kv_base;
      if (ke > fs.ldc) ke = fs.ldc;
      if (ke > k0) {
        const int64_t m = (t * fs.gx + x) * 2;
        sk0 = static_cast<int>(k0);
        ske = static_cast<int>(ke);
        sc0 = fs.cnt[m];
        sc1 = fs.cnt[m + 1];
        sm = fmaxf(fs.msc[m], fs.msc[m + 1]);
        c = static_cast<uint32_t>(sc0 + sc1);
      }
    }
    const uint32_t off = block_excl_scan(c, S.tmp, &C);
    if (tid < nseg) {
      seg_k0[tid] = sk0;
      seg_ke[tid] = ske;
      seg_c0[tid] = sc0;
      seg_c1[tid] = sc1;
      seg_of[tid] = static_cast<int>(off);
    }
    if (C > static_cast<uint32_t>(CCAP) || C < static_cast<uint32_t>(k)) fallback = true;
  }
  const float smax = static_cast<float>(block_max_d(static_cast<double>(sm), L.redd));
  uint32_t theta = 0;
  if (!fallback) {
    // ---- 2. candidates into LDS: wave w copies the ranges w, w + 16, .. ----
    for (int sgi = wave; sgi < nseg; sgi += TK_WAVES) {
      const uint2* crow = fs.cand + t * fs.ldc;
      const int c0 = seg_c0[sgi], c1 = seg_c1[sgi], o = seg_of[sgi];
      const int k0 = seg_k0[sgi], ke = seg_ke[sgi];
      for (int i = lane; i < c0 + c1; i += 64) {
        const uint2 e = i < c0 ? crow[k0 + i] : crow[ke - 1 - (i - c0)];
        ckey[o + i] = order_key(__uint_as_float(e.x));
        cpos[o + i] = static_cast<int32_t>(e.y);
      }
    }
    // ---- 3. theta: the k-th largest candidate key ----
    __syncthreads();  // the candidates are in LDS
    constexpr int PERC = CCAP / TK_THREADS;
    uint32_t key[PERC];
    bool live[PERC];
#pragma unroll
    for (int j = 0; j < PERC; ++j) {
      const uint32_t i = tid + TK_THREADS * j;
      live[j] = i < C;
      key[j] = live[j] ? ckey[i] : 0u;
    }
    theta = block_kth_largest<PERC>(key, live, static_cast<uint32_t>(k), S.fhist, S.tmp, S.sel,
                                    &S.smax);
  }
  // ---- 4. eps, and whether every key of the band is among the candidates ----
  double eps = 0.0;
  float lo_f = 0.0f, hi_f = 0.0f;
  if (!fallback) {
    const float th = __uint_as_float((theta & 0x80000000u) ? (theta & 0x7FFFFFFFu) : ~theta);
    rr.rf.kmax = nullptr;
    rr.rf.smax_given = smax;
    refine_prefetch(rr, n, S.rf_a, S.rf_s);
    if (tid < 4) L.counters[tid] = 0;
    __syncthreads();
    eps = refine_eps(rr.rf, th, S.rf_a, S.rf_s);
    if (!__builtin_isfinite(th) || !__builtin_isfinite(eps)) {
      fallback = true;
    } else {
      band_edges(th, eps, &lo_f, &hi_f);
      if (lo_f < fs.tau[t]) fallback = true;  // keys in the band may have been left out
    }
    eps_f = static_cast<float>(eps);
  }
  int nb = 0, nkept = 0;
  if (!fallback) {
    // ---- 5. kept keys (above the band) and the band ----
    const uint32_t lo_k = order_key(lo_f), hi_k = order_key(hi_f);
    for (uint32_t i0 = 0; i0 < C; i0 += TK_THREADS) {  // block-uniform trips
      const uint32_t i = i0 + tid;
      const bool live = i < C;
      const uint32_t key = live ? ckey[i] : 0u;
      const bool kp = live && key > hi_k;
      const bool bd = live && !kp && key >= lo_k;
      const uint64_t bkp = __builtin_amdgcn_ballot_w64(kp), bbd = __builtin_amdgcn_ballot_w64(bd);
      int basek = 0, baseb = 0;
      if (lane == 0) {
        if (bkp) basek = atomicAdd(&L.counters[1], static_cast<int>(__popcll(bkp)));
        if (bbd) baseb = atomicAdd(&L.counters[0], static_cast<int>(__popcll(bbd)));
      }
      basek = __builtin_amdgcn_readfirstlane(basek);
      baseb = __builtin_amdgcn_readfirstlane(baseb);
      if (kp) {
        const int slot = basek + static_cast<int>(lanes_below(bkp));
        if (slot < RF_MAXK) L.in_pos[slot] = cpos[i];
      }
      if (bd) {
        const int slot = baseb + static_cast<int>(lanes_below(bbd));
        if (slot < BAND_CAP) {
          L.band_pos[slot] = cpos[i];
          reinterpret_cast<float*>(S.fpos)[slot] = __uint_as_float(
              (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);  // its float32 score
        }
      }
    }
    __syncthreads();
    nb = L.counters[0];
    nkept = L.counters[1];
    const int need = k - nkept;
    if (nb > BAND_CAP || need < 1 || need > nb) fallback = true;  // uniform
  }
  if (!fallback) {
    // ---- 6. exact rescore of the band, its best keys, and the ascending emission ----
    const int need = k - nkept;
    const double worst = rescore_band(rr, nullptr, nb, L, false, reinterpret_cast<float*>(L.sel_pos),
                                      reinterpret_cast<float*>(S.fpos));
    choose_band<true>(nb, need, L);
    emit_selected(n, k, out, L.in_pos, nkept, L.sel_pos, need, L, S.tmp);
    if (tid == 0) {
      if (rf.status) rf.status[t] = refine_status(nb, worst, eps);
      if (fs.path) fs.path[t] = 0;
    }
    return;
  }
  // ---- fallback: score the whole row here, then the standard selection and refine ----
  __syncthreads();
  float* frow = reinterpret_cast<float*>(fs.cand + t * fs.ldc);  // this row's own slice
  float fsmax;
  score_row_block(rr, n, frow, &fsmax, L.redd);
  __syncthreads();  // the block's score stores are visible to its own loads after this
  rr.rf.kmax = nullptr;
  rr.rf.smax_given = fsmax;
  select_row(frow, n, k, out, S, rr, true);
  if (tid == 0 && fs.path) fs.path[t] = 1;
  (void)eps_f;
}
}  // namespace
}  // namespace dsa

namespace dsa {
namespace {
// Chunks of rows longer than FAST_MAX, and the stride of the compact candidate rows.
int64_t topk_nchunk(int64_t max_kv_len) { return max_kv_len > FAST_MAX ? ceil_div(max_kv_len, FAST_MAX) : 1; }
int64_t topk_cstride(int64_t nchunk, int k) { return (nchunk * k + 3) / 4 * 4; }
// Bytes of the chunk stage (16-byte multiple); the refine's scale maxima follow.
int64_t topk_chunk_bytes(int32_t T, int64_t max_kv_len, int32_t k) {
  const int64_t nc = topk_nchunk(max_kv_len);
  if (nc <= 1) return 0;
  // chunk indices [T, nc, k] (padded to 16 bytes), then candidate scores [T, cstride]
  return ((static_cast<int64_t>(T) * nc * k + 3) / 4 * 4 + static_cast<int64_t>(T) * topk_cstride(nc, k)) * 4;
}
int64_t topk_nsc(int64_t max_kv_len) { return max_kv_len > 0 ? ceil_div(max_kv_len, SC_CHUNK) : 1; }
// Bytes of the refine's scale maxima (16-byte multiple).
int64_t topk_kmax_bytes(int32_t B, int64_t max_kv_len) {
  return (static_cast<int64_t>(B) * topk_nsc(max_kv_len) * 4 + 15) / 16 * 16;
}
// Bytes of the long-row refine: LongRow[T], band positions [T, BAND_CAP], exact scores
// [T, BAND_CAP] and the kept keys' bitmaps [T, LR_MAX_N / 32] (grids with rows longer than
// FAST_MAX only).
int64_t topk_long_bytes(int32_t T, int64_t max_kv_len) {
  if (topk_nchunk(max_kv_len) <= 1) return 0;
  return static_cast<int64_t>(T) *
         (static_cast<int64_t>(sizeof(LongRow)) + BAND_CAP * (4 + 8) + LR_MAX_N / 32 * 4);
}
}  // namespace
}  // namespace dsa

extern "C" size_t dsa_topk_workspace_size(int32_t B, int32_t T, int64_t max_kv_len, int32_t k,
                                          int32_t refine) {
  using namespace dsa;
  if (B <= 0 || T <= 0 || k <= 0 || max_kv_len < 0) return 0;
  int64_t bytes = topk_chunk_bytes(T, max_kv_len, k);
  if (refine) bytes += topk_kmax_bytes(B, max_kv_len) + topk_long_bytes(T, max_kv_len);
  return static_cast<size_t>(bytes);
}

extern "C" dsa_status dsa_key_scale_max(const float* k_scale, int64_t N, int64_t row_begin,
                                        int64_t row_end, float* k_scale_max, void* stream) {
  using namespace dsa;
  DSA_REQUIRE(N >= 0 && row_begin >= 0 && row_begin <= row_end && row_end <= N,
              "dsa_key_scale_max: need 0 <= row_begin <= row_end <= N");
  if (row_begin == row_end) return ok();
  DSA_REQUIRE(k_scale && k_scale_max, "dsa_key_scale_max: null pointer");
  DSA_REQUIRE((reinterpret_cast<uintptr_t>(k_scale_max) & 3) == 0 &&
                  (reinterpret_cast<uintptr_t>(k_scale) & 3) == 0,
              "dsa_key_scale_max: k_scale and k_scale_max must be 4-byte aligned");
  const int64_t c0 = row_begin / SC_CHUNK, c1 = (row_end - 1) / SC_CHUNK;
  DSA_REQUIRE(c1 - c0 < 0x7FFFFFFF, "dsa_key_scale_max: too many rows");
  hipLaunchKernelGGL(key_scale_table_kernel, dim3(static_cast<unsigned>(c1 - c0 + 1)), dim3(256), 0,
                     as_stream(stream), k_scale, N, c0, k_scale_max);
  return check_launch("dsa_key_scale_max");
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
    DSA_REQUIRE((reinterpret_cast<uintptr_t>(refine->q_fp8) & 15) == 0 &&
                    (reinterpret_cast<uintptr_t>(refine->k_fp8) & 15) == 0,
                "dsa_topk: refine q_fp8 and k_fp8 must be 16-byte aligned");
    DSA_REQUIRE(k <= RF_MAXK, "dsa_topk: the refine supports k <= %d (got %d)", RF_MAXK, k);
    DSA_REQUIRE(refine->D_I == 64 || refine->D_I == 128, "dsa_topk: refine D_I must be 64 or 128");
    DSA_REQUIRE(refine->H_I >= 1 && refine->H_I <= 128, "dsa_topk: refine H_I must be in [1, 128]");
    DSA_REQUIRE(refine->err_scale >= 0.0 && refine->err_scale < 1e30,
                "dsa_topk: refine err_scale must be in [0, 1e30)");
    DSA_REQUIRE(!refine->k_scale_max || refine->k_scale_max_len >= 1,
                "dsa_topk: refine k_scale_max needs k_scale_max_len >= 1");
    DSA_REQUIRE((reinterpret_cast<uintptr_t>(refine->k_scale_max) & 3) == 0,
                "dsa_topk: refine k_scale_max must be 4-byte aligned");
  }
  if (B == 0 || T == 0 || max_q_rows == 0) return ok();
  DSA_REQUIRE(scores && q_row_offsets && kv_row_offsets && topk, "dsa_topk: null pointer");
  DSA_REQUIRE(!refine || (refine->q_fp8 && refine->q_scale && refine->w && refine->k_fp8 &&
                          refine->k_scale),
              "dsa_topk: null refine pointer");
  DSA_REQUIRE((reinterpret_cast<uintptr_t>(scores) & 15) == 0,
              "dsa_topk: scores must be 16-byte aligned");
  DSA_REQUIRE(B <= 65535, "dsa_topk: B must be <= 65535");
  const size_t need = dsa_topk_workspace_size(B, T, max_kv_len, k, refine ? 1 : 0);
  if (need && (ws_bytes < need || !ws))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "dsa_topk: the workspace needs %zu bytes (got %zu)",
                need, ws_bytes);
  DSA_REQUIRE(!need || (reinterpret_cast<uintptr_t>(ws) & 15) == 0,
              "dsa_topk: ws must be 16-byte aligned");
  const int64_t nchunk = topk_nchunk(max_kv_len);
  DSA_REQUIRE(max_q_rows * nchunk <= 0x7FFFFFFF, "dsa_topk: too many chunks");
  DSA_REQUIRE(static_cast<int64_t>(max_q_rows) * (LR_MAX_N / LR_CLS > LR_RESCORE_X ? LR_MAX_N / LR_CLS
                                                                                 : LR_RESCORE_X) <= 0x7FFFFFFF,
              "dsa_topk: max_q_rows too large");
  const int64_t chunk_bytes = topk_chunk_bytes(T, max_kv_len, k);
  hipStream_t st = as_stream(stream);
  Refine rf{};
  LongRefine lr{nullptr, nullptr, nullptr, nullptr};
  if (refine) {
    const int64_t nsc = topk_nsc(max_kv_len);
    DSA_REQUIRE(nsc <= 65535, "dsa_topk: max_kv_len too large for the refine");
    rf.q_fp8 = refine->q_fp8;
    rf.q_scale = refine->q_scale;
    rf.w = refine->w;
    rf.k_fp8 = refine->k_fp8;
    rf.k_scale = refine->k_scale;
    rf.status = refine->status;
    rf.C = refine->err_scale;
    rf.H = refine->H_I;
    rf.D = refine->D_I;
    rf.nsc = static_cast<int>(nsc);
    if (refine->k_scale_max) {  // the caller's table: no pre-pass
      rf.kglob = refine->k_scale_max;
      rf.kglob_len = refine->k_scale_max_len;
    } else {
      rf.kmax = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + chunk_bytes);
      hipLaunchKernelGGL(topk_scale_max_kernel, dim3((unsigned)nsc, (unsigned)B), dim3(256), 0, st,
                         refine->k_scale, kv_row_offsets, (int)nsc, const_cast<float*>(rf.kmax));
    }
    if (nchunk > 1) {
      uint8_t* p = static_cast<uint8_t*>(ws) + chunk_bytes + topk_kmax_bytes(B, max_kv_len);
      lr.rows = reinterpret_cast<LongRow*>(p);
      lr.band_pos = reinterpret_cast<int32_t*>(p + static_cast<int64_t>(T) * sizeof(LongRow));
      lr.band_ex = reinterpret_cast<double*>(p + static_cast<int64_t>(T) * sizeof(LongRow) +
                                             static_cast<int64_t>(T) * BAND_CAP * 4);
      lr.kept = reinterpret_cast<uint32_t*>(p + static_cast<int64_t>(T) * sizeof(LongRow) +
                                            static_cast<int64_t>(T) * BAND_CAP * 12);
    }
  }
  dim3 grid((unsigned)max_q_rows, (unsigned)B);
  if (nchunk > 1) {
    int32_t* widx = static_cast<int32_t*>(ws);
    const int64_t cstride = topk_cstride(nchunk, k);
    float* cand_s = reinterpret_cast<float*>(widx + (static_cast<int64_t>(T) * nchunk * k + 3) / 4 * 4);
    hipLaunchKernelGGL(topk_chunk_kernel, dim3((unsigned)(max_q_rows * nchunk), (unsigned)B),
                       dim3(TK_THREADS), 0, st, scores, score_ld, q_row_offsets, kv_row_offsets, k,
                       (int)nchunk, cstride, widx, cand_s, topk, rf);
    hipLaunchKernelGGL(topk_merge_kernel, grid, dim3(TK_THREADS), 0, st, scores, q_row_offsets,
                       kv_row_offsets, score_ld, k, (int)nchunk, cstride, widx, cand_s, topk, rf, lr);
    if (lr.rows) {
      const int64_t ncls = ceil_div(max_kv_len < LR_MAX_N ? max_kv_len : LR_MAX_N, LR_CLS);
      hipLaunchKernelGGL(topk_band_classify_kernel,
                         dim3((unsigned)(ncls * max_q_rows), (unsigned)B), dim3(TK_THREADS), 0, st,
                         scores, q_row_offsets, kv_row_offsets, score_ld, (int)ncls, lr);
      hipLaunchKernelGGL(topk_band_rescore_kernel,
                         dim3((unsigned)(static_cast<int64_t>(LR_RESCORE_X) * max_q_rows), (unsigned)B),
                         dim3(TK_THREADS), 0, st, scores, q_row_offsets, kv_row_offsets, score_ld,
                         max_q_rows, B, rf, lr);
      hipLaunchKernelGGL(topk_band_finish_kernel, grid, dim3(TK_THREADS), 0, st, scores,
                         q_row_offsets, kv_row_offsets, score_ld, k, topk, rf.status, lr);
    }
  } else {
    hipLaunchKernelGGL(topk_kernel, grid, dim3(TK_THREADS), 0, st, scores, score_ld, q_row_offsets,
                       kv_row_offsets, k, topk, rf);
  }
  return check_launch("dsa_topk");
}

namespace dsa {

int fused_sample_count(int64_t max_kv_len) {
  int64_t S = 1024;
  while (S < 8192 && S * 32 < max_kv_len) S *= 2;
  return static_cast<int>(S);
}

void launch_sample_tau(const float* samples, int S, const int32_t* q_off, const int64_t* kv_off,
                       int B, int max_q_rows, int k, float* tau, hipStream_t st) {
  hipLaunchKernelGGL(sample_tau_kernel, dim3((unsigned)max_q_rows, (unsigned)B), dim3(TK_THREADS), 0,
                     st, samples, S, q_off, kv_off, k, tau);
}

void launch_fused_select(const FusedSelectLaunch& a, const int32_t* q_off, const int64_t* kv_off,
                         int B, int max_q_rows, int k, int32_t* topk, hipStream_t st) {
  FusedSel fs;
  fs.cand = static_cast<uint2*>(a.cand);
  fs.ldc = a.ldc;
  fs.cnt = a.cnt;
  fs.msc = a.msc;
  fs.tau = a.tau;
  fs.path = a.path;
  fs.gx = a.gx;
  Refine rf{};
  rf.q_fp8 = a.q_fp8;
  rf.q_scale = a.q_scale;
  rf.w = a.w;
  rf.k_fp8 = a.k_fp8;
  rf.k_scale = a.k_scale;
  rf.kmax = nullptr;
  rf.status = a.status;
  rf.C = a.err_scale;
  rf.H = a.H;
  rf.D = a.D;
  rf.nsc = 0;
  rf.smax_given = 0.0f;
  hipLaunchKernelGGL(fused_select_kernel, dim3((unsigned)max_q_rows, (unsigned)B), dim3(TK_THREADS), 0,
                     st, fs, rf, q_off, kv_off, B, k, topk);
}

}  // namespace dsa
