// fused.hpp -- launch helpers of the fused scoring and selection (dsa_index_topk), shared by
// index_score.hip (the entry point and the scoring launches) and topk.hip (the threshold and
// selection kernels). Internal to libdsa.so.
#pragma once

#include "common.hpp"

namespace dsa {

// Samples per request for the candidate threshold: about one key in 32 of the longest
// request, between 1024 and 8192.
int fused_sample_count(int64_t max_kv_len);

// tau[t]: the candidate threshold of every row from its sample scores samples[T, S].
void launch_sample_tau(const float* samples, int S, const int32_t* q_off, const int64_t* kv_off,
                       int B, int max_q_rows, int k, float* tau, hipStream_t st);

// Everything fused_select_kernel reads: the candidates of the compaction launch and the
// refine inputs.
struct FusedSelectLaunch {
  void* cand;          // uint2 [T, ldc]
  int64_t ldc;
  const int32_t* cnt;  // [T, gx, 2]
  const float* msc;    // [T, gx, 2]
  const float* tau;    // [T]
  int32_t* path;       // [T] or nullptr
  int gx;
  const uint8_t* q_fp8;
  const float* q_scale;
  const float* w;
  const uint8_t* k_fp8;
  const float* k_scale;
  int32_t* status;     // [T] or nullptr
  double err_scale;
  int H, D;
};

void launch_fused_select(const FusedSelectLaunch& a, const int32_t* q_off, const int64_t* kv_off,
                         int B, int max_q_rows, int k, int32_t* topk, hipStream_t st);

}  // namespace dsa
