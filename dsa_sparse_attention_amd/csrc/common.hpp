// common.hpp -- shared host/device helpers of libdsa.so (HIP, gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

// ---- host-side error reporting (thread-local message, see dsa_last_error) ----
dsa_status fail(dsa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
dsa_status ok();
// Turns the launch error state into a status (no synchronisation).
dsa_status check_launch(const char* what);

#define DSA_REQUIRE(cond, ...)                                                   \
  do {                                                                           \
    if (!(cond)) return ::dsa::fail(DSA_ERR_INVALID_ARGUMENT, __VA_ARGS__);      \
  } while (0)

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---- device helpers ----
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float32 -> bfloat16 bits, round-to-nearest-even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return static_cast<uint16_t>(u >> 16);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// 16-byte LDS DMA (global_load_lds_dwordx4): lane l copies 16 bytes from `gsrc` to
// LDS byte lds_base + 16*l; lds_base must be wave-uniform. Issued from inline asm
// so the compiler keeps no wait bookkeeping of its own for it (it would otherwise
// wait for every pending DMA before any LDS read it cannot prove disjoint): the
// caller retires these loads itself with s_waitcnt vmcnt and a barrier before
// reading the data. Loads retire in order, so the compiler's own vmcnt waits for
// its loads stay correct (only stricter) while such DMAs are in flight. The
// instruction's offset field is not used: it would move the LDS destination too.
__device__ __forceinline__ void lds_dma16(const void* gsrc, const lds_void* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_base)));
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "s"(m0)
               : "memory");
}

// 4-byte LDS DMA (global_load_lds_dword): lane l copies 4 bytes from `gsrc` to LDS byte
// lds_base + 4*l; same rules as lds_dma16.
__device__ __forceinline__ void lds_dma4(const void* gsrc, const lds_void* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_base)));
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(gsrc), "s"(m0)
               : "memory");
}

// s_waitcnt vmcnt(n) (expcnt and lgkmcnt left alone), constant n <= 63: vmcnt is
// split over bits 3:0 and 15:14 of the immediate.
#define DSA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))

// Row bookkeeping of the ragged verify batch: request b, row r of R_b rows,
// L_b cached positions; the row sits at position L_b - R_b + r.
struct RowInfo {
  int64_t kv_base;  // kv_row_offsets[b]
  int64_t L;        // cached positions of the request
  int32_t R;        // verify rows of the request
  int32_t t0;       // first query row of the request
};

__device__ __forceinline__ RowInfo load_row_info(const int32_t* q_off, const int64_t* kv_off,
                                                 int b) {
  RowInfo ri;
  ri.t0 = q_off[b];
  ri.R = q_off[b + 1] - ri.t0;
  ri.kv_base = kv_off[b];
  ri.L = kv_off[b + 1] - ri.kv_base;
  return ri;
}

// Number of positions row r may see (p + 1, clamped to [0, L]).
__device__ __forceinline__ int64_t visible_count(const RowInfo& ri, int r) {
  int64_t v = ri.L - ri.R + r + 1;
  return v < 0 ? 0 : (v > ri.L ? ri.L : v);
}

}  // namespace dsa
