// Shared device helpers for the gfx950 (CDNA4) attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// v_exp_f32 / v_log_f32: base-2 exponential and logarithm of the hardware.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// The value held by the lane 32 positions away (lane l reads lane l ^ 32).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

// Work-group id remapped so that consecutive logical ids land on the same XCD.  The dispatcher hands
// work-groups to the 8 XCDs round-robin; XCD x receives physical ids x, x+8, x+16, ...  This maps them
// to the contiguous logical range of that XCD, so tiles that share K/V also share one L2.
__device__ __forceinline__ int xcd_logical_id(int bid, int total) {
  constexpr int kXcd = 8;
  const int x = bid % kXcd, k = bid / kXcd;
  const int base = total / kXcd, rem = total % kXcd;
  return x * base + (x < rem ? x : rem) + k;
}

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void store16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

}  // namespace fa
