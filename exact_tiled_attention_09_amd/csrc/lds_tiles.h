// Helpers shared by the gfx950 kernels that stream K / V (or Q / dO) tiles through LDS and read MFMA
// fragments from them: row swizzles, buffer-resource loads straight into LDS, transposing LDS reads and
// the half-wave pair reductions of the 32x32 MFMA output layout.
#pragma once

#include "common.h"

namespace fa {

// 16-byte-chunk XOR swizzles within a row, chosen so that the fragment reads below hit distinct banks:
//  K (16 lanes read 16 rows at one logical chunk): spread the rows over all chunk positions;
//  V (ds_read_b64_tr_b16: 32 lanes read 4 rows x 4 chunks): spread the 4 rows by chunk xor 4k.
template <int D>
__device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

// Buffer resource over `bytes` bytes at `base` (raw buffer: stride 0, byte offsets).  Loads at offsets
// at or past `bytes` return zeros instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
// 16 bytes per lane from rsrc + voff into LDS: the wave's 64 x 16 bytes land contiguously at lds_block.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, int voff, void* lds_block) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_block, 16, voff, 0, 0, 0);
}

// The same with the non-temporal cache policy, for data that is read exactly once.
__device__ __forceinline__ void load_lds16_nt(__amdgpu_buffer_rsrc_t r, int voff, void* lds_block) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_block, 16, voff, 0, 0, 2);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}

// max / sum of x over lanes l and l^32 (v_permlane32_swap exchanges the two half-waves).
__device__ __forceinline__ float pair_max(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

}  // namespace fa
