// LDS tile layouts and lane exchanges shared by the gather-attention kernels.
#pragma once

#include "absa_device.h"

namespace absa {

// LDS tiles hold 64 keys x D bf16 row-major, 16-byte chunks xor-swizzled by row.
// K tile: chunk c of row kk at c ^ (kk & 15) (D = 128) so that the 16 rows read
// by a quarter-wave (one 16-byte chunk each) hit distinct bank groups.
template <int D>
__device__ __forceinline__ int k_off(int kk, int c) {
  if constexpr (D == 128) return kk * 256 + ((c ^ (kk & 15)) << 4);
  else return kk * 128 + ((c ^ ((kk >> 1) & 7)) << 4);
}

// V tile: chunk c of row kk at c ^ 4 (kk & 3) (D = 128; D = 64: c ^ 4 ((kk >> 1) & 1)).
// V is read with ds_read_b64_tr_b16: a half-wave reads 4 consecutive rows x 64
// bytes (chunks 4 db .. 4 db + 3); the xor moves each row's four chunks to a
// different quarter of the banks (for D = 64, rows of equal parity share a bank
// half and the xor separates them).
template <int D>
__device__ __forceinline__ int v_off(int kk, int c) {
  if constexpr (D == 128) return kk * 256 + ((c ^ ((kk & 3) << 2)) << 4);
  else return kk * 128 + ((c ^ (((kk >> 1) & 1) << 2)) << 4);
}

// The chunk a lane fetches for row kk when a direct load writes LDS lane by
// lane: the swizzle is applied on the global side.
template <int D>
__device__ __forceinline__ int k_chunk(int kk, int cp) {
  return (D == 128) ? (cp ^ (kk & 15)) : (cp ^ ((kk >> 1) & 7));
}
template <int D>
__device__ __forceinline__ int v_chunk(int kk, int cp) {
  return (D == 128) ? (cp ^ ((kk & 3) << 2)) : (cp ^ (((kk >> 1) & 1) << 2));
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // a first-class vector, kept in VGPRs
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Lanes l and l + 32 hold the same query (different keys): v_permlane32_swap
// exchanges the two halves of a register, giving each lane its partner's value.
__device__ __forceinline__ float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace absa
