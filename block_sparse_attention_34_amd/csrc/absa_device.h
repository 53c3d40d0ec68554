// Device helpers shared by the gfx950 kernels: bf16 conversion, wave/block
// reductions, and a Philox4x32-10 generator written from its definition in
// Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
// (SC'11).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace absa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Four bf16 values packed in two dwords -> four floats.
__device__ __forceinline__ void unpack_bf16x2(uint32_t w, float& lo, float& hi) {
  lo = __uint_as_float(w << 16);
  hi = __uint_as_float(w & 0xFFFF0000u);
}

// ----------------------------------------------------------------------------- scalar pointers
// A wave-uniform pointer rebuilt from the first lane's two 32-bit halves, for
// buffer resources (which live in scalar registers).  The halves are taken as
// unsigned: readfirstlane returns int, and a sign-extended low half would fill
// the high half with ones whenever bit 31 of the address is set.
__device__ __forceinline__ void* uniform_ptr(const void* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a))));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a >> 32))));
  return reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// ----------------------------------------------------------------------------- Philox4x32-10
// One round: the two 32x32->64 products of words 0 and 2 with the round
// multipliers feed a xor with words 1/3 and the round key; the key advances by
// the two Weyl increments between rounds.
struct philox_u4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ philox_u4 philox4x32_10(philox_u4 c, uint32_t k0, uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    // (one 32 x 32 -> 64-bit product each: a single v_mad_u64_u32)
    const uint64_t p0 = (uint64_t)M0 * c.x, p1 = (uint64_t)M1 * c.z;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    philox_u4 n;
    n.x = hi1 ^ c.y ^ k0;
    n.y = lo1;
    n.z = hi0 ^ c.w ^ k1;
    n.w = lo0;
    c = n;
    k0 += W0;
    k1 += W1;
  }
  return c;
}

// ----------------------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Block-wide reductions for NT threads (NT a multiple of 64, <= 1024).  `red`
// is LDS scratch of at least NT/64 entries; ends with all threads holding the
// result.  Fixed combination order, so results are deterministic.
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) t += red[w];
  return t;
}

template <int NT>
__device__ __forceinline__ int block_sum_i(int v, int* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  v = wave_sum_i(v);
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) t += red[w];
  return t;
}

// Wave totals through DPP: pairwise within quads, then rotations within each
// 16-lane row, then the four row sums read in lane order.  Every lane returns
// the same value, and it does not depend on lane timing (only lanes 0, 16, 32
// and 48 are read after the rotations).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float wave_total(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x124>(v);  // row_ror:4
  v += dpp_f<0x128>(v);  // row_ror:8
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ int wave_total_i(int v) {
  v += __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);
  v += __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);
  v += __builtin_amdgcn_mov_dpp(v, 0x124, 0xF, 0xF, true);
  v += __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, true);
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}

// Block totals of a float and an int together, one barrier: `redf`/`redi` hold
// two buffers of NT/64 entries used alternately (`parity`), so a buffer is only
// rewritten after every thread has passed the barrier that follows its last read.
template <int NT>
__device__ __forceinline__ void block_total2(float& fv, int& iv, float* redf, int* redi, int parity) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  fv = wave_total(fv);
  iv = wave_total_i(iv);
  float* rf = redf + parity * (NT / 64);
  int* ri = redi + parity * (NT / 64);
  if (lane == 0) {
    rf[wid] = fv;
    ri[wid] = iv;
  }
  __syncthreads();
  float t = 0.f;
  int c = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    t += rf[w];
    c += ri[w];
  }
  fv = t;
  iv = c;
}

// Exclusive prefix sum in thread order and the total.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* red, int& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan(v, lane);
  __syncthreads();
  if (lane == 63) red[wid] = inc;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int x = red[w];
    before += (w < wid) ? x : 0;
    tot += x;
  }
  total = tot;
  return before + inc - v;
}

}  // namespace absa
