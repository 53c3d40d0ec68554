// Measurement support (not part of the library): issue rates of the units the
// gather-attention kernel leans on, per CU, on gfx950.  One workgroup of 8
// waves per CU (96 KB of LDS each, so no second workgroup fits); wave w and
// wave w + 4 share a SIMD.  Each wave runs `iters` iterations of one
// instruction mix, chosen per wave:
//   0  nothing (the wave waits at the end)
//   1  8 ds_read_b128 (16 B per lane) per iteration
//   2  8 ds_read_b64_tr_b16 (8 B per lane, transposing) per iteration
//   3  16 independent v_exp_f32 per iteration
//   4  16 independent v_fma_f32 per iteration
//   5  4 independent v_mfma_f32_32x32x16_bf16 per iteration
// and records the shader-clock counter (s_memtime) and the 100 MHz real-time
// counter (s_memrealtime) at the start and at the end of its loop, so that the
// span over the waves that share a unit gives rates per clock cycle whatever
// clock the chip runs at.  All LDS addresses stay inside the 96 KB
// array; nothing is written outside `cyc` and `sink`.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int LDS_BYTES = 96 * 1024;

__global__ __launch_bounds__(512, 1) void unit_rates_kernel(const int* modes, int iters, unsigned long long* cyc,
                                                            float* sink) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < LDS_BYTES / 4; i += 512) reinterpret_cast<uint32_t*>(lds)[i] = (uint32_t)i * 2654435761u;
  __syncthreads();
  const int mode = __builtin_amdgcn_readfirstlane(modes[w]);
  uint32_t xo = 0;
  float xf[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) xf[j] = -0.01f * (float)(j + 1) - 0.001f * (float)lane;
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  bf16x8 a, b;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    a[r] = (__bf16)(0.001f * (float)(lane + r));
    b[r] = (__bf16)(0.002f * (float)(lane - r));
  }
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  __builtin_amdgcn_sched_barrier(0);
  if (mode == 1) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // 16-byte lanes, 1 KB per wave-wide read, wrapping inside the first 64 KB
        const int off = (lane * 16 + ((it * 8 + j) & 63) * 1024) & 0xFFFF;
        const u32x4 v = *reinterpret_cast<const u32x4*>(lds + off);
        xo ^= v[0] ^ v[1] ^ v[2] ^ v[3];
      }
    }
  } else if (mode == 2) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // 8-byte aligned lane addresses, 512 B per wave-wide read, inside the first 64 KB
        const int off = (lane * 8 + ((it * 8 + j) & 127) * 512) & 0xFFFF;
        const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds + off));
        const uint2 u = __builtin_bit_cast(uint2, v);
        xo ^= u.x ^ u.y;
      }
    }
  } else if (mode == 3) {
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 16; ++j) xf[j] = __builtin_amdgcn_exp2f(xf[j]);
  } else if (mode == 4) {
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 16; ++j) xf[j] = __builtin_fmaf(xf[j], 0.999f, 0.001f);
  } else if (mode == 5) {
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  // the loop's results are complete before the clock is read again
  float s = (float)xo;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += xf[j];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_sched_barrier(0);
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  __builtin_amdgcn_sched_barrier(0);
  sink[(size_t)blockIdx.x * 512 + tid] = s;
  if (lane == 0) {
    unsigned long long* c = cyc + ((size_t)blockIdx.x * 8 + w) * 4;
    c[0] = t0;
    c[1] = t1;
    c[2] = r0;
    c[3] = r1;
  }
}

// modes: 8 ints (device), one per wave of a workgroup; cyc: nblocks * 32 uint64 (device), per
// wave the clock counter at the start and end of its loop, then the real-time counter at both;
// sink: nblocks * 512 floats (device).
extern "C" int unit_rates_probe(const void* modes, int iters, void* cyc, void* sink, int nblocks, void* stream) {
  if (nblocks <= 0 || iters <= 0) return 0;
  unit_rates_kernel<<<nblocks, 512, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const int*>(modes), iters, static_cast<unsigned long long*>(cyc), static_cast<float*>(sink));
  return (int)hipGetLastError();
}
