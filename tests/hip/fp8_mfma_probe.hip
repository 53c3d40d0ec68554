// Test support (not part of the library): runs single FP8 matrix instructions
// (v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 x E4M3, unit scales) on given
// operands so a test can compare their sums with exact ones.  Lane l of the one
// wave holds 32 bytes of A (row l % 32, k = 32 (l / 32) + byte) and of B
// (column l % 32, same k), and 16 floats of C / D (row 8 (r / 4) + 4 (l / 32)
// + r % 4 of register r, column l % 32).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(64) void fp8_mfma_probe_kernel(const int* a, const int* b, const float* c, float* d) {
  const int l = threadIdx.x;
  const size_t i = blockIdx.x;
  v8i av, bv;
  for (int j = 0; j < 8; ++j) {
    av[j] = a[(i * 64 + l) * 8 + j];
    bv[j] = b[(i * 64 + l) * 8 + j];
  }
  f32x16 acc;
  for (int r = 0; r < 16; ++r) acc[r] = c[(i * 64 + l) * 16 + r];
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 0, 0, 0);
  for (int r = 0; r < 16; ++r) d[(i * 64 + l) * 16 + r] = acc[r];
}

// n independent instructions: a, b hold n * 2048 bytes, c and d n * 1024 floats (device pointers).
extern "C" int fp8_mfma_probe(const void* a, const void* b, const void* c, void* d, int n, void* stream) {
  if (n <= 0) return 0;
  fp8_mfma_probe_kernel<<<n, 64, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const int*>(a), static_cast<const int*>(b), static_cast<const float*>(c), static_cast<float*>(d));
  return (int)hipGetLastError();
}
