// Test support (not part of the library): v_exp_f32 (the selection kernels'
// 2^x) applied element by element, so a test can compare its values with exact
// powers of two.
#include <hip/hip_runtime.h>

__global__ __launch_bounds__(256) void exp2_probe_kernel(const float* x, float* y, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) y[i] = __builtin_amdgcn_exp2f(x[i]);
}

// y[i] = 2^x[i] for i < n (device pointers).
extern "C" int exp2_probe(const void* x, void* y, int n, void* stream) {
  if (n <= 0) return 0;
  exp2_probe_kernel<<<(n + 255) / 256, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const float*>(x), static_cast<float*>(y), n);
  return (int)hipGetLastError();
}
