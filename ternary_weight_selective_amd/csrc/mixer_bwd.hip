// Element-wise pieces of the mixer backward (the chain itself is sequenced in api.cpp): the sum
// of the two gradients that reach the in_proj output (through the scan and through x_proj), the
// residual gradient, and the placement of dB and dC into the x_proj output's gradient.
#include "mixer_bwd.hpp"

namespace ssm {

namespace {
// a[i] += b[i], four elements per thread when aligned
__global__ __launch_bounds__(256) void k_add_f32(float* __restrict__ a, const float* __restrict__ b, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 3 < n) {
    float4 x = *(float4*)(a + i);
    const float4 y = *(const float4*)(b + i);
    x.x += y.x; x.y += y.y; x.z += y.z; x.w += y.w;
    *(float4*)(a + i) = x;
  } else {
    for (int64_t j = i; j < n; ++j) a[j] += b[j];
  }
}

// dst[r * ld_dst + c] = src[r * n + c] for c < n
__global__ __launch_bounds__(256) void k_copy_cols(const float* __restrict__ src, int64_t m, int64_t n,
                                                   float* __restrict__ dst, int64_t ld_dst) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= m * n) return;
  dst[(e / n) * ld_dst + e % n] = src[e];
}
}  // namespace

hipError_t launch_add_f32(float* a, const float* b, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (((uintptr_t)a | (uintptr_t)b) % 16 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_add_f32, dim3((unsigned)cdiv(cdiv(n, 4), 256)), dim3(256), 0, s, a, b, n);
  return hipGetLastError();
}

hipError_t launch_copy_cols(const float* src, int64_t m, int64_t n, float* dst, int64_t ld_dst, hipStream_t s) {
  if (m * n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_copy_cols, dim3((unsigned)cdiv(m * n, 256)), dim3(256), 0, s, src, m, n, dst, ld_dst);
  return hipGetLastError();
}

}  // namespace ssm
