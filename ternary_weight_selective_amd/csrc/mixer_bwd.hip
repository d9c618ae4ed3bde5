// Element-wise piece of the mixer backward (the chain itself is sequenced in api.cpp): the
// placement of dB and dC into the x_proj output's gradient.  The two sums of the chain (the
// gradients that reach the in_proj output through the scan and through x_proj, and the
// residual) are taken in the STE backward's epilogue (launch_ste_bwd_add).
#include "mixer_bwd.hpp"

namespace ssm {

namespace {
// dst[r * ld_dst + c] = src[r * n + c] for c < n
__global__ __launch_bounds__(256) void k_copy_cols(const float* __restrict__ src, int64_t m, int64_t n,
                                                   float* __restrict__ dst, int64_t ld_dst) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= m * n) return;
  dst[(e / n) * ld_dst + e % n] = src[e];
}
}  // namespace

hipError_t launch_copy_cols(const float* src, int64_t m, int64_t n, float* dst, int64_t ld_dst, hipStream_t s) {
  if (m * n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_copy_cols, dim3((unsigned)cdiv(m * n, 256)), dim3(256), 0, s, src, m, n, dst, ld_dst);
  return hipGetLastError();
}

}  // namespace ssm
