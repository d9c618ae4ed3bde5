// Absmean ternarisation and 2-bit packing of latent weights (BitNet b1.58 absmean scale,
// cited by title in "Baseline Shape Decides the Verdict ...", Builds on; per-group scales
// and the zero ratio from the Ternary Mamba abstract).  Offline: runs once per weight.
#include "launch.hpp"

namespace ssm {

// One thread per row-group (or per row for a tensor scale): fp64 sum of |w| in ascending k.
__global__ void k_abs_partials(const float* __restrict__ w, int64_t n, int64_t k, int64_t glen,
                               int64_t ng, double* __restrict__ part) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n * ng) return;
  const float* p = w + (i / ng) * k + (i % ng) * glen;
  double s = 0.0;
  for (int64_t j = 0; j < glen; ++j) s += fabs((double)p[j]);
  part[i] = s;
}

// Tensor scale: the row sums are added in ascending row order by one thread.
__global__ void k_scale_tensor(const double* __restrict__ part, int64_t n, int64_t count,
                               float* __restrict__ scale) {
  if (blockIdx.x != 0 || threadIdx.x != 0) return;
  double s = 0.0;
  for (int64_t i = 0; i < n; ++i) s += part[i];
  scale[0] = (float)(s / (double)count);
}

__global__ void k_scale_groups(const double* __restrict__ part, int64_t cnt, int64_t glen,
                               float* __restrict__ scale) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < cnt) scale[i] = (float)(part[i] / (double)glen);
}

__global__ void k_copy_f32(const float* __restrict__ src, int64_t cnt, float* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < cnt) dst[i] = src[i];
}

__global__ void k_zero_i64(int64_t* p) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *p = 0;
}

// One thread per packed word (16 weights of a row).  code = clamp(rint(w / g), -1, 1) with
// g = max(gamma, 1e-5) and an IEEE division; weight i = 4j + p of the word goes to byte p,
// bits 2j.  Zero codes are counted per wave and added with one integer atomic per wave.
__global__ __launch_bounds__(256) void k_pack(const float* __restrict__ w, int64_t n, int64_t k,
                                              int64_t group, const float* __restrict__ scale,
                                              uint32_t* __restrict__ packed, int64_t rw,
                                              int64_t* __restrict__ zero_count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int zeros = 0;
  if (i < n * rw) {
    const int64_t row = i / rw, wd = i % rw;
    const int64_t ng = group ? k / group : 1;
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t c = wd * 16 + e;
      if (c < k) {
        const float gamma = group ? scale[row * ng + c / group] : scale[0];
        const float g = fmaxf(gamma, 1e-5f);
        const float r = rintf(__fdiv_rn(w[row * k + c], g));
        const uint32_t code = r >= 1.0f ? 1u : (r <= -1.0f ? 3u : 0u);
        zeros += (code == 0u);
        word |= code << (8 * (e & 3) + 2 * (e >> 2));
      }
    }
    packed[i] = word;
  }
  if (zero_count) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) zeros += __shfl_xor(zeros, d, 64);
    if ((threadIdx.x & 63) == 0 && zeros) atomicAdd((unsigned long long*)zero_count, (unsigned long long)zeros);
  }
}

hipError_t launch_abs_partials(const float* w, int64_t n, int64_t k, int64_t group, double* part,
                               hipStream_t s) {
  const int64_t ng = group ? k / group : 1, glen = group ? group : k;
  const int64_t cnt = n * ng;
  hipLaunchKernelGGL(k_abs_partials, dim3((unsigned)cdiv(cnt, 256)), dim3(256), 0, s, w, n, k, glen, ng, part);
  return hipGetLastError();
}

hipError_t launch_scales(const double* part, int64_t n, int64_t k, int64_t group, const float* scale_in,
                         float* scale, hipStream_t s) {
  const int64_t cnt = group ? n * (k / group) : 1;
  if (scale_in) {
    hipLaunchKernelGGL(k_copy_f32, dim3((unsigned)cdiv(cnt, 256)), dim3(256), 0, s, scale_in, cnt, scale);
  } else if (group == 0) {
    hipLaunchKernelGGL(k_scale_tensor, dim3(1), dim3(64), 0, s, part, n, n * k, scale);
  } else {
    hipLaunchKernelGGL(k_scale_groups, dim3((unsigned)cdiv(cnt, 256)), dim3(256), 0, s, part, cnt, group, scale);
  }
  return hipGetLastError();
}

hipError_t launch_pack(const float* w, int64_t n, int64_t k, int64_t group, const float* scale,
                       uint32_t* packed, int64_t* zero_count, hipStream_t s) {
  const int64_t rw = cdiv(k, 16);
  if (zero_count) hipLaunchKernelGGL(k_zero_i64, dim3(1), dim3(64), 0, s, zero_count);
  hipLaunchKernelGGL(k_pack, dim3((unsigned)cdiv(n * rw, 256)), dim3(256), 0, s, w, n, k, group, scale, packed,
                     rw, zero_count);
  return hipGetLastError();
}

}  // namespace ssm
