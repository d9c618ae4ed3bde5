// Device helpers shared by the gfx950 kernels of the ternary selective-SSM library.
// Compiled with -ffp-contract=off: every fused multiply-add below is written out.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

typedef uint16_t bf16_t;  // bf16 bit pattern as stored in memory

__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// round to nearest, ties to even (inputs are finite)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ float ld_act(const T* p);
template <> __device__ __forceinline__ float ld_act<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld_act<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }

template <typename T> __device__ __forceinline__ void st_act(T* p, float v);
template <> __device__ __forceinline__ void st_act<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void st_act<bf16_t>(bf16_t* p, float v) { *p = f32_to_bf16(v); }

// Sum over the 64 lanes of a wave as six rounds in which lane j adds lane j ^ d,
// d = 32, 16, 8, 4, 2, 1.  fp32 addition is commutative, so every lane ends with the
// same value and the order of the additions is fixed.
__device__ __forceinline__ float wave_sum_butterfly(float s) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) s = s + __shfl_xor(s, d, 64);
  return s;
}

__device__ __forceinline__ float wave_max(float m) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
  return m;
}

// 16 ternary codes of one packed word -> 16 int8 in weight order.  Dword j of the
// result holds weights 4j..4j+3; their 2-bit codes sit at bits 2j of bytes 0..3, so a
// shift and mask leave one code per byte and a byte permute maps code 0/1/3 to
// 0x00/0x01/0xFF through the table 0xFF000100.
__device__ __forceinline__ v4i unpack16_i8(uint32_t w) {
  v4i r;
  r[0] = (int)__builtin_amdgcn_perm(0u, 0xFF000100u, w & 0x03030303u);
  r[1] = (int)__builtin_amdgcn_perm(0u, 0xFF000100u, (w >> 2) & 0x03030303u);
  r[2] = (int)__builtin_amdgcn_perm(0u, 0xFF000100u, (w >> 4) & 0x03030303u);
  r[3] = (int)__builtin_amdgcn_perm(0u, 0xFF000100u, (w >> 6) & 0x03030303u);
  return r;
}

// Two int8 ternary values (low two bytes of b) -> two bf16 (+1 = 0x3F80, -1 = 0xBF80, 0 = 0).
__device__ __forceinline__ uint32_t tern2_to_bf16x2(uint32_t b) {
  uint32_t lo = b & 0xFFu, hi = (b >> 8) & 0xFFu;
  uint32_t vlo = lo ? (0x3F80u | ((lo & 0x80u) << 8)) : 0u;
  uint32_t vhi = hi ? (0x3F80u | ((hi & 0x80u) << 8)) : 0u;
  return vlo | (vhi << 16);
}

// Correctly rounded fp32 square root.  The device's fp32 sqrt instruction sequence is not
// correctly rounded (it is off by one ulp on some inputs); a correctly rounded fp64 square
// root rounded once to fp32 is, because 53 >= 2 * 24 + 2 bits make the double rounding
// innocuous for square roots.
__device__ __forceinline__ float sqrt_rn(float x) { return (float)__dsqrt_rn((double)x); }

__host__ __device__ constexpr int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ constexpr int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

}  // namespace ssm
